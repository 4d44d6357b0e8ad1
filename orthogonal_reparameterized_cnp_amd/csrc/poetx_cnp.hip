// Cayley-Neumann blocks: build G - I from packed skew parameters, and the
// chain rule from block gradients dG back to the packed parameters.
//
// Build (POET-X blog on zhichai.net, 第四斧: Q^2 once, Q^3 and Q^4 from it):
//   S = Q^2, N = 2Q + S,  G - I = 2Q + 2S + S N  (= 2Q + 2Q^2 + 2Q^3 + Q^4).
// Chain rule of G = I + 2(Q + Q^2 + Q^3) + Q^4 with Q^T = -Q, grouped by powers
// of Q on the left: with U = dL/dG (the block gradient, summed over tokens
// here too), V1 = U Q, V2 = V1 Q, V3 = V2 Q,
//   dQ = X0 + Q (X1 + Q (X2 + Q X3)),
//   X0 = 2U - 2V1 + 2V2 - V3, X1 = -2U + 2V1 - V2, X2 = 2U - V1, X3 = -U,
// then dq[p(i,j)] = dQ[i][j] - dQ[j][i] on the packed slots.
//
// Q is unpacked once into a dense block buffer; every product reads plain
// row-major operands.  Products with Q on the right load Q's rows as the B
// operand, which yields X Q^T = -X Q (the sign is folded into the epilogue);
// products with a non-symmetric matrix on the right read the transpose that
// the producing epilogue wrote.
#include "kernel_util.h"

using namespace px;

namespace {

// Up to two sides of one linear share a launch: block z < nb0 belongs to side 0.
struct Sides {
  const float* q[2];
  int d[2];
  int nb0;
  PX_DEV void at(int z, int b, const float*& qk, int& r) const {
    const int s = z >= nb0;
    const int blk = z - s * nb0;
    r = min(b, d[s] - blk * b);
    qk = q[s] + (int64_t)blk * ((int64_t)b * (b - 1) / 2);
  }
};

template <typename T>
__global__ void k_unpack_q(Sides sd, int b, T* __restrict__ Qb) {
  const int z = blockIdx.y;
  const float* qk;
  int r;
  sd.at(z, b, qk, r);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)b * b) return;
  const int i = (int)(e / b), j = (int)(e % b);
  Qb[(int64_t)z * b * b + e] = from_f32<T>(skew_at(qk, i, j, r, b));
}

// S = Q Q = -(Q Q^T); writes S (fp32 and operand dtype) and N^T = S - 2Q.
template <class C, typename T>
__global__ __launch_bounds__(C::NT) void k_cnp_square(Sides sd, int b, const T* __restrict__ Qb,
                                                      float* __restrict__ S32, T* __restrict__ Sb,
                                                      T* __restrict__ Ntb) {
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);
  const int z = blockIdx.z;
  const float* qk;
  int r;
  sd.at(z, b, qk, r);
  const int m0 = blockIdx.y * C::BM, n0 = blockIdx.x * C::BN;
  if (m0 >= r || n0 >= r) return;  // nothing outside the live corner is read later
  const int64_t off = (int64_t)z * b * b;
  LoadK<C::BM, C::BK, C::NT, T, T> la;
  la.init(Qb + off + (int64_t)m0 * b, b, r - m0, r);
  LoadK<C::BN, C::BK, C::NT, T, T> lb;
  lb.init(Qb + off + (int64_t)n0 * b, b, r - n0, r);
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, T>(lds, la, lb, r, acc, p.wm, p.wn, p.lane);
  each_acc<C>(acc, [&](int i, int j, float v) {
    i += m0;
    j += n0;
    if (i < r && j < r) {
      const int64_t e = off + (int64_t)i * b + j;
      const float s = -v;
      S32[e] = s;
      Sb[e] = from_f32<T>(s);
      Ntb[e] = from_f32<T>(s - 2.f * skew_at(qk, i, j, r, b));
    }
  });
}

// G - I = 2Q + 2S + S N, written as slice 0 (row-major) and slice 1 (transposed)
template <class C, typename T>
__global__ __launch_bounds__(C::NT) void k_cnp_delta(Sides sd, int b, int nb_all, const float* __restrict__ S32,
                                                     const T* __restrict__ Sb, const T* __restrict__ Ntb,
                                                     T* __restrict__ g) {
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);
  const int z = blockIdx.z;
  const float* qk;
  int r;
  sd.at(z, b, qk, r);
  const int m0 = blockIdx.y * C::BM, n0 = blockIdx.x * C::BN;
  const int64_t off = (int64_t)z * b * b;
  LoadK<C::BM, C::BK, C::NT, T, T> la;
  la.init(Sb + off + (int64_t)m0 * b, b, r - m0, r);
  LoadK<C::BN, C::BK, C::NT, T, T> lb;
  lb.init(Ntb + off + (int64_t)n0 * b, b, r - n0, r);
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, T>(lds, la, lb, r, acc, p.wm, p.wn, p.lane);
  T* g0 = g + off;
  T* g1 = g + (int64_t)nb_all * b * b + off;
  each_acc4<C>(acc, [&](int i0, int j, const float* v) {
    i0 += m0;
    j += n0;
    if (j >= b || i0 >= b) return;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + e;
      o[e] = (i < r && j < r) ? v[e] + 2.f * skew_at(qk, i, j, r, b) + 2.f * S32[off + (int64_t)i * b + j] : 0.f;
      if (i < b) g0[(int64_t)i * b + j] = from_f32<T>(o[e]);
    }
    if (i0 + 4 <= b)
      store4<T>(g1 + (int64_t)j * b + i0, o);
    else
      for (int e = 0; e < 4 && i0 + e < b; ++e) g1[(int64_t)j * b + i0 + e] = from_f32<T>(o[e]);
  });
}

// Block gradients U = dL/dG summed over all tokens, both sides in one launch:
// side s, block blk: U[i][j] = sum_t A_s[t][kb + i] * B_s[t][kb + j] (R side:
// A = Xt, B = dA; P side: A = H, B = dZt).  Each workgroup owns one output
// tile and runs the whole token range, so the sum order is fixed.  Written as
// fp32, operand dtype and operand-dtype transpose, the forms the chain reads.
template <typename T> struct GradSides {
  const T* A[2];
  const T* B[2];
  int64_t lda[2], ldb[2];
};

template <typename T> struct Chain {
  const T* Qb;
  float* U32;
  T* Ub;
  T* Utb;
  float* V1_32;
  T* V1b;
  float* P2_32;  // Q U
  float* V2_32;
  T* V2b;
  float* V3_32;
  T* Y1tb;
  T* Y2tb;
  float* dQ32;
};

template <class C, typename T>
__global__ __launch_bounds__(C::NT) void k_block_grads(Sides sd, GradSides<T> gs, int rows, int b, Chain<T> ch) {
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);
  const int z = blockIdx.y;
  const int s = z >= sd.nb0;
  const int blk = z - s * sd.nb0;
  const int kb = blk * b, r = min(b, sd.d[s] - kb);
  const int tiles_n = (b + C::BN - 1) / C::BN;
  const int m0 = (blockIdx.x / tiles_n) * C::BM, n0 = (blockIdx.x % tiles_n) * C::BN;
  if (m0 >= r || n0 >= r) return;  // only the live corner is read later
  LoadMN<C::BM, C::BK, C::NT, T, T> la;
  la.init(gs.A[s] + kb + m0, gs.lda[s], r - m0, rows);
  LoadMN<C::BN, C::BK, C::NT, T, T> lb;
  lb.init(gs.B[s] + kb + n0, gs.ldb[s], r - n0, rows);
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, T>(lds, la, lb, rows, acc, p.wm, p.wn, p.lane);
  const int64_t off = (int64_t)z * b * b;
  each_acc4<C>(acc, [&](int i0, int j, const float* v) {
    i0 += m0;
    j += n0;
    if (j >= r || i0 >= r) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e >= r) continue;
      const int64_t x = off + (int64_t)(i0 + e) * b + j;
      ch.U32[x] = v[e];
      ch.Ub[x] = from_f32<T>(v[e]);
    }
    T* dst = ch.Utb + off + (int64_t)j * b + i0;
    if (i0 + 4 <= r)
      store4<T>(dst, v);
    else
      for (int e = 0; e < 4 && i0 + e < r; ++e) dst[e] = from_f32<T>(v[e]);
  });
}

// Chain rule in four launches (see the file header for V1..V3, X0..X3):
//   step 1: V1 = U Q            and  P2 = Q U          (2 NB blocks of work)
//   step 2: V2 = V1 Q           with Y1 = 2U - V1 - P2 written transposed
//   step 3: V3 = V2 Q           and  Y2 = -2U + 2V1 - V2 + Q Y1 (transposed)
//   step 4: dQ = 2U - 2V1 + 2V2 - V3 + Q Y2
// Products X Q load Q's rows as the B operand and negate (X Q^T = -X Q).
template <class C, typename T, int STEP>
__global__ __launch_bounds__(C::NT) void k_cnp_chain(Sides sd, int b, int NB, Chain<T> ch) {
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);
  const bool second = (STEP == 1 || STEP == 3) && (int)blockIdx.z >= NB;
  const int z = blockIdx.z - (second ? NB : 0);
  const float* qk;
  int r;
  sd.at(z, b, qk, r);
  const int m0 = blockIdx.y * C::BM, n0 = blockIdx.x * C::BN;
  if (m0 >= r || n0 >= r) return;  // later steps and the packing read only the live corner
  const int64_t off = (int64_t)z * b * b;
  // right-multiplication by Q (first products of steps 1-3) or left-multiplication (the rest)
  const bool right = (STEP <= 3) && !second;
  LoadK<C::BM, C::BK, C::NT, T, T> la;
  LoadK<C::BN, C::BK, C::NT, T, T> lb;
  if (right) {
    const T* src = STEP == 1 ? ch.Ub : STEP == 2 ? ch.V1b : ch.V2b;
    la.init(src + off + (int64_t)m0 * b, b, r - m0, r);
    lb.init(ch.Qb + off + (int64_t)n0 * b, b, r - n0, r);
  } else {
    const T* srcT = STEP == 1 ? ch.Utb : STEP == 3 ? ch.Y1tb : ch.Y2tb;
    la.init(ch.Qb + off + (int64_t)m0 * b, b, r - m0, r);
    lb.init(srcT + off + (int64_t)n0 * b, b, r - n0, r);
  }
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, T>(lds, la, lb, r, acc, p.wm, p.wn, p.lane);
  each_acc4<C>(acc, [&](int i0, int j, const float* v) {
    i0 += m0;
    j += n0;
    if (j >= r || i0 >= r) return;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e >= r) continue;
      const int64_t x = off + (int64_t)(i0 + e) * b + j;
      if (right) {
        const float val = -v[e];
        if (STEP == 1) {
          ch.V1_32[x] = val;
          ch.V1b[x] = from_f32<T>(val);
        } else if (STEP == 2) {
          ch.V2_32[x] = val;
          ch.V2b[x] = from_f32<T>(val);
          o[e] = 2.f * ch.U32[x] - ch.V1_32[x] - ch.P2_32[x];  // Y1
        } else {
          ch.V3_32[x] = val;
        }
      } else if (STEP == 1) {
        ch.P2_32[x] = v[e];
      } else if (STEP == 3) {
        o[e] = -2.f * ch.U32[x] + 2.f * ch.V1_32[x] - ch.V2_32[x] + v[e];  // Y2
      } else {
        ch.dQ32[x] = 2.f * ch.U32[x] - 2.f * ch.V1_32[x] + 2.f * ch.V2_32[x] - ch.V3_32[x] + v[e];
      }
    }
    const bool wr = (STEP == 2 && right) || (STEP == 3 && !right);
    if (wr) {
      T* dst = (STEP == 2 ? ch.Y1tb : ch.Y2tb) + off + (int64_t)j * b + i0;
      if (i0 + 4 <= r)
        store4<T>(dst, o);
      else
        for (int e = 0; e < 4 && i0 + e < r; ++e) dst[e] = from_f32<T>(o[e]);
    }
  });
}

struct DqOut {
  float* dq[2];
};

__global__ void k_pack_dq(Sides sd, int b, const float* __restrict__ dQ32, DqOut out) {
  const int z = blockIdx.y;
  const int s = z >= sd.nb0;
  const int blk = z - s * sd.nb0;
  const int r = min(b, sd.d[s] - blk * b);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)b * b) return;
  const int i = (int)(e / b), j = (int)(e % b);
  if (i >= j) return;
  const float* Qb = dQ32 + (int64_t)z * b * b;
  const float v = (j < r) ? Qb[(int64_t)i * b + j] - Qb[(int64_t)j * b + i] : 0.f;
  out.dq[s][(int64_t)blk * ((int64_t)b * (b - 1) / 2) + packed_slot(i, j, b)] = v;
}

template <typename T> struct CnpTile;
template <> struct CnpTile<bf16_t> { using C = TSq; };
template <> struct CnpTile<float> { using C = TF; };

inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

template <typename T>
hipError_t build_t(const float* q, int d, int b, T* g, void* ws, hipStream_t s) {
  using C = typename CnpTile<T>::C;
  const int nb = pxk::nblocks(d, b);
  const size_t E = (size_t)nb * b * b;
  char* w = reinterpret_cast<char*>(ws);
  T* Qb = reinterpret_cast<T*>(w);
  w += al256(E * sizeof(T));
  float* S32 = reinterpret_cast<float*>(w);
  w += al256(E * 4);
  T* Sb = reinterpret_cast<T*>(w);
  w += al256(E * sizeof(T));
  T* Ntb = reinterpret_cast<T*>(w);
  Sides sd{{q, q}, {d, d}, nb};
  const int lds = Lay<C, T>::BYTES;
  hipError_t e = allow_lds(k_cnp_square<C, T>, lds);
  if (e == hipSuccess) e = allow_lds(k_cnp_delta<C, T>, lds);
  if (e != hipSuccess) return e;
  k_unpack_q<T><<<dim3(cdiv((int64_t)b * b, 256), nb), 256, 0, s>>>(sd, b, Qb);
  dim3 grid(cdiv(b, C::BN), cdiv(b, C::BM), nb);
  k_cnp_square<C, T><<<grid, C::NT, lds, s>>>(sd, b, Qb, S32, Sb, Ntb);
  k_cnp_delta<C, T><<<grid, C::NT, lds, s>>>(sd, b, nb, S32, Sb, Ntb, g);
  return hipGetLastError();
}

template <typename T> Chain<T> carve(void* ws, size_t E) {
  char* w = reinterpret_cast<char*>(ws);
  auto takeT = [&]() {
    T* p = reinterpret_cast<T*>(w);
    w += al256(E * sizeof(T));
    return p;
  };
  auto takeF = [&]() {
    float* p = reinterpret_cast<float*>(w);
    w += al256(E * 4);
    return p;
  };
  Chain<T> ch;
  ch.Qb = takeT();
  ch.U32 = takeF();
  ch.Ub = takeT();
  ch.Utb = takeT();
  ch.V1_32 = takeF();
  ch.V1b = takeT();
  ch.P2_32 = takeF();
  ch.V2_32 = takeF();
  ch.V2b = takeT();
  ch.V3_32 = takeF();
  ch.Y1tb = takeT();
  ch.Y2tb = takeT();
  ch.dQ32 = takeF();
  return ch;
}

template <typename T>
hipError_t grads_t(const pxk::CnpSide* sides, int rows, int b, void* ws, hipStream_t s) {
  using C = typename CnpTile<T>::C;
  const int nb0 = pxk::nblocks(sides[0].d, b), nb1 = pxk::nblocks(sides[1].d, b);
  const int NB = nb0 + nb1;
  Chain<T> ch = carve<T>(ws, (size_t)NB * b * b);
  Sides sd{{sides[0].q, sides[1].q}, {sides[0].d, sides[1].d}, nb0};
  GradSides<T> gs;
  for (int k = 0; k < 2; ++k) {
    gs.A[k] = reinterpret_cast<const T*>(sides[k].A);
    gs.B[k] = reinterpret_cast<const T*>(sides[k].B);
    gs.lda[k] = sides[k].lda;
    gs.ldb[k] = sides[k].ldb;
  }
  k_unpack_q<T><<<dim3(cdiv((int64_t)b * b, 256), NB), 256, 0, s>>>(sd, b, const_cast<T*>(ch.Qb));
  const int lds = smem_bytes<C, T, T>();
  hipError_t e = allow_lds(k_block_grads<C, T>, lds);
  if (e != hipSuccess) return e;
  dim3 grid(cdiv(b, C::BM) * cdiv(b, C::BN), NB);
  k_block_grads<C, T><<<grid, C::NT, lds, s>>>(sd, gs, rows, b, ch);
  return hipGetLastError();
}

template <typename T>
hipError_t chain_t(const pxk::CnpSide* sides, int b, void* ws, hipStream_t s) {
  using C = typename CnpTile<T>::C;
  const int nb0 = pxk::nblocks(sides[0].d, b), nb1 = pxk::nblocks(sides[1].d, b);
  const int NB = nb0 + nb1;
  Chain<T> ch = carve<T>(ws, (size_t)NB * b * b);
  Sides sd{{sides[0].q, sides[1].q}, {sides[0].d, sides[1].d}, nb0};
  DqOut out{{sides[0].dq, sides[1].dq}};
  const int lds = smem_bytes<C, T, T>();
  hipError_t e = hipSuccess;
#define PX_CHAIN(K, MULT)                                                                  \
  e = allow_lds(k_cnp_chain<C, T, K>, lds);                                                 \
  if (e != hipSuccess) return e;                                                            \
  k_cnp_chain<C, T, K><<<dim3(cdiv(b, C::BN), cdiv(b, C::BM), (MULT) * NB), C::NT, lds, s>>>(sd, b, NB, ch);
  PX_CHAIN(1, 2)
  PX_CHAIN(2, 1)
  PX_CHAIN(3, 2)
  PX_CHAIN(4, 1)
#undef PX_CHAIN
  k_pack_dq<<<dim3(cdiv((int64_t)b * b, 256), NB), 256, 0, s>>>(sd, b, ch.dQ32, out);
  return hipGetLastError();
}

}  // namespace

namespace pxk {

size_t cnp_build_ws_bytes(int dt, int d, int b) {
  const size_t E = (size_t)nblocks(d, b) * b * b, es = dt_size(dt);
  return al256(E * es) * 3 + al256(E * 4);
}

size_t cnp_backward_ws_bytes(int dt, int d0, int d1, int b) {
  const size_t E = (size_t)(nblocks(d0, b) + nblocks(d1, b)) * b * b, es = dt_size(dt);
  return al256(E * es) * 7 + al256(E * 4) * 6;
}

hipError_t cnp_build(int dt, const float* q, int d, int b, void* g, void* ws, hipStream_t s) {
  if (dt == BF16) return build_t<bf16_t>(q, d, b, reinterpret_cast<bf16_t*>(g), ws, s);
  return build_t<float>(q, d, b, reinterpret_cast<float*>(g), ws, s);
}

hipError_t block_grads(int cdt, const CnpSide* sides, int rows, int b, void* ws, hipStream_t s) {
  if (cdt == BF16) return grads_t<bf16_t>(sides, rows, b, ws, s);
  return grads_t<float>(sides, rows, b, ws, s);
}

hipError_t cnp_chain(int cdt, const CnpSide* sides, int b, void* ws, hipStream_t s) {
  if (cdt == BF16) return chain_t<bf16_t>(sides, b, ws, s);
  return chain_t<float>(sides, b, ws, s);
}

}  // namespace pxk
