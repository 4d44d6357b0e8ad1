// HIP kernels of libpoetx for gfx950 and their typed launchers.
//
// Every dense contraction of the layer (CNP block squares, block-diagonal
// products, the W~ contractions, the block gradients and the CNP chain rule)
// is an instance of the LDS-staged MFMA tile loop in mfma_tile.h with a
// suitable pair of operand loaders and an epilogue.  Permutations are index
// arrays applied by row-staged gathers through LDS.
#include "kernel_util.h"

using namespace px;

namespace {

// ============================================================================
// block-diagonal product over token rows, identity added in fp32:
//   out[t][kb+j] = (in[t][kb+j] + sum_k in[t][kb+k] dT[blk][j][k]) * scale[kb+j]
// ============================================================================
// The identity term is added from the A tile in LDS: the block's output column
// c equals K index c, so during the K tile that holds columns [k0, k0 + BK)
// each wave adds A[row][c - k0] to the accumulators of its column groups that
// fall in that range.
template <class C, typename T> struct IdentityHook {
  Acc<C>* acc;
  int n0;
  PX_DEV void operator()(int kt, const T* A) const {
    constexpr int LDK = Lay<C, T>::LDK;
    const AccPos<C> p = acc_pos<C>();
    const int k0 = kt * C::BK;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int g = n0 + p.wn * C::WTN + j * 32;  // first column of this wave's group
      if (g < k0 || g >= k0 + C::BK) continue;
      const int kc = n0 + p.col(j) - k0;
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc->v[i][j][e] += to_f32<T>(A[p.row(i, e) * LDK + kc]);
    }
  }
};

template <class C, typename T, typename IT, typename GT, typename OT>
__global__ __launch_bounds__(C::NT) void k_apply(const IT* __restrict__ in, int64_t ld_in, int rows, int d, int b,
                                                  const GT* __restrict__ dT, const float* __restrict__ colscale,
                                                  OT* __restrict__ out, int64_t ld_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);
  const int blk = blockIdx.z, kb = blk * b, r = min(b, d - kb);
  const int m0 = blockIdx.x * C::BM, n0 = blockIdx.y * C::BN;
  if (n0 >= r) return;
  LoadK<C::BM, C::BK, C::NT, IT, T> la;
  la.init(in + (int64_t)m0 * ld_in + kb, ld_in, rows - m0, r);
  LoadK<C::BN, C::BK, C::NT, GT, T> lb;
  lb.init(dT + ((int64_t)blk * b + n0) * b, b, r - n0, r);
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, T>(lds, la, lb, r, acc, p.wm, p.wn, p.lane, IdentityHook<C, T>{&acc, n0});
  const float* cs = colscale ? colscale + kb + n0 : nullptr;
  store_tile<C, OT>(acc, smem, out + (int64_t)m0 * ld_out + kb + n0, ld_out, rows - m0, r - n0,
                    [&](int c) { return cs ? cs[c] : 1.f; });
}

// ============================================================================
// plain contraction out = A * B (* colscale)
// ============================================================================
// Workgroups are dealt to the 8 XCDs round robin by launch order.  The launch
// index is remapped so that each XCD receives a contiguous range of tile
// numbers, and tile numbers run through groups of GM row tiles, so the
// workgroups sharing one XCD's L2 work on a compact patch of A rows and B
// columns.
struct TileMap {
  int tm, tn;
  static constexpr int GM = 8;
  PX_DEV void at(int id, int& bm, int& bn) const {
    const int total = tm * tn;
    if (total % 8 == 0) id = (id % 8) * (total / 8) + id / 8;
    const int group = id / (GM * tn);
    const int first = group * GM;
    const int gsize = min(tm - first, GM);
    bm = first + (id % (GM * tn)) % gsize;
    bn = (id % (GM * tn)) / gsize;
  }
};

template <class C, typename T, typename AT, typename BT, typename OT, bool BKN>
__global__ __launch_bounds__(C::NT) void k_gemm(const AT* __restrict__ A, int64_t lda, const BT* __restrict__ B,
                                                 int64_t ldb, int M, int N, int K, const float* __restrict__ colscale,
                                                 OT* __restrict__ out, int64_t ldo, TileMap map) {
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);
  int bm, bn;
  map.at(blockIdx.x, bm, bn);
  const int m0 = bm * C::BM, n0 = bn * C::BN;
  LoadK<C::BM, C::BK, C::NT, AT, T> la;
  la.init(A + (int64_t)m0 * lda, lda, M - m0, K);
  using LB = typename std::conditional<BKN, LoadMN<C::BN, C::BK, C::NT, BT, T>, LoadK<C::BN, C::BK, C::NT, BT, T>>::type;
  LB lb;
  if constexpr (BKN)
    lb.init(B + n0, ldb, N - n0, K);
  else
    lb.init(B + (int64_t)n0 * ldb, ldb, N - n0, K);
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, T>(lds, la, lb, K, acc, p.wm, p.wn, p.lane);
  const float* cs = colscale ? colscale + n0 : nullptr;
  store_tile<C, OT>(acc, smem, out + (int64_t)m0 * ldo + n0, ldo, M - m0, N - n0,
                    [&](int c) { return cs ? cs[c] : 1.f; });
}

// ============================================================================
// permutations
// ============================================================================
// Row-staged gather: the workgroup copies whole source rows into LDS with
// 16-byte coalesced loads, then writes each output row with 16-byte stores,
// every lane gathering its 16 bytes from LDS at the permuted positions.
// Indices are clamped into range so that a malformed permutation cannot
// address outside the staged rows.
template <typename E>
__global__ __launch_bounds__(256) void k_permute_lds(const E* __restrict__ in, int64_t ld_in,
                                                     const int32_t* __restrict__ rowmap,
                                                     const int32_t* __restrict__ colmap, E* __restrict__ out,
                                                     int64_t ld_out, int rows, int d_in, int d_out, int rpw) {
  extern __shared__ __align__(16) unsigned char smem[];
  E* buf = reinterpret_cast<E*>(smem);
  constexpr int V = 16 / sizeof(E);
  const int pitch = (d_in + V - 1) / V * V;
  const int t0 = blockIdx.x * rpw;
  const int nr = min(rpw, rows - t0);
  const bool vin = (reinterpret_cast<uintptr_t>(in) % 16 == 0) && (ld_in % V == 0) && (d_in % V == 0);
  for (int rr = 0; rr < nr; ++rr) {
    int src = t0 + rr;
    if (rowmap) src = min(max(rowmap[src], 0), rows - 1);
    const E* row = in + (int64_t)src * ld_in;
    E* dst = buf + rr * pitch;
    if (vin) {
      for (int i = threadIdx.x; i < d_in / V; i += blockDim.x)
        reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(row)[i];
    } else {
      for (int i = threadIdx.x; i < d_in; i += blockDim.x) dst[i] = row[i];
    }
  }
  __syncthreads();
  const bool vout = (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (ld_out % V == 0) &&
                    (reinterpret_cast<uintptr_t>(colmap) % 16 == 0);
  const int nchunk = (d_out + V - 1) / V;
  for (int rr = 0; rr < nr; ++rr) {
    E* o = out + (int64_t)(t0 + rr) * ld_out;
    const E* srow = buf + rr * pitch;
    for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
      const int i0 = c * V;
      if (vout && i0 + V <= d_out) {
        int32_t idx[V];
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
          const int4 w = reinterpret_cast<const int4*>(colmap + i0)[q];
          idx[4 * q] = w.x;
          idx[4 * q + 1] = w.y;
          idx[4 * q + 2] = w.z;
          idx[4 * q + 3] = w.w;
        }
        E vals[V];
#pragma unroll
        for (int e = 0; e < V; ++e) vals[e] = srow[min(max(idx[e], 0), d_in - 1)];
        *reinterpret_cast<uint4*>(o + i0) = *reinterpret_cast<const uint4*>(vals);
      } else {
        for (int e = 0; e < V && i0 + e < d_out; ++e) o[i0 + e] = srow[min(max(colmap[i0 + e], 0), d_in - 1)];
      }
    }
  }
}

template <typename E>
__global__ __launch_bounds__(256) void k_permute_direct(const E* __restrict__ in, int64_t ld_in,
                                                        const int32_t* __restrict__ rowmap,
                                                        const int32_t* __restrict__ colmap, E* __restrict__ out,
                                                        int64_t ld_out, int rows, int d_in, int d_out) {
  const int t = blockIdx.x;
  int src = t;
  if (rowmap) src = min(max(rowmap[t], 0), rows - 1);
  for (int i = threadIdx.x; i < d_out; i += blockDim.x) {
    const int c = min(max(colmap[i], 0), d_in - 1);
    out[(int64_t)t * ld_out + i] = in[(int64_t)src * ld_in + c];
  }
}

__global__ void k_inverse_perm(const int32_t* __restrict__ perm, int d, int32_t* __restrict__ inv) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < d) inv[min(max(perm[i], 0), d - 1)] = i;
}

__global__ void k_compose_perm(const int32_t* __restrict__ a, const int32_t* __restrict__ bm, int d,
                               int32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < d) out[i] = a[min(max(bm[i], 0), d - 1)];
}

// SplitMix64 output number k (0-based) of the stream seeded with `seed`:
// the state after k + 1 golden-ratio increments, through the finaliser.
PX_DEV uint64_t splitmix64_at(uint64_t seed, uint64_t k) {
  uint64_t z = seed + (k + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Durstenfeld shuffle.  The swap partners j_i = floor(u * (i + 1) / 2^64),
// with u the (d-1-i)-th output, are drawn in parallel; the swaps themselves are
// inherently sequential and are made by one lane in LDS (or in global memory
// when d does not fit).
__global__ __launch_bounds__(256) void k_perm_shuffle(uint64_t seed, int d, int32_t* __restrict__ out,
                                                      int32_t* __restrict__ jglob, int use_lds) {
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* p = use_lds ? reinterpret_cast<int32_t*>(smem) : out;
  int32_t* jb = use_lds ? reinterpret_cast<int32_t*>(smem) + d : jglob;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    p[i] = i;
    if (i >= 1) jb[i] = (int32_t)__umul64hi(splitmix64_at(seed, (uint64_t)(d - 1 - i)), (uint64_t)(i + 1));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = d - 1; i >= 1; --i) {
      const int j = jb[i];
      const int32_t a = p[i], c = p[j];
      p[i] = c;
      p[j] = a;
    }
  }
  __syncthreads();
  if (use_lds)
    for (int i = threadIdx.x; i < d; i += blockDim.x) out[i] = p[i];
}

// ============================================================================
// merge-then-reinitialise
// ============================================================================
// M1[kb+i][c] = (W[kb+i][c] + sum_k DeltaR[blk][i][k] W[kb+k][c]) * wscale[c]
template <class C, typename GT, typename WT>
__global__ __launch_bounds__(C::NT) void k_merge_left(const GT* __restrict__ gR, const WT* __restrict__ W, int64_t ldw,
                                                       const float* __restrict__ wscale, int m, int n, int b,
                                                       float* __restrict__ M1, int64_t ldm) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* lds = reinterpret_cast<float*>(smem);
  const int blk = blockIdx.z, kb = blk * b, r = min(b, m - kb);
  const int m0 = blockIdx.y * C::BM, n0 = blockIdx.x * C::BN;
  if (m0 >= r) return;
  LoadK<C::BM, C::BK, C::NT, GT, float> la;
  la.init(gR + ((int64_t)blk * b + m0) * b, b, r - m0, r);
  LoadMN<C::BN, C::BK, C::NT, WT, float> lb;
  lb.init(W + (int64_t)kb * ldw + n0, ldw, n - n0, r);
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, float>(lds, la, lb, r, acc, p.wm, p.wn, p.lane);
  each_acc<C>(acc, [&](int i, int j, float v) {
    const int ii = m0 + i, c = n0 + j;
    if (ii < r && c < n) {
      v += to_f32<WT>(W[(int64_t)(kb + ii) * ldw + c]);
      if (wscale) v *= wscale[c];
      M1[(int64_t)(kb + ii) * ldm + c] = v;
    }
  });
}

__global__ void k_col_absmax(const float* __restrict__ M, int64_t ld, int rows, int n, int rows_per,
                             uint32_t* __restrict__ amax) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  const int r0 = blockIdx.y * rows_per, r1 = min(rows, r0 + rows_per);
  float mx = 0.f;
  for (int r = r0; r < r1; ++r) mx = fmaxf(mx, fabsf(M[(int64_t)r * ld + c]));
  // non-negative floats order like their bit patterns, so max is exact and order-free
  atomicMax(amax + c, __float_as_uint(mx));
}

PX_DEV float int8_scale(uint32_t amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a == 0.f ? 1.f : a / 127.f;
}

template <typename WT>
__global__ void k_store_weight(const float* __restrict__ M, int64_t ld, int rows, int n, WT* __restrict__ W,
                               int64_t ldw, const uint32_t* __restrict__ amax, float* __restrict__ wscale) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  float s = 1.f;
  if constexpr (sizeof(WT) == 1) {
    s = int8_scale(amax[c]);
    if (blockIdx.y == 0) wscale[c] = s;
  }
  for (int r = blockIdx.y; r < rows; r += gridDim.y) {
    const float v = M[(int64_t)r * ld + c];
    if constexpr (sizeof(WT) == 1) {
      float code = rintf(v / s);
      code = fminf(fmaxf(code, -127.f), 127.f);
      W[(int64_t)r * ldw + c] = (int8_t)code;
    } else {
      W[(int64_t)r * ldw + c] = from_f32<WT>(v);
    }
  }
}

__global__ void k_fill_zero(uint8_t* __restrict__ p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(p)[i] = make_uint4(0, 0, 0, 0);
  const size_t tail = bytes - n16 * 16;
  if (blockIdx.x == 0 && threadIdx.x < tail) p[n16 * 16 + threadIdx.x] = 0;
}

}  // namespace

// ============================================================================
// launchers
// ============================================================================
namespace pxk {

hipError_t fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>(4096, (bytes / 16 + 255) / 256 + 1);
  k_fill_zero<<<grid, 256, 0, s>>>(reinterpret_cast<uint8_t*>(p), bytes);
  return hipGetLastError();
}

hipError_t permute(int dt, const void* in, int64_t ld_in, const int32_t* rowmap, const int32_t* colmap, void* out,
                   int64_t ld_out, int rows, int d_in, int d_out, hipStream_t s) {
  if (rows <= 0 || d_out <= 0) return hipSuccess;
  const size_t es = dt_size(dt);
  const size_t row_bytes = (size_t)d_in * es;
  const size_t budget = 64 * 1024;
  auto go = [&](auto tag) -> hipError_t {
    using E = decltype(tag);
    const size_t pitch_bytes = (row_bytes + 15) / 16 * 16;
    if (pitch_bytes <= budget) {
      const int rpw = (int)std::max<size_t>(1, std::min<size_t>(16, budget / pitch_bytes));
      k_permute_lds<E><<<cdiv(rows, rpw), 256, rpw * pitch_bytes, s>>>(
          reinterpret_cast<const E*>(in), ld_in, rowmap, colmap, reinterpret_cast<E*>(out), ld_out, rows, d_in, d_out,
          rpw);
    } else {
      k_permute_direct<E><<<rows, 256, 0, s>>>(reinterpret_cast<const E*>(in), ld_in, rowmap, colmap,
                                               reinterpret_cast<E*>(out), ld_out, rows, d_in, d_out);
    }
    return hipGetLastError();
  };
  if (dt == F32) return go(float{});
  if (dt == BF16) return go(bf16_t{});
  return go(int8_t{});
}

hipError_t inverse_perm(const int32_t* perm, int d, int32_t* inv, hipStream_t s) {
  k_inverse_perm<<<cdiv(d, 256), 256, 0, s>>>(perm, d, inv);
  return hipGetLastError();
}

hipError_t compose_perm(const int32_t* a, const int32_t* b, int d, int32_t* out, hipStream_t s) {
  k_compose_perm<<<cdiv(d, 256), 256, 0, s>>>(a, b, d, out);
  return hipGetLastError();
}

hipError_t perm_from_seed_device(uint64_t seed, int d, int32_t* out, int32_t* scratch, hipStream_t s) {
  const size_t lds = (size_t)d * 8;
  const int use_lds = lds <= 160 * 1024;
  if (use_lds) {
    hipError_t e = allow_lds(k_perm_shuffle, (int)lds);
    if (e != hipSuccess) return e;
  }
  k_perm_shuffle<<<1, 256, use_lds ? lds : 0, s>>>(seed, d, out, scratch, use_lds);
  return hipGetLastError();
}

template <class C, typename T, typename IT, typename GT, typename OT>
static hipError_t apply_t(const void* in, int64_t ld_in, int rows, int d, int b, const void* dT, const float* cs,
                          void* out, int64_t ld_out, hipStream_t s) {
  const int lds = smem_bytes<C, T, OT>();
  auto k = k_apply<C, T, IT, GT, OT>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  dim3 grid(cdiv(rows, C::BM), cdiv(b, C::BN), nblocks(d, b));
  k<<<grid, C::NT, lds, s>>>(reinterpret_cast<const IT*>(in), ld_in, rows, d, b, reinterpret_cast<const GT*>(dT), cs,
                             reinterpret_cast<OT*>(out), ld_out);
  return hipGetLastError();
}

hipError_t apply(int cdt, int in_dt, const void* in, int64_t ld_in, int rows, int d, int b, int dT_dt, const void* dT,
                 const float* colscale, int out_dt, void* out, int64_t ld_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (cdt == BF16 && in_dt == BF16 && dT_dt == BF16 && out_dt == BF16)
    return apply_t<TGemm, bf16_t, bf16_t, bf16_t, bf16_t>(in, ld_in, rows, d, b, dT, colscale, out, ld_out, s);
  if (cdt == F32 && in_dt == F32 && dT_dt == F32 && out_dt == F32)
    return apply_t<TF, float, float, float, float>(in, ld_in, rows, d, b, dT, colscale, out, ld_out, s);
  // merge products: fp32 rows times the stored blocks
  if (cdt == F32 && in_dt == F32 && dT_dt == BF16 && out_dt == F32)
    return apply_t<TFM, float, float, bf16_t, float>(in, ld_in, rows, d, b, dT, colscale, out, ld_out, s);
  if (cdt == F32 && in_dt == F32 && dT_dt == F32 && out_dt == F32)
    return apply_t<TFM, float, float, float, float>(in, ld_in, rows, d, b, dT, colscale, out, ld_out, s);
  return hipErrorInvalidValue;
}

template <class C, typename T, typename AT, typename BT, typename OT, bool BKN>
static hipError_t gemm_t(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K, const float* cs,
                         void* out, int64_t ldo, hipStream_t s) {
  const int lds = smem_bytes<C, T, OT>();
  auto k = k_gemm<C, T, AT, BT, OT, BKN>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  const TileMap map{(int)cdiv(M, C::BM), (int)cdiv(N, C::BN)};
  k<<<map.tm * map.tn, C::NT, lds, s>>>(reinterpret_cast<const AT*>(A), lda, reinterpret_cast<const BT*>(B), ldb, M, N,
                                        K, cs, reinterpret_cast<OT*>(out), ldo, map);
  return hipGetLastError();
}

// bf16 contraction: the 256 x 256 tile when it yields at least one workgroup
// per CU, else the 256 x 128 tile.
template <typename BT, bool BKN>
static hipError_t gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K,
                            const float* cs, void* out, int64_t ldo, hipStream_t s) {
  if ((int64_t)cdiv(M, 256) * cdiv(N, 256) >= 256)
    return gemm_t<TGemm, bf16_t, bf16_t, BT, bf16_t, BKN>(A, lda, B, ldb, M, N, K, cs, out, ldo, s);
  return gemm_t<TBig, bf16_t, bf16_t, BT, bf16_t, BKN>(A, lda, B, ldb, M, N, K, cs, out, ldo, s);
}

hipError_t gemm(int cdt, int a_dt, const void* A, int64_t lda, int b_dt, const void* B, int64_t ldb, bool b_kn, int M,
                int N, int K, const float* colscale, int out_dt, void* out, int64_t ldo, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (cdt == BF16 && a_dt == BF16 && out_dt == BF16) {
    if (b_dt == BF16)
      return b_kn ? gemm_bf16<bf16_t, true>(A, lda, B, ldb, M, N, K, colscale, out, ldo, s)
                  : gemm_bf16<bf16_t, false>(A, lda, B, ldb, M, N, K, colscale, out, ldo, s);
    if (b_dt == I8)
      return b_kn ? gemm_bf16<int8_t, true>(A, lda, B, ldb, M, N, K, colscale, out, ldo, s)
                  : gemm_bf16<int8_t, false>(A, lda, B, ldb, M, N, K, colscale, out, ldo, s);
  }
  if (cdt == F32 && a_dt == F32 && b_dt == F32 && out_dt == F32)
    return b_kn ? gemm_t<TF, float, float, float, float, true>(A, lda, B, ldb, M, N, K, colscale, out, ldo, s)
                : gemm_t<TF, float, float, float, float, false>(A, lda, B, ldb, M, N, K, colscale, out, ldo, s);
  return hipErrorInvalidValue;
}

template <typename GT, typename WT>
static hipError_t merge_left_t(const void* gR, const void* W, int64_t ldw, const float* wscale, int m, int n, int b,
                               float* M1, int64_t ldm, hipStream_t s) {
  using C = TFM;
  const int lds = Lay<C, float>::BYTES;
  auto k = k_merge_left<C, GT, WT>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  dim3 grid(cdiv(n, C::BN), cdiv(b, C::BM), nblocks(m, b));
  k<<<grid, C::NT, lds, s>>>(reinterpret_cast<const GT*>(gR), reinterpret_cast<const WT*>(W), ldw, wscale, m, n, b,
                             M1, ldm);
  return hipGetLastError();
}

hipError_t merge_left(int g_dt, const void* gR, int w_dt, const void* W, int64_t ldw, const float* wscale, int m, int n,
                      int b, float* M1, int64_t ldm, hipStream_t s) {
  if (g_dt == F32 && w_dt == F32) return merge_left_t<float, float>(gR, W, ldw, wscale, m, n, b, M1, ldm, s);
  if (g_dt == BF16 && w_dt == BF16) return merge_left_t<bf16_t, bf16_t>(gR, W, ldw, wscale, m, n, b, M1, ldm, s);
  if (g_dt == BF16 && w_dt == I8) return merge_left_t<bf16_t, int8_t>(gR, W, ldw, wscale, m, n, b, M1, ldm, s);
  return hipErrorInvalidValue;
}

hipError_t col_absmax(const float* M, int64_t ld, int rows, int n, uint32_t* amax, hipStream_t s) {
  const int rows_per = 256;
  dim3 grid(cdiv(n, 256), cdiv(rows, rows_per));
  k_col_absmax<<<grid, 256, 0, s>>>(M, ld, rows, n, rows_per, amax);
  return hipGetLastError();
}

hipError_t store_weight(const float* M, int64_t ld, int rows, int n, int w_dt, void* W, int64_t ldw,
                        const uint32_t* amax, float* wscale, hipStream_t s) {
  dim3 grid(cdiv(n, 256), std::min(rows, 4096));
  if (w_dt == F32)
    k_store_weight<float><<<grid, 256, 0, s>>>(M, ld, rows, n, reinterpret_cast<float*>(W), ldw, amax, wscale);
  else if (w_dt == BF16)
    k_store_weight<bf16_t><<<grid, 256, 0, s>>>(M, ld, rows, n, reinterpret_cast<bf16_t*>(W), ldw, amax, wscale);
  else
    k_store_weight<int8_t><<<grid, 256, 0, s>>>(M, ld, rows, n, reinterpret_cast<int8_t*>(W), ldw, amax, wscale);
  return hipGetLastError();
}

}  // namespace pxk
