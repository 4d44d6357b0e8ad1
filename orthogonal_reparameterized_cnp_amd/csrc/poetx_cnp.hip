// Cayley-Neumann blocks: build G - I from packed skew parameters, and the
// chain rule from block gradients dG back to the packed parameters.
//
// Build (POET-X blog on zhichai.net, 第四斧: Q^2 once, Q^3 and Q^4 from it):
//   S = Q^2, N = 2Q + S,  G - I = (N + S) + N S  (= 2Q + 2Q^2 + 2Q^3 + Q^4).
// Chain rule of G = I + 2(Q + Q^2 + Q^3) + Q^4 with Q^T = -Q: with U = dL/dG
// (the block gradient, summed over tokens here too), the derivative of L with
// respect to the entries of Q is
//   D = 2U - 2(UQ + QU) + 2(UQ^2 + QUQ + Q^2U) - (UQ^3 + QUQ^2 + Q^2UQ + Q^3U),
// the ten terms of dG paired with U.  With V1 = U Q, P = Q U, S = Q^2 and
// W = 2U - V1 - P the same sum is
//   D = (2U - 2V1 - 2P) + 2 Q V1 + W S + S W,
// six b x b products in two launches; then dq[p(i,j)] = D[i][j] - D[j][i] on
// the packed slots.
//
// Q is unpacked once into a dense block buffer; every product reads plain
// row-major operands.  Products with Q on the right load Q's rows as the B
// operand, which yields X Q^T = -X Q (the sign is folded into the epilogue);
// products with a non-symmetric matrix on the right read the transpose that
// the producing epilogue wrote.  The fp32 part of D is carried in one array
// that each launch updates in place.
#include "kernel_util.h"

using namespace px;

namespace {

// The sides of one launch (the two sides of a linear, or every side of a
// batch): their blocks are numbered consecutively, side s owning global blocks
// [first[s], first[s + 1]).  Passed by value as a kernel argument.
struct SideTable {
  const float* q[pxk::kMaxSides];
  int d[pxk::kMaxSides];
  int first[pxk::kMaxSides + 1];
  int count;
  PX_DEV int side_of(int z) const {
    int s = 0;
    while (s + 1 < count && z >= first[s + 1]) ++s;
    return s;
  }
  // side s, block blk of that side, its live size r and its packed parameters
  // (null for a table built without them: the block gradients do not read q)
  PX_DEV void at(int z, int b, int& s, int& blk, int& r, const float*& qk) const {
    s = side_of(z);
    blk = z - first[s];
    r = min(b, d[s] - blk * b);
    qk = q[s] ? q[s] + (int64_t)blk * ((int64_t)b * (b - 1) / 2) : nullptr;
  }
  PX_DEV void at(int z, int b, const float*& qk, int& r) const {
    int s, blk;
    at(z, b, s, blk, r, qk);
  }
};

// Workgroups are dealt to the 8 XCDs round robin by launch index, so
// consecutive indices land on different L2s.  The product kernels remap the
// launch index to a unit number that gives each XCD a contiguous range of
// units (the first units % 8 XCDs one more); units run tile-fastest within a
// block, so the tiles that share a block's operand panels run together on one
// XCD and fetch those panels into its L2 once.
PX_DEV int xcd_unit(int id, int units) {
  const int x = id % 8, k = id / 8, q = units / 8, r = units % 8;
  return x * q + min(x, r) + k;
}

// K loop over two K-contiguous bf16/fp32 operand tiles (row pitch b): the
// direct-to-LDS loop for interior bf16 tiles, else the checked register loop.
template <class C, typename T, class Epi>
PX_DEV void run_kk(unsigned char* smem, const T* a0, int rows_a, const T* b0, int rows_b, int b, int K, Epi&& epi) {
  if constexpr (std::is_same<T, bf16_t>::value && C::BM == DSq::BM && C::BN == DSq::BN && C::NT == DSq::NT) {
    if (dma_rows_ok(a0, b, rows_a, DSq::BM) && dma_rows_ok(b0, b, rows_b, DSq::BN) && K % DSq::BK == 0) {
      Acc<DSq> acc;
      const AccPos<DSq> p = acc_pos<DSq>();
      const DmaSrc src{reinterpret_cast<const bf16_t*>(a0), b, reinterpret_cast<const bf16_t*>(b0), b};
      dma_mainloop<DSq>(reinterpret_cast<char*>(smem), src, K / DSq::BK, acc, p.wm, p.wn, p.lane, NoHook());
      epi(acc);
      return;
    }
  }
  LoadK<C::BM, C::BK, C::NT, T, T> la;
  la.init(a0, b, rows_a, K);
  LoadK<C::BN, C::BK, C::NT, T, T> lb;
  lb.init(b0, b, rows_b, K);
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, T>(reinterpret_cast<T*>(smem), la, lb, K, acc, p.wm, p.wn, p.lane);
  epi(acc);
}

// Two products of the same shape, X0 Y0^T and X1 Y1^T, one after the other in
// the same workgroup; epi(acc0, acc1).  Both take the same loop.  (One
// pipeline over both, with the accumulator chosen per K tile, needs more than
// the 256 registers of two waves per SIMD.)
template <class C, typename T, class Epi>
PX_DEV void run_kk2(unsigned char* smem, const T* x0, const T* y0, const T* x1, const T* y1, int rows_x, int rows_y,
                    int b, int K, Epi&& epi) {
  if constexpr (std::is_same<T, bf16_t>::value && C::BM == DSq::BM && C::BN == DSq::BN && C::NT == DSq::NT) {
    if (dma_rows_ok(x0, b, rows_x, DSq::BM) && dma_rows_ok(x1, b, rows_x, DSq::BM) &&
        dma_rows_ok(y0, b, rows_y, DSq::BN) && dma_rows_ok(y1, b, rows_y, DSq::BN) && K % DSq::BK == 0) {
      Acc<DSq> a0, a1;
      const AccPos<DSq> p = acc_pos<DSq>();
      const DmaSrc s0{reinterpret_cast<const bf16_t*>(x0), b, reinterpret_cast<const bf16_t*>(y0), b};
      dma_mainloop<DSq>(reinterpret_cast<char*>(smem), s0, K / DSq::BK, a0, p.wm, p.wn, p.lane, NoHook());
      const DmaSrc s1{reinterpret_cast<const bf16_t*>(x1), b, reinterpret_cast<const bf16_t*>(y1), b};
      dma_mainloop<DSq>(reinterpret_cast<char*>(smem), s1, K / DSq::BK, a1, p.wm, p.wn, p.lane, NoHook());
      epi(a0, a1);
      return;
    }
  }
  const AccPos<C> p = acc_pos<C>();
  Acc<C> a0, a1;
  {
    LoadK<C::BM, C::BK, C::NT, T, T> la;
    la.init(x0, b, rows_x, K);
    LoadK<C::BN, C::BK, C::NT, T, T> lb;
    lb.init(y0, b, rows_y, K);
    mainloop<C, T>(reinterpret_cast<T*>(smem), la, lb, K, a0, p.wm, p.wn, p.lane);
  }
  __syncthreads();
  {
    LoadK<C::BM, C::BK, C::NT, T, T> la;
    la.init(x1, b, rows_x, K);
    LoadK<C::BN, C::BK, C::NT, T, T> lb;
    lb.init(y1, b, rows_y, K);
    mainloop<C, T>(reinterpret_cast<T*>(smem), la, lb, K, a1, p.wm, p.wn, p.lane);
  }
  epi(a0, a1);
}

// Three products of the same shape added in one accumulator,
// X0 Y0^T + X1 Y1^T + X2 Y2^T; epi(acc).  All three take the same loop.
template <class C, typename T, class Epi>
PX_DEV void run_kk_sum3(unsigned char* smem, const T* x0, const T* y0, const T* x1, const T* y1, const T* x2,
                        const T* y2, int rows_x, int rows_y, int b, int K, Epi&& epi) {
  if constexpr (std::is_same<T, bf16_t>::value && C::BM == DSq::BM && C::BN == DSq::BN && C::NT == DSq::NT) {
    if (dma_rows_ok(x0, b, rows_x, DSq::BM) && dma_rows_ok(x1, b, rows_x, DSq::BM) &&
        dma_rows_ok(x2, b, rows_x, DSq::BM) && dma_rows_ok(y0, b, rows_y, DSq::BN) &&
        dma_rows_ok(y1, b, rows_y, DSq::BN) && dma_rows_ok(y2, b, rows_y, DSq::BN) && K % DSq::BK == 0) {
      Acc<DSq> acc;
      const AccPos<DSq> p = acc_pos<DSq>();
      const DmaSrc s0{reinterpret_cast<const bf16_t*>(x0), b, reinterpret_cast<const bf16_t*>(y0), b};
      const DmaSrc s1{reinterpret_cast<const bf16_t*>(x1), b, reinterpret_cast<const bf16_t*>(y1), b};
      const DmaSrc s2{reinterpret_cast<const bf16_t*>(x2), b, reinterpret_cast<const bf16_t*>(y2), b};
      dma_mainloop_sum3<DSq>(reinterpret_cast<char*>(smem), s0, s1, s2, K / DSq::BK, acc, p.wm, p.wn, p.lane);
      epi(acc);
      return;
    }
  }
  const AccPos<C> p = acc_pos<C>();
  Acc<C> acc;
  auto add = [&](const T* x, const T* y, bool first) {
    LoadK<C::BM, C::BK, C::NT, T, T> la;
    la.init(x, b, rows_x, K);
    LoadK<C::BN, C::BK, C::NT, T, T> lb;
    lb.init(y, b, rows_y, K);
    mainloop<C, T>(reinterpret_cast<T*>(smem), la, lb, K, acc, p.wm, p.wn, p.lane, NoHook(), first);
  };
  add(x0, y0, true);
  __syncthreads();
  add(x1, y1, false);
  __syncthreads();
  add(x2, y2, false);
  epi(acc);
}

// A tile stored transposed through LDS: the epilogue puts tile rows i0 .. i0 + 3
// of tile column j (tile-local) with put(); after a barrier, flush() writes the
// tile transposed, dst[(col0 + j) * ld + row0 + i] for j < ncols, i < nrows,
// in row-contiguous pieces of 4 elements, instead of one 4-element piece per
// lane in 64 different rows.  The LDS must be free (after a K loop's final
// barrier) and hold BYTES per stage.
template <class CC, typename T> struct TStage {
  static constexpr int PITCH = CC::BM + 4;  // elements per staged row (one tile column); 8 / 16-byte aligned
  static constexpr int BYTES = CC::BN * PITCH * (int)sizeof(T);
  T* t;
  PX_DEV explicit TStage(void* lds) : t(reinterpret_cast<T*>(lds)) {}
  PX_DEV void put(int i0, int j, const float v[4]) const { store4<T>(t + j * PITCH + i0, v); }
  PX_DEV void flush(T* dst, int64_t ld, int row0, int col0, int nrows, int ncols) const {
    constexpr int Q = CC::BM / 4;  // 4-element pieces per staged row
    using V = typename std::conditional<sizeof(T) == 2, uint2, uint4>::type;
    const bool vec = reinterpret_cast<uintptr_t>(dst) % sizeof(V) == 0 && ld % 4 == 0 && row0 % 4 == 0;
    for (int c = threadIdx.x; c < CC::BN * Q; c += blockDim.x) {
      const int j = c / Q, i = (c % Q) * 4;
      if (j >= ncols || i >= nrows) continue;
      const T* s = t + j * PITCH + i;
      T* d = dst + (int64_t)(col0 + j) * ld + row0 + i;
      if (vec && i + 4 <= nrows)
        *reinterpret_cast<V*>(d) = *reinterpret_cast<const V*>(s);
      else
        for (int e = 0; e < 4 && i + e < nrows; ++e) d[e] = s[e];
    }
  }
  // the staged tile itself, untransposed: dst[(row0 + i) * ld + col0 + j] = value put at (i, j), in
  // 16-byte pieces of 16 / sizeof(T) consecutive j read down the staged rows
  PX_DEV void flush_rows(T* dst, int64_t ld, int row0, int col0, int nrows, int ncols) const {
    constexpr int V = 16 / (int)sizeof(T), Q = CC::BN / V;  // pieces per output row
    const bool vec = reinterpret_cast<uintptr_t>(dst) % 16 == 0 && ld % V == 0 && col0 % V == 0;
    for (int c = threadIdx.x; c < CC::BM * Q; c += blockDim.x) {
      const int i = c / Q, j = (c % Q) * V;
      if (i >= nrows || j >= ncols) continue;
      T* d = dst + (int64_t)(row0 + i) * ld + col0 + j;
      T vals[V];
#pragma unroll
      for (int e = 0; e < V; ++e) vals[e] = t[(j + e) * PITCH + i];
      if (vec && j + V <= ncols) {
        *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(vals);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (j + e < ncols) d[e] = vals[e];
      }
    }
  }
};

// Dense Q from the packed parameters.  A workgroup takes one tile (ti, tj),
// ti <= tj, of 64 x 64: it reads the packed slots of the tile's entries above
// the diagonal along packed rows into LDS, then writes the tile (for a
// diagonal tile also its entries below the diagonal, negated from the
// mirrored ones) and, off the diagonal, the mirrored tile (tj, ti) = -(its
// transpose), in 16-byte pieces of rows.  Entries outside the live r x r
// corner, and the diagonal, are zero.  Writes Q in the operand dtype.
template <typename T>
__global__ __launch_bounds__(256) void k_unpack_q(SideTable sd, int b, T* __restrict__ Qb) {
  __shared__ float t[64][65];
  const int z = blockIdx.y;
  const float* qk;
  int r;
  sd.at(z, b, qk, r);
  const int tiles = (b + 63) / 64;
  int u = blockIdx.x, ti = 0;
  while (u >= tiles - ti) {
    u -= tiles - ti;
    ++ti;
  }
  const int tj = ti + u, i0 = ti * 64, j0 = tj * 64;
  const int c = threadIdx.x & 63, rr = threadIdx.x >> 6;
  // every load reads a valid slot (slot 0 stands in for masked ones); a block
  // of size b has b (b - 1) / 2 slots, none for b = 1 (Q is zero)
  const bool any = b > 1;
  float v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = i0 + rr + 4 * k, j = j0 + c;
    const bool ok = any && i < j && j < r;
    v[k] = qk[ok ? packed_slot(i, j, b) : 0];
    v[k] = ok ? v[k] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) t[rr + 4 * k][c] = v[k];
  __syncthreads();
  T* Q = Qb + (int64_t)z * b * b;
  constexpr int V = 16 / sizeof(T);
  const bool vec = b % V == 0;
  // one 64 x 64 output tile at (row0, col0): value(row, col) from LDS
  auto put = [&](int row0, int col0, auto value) {
    for (int w = threadIdx.x; w < 64 * 64 / V; w += blockDim.x) {
      const int row = w / (64 / V), col = (w % (64 / V)) * V;
      if (row0 + row >= b || col0 + col >= b) continue;
      T* o = Q + (int64_t)(row0 + row) * b + col0 + col;
      if (vec) {
        T vals[V];
#pragma unroll
        for (int e = 0; e < V; ++e) vals[e] = from_f32<T>(value(row, col + e));
        *reinterpret_cast<uint4*>(o) = *reinterpret_cast<const uint4*>(vals);
      } else {
        for (int e = 0; e < V && col0 + col + e < b; ++e) o[e] = from_f32<T>(value(row, col + e));
      }
    }
  };
  if (ti == tj) {
    // diagonal tile: above the diagonal as read, below it the negated mirror
    put(i0, j0, [&](int i, int j) { return i < j ? t[i][j] : i > j ? -t[j][i] : 0.f; });
  } else {
    put(i0, j0, [&](int i, int j) { return t[i][j]; });
    put(j0, i0, [&](int j, int i) { return -t[i][j]; });
  }
}

// S = Q Q = -(Q Q^T).  Writes S and N = 2Q + S in the operand dtype (the
// epilogue reads Q at its accumulators' positions).
template <class C, typename T>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2))) void k_cnp_square(SideTable sd, int b, const T* __restrict__ Qb,
                                                      T* __restrict__ Nb, T* __restrict__ Sb) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tn = (b + C::BN - 1) / C::BN, tm = (b + C::BM - 1) / C::BM;
  const int u = xcd_unit(blockIdx.x, gridDim.x), z = u / (tm * tn);
  const float* qk;
  int r;
  sd.at(z, b, qk, r);
  const int m0 = (u % (tm * tn) / tn) * C::BM, n0 = (u % tn) * C::BN;
  if (m0 >= r || n0 >= r) return;  // nothing outside the live corner is read later
  const int64_t off = (int64_t)z * b * b;
  run_kk<C, T>(smem, Qb + off + (int64_t)m0 * b, r - m0, Qb + off + (int64_t)n0 * b, r - n0, b, r, [&](auto& acc) {
    using CC = cfg_of<decltype(acc)>;
    float q[CC::TM][CC::TN][16];
    load_at_acc<CC>(q, Qb + off, b, m0, n0, r, r);
    // the two outputs over the live corner, each staged in LDS and written in 16-byte row pieces
    const int rows = min(CC::BM, r - m0), cols = min(CC::BN, r - n0);
    const int64_t at = off + (int64_t)m0 * b + n0;
    store_tile_fn<CC, T>(smem, Sb + at, b, rows, cols, [&](int i, int j, int e) { return -acc.v[i][j][e]; });
    store_tile_fn<CC, T>(smem, Nb + at, b, rows, cols,
                         [&](int i, int j, int e) { return 2.f * q[i][j][e] - acc.v[i][j][e]; });
  });
}

// G - I = (N + S) + N S (N S = S N: both are polynomials in Q, and N + S = 2Q + 2S),
// written as slice 0 (row-major) and slice 1 (transposed); zero outside the live
// r x r corner.  S is symmetric, so its rows serve as the B operand.
struct GOut {
  void* g[pxk::kMaxSides];  // side s: [2][nb_s][b][b], slice 0 = G - I, slice 1 = its transpose
};

template <class C, typename T>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2))) void k_cnp_delta(SideTable sd, int b, const T* __restrict__ Nb,
                                                     const T* __restrict__ Sb, GOut go) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tn = (b + C::BN - 1) / C::BN, tm = (b + C::BM - 1) / C::BM;
  const int u = xcd_unit(blockIdx.x, gridDim.x), z = u / (tm * tn);
  const float* qk;
  int side, blk, r;
  sd.at(z, b, side, blk, r, qk);
  const int m0 = (u % (tm * tn) / tn) * C::BM, n0 = (u % tn) * C::BN;
  const int64_t off = (int64_t)z * b * b;
  const int64_t nb_s = sd.first[side + 1] - sd.first[side];
  T* g0 = reinterpret_cast<T*>(go.g[side]) + (int64_t)blk * b * b;
  T* g1 = reinterpret_cast<T*>(go.g[side]) + (nb_s + blk) * b * b;
  run_kk<C, T>(smem, Nb + off + (int64_t)m0 * b, r - m0, Sb + off + (int64_t)n0 * b, r - n0, b, r, [&](auto& acc) {
    using CC = cfg_of<decltype(acc)>;
    // t2 = N + S = 2Q + 2S at the accumulators' positions (S added one row group at a time)
    float t2[CC::TM][CC::TN][16];
    load_at_acc<CC>(t2, Nb + off, b, m0, n0, max(r, 1), max(r, 1));
#pragma unroll
    for (int ti = 0; ti < CC::TM; ++ti) {
      float sv[CC::TN][16];
      load_at_acc_i<CC>(sv, Sb + off, b, m0, n0, max(r, 1), max(r, 1), ti);
#pragma unroll
      for (int tj = 0; tj < CC::TN; ++tj)
#pragma unroll
        for (int e = 0; e < 16; ++e) t2[ti][tj][e] += sv[tj][e];
    }
    const AccPos<CC> p = acc_pos<CC>();
    // G - I over the whole b x b block (zero outside the live corner)
    auto value = [&](int ti, int tj, int e) {
      const int i = m0 + p.row(ti, e), j = n0 + p.col(tj);
      return (i < r && j < r) ? acc.v[ti][tj][e] + t2[ti][tj][e] : 0.f;
    };
    // slice 0 (row-major) staged in LDS and written in 16-byte row pieces; slice 1 (the transpose)
    // through a second LDS area past the first
    const int rows = min(CC::BM, b - m0), cols = min(CC::BN, b - n0);
    store_tile_fn<CC, T>(smem, g0 + (int64_t)m0 * b + n0, b, rows, cols, value);
    constexpr int EPI = (CC::BM * (CC::BN + 16 / (int)sizeof(T)) * (int)sizeof(T) + 15) / 16 * 16;
    const TStage<CC, T> st(smem + EPI);
#pragma unroll
    for (int ti = 0; ti < CC::TM; ++ti)
#pragma unroll
      for (int tj = 0; tj < CC::TN; ++tj) {
        const int j = n0 + p.col(tj);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int i0 = m0 + p.row(ti, 4 * g);
          if (j >= b || i0 >= b) continue;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = value(ti, tj, 4 * g + e);
          st.put(i0 - m0, j - n0, o);
        }
      }
    __syncthreads();
    st.flush(g1, b, m0, n0, rows, cols);
  });
}

// Block gradients U = dL/dG summed over all tokens, both sides in one launch:
// side s, block blk: U[i][j] = sum_t A_s[t][kb + i] * B_s[t][kb + j] (R side:
// A = Xt, B = dA; P side: A = H, B = dZt).  Each workgroup owns one output
// tile and runs the whole token range, so the sum order is fixed.  Written as
// fp32, operand dtype and operand-dtype transpose, the forms the chain reads.
template <typename T> struct GradSides {
  const T* A[pxk::kGradSides];
  const T* B[pxk::kGradSides];
  int64_t lda[pxk::kGradSides], ldb[pxk::kGradSides];
};

template <typename T> struct Chain {
  const T* Qb;
  float* F32;  // U, then 2U - 2V1 - 2P, then D (updated in place)
  T* Ub;       // U
  T* Utb;      // U^T
  T* Wb;       // W = 2U - V1 - P
  T* Wtb;      // W^T
  T* V1tb;     // (2 V1)^T
  T* Sb;       // S = Q^2
};

// G groups of C::NT threads split the token range of one output tile; their
// partial sums are added in group order through LDS, so results do not depend
// on timing.  The launcher uses G > 1 only when rows is a multiple of G * BK,
// so that every group runs the same number of K steps (and barriers).
template <class C, typename T, int G>
__global__ __launch_bounds__(C::NT * G) void k_block_grads(SideTable sd, GradSides<T> gs, int rows, int b, Chain<T> ch,
                                                           int64_t zoff) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int grp = G == 1 ? 0 : (int)(threadIdx.x / C::NT);
  T* lds = reinterpret_cast<T*>(smem + grp * Lay<C, T>::BYTES);
  const int tiles_n = (b + C::BN - 1) / C::BN, tiles = tiles_n * ((b + C::BM - 1) / C::BM);
  const int u = xcd_unit(blockIdx.x, gridDim.x);
  const int zl = u / tiles;  // block of this linear; zoff + zl is its place in the gradient arrays
  int s, blk, r;
  const float* qk;
  sd.at(zl, b, s, blk, r, qk);
  const int kb = blk * b;
  const int m0 = (u % tiles / tiles_n) * C::BM, n0 = (u % tiles_n) * C::BN;
  if (m0 >= r || n0 >= r) return;  // only the live corner is read later
  const int per = rows / G;
  const int64_t t0 = (int64_t)grp * per;
  LoadMN<C::BM, C::BK, C::NT, T, T> la;
  la.init(gs.A[s] + t0 * gs.lda[s] + kb + m0, gs.lda[s], r - m0, per);
  LoadMN<C::BN, C::BK, C::NT, T, T> lb;
  lb.init(gs.B[s] + t0 * gs.ldb[s] + kb + n0, gs.ldb[s], r - n0, per);
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, T>(lds, la, lb, per, acc, p.wm, p.wn, p.lane);
  if constexpr (G > 1) {
    // the loop ended with a barrier: the operand tiles are free for the fold
    constexpr int PITCH = C::BN + 4;
    float* red = reinterpret_cast<float*>(smem);
    for (int g = 1; g < G; ++g) {
      if (grp == g)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[p.row(i, e) * PITCH + p.col(j)] = acc.v[i][j][e];
      __syncthreads();
      if (grp == 0)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc.v[i][j][e] += red[p.row(i, e) * PITCH + p.col(j)];
      __syncthreads();
    }
    if (grp != 0) return;
  }
  const int64_t off = (zoff + zl) * b * b;
  each_acc4<C>(acc, [&](int i0, int j, const float* v) {
    i0 += m0;
    j += n0;
    if (j >= r || i0 >= r) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e >= r) continue;
      const int64_t x = off + (int64_t)(i0 + e) * b + j;
      ch.F32[x] = v[e];
      ch.Ub[x] = from_f32<T>(v[e]);
    }
    T* dst = ch.Utb + off + (int64_t)j * b + i0;
    if (i0 + 4 <= r)
      store4<T>(dst, v);
    else
      for (int e = 0; e < 4 && i0 + e < r; ++e) dst[e] = from_f32<T>(v[e]);
  });
}

// Block gradients of large blocks (b a multiple of 256), split over tokens:
// workgroup (tile, block, s) sums the rows of 64-row K tiles
// [s * KT / S, (s + 1) * KT / S) (KT = rows / 64; S = 1 takes all rows) of its
// 256 x 256 tile and writes the fp32 partial to part[s][block].  Big tiles
// give each K step enough MFMA work to cover its loads, and the token split
// gives the grid enough workgroups; k_block_grads_reduce then adds the S
// partials in split order.
template <class C, typename T>
__global__ __launch_bounds__(C::NT) void k_block_grads_part(SideTable sd, GradSides<T> gs, int rows, int b, int S,
                                                            float* __restrict__ part) {
  extern __shared__ __align__(16) unsigned char smem[];
  // units: tile fastest, then split, then block
  const int tiles_n = (b + C::BN - 1) / C::BN, tiles = tiles_n * ((b + C::BM - 1) / C::BM);
  const int u = xcd_unit(blockIdx.x, gridDim.x);
  const int sp = u / tiles % S, zl = u / tiles / S, NB = sd.first[sd.count];
  int s, blk, r;
  const float* qk;
  sd.at(zl, b, s, blk, r, qk);
  const int kb = blk * b;
  const int m0 = (u % tiles / tiles_n) * C::BM, n0 = (u % tiles_n) * C::BN;
  if (m0 >= r || n0 >= r) return;  // only the live corner is read later
  int64_t t0 = 0;
  int per = rows;
  if (S > 1) {  // rows is a multiple of 64 (checked by the launcher)
    const int KT = rows / 64, k0 = (int)((int64_t)sp * KT / S), k1 = (int)((int64_t)(sp + 1) * KT / S);
    t0 = (int64_t)k0 * 64;
    per = (k1 - k0) * 64;
  }
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  bool done = false;
  if constexpr (std::is_same<T, bf16_t>::value && C::BK == 64) {
    // whole tile inside the block and whole 64-row K tiles: the line-wide
    // transposing loader into the swizzled unpadded tile
    const T* pa = gs.A[s] + t0 * gs.lda[s] + kb + m0;
    const T* pb = gs.B[s] + t0 * gs.ldb[s] + kb + n0;
    if (r - m0 >= C::BM && r - n0 >= C::BN && per % 64 == 0 && aligned8(pa, gs.lda[s]) && aligned8(pb, gs.ldb[s])) {
      constexpr int TA = C::BM * 128, STG = (C::BM + C::BN) * 128;
      char* lds = reinterpret_cast<char*>(smem);
      // the first half of the workgroup loads the A tile, the second half the B tile
      static_assert(C::BM == C::BN, "one loader shape for both operands");
      const bool is_b = threadIdx.x >= C::NT / 2;
      LoadT<C::BM, C::NT / 2> ld;
      ld.init(is_b ? pb : pa, is_b ? gs.ldb[s] : gs.lda[s]);
      const int mine = is_b ? TA : 0;
      acc.zero();
      const int NK = per / 64;
      ld.fetch(0);
      ld.stash(lds + mine);
      __syncthreads();
      for (int kt = 0; kt < NK; ++kt) {
        const char* cur = lds + (kt & 1) * STG;
        char* nxt = lds + ((kt + 1) & 1) * STG;
        const bool more = kt + 1 < NK;
        if (more) ld.fetch((kt + 1) * 64);
        mma_stage_t<C>(cur, cur + TA, acc, p.wm, p.wn, p.lane);
        if (more) ld.stash(nxt + mine);
        __syncthreads();
      }
      done = true;
    }
  }
  if (!done) {
    LoadMN<C::BM, C::BK, C::NT, T, T> la;
    la.init(gs.A[s] + t0 * gs.lda[s] + kb + m0, gs.lda[s], r - m0, per);
    LoadMN<C::BN, C::BK, C::NT, T, T> lb;
    lb.init(gs.B[s] + t0 * gs.ldb[s] + kb + n0, gs.ldb[s], r - n0, per);
    mainloop<C, T>(reinterpret_cast<T*>(smem), la, lb, per, acc, p.wm, p.wn, p.lane);
  }
  float* P = part + ((int64_t)sp * NB + zl) * b * b;
  each_acc<C>(acc, [&](int i, int j, float v) {
    i += m0;
    j += n0;
    if (i < r && j < r) P[(int64_t)i * b + j] = v;
  });
}

// U = part[0] + part[1] + ... + part[S-1] (in that order) over the live corner
// of every block, written as the chain rule reads it: fp32, operand dtype and
// operand-dtype transpose (through an LDS tile so every access is
// row-contiguous).  One 64 x 64 tile per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void k_block_grads_reduce(SideTable sd, int b, int S, const float* __restrict__ part,
                                                            Chain<T> ch, int64_t zoff) {
  __shared__ float t[64][65];
  const int zl = blockIdx.y;
  int s, blk, r;
  const float* qk;
  sd.at(zl, b, s, blk, r, qk);
  const int tiles = (b + 63) / 64;
  const int i0 = (blockIdx.x / tiles) * 64, j0 = (blockIdx.x % tiles) * 64;
  if (i0 >= r || j0 >= r) return;
  const int c = threadIdx.x & 63, rr = threadIdx.x >> 6;
  float u[16];
  for (int sp = 0; sp < S; ++sp) {
    const float* P = part + ((int64_t)sp * gridDim.y + zl) * b * b;
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = min(i0 + rr + 4 * k, r - 1), j = min(j0 + c, r - 1);
      v[k] = P[(int64_t)i * b + j];
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) u[k] = sp == 0 ? v[k] : u[k] + v[k];
  }
  const int64_t off = (zoff + zl) * b * b;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = i0 + rr + 4 * k, j = j0 + c;
    t[rr + 4 * k][c] = u[k];
    if (i < r && j < r) {
      ch.F32[off + (int64_t)i * b + j] = u[k];
      ch.Ub[off + (int64_t)i * b + j] = from_f32<T>(u[k]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int jj = rr + 4 * k, j = j0 + jj, i = i0 + c;  // Utb[j][i] = U[i][j]
    if (i < r && j < r) ch.Utb[off + (int64_t)j * b + i] = from_f32<T>(t[c][jj]);
  }
}

// Chain rule, first launch, two workgroups per output tile (both on the XCD
// of their block).  The first forms U Q^T = -V1 and Q U = P (the rows of U^T
// as B operand) and writes W = 2U - V1 - P (row-major and transposed),
// (2 V1)^T and the fp32 part 2U - 2V1 - 2P over U; the second forms
// Q Q^T = -S and writes S.
template <class C, typename T>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2))) void k_cnp_grad1(SideTable sd, int b,
                                                                                            Chain<T> ch, int kinds) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tn = (b + C::BN - 1) / C::BN, tm = (b + C::BM - 1) / C::BM, tiles = tm * tn;
  // units: tile fastest, then the kind of workgroup (kinds = 1: S is given, only the first kind), then the block
  const int u = xcd_unit(blockIdx.x, gridDim.x), z = u / (kinds * tiles), kind = kinds == 2 ? u / tiles % 2 : 0;
  const float* qk;
  int r;
  sd.at(z, b, qk, r);
  const int m0 = (u % tiles / tn) * C::BM, n0 = (u % tn) * C::BN;
  if (m0 >= r || n0 >= r) return;  // the second launch and the packing read only the live corner
  const int64_t off = (int64_t)z * b * b;
  const T* Qm = ch.Qb + off + (int64_t)m0 * b;
  const T* Qn = ch.Qb + off + (int64_t)n0 * b;
  if (kind == 1) {
    run_kk<C, T>(smem, Qm, r - m0, Qn, r - n0, b, r, [&](auto& qq) {
      using CC = cfg_of<decltype(qq)>;
      each_acc4<CC>(qq, [&](int i0, int j, const float* v) {
        i0 += m0;
        j += n0;
        if (j >= r || i0 >= r) return;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (i0 + e < r) ch.Sb[off + (int64_t)(i0 + e) * b + j] = from_f32<T>(-v[e]);
      });
    });
    return;
  }
  run_kk2<C, T>(smem, ch.Ub + off + (int64_t)m0 * b, Qn, Qm, ch.Utb + off + (int64_t)n0 * b, r - m0, r - n0, b, r,
                [&](auto& uq, auto& qu) {
    using CC = cfg_of<decltype(uq)>;
    const AccPos<CC> p = acc_pos<CC>();
    // W^T and (2 V1)^T leave through LDS
    const TStage<CC, T> sw(smem), sv(smem + TStage<CC, T>::BYTES);
#pragma unroll
    for (int ti = 0; ti < CC::TM; ++ti) {
      // one row group of U at a time keeps the epilogue's registers down
      float f[CC::TN][16];
      load_at_acc_i<CC>(f, ch.F32 + off, b, m0, n0, r, r, ti);
#pragma unroll
      for (int tj = 0; tj < CC::TN; ++tj) {
        const int j = n0 + p.col(tj);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int i0 = m0 + p.row(ti, 4 * g);
          if (j >= r || i0 >= r) continue;
          float w[4] = {0.f, 0.f, 0.f, 0.f}, v2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (i0 + e >= r) continue;
            const int k = 4 * g + e;
            const int64_t x = off + (int64_t)(i0 + e) * b + j;
            const float uv = f[tj][k], v1 = -uq.v[ti][tj][k], pv = qu.v[ti][tj][k];
            w[e] = 2.f * uv - v1 - pv;
            v2[e] = 2.f * v1;
            ch.F32[x] = 2.f * uv - 2.f * v1 - 2.f * pv;
          }
          sw.put(i0 - m0, j - n0, w);
          sv.put(i0 - m0, j - n0, v2);
        }
      }
    }
    __syncthreads();
    const int nr = min(CC::BM, r - m0), nc = min(CC::BN, r - n0);
    sw.flush(ch.Wtb + off, b, m0, n0, nr, nc);
    sv.flush(ch.V1tb + off, b, m0, n0, nr, nc);
    sw.flush_rows(ch.Wb + off, b, m0, n0, nr, nc);  // W itself, from the same stage
  });
}

// Chain rule, second launch: D = F + Q (2 V1) + W S + S W over F in place,
// one output tile per workgroup, the three products added in one
// accumulator (S is symmetric, so its rows serve as the B operand of W S).
template <class C, typename T>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2))) void k_cnp_grad2(SideTable sd, int b,
                                                                                            Chain<T> ch) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tn = (b + C::BN - 1) / C::BN, tm = (b + C::BM - 1) / C::BM;
  const int u = xcd_unit(blockIdx.x, gridDim.x), z = u / (tm * tn);
  const float* qk;
  int r;
  sd.at(z, b, qk, r);
  const int m0 = (u % (tm * tn) / tn) * C::BM, n0 = (u % tn) * C::BN;
  if (m0 >= r || n0 >= r) return;  // the packing reads only the live corner
  const int64_t off = (int64_t)z * b * b, om = off + (int64_t)m0 * b, on = off + (int64_t)n0 * b;
  run_kk_sum3<C, T>(smem, ch.Qb + om, ch.V1tb + on, ch.Wb + om, ch.Sb + on, ch.Sb + om, ch.Wtb + on, r - m0, r - n0, b,
                    r, [&](auto& acc) {
    using CC = cfg_of<decltype(acc)>;
    const AccPos<CC> p = acc_pos<CC>();
#pragma unroll
    for (int ti = 0; ti < CC::TM; ++ti) {
      float f[CC::TN][16];
      load_at_acc_i<CC>(f, ch.F32 + off, b, m0, n0, r, r, ti);
#pragma unroll
      for (int tj = 0; tj < CC::TN; ++tj) {
        const int j = n0 + p.col(tj);
        if (j >= r) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int i = m0 + p.row(ti, e);
          if (i < r) ch.F32[off + (int64_t)i * b + j] = f[tj][e] + acc.v[ti][tj][e];
        }
      }
    }
  });
}

struct DqOut {
  float* dq[pxk::kMaxSides];
};

// dq[p(i, j)] = dQ[i][j] - dQ[j][i] for i < j (zero where j >= r), one 64 x 64
// tile on or above the diagonal per workgroup; the mirrored tile is staged
// through LDS so that reads and writes are row-contiguous.
__global__ __launch_bounds__(256) void k_pack_dq(SideTable sd, int b, const float* __restrict__ dQ32, DqOut out) {
  __shared__ float t[64][65];
  const int z = blockIdx.y;
  int s, blk, r;
  const float* qk;
  sd.at(z, b, s, blk, r, qk);
  // one workgroup per tile on or above the diagonal (ti <= tj)
  const int tiles = (b + 63) / 64;
  int w = blockIdx.x, ti = 0;
  while (w >= tiles - ti) {
    w -= tiles - ti;
    ++ti;
  }
  const int i0 = ti * 64, j0 = (ti + w) * 64;
  const float* D = dQ32 + (int64_t)z * b * b;
  const int c = threadIdx.x & 63, rr = threadIdx.x >> 6;
  // loads from positions clamped into the live corner, all issued up front
  float v[16], u[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int j = min(j0 + rr + 4 * k, r - 1), i = min(i0 + c, r - 1);
    v[k] = D[(int64_t)j * b + i];
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = min(i0 + rr + 4 * k, r - 1), j = min(j0 + c, r - 1);
    u[k] = D[(int64_t)i * b + j];
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) t[rr + 4 * k][c] = v[k];
  __syncthreads();
  float* dq = out.dq[s] + (int64_t)blk * ((int64_t)b * (b - 1) / 2);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int ii = rr + 4 * k, i = i0 + ii, j = j0 + c;
    if (i < j && j < b) dq[packed_slot(i, j, b)] = (j < r) ? u[k] - t[c][ii] : 0.f;
  }
}

template <typename T> struct CnpTile;
template <> struct CnpTile<bf16_t> { using C = TSq; };
template <> struct CnpTile<float> { using C = TF; };

inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

template <typename T>
hipError_t build_t(const SideTable& sd, int b, const GOut& go, void* ws, hipStream_t s) {
  using C = typename CnpTile<T>::C;
  const int nb = sd.first[sd.count];
  const size_t E = (size_t)nb * b * b;
  char* w = reinterpret_cast<char*>(ws);
  T* Qb = reinterpret_cast<T*>(w);
  w += al256(E * sizeof(T));
  T* Nb = reinterpret_cast<T*>(w);  // 2Q + S
  w += al256(E * sizeof(T));
  T* Sb = reinterpret_cast<T*>(w);  // third: the chain rule's reuse of a build reads S here
  const int lds = std::max(Lay<C, T>::BYTES, std::is_same<T, bf16_t>::value ? DSq::LDS_BYTES : 0);
  hipError_t e = allow_lds(k_cnp_square<C, T>, lds);
  if (e == hipSuccess) e = allow_lds(k_cnp_delta<C, T>, lds);
  static_assert((C::BM * (C::BN + 16 / (int)sizeof(T)) * (int)sizeof(T) + 15) / 16 * 16 + TStage<C, T>::BYTES <=
                    std::max(Lay<C, T>::BYTES, std::is_same<T, bf16_t>::value ? DSq::LDS_BYTES : 0),
                "the two output stages of k_cnp_delta fit the K loop's LDS");
  if (e != hipSuccess) return e;
  const unsigned t64 = cdiv(b, 64);
  k_unpack_q<T><<<dim3(t64 * (t64 + 1) / 2, nb), 256, 0, s>>>(sd, b, Qb);
  const unsigned grid = cdiv(b, C::BN) * cdiv(b, C::BM) * nb;
  k_cnp_square<C, T><<<grid, C::NT, lds, s>>>(sd, b, Qb, Nb, Sb);
  k_cnp_delta<C, T><<<grid, C::NT, lds, s>>>(sd, b, Nb, Sb, go);
  return hipGetLastError();
}

template <typename T> Chain<T> carve(void* ws, size_t E) {
  char* w = reinterpret_cast<char*>(ws);
  auto takeT = [&]() {
    T* p = reinterpret_cast<T*>(w);
    w += al256(E * sizeof(T));
    return p;
  };
  Chain<T> ch;
  ch.F32 = reinterpret_cast<float*>(w);
  w += al256(E * 4);
  ch.Qb = takeT();
  ch.Ub = takeT();
  ch.Utb = takeT();
  ch.Wb = takeT();
  ch.Wtb = takeT();
  ch.V1tb = takeT();
  ch.Sb = takeT();
  return ch;
}

SideTable make_table(int count, const float* const* q, const int* d, int b) {
  SideTable t{};
  t.count = count;
  t.first[0] = 0;
  for (int i = 0; i < count; ++i) {
    t.q[i] = q[i];
    t.d[i] = d[i];
    t.first[i + 1] = t.first[i] + pxk::nblocks(d[i], b);
  }
  return t;
}

template <typename T>
hipError_t grads_t(int count, const pxk::CnpSide* sides, int rows, int b, void* dg, int64_t zoff, int64_t total,
                   float* part, hipStream_t s) {
  using C = typename CnpTile<T>::C;
  if (count < 1 || count > pxk::kGradSides) return hipErrorInvalidValue;
  const float* q[pxk::kGradSides];
  int d[pxk::kGradSides];
  for (int k = 0; k < count; ++k) {
    q[k] = sides[k].q;
    d[k] = sides[k].d;
  }
  const SideTable sd = make_table(count, q, d, b);
  const int NB = sd.first[count];
  Chain<T> ch = carve<T>(dg, (size_t)total * b * b);
  GradSides<T> gs{};
  for (int k = 0; k < count; ++k) {
    gs.A[k] = reinterpret_cast<const T*>(sides[k].A);
    gs.B[k] = reinterpret_cast<const T*>(sides[k].B);
    gs.lda[k] = sides[k].lda;
    gs.ldb[k] = sides[k].ldb;
  }
  hipError_t e;
  const int S = pxk::block_grads_splits(sizeof(T) == 2 ? pxk::BF16 : pxk::F32, rows, NB, b);
  if (S > 0) {
    using CB = TGemmI;  // 256 x 256, 8 waves, MFMA / LDS interleave hint
    constexpr int lds = Lay<CB, T>::BYTES;
    e = allow_lds(k_block_grads_part<CB, T>, lds);
    if (e != hipSuccess) return e;
    k_block_grads_part<CB, T><<<cdiv(b, CB::BM) * cdiv(b, CB::BN) * NB * S, CB::NT, lds, s>>>(sd, gs, rows, b, S, part);
    const unsigned t64 = cdiv(b, 64);
    k_block_grads_reduce<T><<<dim3(t64 * t64, NB), 256, 0, s>>>(sd, b, S, part, ch, zoff);
    return hipGetLastError();
  }
  const unsigned grid = cdiv(b, C::BM) * cdiv(b, C::BN) * NB;
  if (rows % (2 * C::BK) == 0) {
    // two groups per tile, each over half of the tokens
    constexpr int lds = std::max(2 * Lay<C, T>::BYTES, C::BM * (C::BN + 4) * 4);
    e = allow_lds(k_block_grads<C, T, 2>, lds);
    if (e != hipSuccess) return e;
    k_block_grads<C, T, 2><<<grid, 2 * C::NT, lds, s>>>(sd, gs, rows, b, ch, zoff);
  } else {
    constexpr int lds = Lay<C, T>::BYTES;
    e = allow_lds(k_block_grads<C, T, 1>, lds);
    if (e != hipSuccess) return e;
    k_block_grads<C, T, 1><<<grid, C::NT, lds, s>>>(sd, gs, rows, b, ch, zoff);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t chain_t(const SideTable& sd, int b, void* dg, const DqOut& out, const void* build, hipStream_t s) {
  using C = typename CnpTile<T>::C;
  const int NB = sd.first[sd.count];
  const size_t E = (size_t)NB * b * b;
  Chain<T> ch = carve<T>(dg, E);
  const unsigned t64 = cdiv(b, 64);
  if (build) {
    // the dense Q and S = Q Q that the build left in its workspace (the same kernels on the same
    // operands form them here otherwise: the results are bit-identical)
    const char* w = reinterpret_cast<const char*>(build);
    ch.Qb = reinterpret_cast<const T*>(w);
    ch.Sb = const_cast<T*>(reinterpret_cast<const T*>(w + 2 * al256(E * sizeof(T))));
  } else {
    k_unpack_q<T><<<dim3(t64 * (t64 + 1) / 2, NB), 256, 0, s>>>(sd, b, const_cast<T*>(ch.Qb));
  }
  const int lds = std::max(Lay<C, T>::BYTES, std::is_same<T, bf16_t>::value ? DSq::LDS_BYTES : 0);
  hipError_t e = hipSuccess;
  const unsigned grid = cdiv(b, C::BN) * cdiv(b, C::BM) * NB;
  // the first launch's epilogue stages two transposed tiles
  const int lds1 = std::max(lds, 2 * TStage<C, T>::BYTES);
  e = allow_lds(k_cnp_grad1<C, T>, lds1);
  if (e == hipSuccess) e = allow_lds(k_cnp_grad2<C, T>, lds);
  if (e != hipSuccess) return e;
  const int kinds = build ? 1 : 2;
  k_cnp_grad1<C, T><<<kinds * grid, C::NT, lds1, s>>>(sd, b, ch, kinds);
  k_cnp_grad2<C, T><<<grid, C::NT, lds, s>>>(sd, b, ch);
  k_pack_dq<<<dim3(t64 * (t64 + 1) / 2, NB), 256, 0, s>>>(sd, b, ch.F32, out);
  return hipGetLastError();
}

}  // namespace

namespace pxk {

size_t cnp_build_ws_bytes(int dt, int64_t blocks, int b) {
  const size_t E = (size_t)blocks * b * b, es = dt_size(dt);
  return al256(E * es) * 3;  // Q, N = 2Q + S, S
}

size_t cnp_grad_bytes(int dt, int64_t blocks, int b) {
  const size_t E = (size_t)blocks * b * b, es = dt_size(dt);
  return al256(E * es) * 7 + al256(E * 4);
}

hipError_t cnp_build_batch(int dt, int count, const float* const* q, const int* d, int b, void* const* g, void* ws,
                           hipStream_t s) {
  if (count < 1 || count > kMaxSides) return hipErrorInvalidValue;
  const SideTable sd = make_table(count, q, d, b);
  GOut go{};
  for (int i = 0; i < count; ++i) go.g[i] = g[i];
  if (dt == BF16) return build_t<bf16_t>(sd, b, go, ws, s);
  return build_t<float>(sd, b, go, ws, s);
}

int block_grads_splits(int dt, int rows, int blocks, int b) {
  // bf16 blocks of a multiple of 256: 256 x 256 tiles, one workgroup per CU
  // at a time.  The token range is cut into S splits of whole 64-row K tiles;
  // S minimises rounds * K tiles per workgroup (rounds = workgroups / CUs,
  // rounded up) plus the cost of writing and re-reading the S partials
  // (about 0.2 K-tile times per 512 x 512 fp32 block and split).
  if (dt != BF16 || b % 256 != 0 || rows <= 0) return 0;
  if (rows % 64 != 0) return 1;
  constexpr int kCUs = 256;
  const int64_t tiles = (int64_t)(b / 256) * (b / 256) * blocks;
  const int KT = rows / 64;
  const double per_split = 0.2 * blocks * ((double)b / 512) * ((double)b / 512);
  int best = 1;
  double best_cost = 0;
  for (int S = 1; S <= 16 && S <= KT; ++S) {
    const int64_t rounds = (tiles * S + kCUs - 1) / kCUs;
    const double cost = (double)rounds * ((KT + S - 1) / S) + per_split * S;
    if (S == 1 || cost < best_cost) {
      best = S;
      best_cost = cost;
    }
  }
  return best;
}

size_t block_grads_part_bytes(int dt, int rows, int blocks, int b) {
  const int S = block_grads_splits(dt, rows, blocks, b);
  return (size_t)S * blocks * b * b * 4;
}

hipError_t block_grads(int cdt, const CnpSide* sides, int rows, int b, void* dg, int64_t zoff, int64_t total,
                       float* part, hipStream_t s) {
  return block_grads_n(cdt, 2, sides, rows, b, dg, zoff, total, part, s);
}

hipError_t block_grads_n(int cdt, int count, const CnpSide* sides, int rows, int b, void* dg, int64_t zoff,
                         int64_t total, float* part, hipStream_t s) {
  if (cdt == BF16) return grads_t<bf16_t>(count, sides, rows, b, dg, zoff, total, part, s);
  return grads_t<float>(count, sides, rows, b, dg, zoff, total, part, s);
}

hipError_t cnp_chain_batch(int cdt, int count, const float* const* q, const int* d, int b, void* dg, float* const* dq,
                           hipStream_t s, const void* build) {
  if (count < 1 || count > kMaxSides) return hipErrorInvalidValue;
  const SideTable sd = make_table(count, q, d, b);
  DqOut out{};
  for (int i = 0; i < count; ++i) out.dq[i] = dq[i];
  if (cdt == BF16) return chain_t<bf16_t>(sd, b, dg, out, build, s);
  return chain_t<float>(sd, b, dg, out, build, s);
}

}  // namespace pxk
