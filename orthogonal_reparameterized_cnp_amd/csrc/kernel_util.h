// Helpers shared by the kernel sources: tile shapes, accumulator iteration and
// launch utilities.
#pragma once

#include <algorithm>
#include <type_traits>

#include "mfma_dma.h"
#include "mfma_tile.h"
#include "poetx_internal.h"

namespace px {

using TGemm = Tile<256, 256, 64, 4, 2>;  // bf16: W~ contractions and block products (8 waves of 64 x 128)
using TGemmI = Tile<256, 256, 64, 4, 2, false, true>;  // the same with the MFMA / LDS interleave hint (bf16 W~)
using TBig = Tile<256, 128, 64, 2, 2>;   // bf16: narrow contractions
using TSq = Tile<128, 128, 64, 2, 2>;   // bf16: block gradients, CNP (b x b outputs)
// direct-to-LDS configurations (K-contiguous operands, interior tiles)
using DGemm = DCfg<256, 256, 64, 2, 4, 2, false, false, true>;  // 8 waves, same block size as TGemm
using DSq = DCfg<128, 128, 64, 2, 2, 2, false, false, true>;    // 4 waves, same block size as TSq
using TNarrow = Tile<256, 128, 64, 4, 2, false, true>;            // bf16 NT narrow contractions, 8 waves
using DNarrow = DCfg<256, 128, 64, 4, 2, 2, false, false, true>;  // its direct-to-LDS loop (waves of 64 x 64)
using TF = Tile<64, 64, 32, 2, 2>;      // fp32: small layers
using TFM = Tile<128, 128, 32, 2, 2>;   // fp32: merge products

// wave position inside the C::NT threads that share one tile (a workgroup may
// hold several such groups, each with its own K range)
template <class C> PX_DEV AccPos<C> acc_pos() {
  const int w = (int)(threadIdx.x % C::NT) >> 6;
  return AccPos<C>{w / C::WN, w % C::WN, (int)(threadIdx.x & 63)};
}

// f(row, col, value) for every accumulator element (tile-local coordinates)
template <class C, class F> PX_DEV void each_acc(const Acc<C>& acc, F&& f) {
  const AccPos<C> p = acc_pos<C>();
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int c = p.col(j);
#pragma unroll
      for (int e = 0; e < 16; ++e) f(p.row(i, e), c, acc.v[i][j][e]);
    }
}

// f(row0, col, v[4]) for runs of 4 consecutive rows of one column, the unit in
// which a lane owns its accumulators (rows row0 .. row0 + 3)
template <class C, class F> PX_DEV void each_acc4(const Acc<C>& acc, F&& f) {
  const AccPos<C> p = acc_pos<C>();
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int c = p.col(j);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float v[4] = {acc.v[i][j][4 * g], acc.v[i][j][4 * g + 1], acc.v[i][j][4 * g + 2], acc.v[i][j][4 * g + 3]};
        f(p.row(i, 4 * g), c, v);
      }
    }
}

// store 4 consecutive elements (one 8- or 16-byte vector store when aligned)
template <typename T> PX_DEV void store4(T* p, const float v[4]) {
  if constexpr (sizeof(T) == 2) {
    if ((reinterpret_cast<uintptr_t>(p) & 7) == 0) {
      uint2 w;
      w.x = f2bf2(v[0], v[1]);
      w.y = f2bf2(v[2], v[3]);
      *reinterpret_cast<uint2*>(p) = w;
    } else {
      for (int e = 0; e < 4; ++e) p[e] = f2bf(v[e]);
    }
  } else {
    if ((reinterpret_cast<uintptr_t>(p) & 15) == 0)
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else
      for (int e = 0; e < 4; ++e) p[e] = v[e];
  }
}

// Store the workgroup's accumulator tile (times scale(col)) to out[rows][cols]
// (row pitch ldo) through LDS: lanes write their accumulators into a padded
// row-major LDS tile, then the workgroup copies rows out in 16-byte chunks.
// `lds` must hold BM x (BN + 16 B) elements of OT; callers pass the mainloop's
// LDS, which is free once the loop has ended.
template <class C, typename OT, class Scale>
PX_DEV void store_tile(const Acc<C>& acc, void* lds, OT* out, int64_t ldo, int rows, int cols, const Scale& scale) {
  constexpr int V = 16 / (int)sizeof(OT);
  constexpr int PITCH = C::BN + V;
  OT* t = reinterpret_cast<OT*>(lds);
  const AccPos<C> p = acc_pos<C>();
  __syncthreads();
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int c = p.col(j);
    const float sc = scale(c);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) t[p.row(i, e) * PITCH + c] = from_f32<OT>(acc.v[i][j][e] * sc);
  }
  __syncthreads();
  constexpr int CPR = C::BN / V;
  const bool vec = (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (ldo % V == 0);
  const bool whole = vec && rows >= C::BM && cols >= C::BN;
  for (int ch = threadIdx.x; ch < C::BM * CPR; ch += C::NT) {
    const int r = ch / CPR, cc = (ch % CPR) * V;
    const OT* src = t + r * PITCH + cc;
    OT* dst = out + (int64_t)r * ldo + cc;
    if (whole || (vec && r < rows && cc + V <= cols)) {
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    } else if (r < rows) {
      for (int e = 0; e < V; ++e)
        if (cc + e < cols) dst[e] = src[e];
    }
  }
}

// store_tile for any value per accumulator element: f(i, j, e) is the value
// of the calling lane's element (i, j, e) (tile row p.row(i, e), column
// p.col(j)).  Staged in the LDS rows [0, BM) x (BN + 16 B), then written out in
// 16-byte chunks; rows >= rows and columns >= cols are not written.
template <class C, typename OT, class F>
PX_DEV void store_tile_fn(void* lds, OT* out, int64_t ldo, int rows, int cols, const F& f) {
  constexpr int V = 16 / (int)sizeof(OT);
  constexpr int PITCH = C::BN + V;
  OT* t = reinterpret_cast<OT*>(lds);
  const AccPos<C> p = acc_pos<C>();
  __syncthreads();
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int c = p.col(j);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) t[p.row(i, e) * PITCH + c] = from_f32<OT>(f(i, j, e));
  }
  __syncthreads();
  constexpr int CPR = C::BN / V;
  const bool vec = (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (ldo % V == 0);
  const bool whole = vec && rows >= C::BM && cols >= C::BN;
  for (int ch = threadIdx.x; ch < C::BM * CPR; ch += C::NT) {
    const int r = ch / CPR, cc = (ch % CPR) * V;
    const OT* src = t + r * PITCH + cc;
    OT* dst = out + (int64_t)r * ldo + cc;
    if (whole || (vec && r < rows && cc + V <= cols)) {
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    } else if (r < rows) {
      for (int e = 0; e < V; ++e)
        if (cc + e < cols) dst[e] = src[e];
    }
  }
}

template <class A> using cfg_of = typename std::decay_t<A>::Cfg;

// f[i][j][e] = src[(row0 + row) * ld + col0 + col] at the calling lane's
// accumulator positions, with row0 + row and col0 + col clamped to
// [0, rmax) x [0, cmax) so that every load is in range and none is predicated:
// all of them are issued before the first is used.
template <class C, typename S>
PX_DEV void load_at_acc(float (&f)[C::TM][C::TN][16], const S* src, int64_t ld, int row0, int col0, int rmax,
                        int cmax) {
  const AccPos<C> p = acc_pos<C>();
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int c = min(col0 + p.col(j), cmax - 1);
#pragma unroll
      for (int e = 0; e < 16; ++e) f[i][j][e] = to_f32<S>(src[(int64_t)min(row0 + p.row(i, e), rmax - 1) * ld + c]);
    }
}

// the same for the accumulator row group ti only: f[j][e] for tile (ti, j)
template <class C, typename S>
PX_DEV void load_at_acc_i(float (&f)[C::TN][16], const S* src, int64_t ld, int row0, int col0, int rmax, int cmax,
                          int ti) {
  const AccPos<C> p = acc_pos<C>();
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int c = min(col0 + p.col(j), cmax - 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) f[j][e] = to_f32<S>(src[(int64_t)min(row0 + p.row(ti, e), rmax - 1) * ld + c]);
  }
}

// true when a K-contiguous operand tile can be copied with 16-byte DMA:
// all rows present, base 16-byte aligned, row pitch a multiple of 8 elements
PX_DEV bool dma_rows_ok(const void* base, int64_t ld, int rows_avail, int rows_tile) {
  return rows_avail >= rows_tile && (reinterpret_cast<uintptr_t>(base) % 16 == 0) && (ld % 8 == 0);
}

// dynamic LDS for a kernel: the double-buffered operand tiles, or the
// epilogue's staging tile if that is larger
template <class C, typename T, typename OT> constexpr int smem_bytes() {
  constexpr int epi = C::BM * (C::BN + 16 / (int)sizeof(OT)) * (int)sizeof(OT);
  return Lay<C, T>::BYTES > epi ? Lay<C, T>::BYTES : epi;
}

template <class CD> constexpr int dma_smem_bytes() {
  if constexpr (std::is_same<CD, void>::value) {
    return 0;
  } else {
    // bf16 staging of the whole tile (either orientation)
    constexpr int epi = (CD::BM > CD::BN ? CD::BM : CD::BN) * ((CD::BM > CD::BN ? CD::BM : CD::BN) + 8) * 2;
    return CD::LDS_BYTES > epi ? CD::LDS_BYTES : epi;
  }
}

struct Unit {
  PX_DEV float operator()(int) const { return 1.f; }
};

// Kernels whose dynamic LDS exceeds the default 64 KB must opt in.
template <typename K> hipError_t allow_lds(K kernel, int bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace px
