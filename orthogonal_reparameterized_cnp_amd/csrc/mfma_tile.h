// Workgroup-level MFMA tile loop for gfx950 (CDNA4, wave64).
//
// One workgroup computes a BM x BN tile of C = A * B with fp32 accumulation.
// Both operands are staged in LDS as [rows][BK] with K contiguous, which is the
// order in which v_mfma_f32_32x32x16_bf16 (bf16 path) and v_mfma_f32_32x32x2f32
// (fp32 path) consume them: each lane supplies a run of consecutive K values
// for one row of A and one column of B.  Operand loaders turn whatever layout
// the source has (K contiguous, or M/N contiguous and transposed on the way
// into LDS, or generated on the fly) into that LDS tile; the K loop is double
// buffered in LDS with the next tile's global loads issued before the MFMAs
// of the current one, so one barrier per K tile suffices.
#pragma once

#include "common.h"

namespace px {

template <int BM_, int BN_, int BK_, int WM_, int WN_, bool PF2 = false, bool IG = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr bool PREFETCH2 = PF2;  // two K tiles of global loads in flight
  static constexpr bool INTERLEAVE = IG;  // ask the compiler to interleave MFMAs and LDS reads
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
};

// LDS row pitch: BK plus 16 bytes, so that the 8 lanes served together by a
// 128-bit LDS read (8 consecutive rows, same K offset) hit 8 distinct 16-byte
// bank groups.
template <typename T> struct LdsPad;
template <> struct LdsPad<bf16_t> { static constexpr int v = 8; };
template <> struct LdsPad<float> { static constexpr int v = 4; };

template <class C, typename T> struct Lay {
  static constexpr int LDK = C::BK + LdsPad<T>::v;
  static constexpr int A_ELEMS = C::BM * LDK;
  static constexpr int B_ELEMS = C::BN * LDK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int BYTES = 2 * STAGE * (int)sizeof(T);
};

template <class C> struct Acc {
  using Cfg = C;
  f32x16_v v[C::TM][C::TN];
  PX_DEV void zero() {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) v[i][j][e] = 0.f;
  }
};

// Coordinates of accumulator register e of MFMA tile (i, j) within the workgroup
// tile: a 32x32 fp32 result is spread so that lane l owns column l % 32 and the
// rows 8*(e/4) + 4*(l/32) + e%4.
template <class C> struct AccPos {
  int wm, wn, lane;
  PX_DEV int row(int i, int e) const { return wm * C::WTM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }
  PX_DEV int col(int j) const { return wn * C::WTN + j * 32 + (lane & 31); }
};

template <class C, bool IGLP = false>
PX_DEV void mma_stage(const bf16_t* As, const bf16_t* Bs, Acc<C>& acc, int wm, int wn, int lane) {
  constexpr int LDK = Lay<C, bf16_t>::LDK;
  constexpr int KS = C::BK / 16;
  const int r = lane & 31, kg = (lane >> 5) * 8;
  const bf16_t* pa = As + (wm * C::WTM + r) * LDK + kg;
  const bf16_t* pb = Bs + (wn * C::WTN + r) * LDK + kg;
  // fragments of k-step s + 1 are read while the MFMAs of step s run
  bf16x8_v a[2][C::TM], b[2][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) a[0][i] = *reinterpret_cast<const bf16x8_v*>(pa + i * 32 * LDK);
#pragma unroll
  for (int j = 0; j < C::TN; ++j) b[0][j] = *reinterpret_cast<const bf16x8_v*>(pb + j * 32 * LDK);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        a[cur ^ 1][i] = *reinterpret_cast<const bf16x8_v*>(pa + i * 32 * LDK + (ks + 1) * 16);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        b[cur ^ 1][j] = *reinterpret_cast<const bf16x8_v*>(pb + j * 32 * LDK + (ks + 1) * 16);
    }
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j], acc.v[i][j], 0, 0, 0);
    if constexpr (IGLP) __builtin_amdgcn_iglp_opt(1);
  }
}

template <class C, bool IGLP = false>
PX_DEV void mma_stage(const float* As, const float* Bs, Acc<C>& acc, int wm, int wn, int lane) {
  constexpr int LDK = Lay<C, float>::LDK;
  const int r = lane & 31, kg = (lane >> 5) * 4;
#pragma unroll
  for (int kk = 0; kk < C::BK; kk += 8) {
    f32x4_v a[C::TM], b[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      a[i] = *reinterpret_cast<const f32x4_v*>(As + (wm * C::WTM + i * 32 + r) * LDK + kk + kg);
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      b[j] = *reinterpret_cast<const f32x4_v*>(Bs + (wn * C::WTN + j * 32 + r) * LDK + kk + kg);
    // element e of the lane's 4 K values feeds the e-th MFMA; the two lane
    // halves cover K offsets {e, 4 + e}, so the four MFMAs cover all 8.
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc.v[i][j], 0, 0, 0);
  }
}

struct NoHook {
  template <typename T> PX_DEV void operator()(int, const T*) const {}
};

// K loop.  `K` is the contraction length; loaders zero-fill past it.  After the
// MFMAs of K tile kt, hook(kt, A tile in LDS) runs (before the barrier that
// lets the tile be overwritten).
template <bool FAST, class C, typename T, class LA, class LB, class H>
PX_DEV void mainloop_t(T* lds, LA& la, LB& lb, int KT, Acc<C>& acc, int wm, int wn, int lane, const H& hook) {
  using L = Lay<C, T>;
  la.template fetch<FAST>(0);
  lb.template fetch<FAST>(0);
  la.stash(lds);
  lb.stash(lds + L::A_ELEMS);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    T* cur = lds + (kt & 1) * L::STAGE;
    T* nxt = lds + ((kt + 1) & 1) * L::STAGE;
    const bool more = kt + 1 < KT;
    if (more) {
      la.template fetch<FAST>((kt + 1) * C::BK);
      lb.template fetch<FAST>((kt + 1) * C::BK);
    }
    // the interleave hint only in the unchecked loop without a per-tile hook (with either, the
    // compiler's scheduling of the larger region takes minutes and tens of GB)
    mma_stage<C, FAST && C::INTERLEAVE && std::is_same<H, NoHook>::value>(cur, cur + L::A_ELEMS, acc, wm, wn, lane);
    hook(kt, cur);
    if (more) {
      la.stash(nxt);
      lb.stash(nxt + L::A_ELEMS);
    }
    __syncthreads();
  }
}

// Two register sets per operand: the global loads of K tile kt + 2 are issued
// while tile kt is multiplied, so each load has two tiles of MFMA time to land.
template <bool FAST, class C, typename T, class LA, class LB, class H>
PX_DEV void mainloop2_t(T* lds, LA& la0, LB& lb0, int KT, Acc<C>& acc, int wm, int wn, int lane, const H& hook) {
  using L = Lay<C, T>;
  LA la1 = la0;
  LB lb1 = lb0;
  la0.template fetch<FAST>(0);
  lb0.template fetch<FAST>(0);
  la0.stash(lds);
  lb0.stash(lds + L::A_ELEMS);
  if (KT > 1) {
    la0.template fetch<FAST>(C::BK);
    lb0.template fetch<FAST>(C::BK);
  }
  __syncthreads();
  // step(kt): tile kt + 1 sits in set P, tile kt + 2 goes into set Q
  auto step = [&](int kt, LA& laP, LB& lbP, LA& laQ, LB& lbQ) {
    T* cur = lds + (kt & 1) * L::STAGE;
    T* nxt = lds + ((kt + 1) & 1) * L::STAGE;
    if (kt + 2 < KT) {
      laQ.template fetch<FAST>((kt + 2) * C::BK);
      lbQ.template fetch<FAST>((kt + 2) * C::BK);
    }
    mma_stage<C>(cur, cur + L::A_ELEMS, acc, wm, wn, lane);
    hook(kt, cur);
    if (kt + 1 < KT) {
      laP.stash(nxt);
      lbP.stash(nxt + L::A_ELEMS);
    }
    __syncthreads();
  };
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, la0, lb0, la1, lb1);
    if (kt + 1 < KT) step(kt + 1, la1, lb1, la0, lb0);
  }
}

// acc = A B^T over K; with zero false, acc += A B^T
template <class C, typename T, class LA, class LB, class H = NoHook>
PX_DEV void mainloop(T* lds, LA& la, LB& lb, int K, Acc<C>& acc, int wm, int wn, int lane, const H& hook = H(),
                     bool zero = true) {
  if (zero) acc.zero();
  const int KT = (K + C::BK - 1) / C::BK;
  if (KT <= 0) return;
  // tiles entirely inside both operands take the loop without bounds checks
  if (la.full() && lb.full() && K % C::BK == 0) {
    if constexpr (C::PREFETCH2)
      mainloop2_t<true, C>(lds, la, lb, KT, acc, wm, wn, lane, hook);
    else
      mainloop_t<true, C>(lds, la, lb, KT, acc, wm, wn, lane, hook);
  } else {
    mainloop_t<false, C>(lds, la, lb, KT, acc, wm, wn, lane, hook);
  }
}

// ---------------------------------------------------------------------------
// 8-element chunks held in registers between the global load and the LDS store
// ---------------------------------------------------------------------------
template <typename D> struct Chunk8;
template <> struct Chunk8<bf16_t> {
  uint4 w;  // 8 bf16
  PX_DEV void zero() { w = make_uint4(0, 0, 0, 0); }
  PX_DEV void set(int e, bf16_t v) {
    uint32_t* p = reinterpret_cast<uint32_t*>(&w);
    const int s = (e & 1) * 16;
    p[e >> 1] = (p[e >> 1] & ~(0xffffu << s)) | ((uint32_t)v << s);
  }
  PX_DEV bf16_t get(int e) const {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(&w);
    return (bf16_t)(p[e >> 1] >> ((e & 1) * 16));
  }
};
template <> struct Chunk8<float> {
  float4 a, b;
  PX_DEV void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  PX_DEV void set(int e, float v) { (e < 4 ? reinterpret_cast<float*>(&a)[e] : reinterpret_cast<float*>(&b)[e - 4]) = v; }
  PX_DEV float get(int e) const { return e < 4 ? reinterpret_cast<const float*>(&a)[e] : reinterpret_cast<const float*>(&b)[e - 4]; }
};

// vector load of 8 consecutive source elements (address aligned to 8 elements)
template <typename D, typename S> struct Load8;
template <> struct Load8<bf16_t, bf16_t> {
  static PX_DEV void go(const bf16_t* p, Chunk8<bf16_t>& c) { c.w = *reinterpret_cast<const uint4*>(p); }
};
template <> struct Load8<float, float> {
  static PX_DEV void go(const float* p, Chunk8<float>& c) {
    c.a = reinterpret_cast<const float4*>(p)[0];
    c.b = reinterpret_cast<const float4*>(p)[1];
  }
};
template <> struct Load8<float, bf16_t> {
  static PX_DEV void go(const bf16_t* p, Chunk8<float>& c) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) c.set(e, __uint_as_float((e & 1) ? (u[e >> 1] & 0xffff0000u) : (u[e >> 1] << 16)));
  }
};
template <> struct Load8<bf16_t, float> {
  static PX_DEV void go(const float* p, Chunk8<bf16_t>& c) {
    const float4 x = reinterpret_cast<const float4*>(p)[0], y = reinterpret_cast<const float4*>(p)[1];
    c.w.x = (uint32_t)f2bf(x.x) | ((uint32_t)f2bf(x.y) << 16);
    c.w.y = (uint32_t)f2bf(x.z) | ((uint32_t)f2bf(x.w) << 16);
    c.w.z = (uint32_t)f2bf(y.x) | ((uint32_t)f2bf(y.y) << 16);
    c.w.w = (uint32_t)f2bf(y.z) | ((uint32_t)f2bf(y.w) << 16);
  }
};
template <typename D> struct Load8<D, int8_t> {
  static PX_DEV void go(const int8_t* p, Chunk8<D>& c) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int8_t v = (int8_t)(((e < 4 ? w.x : w.y) >> ((e & 3) * 8)) & 0xff);
      c.set(e, Cvt<D, int8_t>::f(v));
    }
  }
};

template <typename S> PX_DEV bool aligned8(const S* p, int64_t ld) {
  return ((reinterpret_cast<uintptr_t>(p) % (8 * sizeof(S))) == 0) && (ld % 8 == 0);
}

// ---------------------------------------------------------------------------
// Loader: source rows with K contiguous.  Tile row `r` is source row r, K
// offset k is column k (relative to `base`).  Rows >= rows or K >= K read as 0.
// ---------------------------------------------------------------------------
template <int ROWS, int BK, int NT, typename S, typename D>
struct LoadK {
  static constexpr int CPR = BK / 8;
  static constexpr int TOT = ROWS * CPR;
  static constexpr int NCH = (TOT + NT - 1) / NT;
  const S* base;
  int64_t ld;
  int rows, K;
  bool vec;
  Chunk8<D> c[NCH];

  PX_DEV void init(const S* base_, int64_t ld_, int rows_, int K_) {
    base = base_;
    ld = ld_;
    rows = rows_;
    K = K_;
    vec = aligned8(base_, ld_);
  }
  PX_DEV bool full() const { return vec && rows >= ROWS; }
  template <bool FAST> PX_DEV void fetch(int k0) {
    if constexpr (FAST) {  // whole tile inside: unconditional vector loads
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ch = (int)(threadIdx.x % NT) + i * NT;
        if (TOT % NT != 0 && ch >= TOT) break;
        Load8<D, S>::go(base + (int64_t)(ch / CPR) * ld + k0 + (ch % CPR) * 8, c[i]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = (int)(threadIdx.x % NT) + i * NT;
      if (TOT % NT != 0 && ch >= TOT) break;
      const int r = ch / CPR, k = k0 + (ch % CPR) * 8;
      const S* p = base + (int64_t)r * ld + k;
      if (r < rows && k + 8 <= K && vec) {
        Load8<D, S>::go(p, c[i]);
      } else {
        c[i].zero();
        if (r < rows)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k + e < K) c[i].set(e, Cvt<D, S>::f(p[e]));
      }
    }
  }
  PX_DEV void stash(D* lds) const {
    constexpr int LDK = BK + LdsPad<D>::v;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = (int)(threadIdx.x % NT) + i * NT;
      if (TOT % NT != 0 && ch >= TOT) break;
      const int r = ch / CPR, kc = (ch % CPR) * 8;
      if constexpr (sizeof(D) == 2) {
        *reinterpret_cast<uint4*>(lds + r * LDK + kc) = c[i].w;
      } else {
        reinterpret_cast<float4*>(lds + r * LDK + kc)[0] = c[i].a;
        reinterpret_cast<float4*>(lds + r * LDK + kc)[1] = c[i].b;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Loader: source with the tile's row index contiguous (element (k, r) at
// base[k * ld + r]); transposed into the [row][K] LDS tile.  Each thread moves
// units of 4 K values x 8 rows: four 8-wide global loads along the rows, then
// eight 4-wide LDS stores along K.  Consecutive lanes take consecutive K quads
// of the same 8 rows, so the 16 lanes served together by a 64-bit LDS store
// write one contiguous 128-byte row segment (no bank conflicts).
// ---------------------------------------------------------------------------
template <int ROWS, int BK, int NT, typename S, typename D>
struct LoadMN {
  static constexpr int MC = ROWS / 8;
  static constexpr int KQ = BK / 4;
  static constexpr int TOT = MC * KQ;
  static constexpr int NU = (TOT + NT - 1) / NT;
  const S* base;
  int64_t ld;
  int rows, K;
  bool vec;
  Chunk8<D> c[NU][4];

  PX_DEV void init(const S* base_, int64_t ld_, int rows_, int K_) {
    base = base_;
    ld = ld_;
    rows = rows_;
    K = K_;
    vec = aligned8(base_, ld_);
  }
  PX_DEV bool full() const { return vec && rows >= ROWS; }
  template <bool FAST> PX_DEV void fetch(int k0) {
    if constexpr (FAST) {  // whole tile inside: unconditional vector loads
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int unit = (int)(threadIdx.x % NT) + u * NT;
        if (TOT % NT != 0 && unit >= TOT) break;
        const S* p = base + (int64_t)(k0 + (unit % KQ) * 4) * ld + (unit / KQ) * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) Load8<D, S>::go(p + (int64_t)kk * ld, c[u][kk]);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int unit = (int)(threadIdx.x % NT) + u * NT;
      if (TOT % NT != 0 && unit >= TOT) break;
      const int r0 = (unit / KQ) * 8, kq = k0 + (unit % KQ) * 4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k = kq + kk;
        const S* p = base + (int64_t)k * ld + r0;
        if (k < K && r0 + 8 <= rows && vec) {
          Load8<D, S>::go(p, c[u][kk]);
        } else {
          c[u][kk].zero();
          if (k < K)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (r0 + e < rows) c[u][kk].set(e, Cvt<D, S>::f(p[e]));
        }
      }
    }
  }
  PX_DEV void stash(D* lds) const {
    constexpr int LDK = BK + LdsPad<D>::v;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int unit = (int)(threadIdx.x % NT) + u * NT;
      if (TOT % NT != 0 && unit >= TOT) break;
      const int r0 = (unit / KQ) * 8, kq = (unit % KQ) * 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        D* p = lds + (r0 + e) * LDK + kq;
        if constexpr (sizeof(D) == 2) {
          uint2 v;
          v.x = (uint32_t)c[u][0].get(e) | ((uint32_t)c[u][1].get(e) << 16);
          v.y = (uint32_t)c[u][2].get(e) | ((uint32_t)c[u][3].get(e) << 16);
          *reinterpret_cast<uint2*>(p) = v;
        } else {
          *reinterpret_cast<float4*>(p) = make_float4(c[u][0].get(e), c[u][1].get(e), c[u][2].get(e), c[u][3].get(e));
        }
      }
    }
  }
};


// ---------------------------------------------------------------------------
// Transposing loader for bf16 tiles of R rows x 64 K whose source has the row
// index contiguous (element (k, r) at base[k * ld + r]), into an unpadded LDS
// tile [R][64] of 128-byte rows whose 16-byte chunks are XOR-swizzled by
// ((r / 2) ^ (r / 16)) % 8.  A unit is 8 rows x 8 K values: eight 16-byte
// global loads along the rows, an 8 x 8 transpose of 16-bit values in
// registers (v_perm), then eight 16-byte LDS stores along K, one chunk each.
// Units are dealt so that lanes 0-31 and 32-63 of a wave each read 256
// consecutive rows of one K (whole 128-byte lines).  NT2 threads load one
// tile: a contiguous range of thread indices starting at a multiple of NT2.
// The whole tile must lie inside the source (no bounds checks).
// ---------------------------------------------------------------------------
PX_DEV int tswz_chunk(int r, int c) { return r * 8 + (c ^ (((r >> 1) ^ (r >> 4)) & 7)); }
template <int R, int NT2> struct LoadT {
  static constexpr int CG = R / 8;        // 8-row chunks
  static constexpr int UNITS = CG * 8;    // (row chunk, K octet)
  static constexpr int NU = UNITS / NT2;
  static_assert(UNITS % NT2 == 0 && NU >= 1 && CG % 32 == 0, "whole units per thread, 32 row chunks per half wave");
  const bf16_t* base;
  int64_t ld;
  uint4 c[NU][8];
  PX_DEV void init(const bf16_t* b, int64_t l) {
    base = b;
    ld = l;
  }
  // unit u: row chunk u % CG (rows 8 (u % CG) .. + 7), K octet u / CG
  PX_DEV void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = (int)(threadIdx.x % NT2) + i * NT2, cg = u % CG, ko = u / CG;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        c[i][kk] = *reinterpret_cast<const uint4*>(base + (int64_t)(k0 + 8 * ko + kk) * ld + 8 * cg);
    }
  }
  PX_DEV static uint32_t word(const uint4& v, int w) { return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w; }
  PX_DEV void stash(char* tile) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = (int)(threadIdx.x % NT2) + i * NT2, cg = u % CG, ko = u / CG;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // row 8 cg + e: the 16-bit element e of the eight loads, in K order (low halves for even e)
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint4 v;
        v.x = __builtin_amdgcn_perm(word(c[i][1], e / 2), word(c[i][0], e / 2), sel);
        v.y = __builtin_amdgcn_perm(word(c[i][3], e / 2), word(c[i][2], e / 2), sel);
        v.z = __builtin_amdgcn_perm(word(c[i][5], e / 2), word(c[i][4], e / 2), sel);
        v.w = __builtin_amdgcn_perm(word(c[i][7], e / 2), word(c[i][6], e / 2), sel);
        *reinterpret_cast<uint4*>(tile + 16 * tswz_chunk(8 * cg + e, ko)) = v;
      }
    }
  }
};

// MFMAs of one 64-K step from two LoadT tiles (A rows = output rows, B rows =
// output columns); the fragments of each 16-K step are read before its MFMAs.
template <class C>
PX_DEV void mma_stage_t(const char* As, const char* Bs, Acc<C>& acc, int wm, int wn, int lane) {
  static_assert(C::BK == 64, "64-K tiles");
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8_v a[C::TM], b[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      a[i] = *reinterpret_cast<const bf16x8_v*>(As + 16 * tswz_chunk(wm * C::WTM + 32 * i + r, 2 * ks + h));
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      b[j] = *reinterpret_cast<const bf16x8_v*>(Bs + 16 * tswz_chunk(wn * C::WTN + 32 * j + r, 2 * ks + h));
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.v[i][j], 0, 0, 0);
  }
}

}  // namespace px
