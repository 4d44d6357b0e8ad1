// bf16 MFMA tile loop fed by direct global -> LDS loads (gfx950).
//
// Each operand tile is copied into LDS by global_load_lds_dwordx4: every lane
// moves 16 bytes and a wave's instruction fills 1 KB of LDS in lane order, so
// no VGPRs hold tiles in flight and a ring of STAGES tiles keeps STAGES - 1 K
// tiles of loads outstanding while the MFMAs consume the oldest one.
//
// LDS layouts (16-byte chunks XOR-swizzled so that fragment reads are free of
// bank conflicts; the swizzle is applied on the global side of the copy by
// choosing which chunk each lane fetches):
//  * K-contiguous operand (source rows are tile rows): [rows][BK].  Fragments
//    are 128-bit reads of 8 consecutive K for one row.
//  * M/N-contiguous operand (source rows are K): [BK][rows], untransposed.
//    Fragments come from two ds_read_b64_tr_b16: within each group of 16 lanes
//    the instruction hands lane i the i-th 16-bit value of the 4-element
//    pieces read by lanes 4j + i/4 (j = 0..3).  Lane s of the group therefore
//    reads K row kb + s/4 at columns c0 + 4(s%4) .. +3, and lane i receives
//    column c0 + i at K rows kb .. kb + 3, which is the MFMA operand layout.
// Only tiles that lie entirely inside both operands with K a multiple of BK
// use this loop; the caller falls back to the checked loop otherwise.
// The library's kernels use this loop with K-contiguous operands only.
#pragma once

#include "mfma_tile.h"

namespace px {

template <int BM_, int BN_, int BK_, int WM_, int WN_, int S_, bool AMN_, bool BMN_, bool IL_ = false>
struct DCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, STAGES = S_;
  static constexpr bool INTERLEAVE = IL_;
  static constexpr bool A_MN = AMN_, B_MN = BMN_;
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int LA = A_BYTES / 1024 / NW, LB = B_BYTES / 1024 / NW;  // DMA instructions per wave per tile
  static constexpr int L = LA + LB;
  static constexpr bool PREFETCH2 = false;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "tile must split into 1 KB per wave");
  static_assert(BK % 16 == 0 && BK <= 64, "BK must be 16, 32, 48 or 64");
  static_assert((STAGES - 2) * L <= 63, "outstanding loads must fit the vmcnt counter");
};

// ---- raw buffer access ------------------------------------------------------
// A resource of 64-bit base, byte size and the gfx9 format
// word.  Reads past the size return zeros and writes past it are dropped,
// which bounds a ragged last row tile without per-row checks.
typedef int i32x4_v __attribute__((ext_vector_type(4)));
PX_DEV i32x4_v buffer_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_v r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)min(bytes, (int64_t)0x7fffffff));
  r[3] = 0x00020000;
  return r;
}
__device__ void raw_buffer_load_lds(i32x4_v rsrc, __attribute__((address_space(3))) uint32_t* lds, int size,
                                    int voffset, int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
__device__ void raw_buffer_store_b128(i32x4_v data, i32x4_v rsrc, int voffset, int soffset,
                                      int aux) __asm("llvm.amdgcn.raw.buffer.store.v4i32");

// ---- layouts ---------------------------------------------------------------
// K-contiguous tile [rows][BK]: row r, 16-byte chunk c (8 K values).
template <int BK> PX_DEV int kmaj_chunk(int r, int c) {
  constexpr int CPR = BK / 8;                // chunks per row
  constexpr int RPL = 16 / CPR;  // rows per 256 bytes (the 64 four-byte LDS banks)
  return r * CPR + (c ^ ((r / RPL) % CPR));
}
// M/N-contiguous tile [BK][R]: K row k, 16-byte chunk c (8 columns).
template <int R> PX_DEV int mn_chunk(int k, int c) {
  constexpr int CPR = R / 8;
  return k * CPR + (c ^ (2 * (k & 3)));
}

// ---- copies ----------------------------------------------------------------
// Issue this wave's share of the DMA copies of one operand tile.
// K-contiguous: element (r, k) at src[(row0 + r) * ld + k0 + k], tile rows R.
template <int R, int BK, int NW>
PX_DEV void dma_kmaj(const bf16_t* src, int64_t ld, int k0, char* lds_tile, int wave, int lane) {
  constexpr int CPR = BK / 8;
  constexpr int RPK = 64 / CPR;  // rows per 1 KB
  constexpr int NKB = R * BK * 2 / 1024;
#pragma unroll
  for (int j = 0; j < NKB / NW; ++j) {
    const int kb = j * NW + wave;
    const int r = kb * RPK + lane / CPR;
    const int phys = lane % CPR;
    constexpr int RPL = 16 / CPR;
    const int c = phys ^ ((r / RPL) % CPR);
    const bf16_t* g = src + (int64_t)r * ld + k0 + 8 * c;
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds_tile + kb * 1024), 16, 0, 0);
  }
}
// M/N-contiguous: element (k, col) at src[(k0 + k) * ld + col], tile columns R.
template <int R, int BK, int NW>
PX_DEV void dma_mn(const bf16_t* src, int64_t ld, int k0, char* lds_tile, int wave, int lane) {
  constexpr int CPR = R / 8;
  constexpr int KPK = 64 / CPR;  // K rows per 1 KB (R = 128: 4, R = 256: 2)
  constexpr int NKB = R * BK * 2 / 1024;
  static_assert(CPR <= 64 && 64 % CPR == 0, "tile width must divide a 1 KB copy");
#pragma unroll
  for (int j = 0; j < NKB / NW; ++j) {
    const int kb = j * NW + wave;
    const int k = kb * KPK + lane / CPR;
    const int phys = lane % CPR;
    const int c = phys ^ (2 * (k & 3));
    const bf16_t* g = src + (int64_t)(k0 + k) * ld + 8 * c;
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds_tile + kb * 1024), 16, 0, 0);
  }
}

// ---- fragments -------------------------------------------------------------
// 32 x 16 operand fragment for MFMA rows/columns t0 .. t0 + 31 at K offset kk.
template <int BK> PX_DEV bf16x8_v frag_kmaj(const char* tile, int t0, int kk, int lane) {
  const int t = t0 + (lane & 31);
  const int c = kk / 8 + (lane >> 5);
  return *reinterpret_cast<const bf16x8_v*>(tile + 16 * kmaj_chunk<BK>(t, c));
}
typedef short v4i16_t __attribute__((ext_vector_type(4)));
template <int R> PX_DEV bf16x8_v frag_mn(const char* tile, int t0, int kk, int lane) {
  const int s = lane & 15;
  const int h = lane >> 5;
  const int col = t0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  v4i16_t p[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int k = kk + 8 * h + 4 * q + (s >> 2);
    const char* a = tile + 16 * mn_chunk<R>(k, col / 8) + 2 * (col % 8);
    p[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(a));
  }
  bf16x8_v f;
  __builtin_memcpy(&f, p, 16);
  return f;
}

template <class C> PX_DEV void load_frags(const char* As, const char* Bs, int kk, int wm, int wn, int lane,
                                          bf16x8_v (&a)[C::TM], bf16x8_v (&b)[C::TN]) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int t0 = wm * C::WTM + i * 32;
    if constexpr (C::A_MN)
      a[i] = frag_mn<C::BM>(As, t0, kk, lane);
    else
      a[i] = frag_kmaj<C::BK>(As, t0, kk, lane);
  }
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int t0 = wn * C::WTN + j * 32;
    if constexpr (C::B_MN)
      b[j] = frag_mn<C::BN>(Bs, t0, kk, lane);
    else
      b[j] = frag_kmaj<C::BK>(Bs, t0, kk, lane);
  }
}

// No extra products per k-step (see FH below).
struct NoFragHook {
  template <class C, class F> PX_DEV void operator()(int, const F*, const F*, Acc<C>&) const {}
};

// Fragments of k-step s + 1 are read while the MFMAs of step s run; with
// INTERLEAVE the compiler is asked to interleave them (iglp_opt) instead of
// batching the reads.  fh(k, a, b, acc) runs after the MFMAs of each 16-wide
// k-step, with that step's fragments (k = K index of the step's first column).
template <class C, class FH = NoFragHook>
PX_DEV void dma_mma_stage(const char* As, const char* Bs, Acc<C>& acc, int wm, int wn, int lane, int k0 = 0,
                          const FH& fh = FH()) {
  constexpr int KS = C::BK / 16;
  bf16x8_v a[2][C::TM], b[2][C::TN];
  load_frags<C>(As, Bs, 0, wm, wn, lane, a[0], b[0]);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) load_frags<C>(As, Bs, (ks + 1) * 16, wm, wn, lane, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j], acc.v[i][j], 0, 0, 0);
    // the compiler's MFMA / LDS-read interleave strategy: +7% on a 256 x 256 x 64 tile over an
    // explicit one-read-per-MFMA-group interleave, which in turn measured slower than no hint
    // (not with a fragment hook: the conditional extra MFMAs make the region's scheduling take
    // minutes and tens of GB of compiler memory)
    if constexpr (C::INTERLEAVE && std::is_same<FH, NoFragHook>::value) __builtin_amdgcn_iglp_opt(1);
    fh(k0 + ks * 16, a[cur], b[cur], acc);
  }
}

// s_waitcnt with only the vector-memory count: vmcnt(N), other counters untouched
template <int N> PX_DEV void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
PX_DEV void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }
PX_DEV void barrier_raw() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <class C, int AHEAD> PX_DEV void wait_ahead(int ahead) {
  if constexpr (AHEAD <= 0) {
    wait_vm<0>();
  } else {
    if (ahead >= AHEAD)
      wait_vm<AHEAD * C::L>();
    else
      wait_ahead<C, AHEAD - 1>(ahead);
  }
}

// Operand sources for the DMA loop: base pointers positioned at the tile's
// first row (K-contiguous) or first column (M/N-contiguous), K offset 0.
struct DmaSrc {
  const bf16_t* a;
  int64_t lda;
  const bf16_t* b;
  int64_t ldb;
};

template <class C> PX_DEV void dma_issue(const DmaSrc& src, char* stage, int k0, int wave, int lane) {
  if constexpr (C::A_MN)
    dma_mn<C::BM, C::BK, C::NW>(src.a, src.lda, k0, stage, wave, lane);
  else
    dma_kmaj<C::BM, C::BK, C::NW>(src.a, src.lda, k0, stage, wave, lane);
  if constexpr (C::B_MN)
    dma_mn<C::BN, C::BK, C::NW>(src.b, src.ldb, k0, stage + C::A_BYTES, wave, lane);
  else
    dma_kmaj<C::BN, C::BK, C::NW>(src.b, src.ldb, k0, stage + C::A_BYTES, wave, lane);
}

// Whole K loop over KT tiles.  hook(kt, A stage) runs after the MFMAs of tile kt.
// With SWAP the MFMAs take the B tile as their first operand, so the
// accumulators hold the transposed tile: acc row index = tile column, acc
// column index = tile row (needs BM == BN).  A lane then owns runs of 4
// consecutive tile columns of one row.
template <class C, class H, bool SWAP = false, class FH = NoFragHook>
PX_DEV void dma_mainloop(char* lds, const DmaSrc& src, int KT, Acc<C>& acc, int wm, int wn, int lane, const H& hook,
                         const FH& fh = FH()) {
  static_assert(!SWAP || C::BM == C::BN, "swapped products need square tiles");
  const int wave = threadIdx.x >> 6;
  acc.zero();
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < KT) dma_issue<C>(src, lds + s * C::STAGE_BYTES, s * C::BK, wave, lane);
  for (int kt = 0; kt < KT; ++kt) {
    // tiles kt + 1 .. kt + STAGES - 2 may stay in flight; tile kt must have landed
    wait_ahead<C, C::STAGES - 2>(min(C::STAGES - 2, KT - 1 - kt));
    wait_lgkm0();
    barrier_raw();
    const int nxt = kt + C::STAGES - 1;
    if (nxt < KT) dma_issue<C>(src, lds + (nxt % C::STAGES) * C::STAGE_BYTES, nxt * C::BK, wave, lane);
    const char* st = lds + (kt % C::STAGES) * C::STAGE_BYTES;
    if constexpr (SWAP)
      dma_mma_stage<C>(st + C::A_BYTES, st, acc, wm, wn, lane, kt * C::BK, fh);
    else
      dma_mma_stage<C>(st, st + C::A_BYTES, acc, wm, wn, lane, kt * C::BK, fh);
    hook(kt, st);
  }
  wait_lgkm0();
  barrier_raw();
}

// One pipelined K loop over three products of the same shape added in acc:
// K tile t (0 <= t < 3 KT) comes from source t / KT at K offset
// (t % KT) * BK, so the copies of the next product are in flight while the
// last tiles of the current one are multiplied.
template <class C>
PX_DEV void dma_mainloop_sum3(char* lds, const DmaSrc& s0, const DmaSrc& s1, const DmaSrc& s2, int KT, Acc<C>& acc,
                              int wm, int wn, int lane) {
  const int wave = threadIdx.x >> 6;
  acc.zero();
  const int TT = 3 * KT;
  // source sg as s0 + [sg == 1] (s1 - s0) + [sg == 2] (s2 - s0), in scalar
  // arithmetic (a select between the three is compiled to a table in scratch)
  auto addr = [](const bf16_t* p) { return reinterpret_cast<uintptr_t>(p); };
  const uintptr_t a1 = addr(s1.a) - addr(s0.a), a2 = addr(s2.a) - addr(s0.a);
  const uintptr_t b1 = addr(s1.b) - addr(s0.b), b2 = addr(s2.b) - addr(s0.b);
  const int64_t la1 = s1.lda - s0.lda, la2 = s2.lda - s0.lda, lb1 = s1.ldb - s0.ldb, lb2 = s2.ldb - s0.ldb;
  auto issue = [&](int t, char* stage) {
    const int sg = t / KT;
    const uintptr_t e1 = sg == 1, e2 = sg == 2;
    const DmaSrc s{reinterpret_cast<const bf16_t*>(addr(s0.a) + e1 * a1 + e2 * a2),
                   s0.lda + (int64_t)e1 * la1 + (int64_t)e2 * la2,
                   reinterpret_cast<const bf16_t*>(addr(s0.b) + e1 * b1 + e2 * b2),
                   s0.ldb + (int64_t)e1 * lb1 + (int64_t)e2 * lb2};
    dma_issue<C>(s, stage, (t - sg * KT) * C::BK, wave, lane);
  };
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < TT) issue(s, lds + s * C::STAGE_BYTES);
  for (int kt = 0; kt < TT; ++kt) {
    wait_ahead<C, C::STAGES - 2>(min(C::STAGES - 2, TT - 1 - kt));
    wait_lgkm0();
    barrier_raw();
    const int nxt = kt + C::STAGES - 1;
    if (nxt < TT) issue(nxt, lds + (nxt % C::STAGES) * C::STAGE_BYTES);
    const char* st = lds + (kt % C::STAGES) * C::STAGE_BYTES;
    dma_mma_stage<C>(st, st + C::A_BYTES, acc, wm, wn, lane);
  }
  wait_lgkm0();
  barrier_raw();
}

}  // namespace px
