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
// fall in that range.  `elem` reads element (row, k) of the staged A tile.
template <class C, class E> struct IdentityHook {
  Acc<C>* acc;
  int n0;
  E elem;
  template <typename P> PX_DEV void operator()(int kt, const P* A) const {
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
        for (int e = 0; e < 16; ++e) acc->v[i][j][e] += elem(A, p.row(i, e), kc);
    }
  }
};
template <class C, typename T> struct PaddedElem {  // register-path LDS layout
  PX_DEV float operator()(const T* A, int r, int k) const { return to_f32<T>(A[r * Lay<C, T>::LDK + k]); }
};

// Identity term of the direct-to-LDS apply, as extra MFMAs.  The loop runs
// with swapped operands (first operand: rows of D^T, i.e. output columns;
// second: rows of the input tile), so out^T += I x in^T adds in[row][col] to
// the accumulator of (col, row) exactly (products with 1 and 0 are exact).
// The identity fragment is built in registers, and only the two 16-wide
// k-steps that cover a 32-column group of output columns need it, so a wave
// adds 2 x TM x TN MFMAs per tile and reads nothing more.
template <class CD> struct IdentityMfma {
  int n0;  // first output column of the tile (block-local, equal to its K index)
  int wm, lane;
  PX_DEV void operator()(int k, const bf16x8_v* /*a*/, const bf16x8_v* b, Acc<CD>& acc) const {
#pragma unroll
    for (int i = 0; i < CD::TM; ++i) {
      const int c0 = n0 + wm * CD::WTM + i * 32;  // first output column of group i
      if (k + 16 <= c0 || k >= c0 + 32) continue;
      // lane holds column c0 + lane % 32 at K indices k + 8 (lane / 32) + e
      const int c = c0 + (lane & 31), kl = k + 8 * (lane >> 5);
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      s16x8 bits;
#pragma unroll
      for (int e = 0; e < 8; ++e) bits[e] = (short)(kl + e == c ? 0x3F80 : 0);  // bf16 1.0 or 0
      bf16x8_v id;
      __builtin_memcpy(&id, &bits, 16);
#pragma unroll
      for (int j = 0; j < CD::TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(id, b[j], acc.v[i][j], 0, 0, 0);
    }
  }
};

// Epilogue of the direct-to-LDS apply, from transposed accumulators (a lane
// owns 4 consecutive columns of one row): out = acc * scale, staged through
// LDS as bf16 with one 8-byte write per 4 values, then written with 16-byte
// row-contiguous stores.  `out` and `cs` point at the tile's first row and
// column; the whole tile is in range and 16-byte aligned (checked by the
// caller).  `lds` holds BN x (BM + 8) bf16; the K loop has ended.
template <class CD>
PX_DEV void apply_store_t(const Acc<CD>& acc, void* lds, const float* cs, bf16_t* out, int64_t ld_out) {
  constexpr int PITCH = CD::BM + 8;  // bf16 per staged row (acc column index = tile row)
  constexpr int CPR = CD::BM / 8;    // 16-byte chunks per row
  bf16_t* t = reinterpret_cast<bf16_t*>(lds);
  const AccPos<CD> p = acc_pos<CD>();
#pragma unroll
  for (int i = 0; i < CD::TM; ++i)
#pragma unroll
    for (int j = 0; j < CD::TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = p.col(j), col = p.row(i, 4 * g);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc.v[i][j][4 * g + e] * (cs ? cs[col + e] : 1.f);
        uint2 w;
        w.x = f2bf2(o[0], o[1]);
        w.y = f2bf2(o[2], o[3]);
        *reinterpret_cast<uint2*>(t + row * PITCH + col) = w;
      }
  __syncthreads();
  static_assert(CD::BN * CPR % CD::NT == 0, "chunks must split evenly");
#pragma unroll
  for (int q = 0; q < CD::BN * CPR / CD::NT; ++q) {
    const int ch = threadIdx.x + q * CD::NT, row = ch / CPR, col = (ch % CPR) * 8;
    *reinterpret_cast<uint4*>(out + (int64_t)row * ld_out + col) = *reinterpret_cast<const uint4*>(t + row * PITCH + col);
  }
}

template <class CD, class C, typename T, typename IT, typename GT, typename OT>
__global__ __launch_bounds__(C::NT) void k_apply(const IT* __restrict__ in, int64_t ld_in, int rows, int d, int b,
                                                  const GT* __restrict__ dT, const float* __restrict__ colscale,
                                                  OT* __restrict__ out, int64_t ld_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);
  // Units run block-major, then row tile, then column tile.  Workgroups are
  // dealt to the 8 XCDs round robin, so the launch index is remapped to give
  // each XCD a contiguous range of units: an XCD then fetches only its own
  // blocks of D^T into its L2, and the column tiles of one row tile, which
  // share their input rows, run back to back on the same XCD.
  const int nrt = (rows + C::BM - 1) / C::BM, nct = (b + C::BN - 1) / C::BN;
  const int units = nrt * nct * ((d + b - 1) / b);
  int u = blockIdx.x;
  if (units % 8 == 0) u = (u % 8) * (units / 8) + u / 8;
  const int blk = u / (nrt * nct), rem = u % (nrt * nct);
  const int kb = blk * b, r = min(b, d - kb);
  const int m0 = (rem / nct) * C::BM, n0 = (rem % nct) * C::BN;
  if (n0 >= r) return;
  const IT* a0 = in + (int64_t)m0 * ld_in + kb;
  const GT* b0 = dT + ((int64_t)blk * b + n0) * b;
  const float* cs = colscale ? colscale + kb + n0 : nullptr;
  auto epi = [&](auto& acc) {
    store_tile<cfg_of<decltype(acc)>, OT>(acc, smem, out + (int64_t)m0 * ld_out + kb + n0, ld_out, rows - m0, r - n0,
                                          [&](int c) { return cs ? cs[c] : 1.f; });
  };
  if constexpr (!std::is_same<CD, void>::value) {
    // the direct-to-LDS loop deals its copies and fragments over CD::NT threads: it must be the launch size
    static_assert(CD::NT == C::NT, "direct-to-LDS configuration and tile loop must use the same workgroup size");
    OT* o0 = out + (int64_t)m0 * ld_out + kb + n0;
    if (dma_rows_ok(a0, ld_in, rows - m0, CD::BM) && dma_rows_ok(b0, b, r - n0, CD::BN) && r % CD::BK == 0 &&
        reinterpret_cast<uintptr_t>(o0) % 16 == 0 && ld_out % 8 == 0) {
      Acc<CD> acc;
      const AccPos<CD> p = acc_pos<CD>();
      const DmaSrc src{reinterpret_cast<const bf16_t*>(a0), ld_in, reinterpret_cast<const bf16_t*>(b0), b};
      dma_mainloop<CD, NoHook, true>(reinterpret_cast<char*>(smem), src, r / CD::BK, acc, p.wm, p.wn, p.lane,
                                     NoHook(), IdentityMfma<CD>{n0, p.wm, p.lane});
      apply_store_t<CD>(acc, smem, cs, reinterpret_cast<bf16_t*>(o0), ld_out);
      return;
    }
  }
  LoadK<C::BM, C::BK, C::NT, IT, T> la;
  la.init(a0, ld_in, rows - m0, r);
  LoadK<C::BN, C::BK, C::NT, GT, T> lb;
  lb.init(b0, b, r - n0, r);
  Acc<C> acc;
  const AccPos<C> p = acc_pos<C>();
  mainloop<C, T>(lds, la, lb, r, acc, p.wm, p.wn, p.lane, IdentityHook<C, PaddedElem<C, T>>{&acc, n0, {}});
  epi(acc);
}

// ============================================================================
// block-diagonal product, streaming form (bf16, blocks of 256 or 512)
// ============================================================================
// A workgroup of 8 waves owns one 256-column group of one block and keeps
// that group's slice of D^T in VGPRs for as long as it works on the block
// (wave w: output columns 32 w .. 32 w + 31 of the group, all B K indices, as
// B / 16 MFMA fragments).  Row tiles of RT tokens x B input columns then
// stream through a ring of S LDS slots, so S - 1 tiles of input are in flight
// while one is multiplied; each tile is read from HBM once, however many
// column groups its block has, because the groups of a block run on one XCD
// over the same tiles at the same time and share it through L2.
// Waves 0-3 issue the tile copies and waves 4-7 the output stores, so each
// wave's vector-memory counter holds one kind of operation and a wait for a
// tile's copies never waits for stores.  The MFMAs take D^T as their first
// operand (accumulators hold the transposed tile: a lane owns 4 consecutive
// output columns of one token row), and the identity term is added by two
// MFMAs against an identity fragment, which is exact.
// Work: items (block, row tile) in block-major order, split into contiguous
// ranges over "pair lanes"; the NH = B / 256 workgroups of a pair lane (one
// per column group) sit on the same XCD and walk the same range.
template <int B, int RT, int S> struct StreamCfg {
  static constexpr int NW = 8, NT = 512, NH = B / 256, NKS = B / 16, NKT = B / 64;
  static constexpr int SLOT = RT * B * 2;            // bytes of one row tile
  static constexpr int SUB = RT * 128;               // bytes of one [RT][64] K sub-tile
  static constexpr int PIECES = SLOT / 1024;          // 1 KB copies per tile
  static constexpr int PPW = PIECES / 4;              // per loader wave
  static constexpr int PITCH = 256 + 8;               // staged output row, bf16
  static constexpr int STAGE = RT * PITCH * 2;
  static constexpr int LDS = S * SLOT + 2 * STAGE;   // ring + two staged output tiles
  static constexpr int TMF = RT / 32;                 // 32-row fragments per tile
  static constexpr int SPL = RT * 32 / 256;           // 16-byte output chunks per store lane
  static_assert(B == 256 || B == 512, "block of 256 or 512 columns");
  static_assert(RT % 32 == 0 && PIECES % 4 == 0 && SPL == 4, "row tile of whole fragments and copies");
  static_assert(S >= 2 && S <= 4 && 2 * PPW <= 63, "outstanding copies must fit the vmcnt counter");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// The sides of one launch: side s has blocks [first[s], first[s + 1]) of the
// launch's block numbering, all with the same rows; cs[s] may be null (scale
// 1) in a CS launch.  Passed by value as a kernel argument.
struct StreamSides {
  const bf16_t* in[pxk::kApplySides];
  const bf16_t* dT[pxk::kApplySides];
  const float* cs[pxk::kApplySides];
  bf16_t* out[pxk::kApplySides];
  int64_t ld_in[pxk::kApplySides], ld_out[pxk::kApplySides];
  int first[pxk::kApplySides + 1];
  int count;
  PX_DEV int side_of(int gb) const {
    int q = 0;
    while (q + 1 < count && gb >= first[q + 1]) ++q;
    return q;
  }
};

template <int B, int RT, int S, bool CS, bool MULTI>
__global__ __launch_bounds__(512) void k_apply_stream(const StreamSides tb, int rows, int items, int pair_lanes) {
  using C = StreamCfg<B, RT, S>;
  extern __shared__ __align__(16) unsigned char smem[];
  char* ring = reinterpret_cast<char*>(smem);
  bf16_t* stage = reinterpret_cast<bf16_t*>(smem + S * C::SLOT);  // two tiles, by item parity
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // launch index -> (XCD, slot on it) -> (pair lane, column group)
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int pl = xcd * (pair_lanes / 8) + slot / C::NH, hc = slot % C::NH;
  const int i0 = (int)((int64_t)pl * items / pair_lanes), i1 = (int)((int64_t)(pl + 1) * items / pair_lanes);
  if (i0 >= i1) return;
  const int rtiles = (rows + RT - 1) / RT;
  const int c0 = hc * 256 + 32 * wave;  // block-local first output column of this wave
  const bool loader = wave < 4;

  // Loader lanes: byte offset of each of their 1 KB copy pieces inside a row
  // tile (piece p = j * 4 + wave: K sub-tile p / (RT / 8), rows 8 (p % (RT / 8))
  // + lane / 8, the 16-byte chunk chosen by the kmaj swizzle).
  auto piece_off = [&](int j, int64_t ld) {
    const int p = j * 4 + (wave & 3);
    const int kt = p / (RT / 8), r = (p % (RT / 8)) * 8 + lane / 8;
    const int c = (lane % 8) ^ ((r / 2) % 8);
    return (int)((int64_t)r * ld * 2) + kt * 128 + 16 * c;
  };
  int voff[C::PPW];
  if constexpr (!MULTI) {
#pragma unroll
    for (int j = 0; j < C::PPW; ++j) voff[j] = piece_off(j, tb.ld_in[0]);
  }
  // launch block gb -> its side and the side's block
  auto locate = [&](int gb, int& sd, int& blk) {
    sd = MULTI ? tb.side_of(gb) : 0;
    blk = gb - (MULTI ? tb.first[sd] : 0);
  };
  // copy of the row tile of item `it` into ring slot `sl` (loader waves only)
  auto issue = [&](int it, int sl) {
    int sd, blk;
    locate(it / rtiles, sd, blk);
    const int m0 = (it % rtiles) * RT;
    const int64_t ld_in = tb.ld_in[sd];
    const i32x4_v rs = buffer_rsrc(tb.in[sd] + (int64_t)m0 * ld_in + (int64_t)blk * B, (int64_t)(rows - m0) * ld_in * 2);
    char* dst = ring + sl * C::SLOT;
#pragma unroll
    for (int j = 0; j < C::PPW; ++j) {
      const int p = j * 4 + wave;
      raw_buffer_load_lds(rs, (__attribute__((address_space(3))) uint32_t*)(dst + (p / (RT / 8)) * C::SUB + (p % (RT / 8)) * 1024),
                          16, MULTI ? piece_off(j, ld_in) : voff[j], 0, 0, 0);
    }
  };
  if (loader) {
#pragma unroll
    for (int q = 0; q < S - 1; ++q)
      if (i0 + q < i1) issue(i0 + q, q);
  }

  // identity fragments for the two k-steps that cover this wave's columns
  bf16x8_v idf[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 bits;
    const int c = c0 + (lane & 31), kl = c0 + 16 * h + 8 * (lane >> 5);
#pragma unroll
    for (int e = 0; e < 8; ++e) bits[e] = (short)(kl + e == c ? 0x3F80 : 0);
    __builtin_memcpy(&idf[h], &bits, 16);
  }
  const int s_id = c0 / 16;
  // store lanes: byte offsets of their 4 staged chunks (row, 8 columns) in LDS and in a row tile of the output
  const int ts = threadIdx.x & 255;
  uint32_t st_lds[C::SPL];
  int st_off[C::SPL];
  auto store_off = [&](int q, int64_t ld) {
    const int ch = ts + 256 * q, row = ch / 32, col = (ch % 32) * 8;
    return (int)((int64_t)row * ld * 2) + col * 2;
  };
#pragma unroll
  for (int q = 0; q < C::SPL; ++q) {
    const int ch = ts + 256 * q, row = ch / 32, col = (ch % 32) * 8;
    st_lds[q] = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)(stage + row * C::PITCH + col);  // tile 0
    st_off[q] = store_off(q, tb.ld_out[0]);
  }

  // store lanes: staged tile `par` (written for item `it`) to the output
  auto store_tile = [&](int par, int it) {
    int sd, blk;
    locate(it / rtiles, sd, blk);
    const int m0 = (it % rtiles) * RT;
    const int64_t ld_out = tb.ld_out[sd];
    const uint32_t sb = par * C::STAGE;
    // read back in assembly, waiting for the four reads inside the block: a
    // compiler-visible LDS read would wait for every copy in flight first
    i32x4_v v0, v1, v2, v3;
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "v"(st_lds[0] + sb), "v"(st_lds[1] + sb), "v"(st_lds[2] + sb), "v"(st_lds[3] + sb)
        : "memory");
    const i32x4_v rs = buffer_rsrc(tb.out[sd] + (int64_t)m0 * ld_out + (int64_t)blk * B + hc * 256,
                                   (int64_t)(rows - m0) * ld_out * 2);
    raw_buffer_store_b128(v0, rs, MULTI ? store_off(0, ld_out) : st_off[0], 0, 0);
    raw_buffer_store_b128(v1, rs, MULTI ? store_off(1, ld_out) : st_off[1], 0, 0);
    raw_buffer_store_b128(v2, rs, MULTI ? store_off(2, ld_out) : st_off[2], 0, 0);
    raw_buffer_store_b128(v3, rs, MULTI ? store_off(3, ld_out) : st_off[3], 0, 0);
  };

  bf16x8_v dfr[C::NKS];
  float scl[16];
  int cur_blk = -1;
  for (int it = i0; it < i1; ++it) {
    const int gb = it / rtiles;
    if (gb != cur_blk) {
      cur_blk = gb;
      int sd, blk;
      locate(gb, sd, blk);
      const float* cs = tb.cs[sd];
      const bf16_t* dp = tb.dT[sd] + ((int64_t)blk * B + c0 + (lane & 31)) * B + 8 * (lane >> 5);
#pragma unroll
      for (int s = 0; s < C::NKS; ++s) dfr[s] = *reinterpret_cast<const bf16x8_v*>(dp + 16 * s);
      if constexpr (CS) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4_v v = cs ? *reinterpret_cast<const f32x4_v*>(cs + (int64_t)blk * B + c0 + 8 * g + 4 * (lane >> 5))
                               : f32x4_v{1.f, 1.f, 1.f, 1.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) scl[4 * g + e] = v[e];
        }
      }
      // wait here, once per block: left to the compiler, the wait for these
      // registers lands before every tile's first MFMA and drains the ring
      wait_vm<0>();
    }
    // tile `it` must have landed: the copies of the tiles after it may stay in flight
    if (loader) {
      const int ahead = min(S - 2, i1 - 1 - it);
      if constexpr (S >= 4) {
        if (ahead >= 2) wait_vm<2 * C::PPW>();
        else if (ahead == 1) wait_vm<C::PPW>();
        else wait_vm<0>();
      } else if constexpr (S == 3) {
        if (ahead >= 1) wait_vm<C::PPW>();
        else wait_vm<0>();
      } else {
        wait_vm<0>();
      }
    }
    wait_lgkm0();
    barrier_raw();
    if (loader && it + S - 1 < i1) issue(it + S - 1, (it - i0 + S - 1) % S);
    // the previous item's tile, staged before the barrier, is stored while this one is multiplied
    if (!loader && it > i0) store_tile((it - 1 - i0) & 1, it - 1);
    const char* tile = ring + ((it - i0) % S) * C::SLOT;
    f32x16_v acc[C::TMF];
#pragma unroll
    for (int i = 0; i < C::TMF; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
    // the fragments of a whole 64-wide K sub-tile are read while the previous
    // sub-tile's MFMAs run
    bf16x8_v fa[2][4][C::TMF];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < C::TMF; ++i) fa[0][q][i] = frag_kmaj<64>(tile, 32 * i, 16 * q, lane);
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
      if (kt + 1 < C::NKT) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < C::TMF; ++i)
            fa[(kt + 1) & 1][q][i] = frag_kmaj<64>(tile + (kt + 1) * C::SUB, 32 * i, 16 * q, lane);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < C::TMF; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dfr[4 * kt + q], fa[kt & 1][q][i], acc[i], 0, 0, 0);
    }
    // keep that order: left alone, the scheduler reads each fragment just
    // before its MFMA and every MFMA waits out an LDS round trip
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * C::TMF, 0);  // LDS reads of sub-tile 0
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
      if (kt + 1 < C::NKT) __builtin_amdgcn_sched_group_barrier(0x100, 4 * C::TMF, 0);  // reads of kt + 1
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * C::TMF, 0);                       // MFMAs of kt
    }
    // identity term: the input fragments of k-steps s_id and s_id + 1 once more
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sh = s_id + h;
#pragma unroll
      for (int i = 0; i < C::TMF; ++i) {
        const bf16x8_v a = frag_kmaj<64>(tile + (sh / 4) * C::SUB, 32 * i, (sh % 4) * 16, lane);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(idf[h], a, acc[i], 0, 0, 0);
      }
    }
    // stage the tile (lane: token row 32 i + lane % 32, columns 32 w + 8 g + 4 (lane / 32) + 0..3)
#pragma unroll
    for (int i = 0; i < C::TMF; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = CS ? acc[i][4 * g + e] * scl[4 * g + e] : acc[i][4 * g + e];
        const uint64_t w = (uint64_t)f2bf2(o[0], o[1]) | ((uint64_t)f2bf2(o[2], o[3]) << 32);
        // written as inline assembly: the compiler cannot tell that the staging
        // area is disjoint from the ring slots that copies are still filling,
        // and would otherwise wait for every copy in flight before the write
        const int row = 32 * i + (lane & 31), col = 32 * wave + 8 * g + 4 * (lane >> 5);
        const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)(stage + row * C::PITCH + col) +
                           ((it - i0) & 1) * C::STAGE;
        asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(w) : "memory");
      }
  }
  // the last item's tile
  wait_lgkm0();
  barrier_raw();
  if (!loader) store_tile((i1 - 1 - i0) & 1, i1 - 1);
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
    at_local(id, bm, bn);
  }
  // tile number id (after the XCD remap) -> (row tile, column tile)
  PX_DEV void at_local(int id, int& bm, int& bn) const {
    const int group = id / (GM * tn);
    const int first = group * GM;
    const int gsize = min(tm - first, GM);
    bm = first + (id % (GM * tn)) % gsize;
    bn = (id % (GM * tn)) / gsize;
  }
};

// One output tile (bm, bn) of out = A * B (* colscale): the direct-to-LDS
// loop when both operand panels and K allow it, else the register loop.
template <class CD, class C, typename T, typename AT, typename BT, typename OT, bool BKN>
PX_DEV void gemm_tile(unsigned char* smem, const AT* __restrict__ A, int64_t lda, const BT* __restrict__ B, int64_t ldb,
                      int M, int N, int K, const float* __restrict__ colscale, OT* __restrict__ out, int64_t ldo,
                      int bm, int bn) {
  T* lds = reinterpret_cast<T*>(smem);
  const int m0 = bm * C::BM, n0 = bn * C::BN;
  const float* cs = colscale ? colscale + n0 : nullptr;
  if constexpr (!std::is_same<CD, void>::value) {
    // the direct-to-LDS loop deals its copies and fragments over CD::NT threads: it must be the launch size
    static_assert(CD::NT == C::NT, "direct-to-LDS configuration and tile loop must use the same workgroup size");
    const AT* a0 = A + (int64_t)m0 * lda;
    const BT* b0 = B + (int64_t)n0 * ldb;
    if (dma_rows_ok(a0, lda, M - m0, CD::BM) && dma_rows_ok(b0, ldb, N - n0, CD::BN) && K % CD::BK == 0) {
      Acc<CD> acc;
      const AccPos<CD> p = acc_pos<CD>();
      const DmaSrc src{reinterpret_cast<const bf16_t*>(a0), lda, reinterpret_cast<const bf16_t*>(b0), ldb};
      dma_mainloop<CD>(reinterpret_cast<char*>(smem), src, K / CD::BK, acc, p.wm, p.wn, p.lane, NoHook());
      store_tile<CD, OT>(acc, smem, out + (int64_t)m0 * ldo + n0, ldo, M - m0, N - n0,
                         [&](int c) { return cs ? cs[c] : 1.f; });
      return;
    }
  }
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
  store_tile<C, OT>(acc, smem, out + (int64_t)m0 * ldo + n0, ldo, M - m0, N - n0,
                    [&](int c) { return cs ? cs[c] : 1.f; });
}

template <class CD, class C, typename T, typename AT, typename BT, typename OT, bool BKN>
__global__ __launch_bounds__(C::NT) void k_gemm(const AT* __restrict__ A, int64_t lda, const BT* __restrict__ B,
                                                 int64_t ldb, int M, int N, int K, const float* __restrict__ colscale,
                                                 OT* __restrict__ out, int64_t ldo, TileMap map) {
  extern __shared__ __align__(16) unsigned char smem[];
  int bm, bn;
  map.at(blockIdx.x, bm, bn);
  gemm_tile<CD, C, T, AT, BT, OT, BKN>(smem, A, lda, B, ldb, M, N, K, colscale, out, ldo, bm, bn);
}

// Several contractions of one tile configuration in one launch: problem q
// owns tiles [first[q], first[q + 1]) of the launch.  Launch indices are
// remapped as in TileMap so that each XCD receives a contiguous range of tile
// numbers; inside a problem, tile numbers run through groups of GM row tiles.
struct GemmTable {
  const bf16_t* A[pxk::kGemmProblems];
  const bf16_t* B[pxk::kGemmProblems];
  const float* cs[pxk::kGemmProblems];
  bf16_t* out[pxk::kGemmProblems];
  int64_t lda[pxk::kGemmProblems], ldb[pxk::kGemmProblems], ldo[pxk::kGemmProblems];
  int M[pxk::kGemmProblems], N[pxk::kGemmProblems], K[pxk::kGemmProblems];
  int first[pxk::kGemmProblems + 1];
  int count;
};

template <class CD, class C>
__global__ __launch_bounds__(C::NT) void k_gemm_group(const GemmTable tb) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int total = tb.first[tb.count];
  int id = blockIdx.x;
  if (total % 8 == 0) id = (id % 8) * (total / 8) + id / 8;
  int q = 0;
  while (q + 1 < tb.count && id >= tb.first[q + 1]) ++q;
  int bm, bn;
  const TileMap map{(tb.M[q] + C::BM - 1) / C::BM, (tb.N[q] + C::BN - 1) / C::BN};
  map.at_local(id - tb.first[q], bm, bn);
  gemm_tile<CD, C, bf16_t, bf16_t, bf16_t, bf16_t, false>(smem, tb.A[q], tb.lda[q], tb.B[q], tb.ldb[q], tb.M[q], tb.N[q],
                                                          tb.K[q], tb.cs[q], tb.out[q], tb.ldo[q], bm, bn);
}

// ============================================================================
// permutations
// ============================================================================
// Rows of a caller's tensor need not start on a 16-byte boundary (a bf16 row
// of odd width puts every other row 2 bytes off).  A staged row therefore
// goes in three parts: the elements before the row's first 16-byte boundary,
// a 16-byte body, and the rest.  Its LDS copy is shifted by lds_shift() so
// that the body lands on 16-byte LDS addresses as well; a row pitch of
// stage_pitch(d) elements leaves room for any shift.

// Elements of p before its first 16-byte boundary, capped at d (all d when p
// is not even aligned to its element).
template <typename E>
__device__ inline int lead16(const E* p, int d) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (a % sizeof(E)) return d;
  return min((int)((16 - a % 16) % 16 / sizeof(E)), d);
}

// Shift of a staged row whose global row leads with h elements: the LDS
// element h then sits on a 16-byte boundary.
template <typename E>
__device__ inline int lds_shift(int h) {
  constexpr int V = 16 / sizeof(E);
  return (V - h % V) % V;
}

// Staged row pitch in elements: d plus room for the largest shift, rounded up
// to 16 bytes.
inline int64_t stage_pitch(int64_t d, size_t es) {
  const int64_t v = 16 / (int64_t)es;
  return (d + 2 * v - 2) / v * v;
}

// dst[0, d) = row[0, d) by the whole workgroup; h = lead16(row, d), and
// dst + h is 16-byte aligned.
template <typename E>
__device__ inline void row_to_lds(const E* __restrict__ row, E* dst, int d, int h) {
  constexpr int V = 16 / sizeof(E);
  const int nb = (d - h) / V, t0 = h + nb * V;
  const uint4* s = reinterpret_cast<const uint4*>(row + h);
  uint4* o = reinterpret_cast<uint4*>(dst + h);
  for (int i = threadIdx.x; i < nb; i += blockDim.x) o[i] = s[i];
  for (int i = threadIdx.x; i < h + d - t0; i += blockDim.x) {
    const int e = i < h ? i : t0 + i - h;
    dst[e] = row[e];
  }
}

// row[0, d) = src[0, d) by the whole workgroup; h = lead16(row, d), and
// src + h is 16-byte aligned.
template <typename E>
__device__ inline void lds_to_row(const E* src, E* __restrict__ row, int d, int h) {
  constexpr int V = 16 / sizeof(E);
  const int nb = (d - h) / V, t0 = h + nb * V;
  const uint4* s = reinterpret_cast<const uint4*>(src + h);
  uint4* o = reinterpret_cast<uint4*>(row + h);
  for (int i = threadIdx.x; i < nb; i += blockDim.x) o[i] = s[i];
  for (int i = threadIdx.x; i < h + d - t0; i += blockDim.x) {
    const int e = i < h ? i : t0 + i - h;
    row[e] = src[e];
  }
}

// Rows t0 .. t0 + nr - 1 of out[:, i] = staged row[colmap[i]] for i < d_out,
// by the whole workgroup: each lane gathers 16 bytes from LDS at the permuted
// positions and writes them with one store.  staged(rr): the LDS copy of the
// rr-th staged row.
template <typename E, class Staged>
PX_DEV void gather_staged(const Staged& staged, int nr, int t0, const int32_t* __restrict__ colmap,
                          E* __restrict__ out, int64_t ld_out, int d_in, int d_out) {
  constexpr int V = 16 / sizeof(E);
  const bool vout = (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (ld_out % V == 0) &&
                    (reinterpret_cast<uintptr_t>(colmap) % 16 == 0);
  const int nchunk = (d_out + V - 1) / V;
  for (int rr = 0; rr < nr; ++rr) {
    E* o = out + (int64_t)(t0 + rr) * ld_out;
    const E* srow = staged(rr);
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

// Row-staged gather: the workgroup copies whole source rows into LDS with
// 16-byte coalesced loads (any row alignment, see row_to_lds), then writes
// each output row with 16-byte stores (gather_staged).  Indices are clamped
// into range so that a malformed permutation cannot address outside the
// staged rows.  pitch = stage_pitch(d_in).
template <typename E>
__global__ __launch_bounds__(256) void k_permute_lds(const E* __restrict__ in, int64_t ld_in,
                                                     const int32_t* __restrict__ rowmap,
                                                     const int32_t* __restrict__ colmap, E* __restrict__ out,
                                                     int64_t ld_out, int rows, int d_in, int d_out, int rpw,
                                                     int pitch) {
  extern __shared__ __align__(16) unsigned char smem[];
  E* buf = reinterpret_cast<E*>(smem);
  const int t0 = blockIdx.x * rpw;
  const int nr = min(rpw, rows - t0);
  auto src_row = [&](int rr) {
    int src = t0 + rr;
    if (rowmap) src = min(max(rowmap[src], 0), rows - 1);
    return in + (int64_t)src * ld_in;
  };
  for (int rr = 0; rr < nr; ++rr) {
    const E* row = src_row(rr);
    const int h = lead16(row, d_in);
    row_to_lds(row, buf + rr * pitch + lds_shift<E>(h), d_in, h);
  }
  __syncthreads();
  gather_staged<E>([&](int rr) -> const E* { return buf + rr * pitch + lds_shift<E>(lead16(src_row(rr), d_in)); },
                   nr, t0, colmap, out, ld_out, d_in, d_out);
}

// The outputs of one multi-output gather: out[k][:, i] = in[:, colmap[k][i]].
struct GatherOuts {
  const int32_t* colmap[pxk::kGatherOuts];
  void* out[pxk::kGatherOuts];
  int64_t ld_out[pxk::kGatherOuts];
  int d_out[pxk::kGatherOuts];
  int count;
};

// k_permute_lds for several outputs from one input: each staged row is read
// from HBM once and gathered into every output.
template <typename E>
__global__ __launch_bounds__(256) void k_permute_lds_multi(const E* __restrict__ in, int64_t ld_in, const GatherOuts go,
                                                           int rows, int d_in, int rpw, int pitch) {
  extern __shared__ __align__(16) unsigned char smem[];
  E* buf = reinterpret_cast<E*>(smem);
  const int t0 = blockIdx.x * rpw;
  const int nr = min(rpw, rows - t0);
  auto src_row = [&](int rr) { return in + (int64_t)(t0 + rr) * ld_in; };
  for (int rr = 0; rr < nr; ++rr) {
    const E* row = src_row(rr);
    const int h = lead16(row, d_in);
    row_to_lds(row, buf + rr * pitch + lds_shift<E>(h), d_in, h);
  }
  __syncthreads();
  for (int k = 0; k < go.count; ++k)
    gather_staged<E>([&](int rr) -> const E* { return buf + rr * pitch + lds_shift<E>(lead16(src_row(rr), d_in)); },
                     nr, t0, go.colmap[k], reinterpret_cast<E*>(go.out[k]), go.ld_out[k], d_in, go.d_out[k]);
}

// dst[c][r] = src[r][c] (bit copy) through a 64 x 64 LDS tile, so that both
// the reads and the writes run along rows; dst columns r in [rows, ld_dst)
// are zero-filled.  Workgroup (x, y) covers dst rows [64y, 64y + 64) and dst
// columns [64x, 64x + 64).
template <typename U>
__global__ __launch_bounds__(256) void k_transpose(const U* __restrict__ src, int64_t ld_src, int rows, int cols,
                                                   U* __restrict__ dst, int64_t ld_dst) {
  __shared__ uint32_t t[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int x = threadIdx.x & 63, y = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + y + 4 * k, c = c0 + x;
    t[y + 4 * k][x] = (r < rows && c < cols) ? (uint32_t)src[(int64_t)r * ld_src + c] : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + y + 4 * k, r = r0 + x;
    if (c < cols && r < ld_dst) dst[(int64_t)c * ld_dst + r] = (U)t[x][y + 4 * k];
  }
}

// int8 codes widened to bf16 (exact: |code| <= 128 needs 8 significant bits),
// so that the int8 contractions take the bf16 direct-to-LDS loop.  Plain:
// dst[r][c] = src[r][c], 16 codes per thread and step; transposed: dst[c][r] =
// src[r][c] through a 64 x 64 LDS tile (as k_transpose), dst columns r in
// [rows, ld_dst) zero-filled.
__global__ __launch_bounds__(256) void k_widen_i8(const int8_t* __restrict__ src, int64_t ld_src, int rows, int cols,
                                                  bf16_t* __restrict__ dst, int64_t ld_dst) {
  const int per_row = (cols + 15) / 16;
  const int64_t total = (int64_t)rows * per_row;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(u / per_row), c0 = (int)(u % per_row) * 16;
    const int8_t* a = src + (int64_t)r * ld_src + c0;
    bf16_t* o = dst + (int64_t)r * ld_dst + c0;
    if (c0 + 16 <= cols && reinterpret_cast<uintptr_t>(a) % 16 == 0 && reinterpret_cast<uintptr_t>(o) % 16 == 0) {
      const int4 v = *reinterpret_cast<const int4*>(a);
      const int8_t* b8 = reinterpret_cast<const int8_t*>(&v);
      uint4 w[2];
      uint32_t* wp = reinterpret_cast<uint32_t*>(w);
#pragma unroll
      for (int k = 0; k < 8; ++k) wp[k] = f2bf2((float)b8[2 * k], (float)b8[2 * k + 1]);
      reinterpret_cast<uint4*>(o)[0] = w[0];
      reinterpret_cast<uint4*>(o)[1] = w[1];
    } else {
      for (int e = 0; e < 16 && c0 + e < cols; ++e) o[e] = f2bf((float)a[e]);
    }
  }
}

// Transposed: a 64 x 64 tile of codes per workgroup.  Each thread reads 16
// codes of one source row (one 16-byte load where the row piece is whole and
// aligned), writes them widened into the LDS tile t[c][r] (bf16 bits, rows of
// 64 + 8 elements), and then stores two 16-byte pieces of destination rows:
// 8 consecutive r of one c each.
__global__ __launch_bounds__(256) void k_widen_i8_t(const int8_t* __restrict__ src, int64_t ld_src, int rows, int cols,
                                                    bf16_t* __restrict__ dst, int64_t ld_dst) {
  constexpr int P = 64 + 8;
  __shared__ __align__(16) uint16_t t[64 * P];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  {
    const int r = threadIdx.x >> 2, cq = (threadIdx.x & 3) * 16;  // source row r0 + r, columns c0 + cq .. + 15
    const int8_t* a = src + (int64_t)(r0 + r) * ld_src + c0 + cq;
    int8_t v[16];
    if (r0 + r < rows && c0 + cq + 16 <= cols && reinterpret_cast<uintptr_t>(a) % 16 == 0) {
      const int4 w = *reinterpret_cast<const int4*>(a);
      __builtin_memcpy(v, &w, 16);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = (r0 + r < rows && c0 + cq + e < cols) ? a[e] : (int8_t)0;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) t[(cq + e) * P + r] = f2bf((float)v[e]);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = threadIdx.x + 256 * h, c = u >> 3, rq = (u & 7) * 8;  // destination row c0 + c, columns r0 + rq .. + 7
    if (c0 + c >= cols) continue;
    bf16_t* o = dst + (int64_t)(c0 + c) * ld_dst + r0 + rq;
    const uint4 w = *reinterpret_cast<const uint4*>(&t[c * P + rq]);
    if (r0 + rq + 8 <= ld_dst && reinterpret_cast<uintptr_t>(o) % 16 == 0) {
      *reinterpret_cast<uint4*>(o) = w;
    } else {
      uint16_t e8[8];
      __builtin_memcpy(e8, &w, 16);
      for (int e = 0; e < 8 && r0 + rq + e < ld_dst; ++e) reinterpret_cast<uint16_t*>(o)[e] = e8[e];
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

// Row-staged scatter, out[t][perm[i]] = in[t][i]: each source row is read with
// 16-byte coalesced loads (the permutation as 16-byte index vectors) and
// written into LDS at the permuted positions; the staged rows then leave with
// 16-byte stores (any output row alignment, see lds_to_row).  Indices are
// clamped into [0, d): a malformed permutation leaves some outputs undefined
// but cannot address outside the staged rows.  pitch = stage_pitch(d).
template <typename E>
__global__ __launch_bounds__(256) void k_scatter_lds(const E* __restrict__ in, int64_t ld_in,
                                                     const int32_t* __restrict__ perm, E* __restrict__ out,
                                                     int64_t ld_out, int rows, int d, int rpw, int pitch) {
  extern __shared__ __align__(16) unsigned char smem[];
  E* buf = reinterpret_cast<E*>(smem);
  constexpr int V = 16 / sizeof(E);
  const int t0 = blockIdx.x * rpw;
  const int nr = min(rpw, rows - t0);
  const int dv = d / V;
  const bool vin = (reinterpret_cast<uintptr_t>(in) % 16 == 0) && (ld_in % V == 0) &&
                   (reinterpret_cast<uintptr_t>(perm) % 16 == 0);
  for (int rr = 0; rr < nr; ++rr) {
    const E* row = in + (int64_t)(t0 + rr) * ld_in;
    E* dst = buf + rr * pitch + lds_shift<E>(lead16(out + (int64_t)(t0 + rr) * ld_out, d));
    int tail = 0;
    if (vin) {
      for (int c = threadIdx.x; c < dv; c += blockDim.x) {
        const uint4 v = reinterpret_cast<const uint4*>(row)[c];
        E vals[V];
        __builtin_memcpy(vals, &v, 16);
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
          const int4 w = reinterpret_cast<const int4*>(perm + c * V)[q];
          dst[min(max(w.x, 0), d - 1)] = vals[4 * q];
          dst[min(max(w.y, 0), d - 1)] = vals[4 * q + 1];
          dst[min(max(w.z, 0), d - 1)] = vals[4 * q + 2];
          dst[min(max(w.w, 0), d - 1)] = vals[4 * q + 3];
        }
      }
      tail = dv * V;
    }
    for (int i = tail + threadIdx.x; i < d; i += blockDim.x) dst[min(max(perm[i], 0), d - 1)] = row[i];
  }
  __syncthreads();
  for (int rr = 0; rr < nr; ++rr) {
    E* o = out + (int64_t)(t0 + rr) * ld_out;
    const int h = lead16(o, d);
    lds_to_row(buf + rr * pitch + lds_shift<E>(h), o, d, h);
  }
}

// The inputs of one summed scatter: out[:, perm[k][i]] += in[k][:, i].
struct ScatterIns {
  const void* in[pxk::kGatherOuts];
  int64_t ld_in[pxk::kGatherOuts];
  const int32_t* perm[pxk::kGatherOuts];
  int count;
};

// Summed row scatter, out[t][perm_k[i]] = sum over k of in_k[t][i] (k in
// order, in fp32, rounded once): each output row is accumulated in an fp32
// LDS row, every input adding its row at its permuted positions (a
// permutation touches every position once, so the adds of one input never
// collide), and leaves with 16-byte stores.  Indices are clamped into [0, d).
template <typename E>
__global__ __launch_bounds__(256) void k_scatter_sum_lds(const ScatterIns si, E* __restrict__ out, int64_t ld_out,
                                                         int rows, int d, int rpw, int pitch) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* acc = reinterpret_cast<float*>(smem);
  constexpr int V = 16 / sizeof(E);
  const int t0 = blockIdx.x * rpw;
  const int nr = min(rpw, rows - t0);
  for (int i = threadIdx.x; i < nr * pitch; i += blockDim.x) acc[i] = 0.f;
  __syncthreads();
  for (int k = 0; k < si.count; ++k) {
    const E* in = reinterpret_cast<const E*>(si.in[k]);
    const int32_t* perm = si.perm[k];
    const bool vin = (reinterpret_cast<uintptr_t>(in) % 16 == 0) && (si.ld_in[k] % V == 0) &&
                     (reinterpret_cast<uintptr_t>(perm) % 16 == 0);
    const int dv = vin ? d / V : 0;
    for (int rr = 0; rr < nr; ++rr) {
      const E* row = in + (int64_t)(t0 + rr) * si.ld_in[k];
      float* a = acc + rr * pitch;
      for (int c = threadIdx.x; c < dv; c += blockDim.x) {
        const uint4 v = reinterpret_cast<const uint4*>(row)[c];
        E vals[V];
        __builtin_memcpy(vals, &v, 16);
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
          const int4 w = reinterpret_cast<const int4*>(perm + c * V)[q];
          a[min(max(w.x, 0), d - 1)] += to_f32(vals[4 * q]);
          a[min(max(w.y, 0), d - 1)] += to_f32(vals[4 * q + 1]);
          a[min(max(w.z, 0), d - 1)] += to_f32(vals[4 * q + 2]);
          a[min(max(w.w, 0), d - 1)] += to_f32(vals[4 * q + 3]);
        }
      }
      for (int i = dv * V + threadIdx.x; i < d; i += blockDim.x) a[min(max(perm[i], 0), d - 1)] += to_f32(row[i]);
    }
    __syncthreads();
  }
  for (int rr = 0; rr < nr; ++rr) {
    E* o = out + (int64_t)(t0 + rr) * ld_out;
    const float* a = acc + rr * pitch;
    const int h = lead16(o, d);
    for (int i = threadIdx.x; i < h; i += blockDim.x) o[i] = from_f32<E>(a[i]);
    const int nb = (d - h) / V, tail = h + nb * V;
    for (int c = threadIdx.x; c < nb; c += blockDim.x) {
      E vals[V];
#pragma unroll
      for (int e = 0; e < V; ++e) vals[e] = from_f32<E>(a[h + c * V + e]);
      *reinterpret_cast<uint4*>(o + h + c * V) = *reinterpret_cast<const uint4*>(vals);
    }
    for (int i = tail + threadIdx.x; i < d; i += blockDim.x) o[i] = from_f32<E>(a[i]);
  }
}

// out[t] = in[t] except out[t][idx[i]] = src[t][i] for i < b: each row of `in`
// is staged in LDS with 16-byte loads, the b values are written over it at
// their positions, and the row leaves with 16-byte stores (one pass over the
// untouched columns instead of a copy followed by a scatter).
// A row is staged at the shift of its input row; it leaves with 16-byte
// stores when its output row has the same shift, element by element
// otherwise.  pitch = stage_pitch(d).
template <typename E>
__global__ __launch_bounds__(256) void k_replace_cols_lds(const E* __restrict__ in, int64_t ld_in,
                                                          const E* __restrict__ src, int64_t ld_src, int b,
                                                          const int32_t* __restrict__ idx, E* __restrict__ out,
                                                          int64_t ld_out, int rows, int d, int rpw, int pitch) {
  extern __shared__ __align__(16) unsigned char smem[];
  E* buf = reinterpret_cast<E*>(smem);
  const int t0 = blockIdx.x * rpw;
  const int nr = min(rpw, rows - t0);
  for (int rr = 0; rr < nr; ++rr) {
    const E* row = in + (int64_t)(t0 + rr) * ld_in;
    const int h = lead16(row, d);
    row_to_lds(row, buf + rr * pitch + lds_shift<E>(h), d, h);
  }
  __syncthreads();
  for (int rr = 0; rr < nr; ++rr) {
    const E* srow = src + (int64_t)(t0 + rr) * ld_src;
    E* dst = buf + rr * pitch + lds_shift<E>(lead16(in + (int64_t)(t0 + rr) * ld_in, d));
    for (int i = threadIdx.x; i < b; i += blockDim.x) dst[min(max(idx[i], 0), d - 1)] = srow[i];
  }
  __syncthreads();
  for (int rr = 0; rr < nr; ++rr) {
    E* o = out + (int64_t)(t0 + rr) * ld_out;
    const int h = lead16(o, d);
    const int sh_in = lds_shift<E>(lead16(in + (int64_t)(t0 + rr) * ld_in, d));
    const E* srow = buf + rr * pitch + sh_in;
    if (lds_shift<E>(h) == sh_in) {
      lds_to_row(srow, o, d, h);
    } else {
      for (int i = threadIdx.x; i < d; i += blockDim.x) o[i] = srow[i];
    }
  }
}

// The same scatter for rows too long to stage (one row per workgroup).
template <typename E>
__global__ __launch_bounds__(256) void k_scatter_direct(const E* __restrict__ in, int64_t ld_in,
                                                        const int32_t* __restrict__ perm, E* __restrict__ out,
                                                        int64_t ld_out, int d) {
  const int64_t t = blockIdx.x;
  for (int i = threadIdx.x; i < d; i += blockDim.x) out[t * ld_out + min(max(perm[i], 0), d - 1)] = in[t * ld_in + i];
}

__global__ void k_inverse_perm(const int32_t* __restrict__ perm, int d, int32_t* __restrict__ inv) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < d) inv[min(max(perm[i], 0), d - 1)] = i;
}

// dst[t][idx[i]] = src[t][i] for i < b (indices clamped into [0, d)); rows in
// a grid-stride loop over blockIdx.y
template <typename T>
__global__ void k_scatter_cols(const T* __restrict__ src, int64_t ld_src, int rows, int b,
                               const int32_t* __restrict__ idx, T* __restrict__ dst, int64_t ld_dst, int d) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= b) return;
  const int64_t c = min(max(idx[i], 0), d - 1);
  for (int t = blockIdx.y; t < rows; t += gridDim.y) dst[(int64_t)t * ld_dst + c] = src[(int64_t)t * ld_src + i];
}

__global__ void k_compose_perm(const int32_t* __restrict__ a, int da, const int32_t* __restrict__ bm, int n,
                               int32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = a[min(max(bm[i], 0), da - 1)];
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

// p[r][c0 .. c0 + w) = 0 for r < rows (row pitch ld elements)
template <typename E>
__global__ void k_zero_cols(E* __restrict__ p, int64_t ld, int rows, int c0, int w) {
  const int64_t total = (int64_t)rows * w;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x)
    p[(u / w) * ld + c0 + u % w] = E(0);
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

hipError_t zero_cols(int dt, void* p, int64_t ld, int rows, int c0, int c1, hipStream_t s) {
  if (rows <= 0 || c1 <= c0) return hipSuccess;
  if (c0 < 0 || c1 > ld) return hipErrorInvalidValue;
  const int w = c1 - c0;
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv((int64_t)rows * w, 256), 4096);
  if (dt == F32)
    k_zero_cols<float><<<grid, 256, 0, s>>>(reinterpret_cast<float*>(p), ld, rows, c0, w);
  else if (dt == BF16)
    k_zero_cols<bf16_t><<<grid, 256, 0, s>>>(reinterpret_cast<bf16_t*>(p), ld, rows, c0, w);
  else
    k_zero_cols<int8_t><<<grid, 256, 0, s>>>(reinterpret_cast<int8_t*>(p), ld, rows, c0, w);
  return hipGetLastError();
}

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
  // Small workgroups keep many rows in flight per CU: about 8 KB of rows per
  // workgroup (one row at d >= 4096 bf16) measured fastest, against 2-3x
  // slower copies with 64 KB per workgroup.
  const size_t budget = 64 * 1024, target = 8 * 1024;
  auto go = [&](auto tag) -> hipError_t {
    using E = decltype(tag);
    const size_t pitch_bytes = (row_bytes + 15) / 16 * 16;
    const int64_t pitch = stage_pitch(d_in, es);
    if ((size_t)pitch * es <= budget) {
      const int rpw = (int)std::max<size_t>(1, std::min<size_t>(16, target / pitch_bytes));
      k_permute_lds<E><<<cdiv(rows, rpw), 256, rpw * pitch * es, s>>>(
          reinterpret_cast<const E*>(in), ld_in, rowmap, colmap, reinterpret_cast<E*>(out), ld_out, rows, d_in, d_out,
          rpw, (int)pitch);
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

hipError_t permute_multi(int dt, const void* in, int64_t ld_in, int count, const int32_t* const* colmap,
                         void* const* out, const int64_t* ld_out, const int* d_out, int rows, int d_in, hipStream_t s) {
  if (rows <= 0 || count <= 0) return hipSuccess;
  if (count > kGatherOuts) return hipErrorInvalidValue;
  const size_t es = dt_size(dt);
  const size_t pitch_bytes = ((size_t)d_in * es + 15) / 16 * 16;
  const int64_t pitch = stage_pitch(d_in, es);
  const size_t budget = 64 * 1024, target = 8 * 1024;  // as for permute
  if ((size_t)pitch * es > budget) {  // rows too long to stage: one gather per output
    for (int k = 0; k < count; ++k) {
      const hipError_t e = permute(dt, in, ld_in, nullptr, colmap[k], out[k], ld_out[k], rows, d_in, d_out[k], s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  GatherOuts go{};
  for (int k = 0; k < count; ++k) {
    if (d_out[k] <= 0) continue;
    const int q = go.count++;
    go.colmap[q] = colmap[k];
    go.out[q] = out[k];
    go.ld_out[q] = ld_out[k];
    go.d_out[q] = d_out[k];
  }
  if (go.count == 0) return hipSuccess;
  const int rpw = (int)std::max<size_t>(1, std::min<size_t>(16, target / pitch_bytes));
  auto go_t = [&](auto tag) -> hipError_t {
    using E = decltype(tag);
    k_permute_lds_multi<E><<<cdiv(rows, rpw), 256, rpw * pitch * es, s>>>(reinterpret_cast<const E*>(in), ld_in, go,
                                                                           rows, d_in, rpw, (int)pitch);
    return hipGetLastError();
  };
  if (dt == F32) return go_t(float{});
  if (dt == BF16) return go_t(bf16_t{});
  return go_t(int8_t{});
}

hipError_t scatter_sum(int dt, int count, const void* const* in, const int64_t* ld_in, const int32_t* const* perm,
                       void* out, int64_t ld_out, int rows, int d, hipStream_t s) {
  if (rows <= 0 || d <= 0) return hipSuccess;
  if (count < 1 || count > kGatherOuts) return hipErrorInvalidValue;
  if (count == 1) return scatter(dt, in[0], ld_in[0], perm[0], out, ld_out, rows, d, s);
  const size_t pitch = ((size_t)d + 3) / 4 * 4;  // fp32 row, 16-byte aligned
  const size_t budget = 64 * 1024, target = 16 * 1024;
  if (pitch * 4 > budget) return hipErrorInvalidValue;
  ScatterIns si{};
  for (int k = 0; k < count; ++k) {
    si.in[k] = in[k];
    si.ld_in[k] = ld_in[k];
    si.perm[k] = perm[k];
  }
  si.count = count;
  const int rpw = (int)std::max<size_t>(1, std::min<size_t>(16, target / (pitch * 4)));
  auto go = [&](auto tag) -> hipError_t {
    using E = decltype(tag);
    k_scatter_sum_lds<E><<<cdiv(rows, rpw), 256, rpw * pitch * 4, s>>>(si, reinterpret_cast<E*>(out), ld_out, rows, d,
                                                                        rpw, (int)pitch);
    return hipGetLastError();
  };
  if (dt == F32) return go(float{});
  if (dt == BF16) return go(bf16_t{});
  return hipErrorInvalidValue;
}

hipError_t scatter(int dt, const void* in, int64_t ld_in, const int32_t* perm, void* out, int64_t ld_out, int rows,
                   int d, hipStream_t s) {
  if (rows <= 0 || d <= 0) return hipSuccess;
  const size_t es = dt_size(dt);
  const size_t budget = 64 * 1024, target = 8 * 1024;  // as for permute
  auto go = [&](auto tag) -> hipError_t {
    using E = decltype(tag);
    const size_t pitch_bytes = ((size_t)d * es + 15) / 16 * 16;
    const int64_t pitch = stage_pitch(d, es);
    if ((size_t)pitch * es <= budget) {
      const int rpw = (int)std::max<size_t>(1, std::min<size_t>(16, target / pitch_bytes));
      k_scatter_lds<E><<<cdiv(rows, rpw), 256, rpw * pitch * es, s>>>(
          reinterpret_cast<const E*>(in), ld_in, perm, reinterpret_cast<E*>(out), ld_out, rows, d, rpw, (int)pitch);
    } else {
      k_scatter_direct<E><<<rows, 256, 0, s>>>(reinterpret_cast<const E*>(in), ld_in, perm,
                                               reinterpret_cast<E*>(out), ld_out, d);
    }
    return hipGetLastError();
  };
  if (dt == F32) return go(float{});
  if (dt == BF16) return go(bf16_t{});
  return go(int8_t{});
}

hipError_t replace_cols(int dt, const void* in, int64_t ld_in, const void* src, int64_t ld_src, int b,
                        const int32_t* idx, void* out, int64_t ld_out, int rows, int d, hipStream_t s) {
  if (rows <= 0 || d <= 0) return hipSuccess;
  const size_t es = dt_size(dt);
  const size_t pitch_bytes = ((size_t)d * es + 15) / 16 * 16;
  const int64_t pitch = stage_pitch(d, es);
  const size_t budget = 64 * 1024, target = 8 * 1024;  // as for permute
  if ((size_t)pitch * es > budget) {  // rows too long to stage: copy, then write the subset
    const hipError_t e = hipMemcpy2DAsync(out, (size_t)ld_out * es, in, (size_t)ld_in * es, (size_t)d * es,
                                          (size_t)rows, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
    return scatter_cols(dt, src, ld_src, rows, b, idx, out, ld_out, d, s);
  }
  const int rpw = (int)std::max<size_t>(1, std::min<size_t>(16, target / pitch_bytes));
  auto go = [&](auto tag) -> hipError_t {
    using E = decltype(tag);
    k_replace_cols_lds<E><<<cdiv(rows, rpw), 256, rpw * pitch * es, s>>>(
        reinterpret_cast<const E*>(in), ld_in, reinterpret_cast<const E*>(src), ld_src, b, idx,
        reinterpret_cast<E*>(out), ld_out, rows, d, rpw, (int)pitch);
    return hipGetLastError();
  };
  if (dt == F32) return go(float{});
  if (dt == BF16) return go(bf16_t{});
  return go(int8_t{});
}

hipError_t widen_i8(const int8_t* src, int64_t ld_src, int rows, int cols, bool trans, bf16_t* dst, int64_t ld_dst,
                    hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (trans) {
    if (ld_dst < rows) return hipErrorInvalidValue;
    const dim3 grid(cdiv(ld_dst, 64), cdiv(cols, 64));
    if (grid.y > 65535) return hipErrorInvalidValue;
    k_widen_i8_t<<<grid, 256, 0, s>>>(src, ld_src, rows, cols, dst, ld_dst);
  } else {
    if (ld_dst < cols) return hipErrorInvalidValue;
    const int64_t units = (int64_t)rows * cdiv(cols, 16);
    k_widen_i8<<<(unsigned)std::min<int64_t>(cdiv(units, 256), 8192), 256, 0, s>>>(src, ld_src, rows, cols, dst, ld_dst);
    // columns [cols, ld_dst) zero as well, as in the transposed form
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return zero_cols(BF16, dst, ld_dst, rows, cols, (int)ld_dst, s);
  }
  return hipGetLastError();
}

hipError_t transpose(int dt, const void* src, int64_t ld_src, int rows, int cols, void* dst, int64_t ld_dst,
                     hipStream_t s) {
  if (rows <= 0 || cols <= 0 || ld_dst < rows) return rows <= 0 || cols <= 0 ? hipSuccess : hipErrorInvalidValue;
  const dim3 grid(cdiv(ld_dst, 64), cdiv(cols, 64));
  if (grid.y > 65535) return hipErrorInvalidValue;
  if (dt == F32)
    k_transpose<uint32_t><<<grid, 256, 0, s>>>(reinterpret_cast<const uint32_t*>(src), ld_src, rows, cols,
                                               reinterpret_cast<uint32_t*>(dst), ld_dst);
  else if (dt == BF16)
    k_transpose<uint16_t><<<grid, 256, 0, s>>>(reinterpret_cast<const uint16_t*>(src), ld_src, rows, cols,
                                               reinterpret_cast<uint16_t*>(dst), ld_dst);
  else
    k_transpose<uint8_t><<<grid, 256, 0, s>>>(reinterpret_cast<const uint8_t*>(src), ld_src, rows, cols,
                                              reinterpret_cast<uint8_t*>(dst), ld_dst);
  return hipGetLastError();
}

hipError_t inverse_perm(const int32_t* perm, int d, int32_t* inv, hipStream_t s) {
  k_inverse_perm<<<cdiv(d, 256), 256, 0, s>>>(perm, d, inv);
  return hipGetLastError();
}

hipError_t scatter_cols(int dt, const void* src, int64_t ld_src, int rows, int b, const int32_t* idx, void* dst,
                        int64_t ld_dst, int d, hipStream_t s) {
  if (rows <= 0 || b <= 0) return hipSuccess;
  const dim3 grid(cdiv(b, 256), (unsigned)std::min(rows, 4096));
  if (dt_size(dt) == 2)
    k_scatter_cols<uint16_t><<<grid, 256, 0, s>>>(reinterpret_cast<const uint16_t*>(src), ld_src, rows, b, idx,
                                                  reinterpret_cast<uint16_t*>(dst), ld_dst, d);
  else if (dt_size(dt) == 4)
    k_scatter_cols<uint32_t><<<grid, 256, 0, s>>>(reinterpret_cast<const uint32_t*>(src), ld_src, rows, b, idx,
                                                  reinterpret_cast<uint32_t*>(dst), ld_dst, d);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t compose_perm(const int32_t* a, const int32_t* b, int d, int32_t* out, hipStream_t s) {
  return compose_idx(a, d, b, d, out, s);
}

hipError_t compose_idx(const int32_t* a, int da, const int32_t* b, int n, int32_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_compose_perm<<<cdiv(n, 256), 256, 0, s>>>(a, da, b, n, out);
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

template <class CD, class C, typename T, typename IT, typename GT, typename OT>
static hipError_t apply_t(const void* in, int64_t ld_in, int rows, int d, int b, const void* dT, const float* cs,
                          void* out, int64_t ld_out, hipStream_t s) {
  const int lds = std::max(smem_bytes<C, T, OT>(), dma_smem_bytes<CD>());
  auto k = k_apply<CD, C, T, IT, GT, OT>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  const int64_t units = (int64_t)cdiv(rows, C::BM) * cdiv(b, C::BN) * nblocks(d, b);
  if (units > INT32_MAX) return hipErrorInvalidValue;
  k<<<(unsigned)units, C::NT, lds, s>>>(reinterpret_cast<const IT*>(in), ld_in, rows, d, b,
                                        reinterpret_cast<const GT*>(dT), cs, reinterpret_cast<OT*>(out), ld_out);
  return hipGetLastError();
}

// bf16 block products on output tiles: 256 x 256 tiles when they give every
// CU a workgroup, else 128 x 128 tiles (two per CU)
static hipError_t apply_bf16_tiled(const void* in, int64_t ld_in, int rows, int d, int b, const void* dT,
                                   const float* cs, void* out, int64_t ld_out, hipStream_t s) {
  if ((int64_t)cdiv(rows, 256) * cdiv(b, 256) * nblocks(d, b) >= 256)
    return apply_t<DGemm, TGemm, bf16_t, bf16_t, bf16_t, bf16_t>(in, ld_in, rows, d, b, dT, cs, out, ld_out, s);
  return apply_t<DSq, TSq, bf16_t, bf16_t, bf16_t, bf16_t>(in, ld_in, rows, d, b, dT, cs, out, ld_out, s);
}

// the streamed whole blocks of the sides in `tb` (tb.first[count] blocks in all)
template <int B, int RT, int S>
static hipError_t apply_stream_t(const StreamSides& tb, int rows, bool cs, hipStream_t s) {
  using C = StreamCfg<B, RT, S>;
  const bool multi = tb.count > 1;
  auto k = multi ? (cs ? k_apply_stream<B, RT, S, true, true> : k_apply_stream<B, RT, S, false, true>)
                 : (cs ? k_apply_stream<B, RT, S, true, false> : k_apply_stream<B, RT, S, false, false>);
  hipError_t e = allow_lds(k, C::LDS);
  if (e != hipSuccess) return e;
  const int64_t items = (int64_t)tb.first[tb.count] * cdiv(rows, RT);
  // one workgroup per CU; pair lanes come in multiples of 8 (one share per XCD)
  const int pair_lanes = (int)(std::min<int64_t>(256 / C::NH, items) / 8 * 8);
  if (pair_lanes < 8 || items > INT32_MAX) return hipErrorInvalidValue;
  k<<<pair_lanes * C::NH, C::NT, C::LDS, s>>>(tb, rows, (int)items, pair_lanes);
  return hipGetLastError();
}

static StreamSides one_side(const void* in, int64_t ld_in, int nbf, const void* dT, const float* cs, void* out,
                            int64_t ld_out) {
  StreamSides tb{};
  tb.in[0] = reinterpret_cast<const bf16_t*>(in);
  tb.dT[0] = reinterpret_cast<const bf16_t*>(dT);
  tb.cs[0] = cs;
  tb.out[0] = reinterpret_cast<bf16_t*>(out);
  tb.ld_in[0] = ld_in;
  tb.ld_out[0] = ld_out;
  tb.first[0] = 0;
  tb.first[1] = nbf;
  tb.count = 1;
  return tb;
}

static bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// bf16 block products: the streaming kernel for the whole blocks of 256 or 512
// columns when there are enough row tiles to occupy the chip, the tiled kernel
// for the rest (other block sizes, a partial last block, small inputs)
constexpr int kStreamRT = 32;

// whole blocks of this side can be streamed (the kernel addresses a row tile
// with 32-bit byte offsets)
static bool streamable(const void* in, int64_t ld_in, int d, int b, const void* dT, const float* cs, const void* out,
                       int64_t ld_out) {
  return (b == 256 || b == 512) && d / b > 0 && ld_in % 8 == 0 && ld_out % 8 == 0 && ld_in < (1 << 25) &&
         ld_out < (1 << 25) && aligned16(in) && aligned16(out) && aligned16(dT) && (!cs || aligned16(cs));
}

static hipError_t apply_stream_sides(const StreamSides& tb, int rows, int b, bool cs, hipStream_t s) {
  return b == 512 ? apply_stream_t<512, kStreamRT, 3>(tb, rows, cs, s) : apply_stream_t<256, kStreamRT, 4>(tb, rows, cs, s);
}

static hipError_t apply_bf16(const void* in, int64_t ld_in, int rows, int d, int b, const void* dT, const float* cs,
                             void* out, int64_t ld_out, hipStream_t s) {
  const int nbf = d / b;
  constexpr int RT = kStreamRT;
  if (streamable(in, ld_in, d, b, dT, cs, out, ld_out) && (int64_t)nbf * cdiv(rows, RT) >= 64) {
    hipError_t e = apply_stream_sides(one_side(in, ld_in, nbf, dT, cs, out, ld_out), rows, b, cs != nullptr, s);
    if (e != hipSuccess || nbf * b == d) return e;
    const int64_t kb = (int64_t)nbf * b;
    return apply_bf16_tiled(reinterpret_cast<const bf16_t*>(in) + kb, ld_in, rows, d - (int)kb, b,
                            reinterpret_cast<const bf16_t*>(dT) + kb * b, cs ? cs + kb : nullptr,
                            reinterpret_cast<bf16_t*>(out) + kb, ld_out, s);
  }
  return apply_bf16_tiled(in, ld_in, rows, d, b, dT, cs, out, ld_out, s);
}

hipError_t apply_batch(int count, const ApplySide* sides, int rows, int b, hipStream_t s) {
  if (rows <= 0 || count <= 0) return hipSuccess;
  if (count > kApplySides) return hipErrorInvalidValue;
  // the streamed whole blocks of the sides that apply() would stream share one launch (so every
  // output is computed as apply() computes it); a side's partial last block, and every other side,
  // take apply_bf16's other paths
  auto in_stream = [&](const ApplySide& a) {
    return streamable(a.in, a.ld_in, a.d, b, a.dT, a.colscale, a.out, a.ld_out) &&
           (int64_t)(a.d / b) * cdiv(rows, kStreamRT) >= 64;
  };
  StreamSides tb{};
  bool cs = false;
  int64_t blocks = 0;
  for (int i = 0; i < count; ++i) {
    const ApplySide& a = sides[i];
    if (!in_stream(a)) continue;
    const int q = tb.count++;
    tb.in[q] = reinterpret_cast<const bf16_t*>(a.in);
    tb.dT[q] = reinterpret_cast<const bf16_t*>(a.dT);
    tb.cs[q] = a.colscale;
    tb.out[q] = reinterpret_cast<bf16_t*>(a.out);
    tb.ld_in[q] = a.ld_in;
    tb.ld_out[q] = a.ld_out;
    tb.first[q] = (int)blocks;
    blocks += a.d / b;
    cs = cs || a.colscale;
  }
  tb.first[tb.count] = (int)blocks;
  if (tb.count > 0) {
    const hipError_t e = apply_stream_sides(tb, rows, b, cs, s);
    if (e != hipSuccess) return e;
  }
  for (int i = 0; i < count; ++i) {
    const ApplySide& a = sides[i];
    hipError_t e = hipSuccess;
    if (in_stream(a)) {
      const int64_t kb = (int64_t)(a.d / b) * b;
      if (kb < a.d)
        e = apply_bf16_tiled(reinterpret_cast<const bf16_t*>(a.in) + kb, a.ld_in, rows, a.d - (int)kb, b,
                             reinterpret_cast<const bf16_t*>(a.dT) + kb * b, a.colscale ? a.colscale + kb : nullptr,
                             reinterpret_cast<bf16_t*>(a.out) + kb, a.ld_out, s);
    } else {
      e = apply_bf16(a.in, a.ld_in, rows, a.d, b, a.dT, a.colscale, a.out, a.ld_out, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t apply(int cdt, int in_dt, const void* in, int64_t ld_in, int rows, int d, int b, int dT_dt, const void* dT,
                 const float* colscale, int out_dt, void* out, int64_t ld_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (cdt == BF16 && in_dt == BF16 && dT_dt == BF16 && out_dt == BF16)
    return apply_bf16(in, ld_in, rows, d, b, dT, colscale, out, ld_out, s);
  // fp32 layers (their merge products included: fp32 weight rows times fp32 blocks)
  if (cdt == F32 && in_dt == F32 && dT_dt == F32 && out_dt == F32)
    return apply_t<void, TF, float, float, float, float>(in, ld_in, rows, d, b, dT, colscale, out, ld_out, s);
  // merge products of bf16 layers: fp32 weight rows times the stored bf16 blocks
  if (cdt == F32 && in_dt == F32 && dT_dt == BF16 && out_dt == F32)
    return apply_t<void, TFM, float, float, bf16_t, float>(in, ld_in, rows, d, b, dT, colscale, out, ld_out, s);
  return hipErrorInvalidValue;
}

template <class CD, class C, typename T, typename AT, typename BT, typename OT, bool BKN>
static hipError_t gemm_t(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K, const float* cs,
                         void* out, int64_t ldo, hipStream_t s) {
  const int lds = std::max(smem_bytes<C, T, OT>(), dma_smem_bytes<CD>());
  auto k = k_gemm<CD, C, T, AT, BT, OT, BKN>;
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
  // the direct-to-LDS loop serves bf16 operands that are both K-contiguous
  using CD = typename std::conditional<!BKN && std::is_same<BT, bf16_t>::value, DGemm, void>::type;
  using C = typename std::conditional<std::is_same<BT, bf16_t>::value, TGemmI, TGemm>::type;
  if ((int64_t)cdiv(M, 256) * cdiv(N, 256) >= 256)
    return gemm_t<CD, C, bf16_t, bf16_t, BT, bf16_t, BKN>(A, lda, B, ldb, M, N, K, cs, out, ldo, s);
  if constexpr (!std::is_same<CD, void>::value)
    return gemm_t<DNarrow, TNarrow, bf16_t, bf16_t, BT, bf16_t, BKN>(A, lda, B, ldb, M, N, K, cs, out, ldo, s);
  return gemm_t<void, TBig, bf16_t, bf16_t, BT, bf16_t, BKN>(A, lda, B, ldb, M, N, K, cs, out, ldo, s);
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
    return b_kn ? gemm_t<void, TF, float, float, float, float, true>(A, lda, B, ldb, M, N, K, colscale, out, ldo, s)
                : gemm_t<void, TF, float, float, float, float, false>(A, lda, B, ldb, M, N, K, colscale, out, ldo, s);
  return hipErrorInvalidValue;
}

int gemm_launches(int count, const GemmProblem* p, int* launch_of) {
  auto tiles_of = [](const GemmProblem& x) { return (int64_t)cdiv(x.M, 256) * cdiv(x.N, 256); };
  // A problem that gives every CU a 256 x 256 tile runs alone, as gemm() runs it: next to another in
  // one launch it would share the Infinity Cache with it, and the XCDs' contiguous shares of the
  // launch would end at different times.  Smaller problems of equal K (equal work per tile) share a
  // launch of 256 x 256 tiles when together they give every CU a tile; the rest run alone.
  auto small = [&](const GemmProblem& x) { return x.M > 0 && x.N > 0 && tiles_of(x) < 256; };
  for (int i = 0; i < count; ++i) launch_of[i] = -1;
  int n = 0;
  for (int i = 0; i < count; ++i) {
    if (launch_of[i] >= 0 || !small(p[i])) continue;
    int64_t tiles = 0;
    int members = 0;
    for (int j = i; j < count; ++j)
      if (launch_of[j] < 0 && small(p[j]) && p[j].K == p[i].K) {
        tiles += tiles_of(p[j]);
        ++members;
      }
    if (members < 2 || tiles < 256) continue;
    for (int j = i; j < count; ++j)
      if (launch_of[j] < 0 && small(p[j]) && p[j].K == p[i].K) launch_of[j] = n;
    ++n;
  }
  for (int i = 0; i < count; ++i)
    if (launch_of[i] < 0) launch_of[i] = n++;
  return n;
}

hipError_t gemm_batch(int count, const GemmProblem* p, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (count > kGemmProblems) return hipErrorInvalidValue;
  int launch_of[kGemmProblems];
  const int n = gemm_launches(count, p, launch_of);
  for (int l = 0; l < n; ++l) {
    GemmTable tb{};
    int64_t tiles = 0;
    int last = -1;
    for (int i = 0; i < count; ++i) {
      if (launch_of[i] != l) continue;
      const GemmProblem& x = p[i];
      last = i;
      if (x.M <= 0 || x.N <= 0) continue;
      const int q = tb.count++;
      tb.A[q] = reinterpret_cast<const bf16_t*>(x.A);
      tb.B[q] = reinterpret_cast<const bf16_t*>(x.B);
      tb.cs[q] = x.colscale;
      tb.out[q] = reinterpret_cast<bf16_t*>(x.out);
      tb.lda[q] = x.lda;
      tb.ldb[q] = x.ldb;
      tb.ldo[q] = x.ldo;
      tb.M[q] = x.M;
      tb.N[q] = x.N;
      tb.K[q] = x.K;
      tb.first[q] = (int)tiles;
      tiles += (int64_t)cdiv(x.M, 256) * cdiv(x.N, 256);
    }
    tb.first[tb.count] = (int)tiles;
    hipError_t e = hipSuccess;
    if (tb.count < 2) {
      const GemmProblem& x = p[last];
      e = gemm(BF16, BF16, x.A, x.lda, BF16, x.B, x.ldb, false, x.M, x.N, x.K, x.colscale, BF16, x.out, x.ldo, s);
    } else {
      using CD = DGemm;
      using C = TGemmI;
      const int lds = std::max(smem_bytes<C, bf16_t, bf16_t>(), dma_smem_bytes<CD>());
      auto k = k_gemm_group<CD, C>;
      e = allow_lds(k, lds);
      if (e == hipSuccess) {
        k<<<(unsigned)tiles, C::NT, lds, s>>>(tb);
        e = hipGetLastError();
      }
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
