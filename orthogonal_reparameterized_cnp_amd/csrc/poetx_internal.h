// Internal launchers shared by the C ABI layer (not part of the public API).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pxk {

enum Dt : int { F32 = 0, BF16 = 1, I8 = 2 };

inline size_t dt_size(int dt) { return dt == F32 ? 4 : dt == BF16 ? 2 : 1; }
inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
inline int64_t packed_len(int64_t b) { return b * (b - 1) / 2; }
inline int nblocks(int d, int b) { return (d + b - 1) / b; }

// Leading dimension of every [rows x d] buffer the library lays out itself
// (pre-merged weight, saved activation, workspace matrices): a multiple of 64
// elements, so rows start 128-byte aligned for bf16 and 256-byte for fp32.
inline int64_t lead(int d) { return round_up(d, 64); }

// out[t][i] = in[rowmap ? rowmap[t] : t][colmap[i]] for t < rows, i < d_out.
hipError_t permute(int dt, const void* in, int64_t ld_in, const int32_t* rowmap, const int32_t* colmap, void* out,
                   int64_t ld_out, int rows, int d_in, int d_out, hipStream_t s);
// out[t][perm[i]] = in[t][i] for t < rows, i < d (the inverse of the gather
// out[t][i] = in[t][perm[i]]), without forming the inverse permutation
hipError_t scatter(int dt, const void* in, int64_t ld_in, const int32_t* perm, void* out, int64_t ld_out, int rows,
                   int d, hipStream_t s);
// dst[c][r] = src[r][c] for r < rows, c < cols; dst[c][r] = 0 for rows <= r < ld_dst
// int8 codes [rows][cols] (pitch ld_src) widened to bf16: dst[r][c], or with
// trans dst[c][r] (dst columns [rows, ld_dst) zero); exact.
hipError_t widen_i8(const int8_t* src, int64_t ld_src, int rows, int cols, bool trans, uint16_t* dst, int64_t ld_dst,
                    hipStream_t s);
hipError_t transpose(int dt, const void* src, int64_t ld_src, int rows, int cols, void* dst, int64_t ld_dst,
                     hipStream_t s);
// dst[t][idx[i]] = src[t][i] for t < rows, i < b (idx values clamped into [0, d))
hipError_t scatter_cols(int dt, const void* src, int64_t ld_src, int rows, int b, const int32_t* idx, void* dst,
                        int64_t ld_dst, int d, hipStream_t s);
// out[t] = in[t] with out[t][idx[i]] = src[t][i] for i < b (out != in), in one pass
hipError_t replace_cols(int dt, const void* in, int64_t ld_in, const void* src, int64_t ld_src, int b,
                        const int32_t* idx, void* out, int64_t ld_out, int rows, int d, hipStream_t s);
// permute without a row map for `count` outputs from one input: out[k][:, i] =
// in[:, colmap[k][i]] for i < d_out[k], each input row read once
constexpr int kGatherOuts = 8;
hipError_t permute_multi(int dt, const void* in, int64_t ld_in, int count, const int32_t* const* colmap,
                         void* const* out, const int64_t* ld_out, const int* d_out, int rows, int d_in, hipStream_t s);
// out[:, perm[k][i]] = sum over k < count of in[k][:, i] (in order, fp32, rounded once to dt; count
// 1 .. kGatherOuts; rows of up to 16 K fp32 values)
hipError_t scatter_sum(int dt, int count, const void* const* in, const int64_t* ld_in, const int32_t* const* perm,
                       void* out, int64_t ld_out, int rows, int d, hipStream_t s);
// inv[perm[i]] = i
hipError_t inverse_perm(const int32_t* perm, int d, int32_t* inv, hipStream_t s);
// out[i] = a[b[i]]
hipError_t compose_perm(const int32_t* a, const int32_t* b, int d, int32_t* out, hipStream_t s);
// out[i] = a[b[i]] for i < n, with a of length da (b's values clamped into [0, da))
hipError_t compose_idx(const int32_t* a, int da, const int32_t* b, int n, int32_t* out, hipStream_t s);
// Durstenfeld shuffle of the identity driven by SplitMix64(seed)
hipError_t perm_from_seed_device(uint64_t seed, int d, int32_t* out, int32_t* scratch, hipStream_t s);

// Most sides in one batched CNP launch (the size of the kernels' side table).
constexpr int kMaxSides = 64;
constexpr int kGradSides = 16;  // sides of one block-gradient launch

// Delta = G - I of every block of `count` sides, and its transpose: side i
// writes g[i] = [2][nb_i][b][b] in dtype dt (F32 or BF16).  Sides are
// independent; the blocks of all of them share each launch.  ws holds
// cnp_build_ws_bytes(dt, sum of nb_i, b) bytes.
hipError_t cnp_build_batch(int dt, int count, const float* const* q, const int* d, int b, void* const* g, void* ws,
                           hipStream_t s);
size_t cnp_build_ws_bytes(int dt, int64_t blocks, int b);

// Row-form block-diagonal product: out[:, kb+j] = (in[:, kb+j] + sum_k in[:, kb+k] D_blk[k][j]) * scale[kb+j]
// where the B operand array `dT` holds D_blk^T, i.e. dT[blk][j][k] = D_blk[k][j].
// Compute dtype cdt; `in`, `dT`, `out` in their own dtypes.
hipError_t apply(int cdt, int in_dt, const void* in, int64_t ld_in, int rows, int d, int b, int dT_dt, const void* dT,
                 const float* colscale, int out_dt, void* out, int64_t ld_out, hipStream_t s);

// `count` bf16 block products of the same rows and b as apply() computes them,
// the streamed whole blocks of all of them in shared launches (the results are
// those of one apply() per side).
constexpr int kApplySides = 8;
struct ApplySide {
  const void* in;
  int64_t ld_in;
  int d;
  const void* dT;
  const float* colscale;
  void* out;
  int64_t ld_out;
};
hipError_t apply_batch(int count, const ApplySide* sides, int rows, int b, hipStream_t s);

// out = A * B (* colscale), A: [M][K] rows (lda); B either [K][N] (b_kn = true) or [N][K] (b_kn = false).
hipError_t gemm(int cdt, int a_dt, const void* A, int64_t lda, int b_dt, const void* B, int64_t ldb, bool b_kn, int M,
                int N, int K, const float* colscale, int out_dt, void* out, int64_t ldo, hipStream_t s);

// `count` bf16 contractions out_q = A_q B_q^T (* colscale_q) (B_q: [N][K] rows):
// those too small to give every CU a 256 x 256 tile on their own, with equal
// K, in one launch of 256 x 256 tiles when together they do, the others one
// gemm() each; the results are those of one gemm() per problem.
constexpr int kGemmProblems = 8;
struct GemmProblem {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  int M, N, K;
  const float* colscale;
  void* out;
  int64_t ldo;
};
hipError_t gemm_batch(int count, const GemmProblem* p, hipStream_t s);
// the launches gemm_batch makes: launch_of[i] (0 .. n - 1) for each problem, n returned
int gemm_launches(int count, const GemmProblem* p, int* launch_of);

// Block gradients and CNP chain rule.  The gradient state `dg` of
// cnp_grad_bytes(dt, blocks, b) bytes holds, for `blocks` CNP blocks of one
// batch of sides, the block gradients and the chain rule's intermediates.
//   block_grads: the two sides of one linear (side 0 = R, side 1 = P),
//     U_s[blk] = sum over all rows t of A_s[t][blk cols]^T B_s[t][blk cols],
//     written to blocks [zoff, zoff + nb_R + nb_P) of dg (which has `total` blocks)
//   cnp_chain_batch: U -> dQ through the CNP chain rule -> packed dq[i]
//     (overwritten) for `count` sides whose blocks fill dg in order
struct CnpSide {
  const float* q;
  int d;
  const void* A;  // [rows][lda]: Xt for R, H for P
  int64_t lda;
  const void* B;  // [rows][ldb]: dA for R, dZt for P
  int64_t ldb;
};
//   Large bf16 blocks are summed in token splits whose fp32 partials go to
//   `part` (block_grads_part_bytes bytes, 0 when no split is used) and are
//   added in split order.
hipError_t block_grads(int cdt, const CnpSide* sides, int rows, int b, void* dg, int64_t zoff, int64_t total,
                       float* part, hipStream_t s);
//   block_grads_n: the same for `count` (1 .. kGradSides) sides in one launch,
//     their blocks numbered consecutively in side order from zoff; q may be null
hipError_t block_grads_n(int cdt, int count, const CnpSide* sides, int rows, int b, void* dg, int64_t zoff,
                         int64_t total, float* part, hipStream_t s);
int block_grads_splits(int dt, int rows, int blocks, int b);
size_t block_grads_part_bytes(int dt, int rows, int blocks, int b);
//   build: null, or the workspace of the cnp_build_batch call for the same sides (its dense Q and
//     S = Q Q are read instead of formed again)
hipError_t cnp_chain_batch(int cdt, int count, const float* const* q, const int* d, int b, void* dg, float* const* dq,
                           hipStream_t s, const void* build = nullptr);
size_t cnp_grad_bytes(int dt, int64_t blocks, int b);

// Merge helpers (fp32 MFMA).
// M1[kb+i][c] = (W[kb+i][c] + sum_k DeltaR_blk[i][k] W[kb+k][c]) * wscale[c]
hipError_t merge_left(int g_dt, const void* gR, int w_dt, const void* W, int64_t ldw, const float* wscale, int m, int n,
                      int b, float* M1, int64_t ldm, hipStream_t s);
// column absmax of M [rows][ld] over rows, as float bits (max over non-negative floats)
hipError_t col_absmax(const float* M, int64_t ld, int rows, int n, uint32_t* amax, hipStream_t s);
// write the final weight from fp32 values: f32/bf16 round, or int8 requantisation with fresh scales
hipError_t store_weight(const float* M, int64_t ld, int rows, int n, int w_dt, void* W, int64_t ldw,
                        const uint32_t* amax, float* wscale, hipStream_t s);
hipError_t fill_zero(void* p, size_t bytes, hipStream_t s);
// p[r][c0 .. c1) = 0 for r < rows of a [rows][ld] matrix of dtype dt
hipError_t zero_cols(int dt, void* p, int64_t ld, int rows, int c0, int c1, hipStream_t s);

// Adam step with decoupled weight decay on `count` fp32 arrays in place:
// side i updates len[i] slots of q[i], m1[i], m2[i] from the gradient g[i].
// Sides are packed into launches of at most kAdamSidesPerLaunch.
constexpr int kAdamSidesPerLaunch = 32;
struct AdamHyper {
  double lr, beta1, beta2, eps, weight_decay;
  int64_t t;  // 1-based steps since the moments were zero
};
hipError_t adam_batch(int count, const int64_t* len, float* const* q, const float* const* g, float* const* m1,
                      float* const* m2, const AdamHyper& hp, hipStream_t s);

}  // namespace pxk
