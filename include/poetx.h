/*
 * libpoetx: the POET-X orthogonal-equivalence linear layer on AMD MI355X (gfx950).
 *
 * The layer (POET paper notes, "Reparameterized LLM Training via Orthogonal
 * Equivalence Transformation", 整体框架) reparameterises a frozen weight W0
 * (m inputs x n outputs) as R W0 P with orthogonal R (m x m) and P (n x n) and
 * computes y = (R W0 P)^T x.  With tokens as rows this is Y = X R W0 P.
 *
 * Each factor is one block-stochastic primitive (same notes, 关键设计 1):
 * R = Psi^T Diag(G^0, ..., G^{nb-1}) Psi with nb = ceil(m / b) blocks, a partial
 * last block of r = m - (nb-1) b rows, and Psi the permutation with
 * Psi[i][perm[i]] = 1 (so X Psi^T = X[:, perm]).  Every block is the
 * Cayley-Neumann form of a skew-symmetric Q (关键设计 2 with k = 3, multiplied out
 * as in the zhichai.net POET-X blog, 第四斧 item 2):
 *     G = I + 2 (Q + Q^2 + Q^3) + Q^4.
 * Q is stored only as its strict upper triangle (第四斧 item 1), row by row with
 * the full block stride b: slot p(i, j) = i*b - i(i+1)/2 + (j - i - 1) holds
 * Q[i][j] for i < j, and Q[j][i] = -Q[i][j].  A side's parameters are one fp32
 * array q[nb][b(b-1)/2]; slots of a partial block with j >= r are ignored.
 *
 * The forward runs in input-centric order (blog 第一斧): gather the input
 * columns by perm_R, apply the R blocks as a batch (第三斧), contract with the
 * pre-merged weight W~ = W0[perm_R, :][:, perm_P] (the two permutations next to
 * W0 are folded into it, 第二斧), apply the P blocks, and scatter the output
 * columns by perm_P.
 *
 * Conventions for every call
 *  - All tensors are caller-owned device memory (plain pointers) unless stated.
 *    Matrices are row-major with the leading dimension stated per argument.
 *  - Every call validates its arguments, then enqueues its kernels on `stream`
 *    (a hipStream_t; NULL means the null stream) and returns without waiting.
 *    On any error nothing is enqueued and nothing is written.
 *  - The library never allocates device memory: scratch space is the caller's
 *    `ws` buffer of at least poetx_workspace_size() bytes, 256-byte aligned.
 *    Calls that share a workspace must not overlap in time.
 *  - The library keeps no state between calls except a per-thread error string
 *    and, while it is enabled, the measurement timer's record.
 *  - Formats the library lays out itself (pre-merged weight, G blocks, saved
 *    activation) are sized by the *_bytes() helpers; their leading dimensions
 *    are rounded up to a multiple of 64 elements.
 */
#ifndef POETX_H
#define POETX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  POETX_OK = 0,
  POETX_E_NULL = 1,        /* a required pointer is NULL */
  POETX_E_SHAPE = 2,       /* m, n, b, d or T out of range */
  POETX_E_DTYPE = 3,       /* unsupported dtype or dtype combination */
  POETX_E_WORKSPACE = 4,   /* ws too small or misaligned */
  POETX_E_PERM = 5,        /* host permutation argument invalid */
  POETX_E_HIP = 6,         /* a HIP runtime call failed (see poetx_last_error) */
  POETX_E_UNSUPPORTED = 7  /* valid request the library does not implement */
} poetx_status;

typedef enum { POETX_F32 = 0, POETX_BF16 = 1, POETX_I8 = 2 } poetx_dtype;

/*
 * Activation saving (gist.science summary, 4. Resultados: the POET-Xfast and
 * POET-Xmem variants).  POETX_XFAST saves H = Xt Diag(G_R) W~ and the gathered
 * input Xt.  POETX_XMEM saves Xt only; the backward recomputes H from it with
 * the forward's own kernels (one more block product and W~ contraction), so its
 * results are bit-identical to POETX_XFAST while the saved state shrinks by
 * T x round_up(n, 64) activations.  POETX_XOUT also saves Xt only and takes H
 * back from the layer's output, H = Y[:, perm_P] Diag(G_P)^T: the checkpoint of
 * the zhichai.net blog, 第五斧 (b = G_P z, one gather and one block product).
 * That inverts the P side exactly only for orthogonal blocks; with the CNP
 * blocks, G G^T = (I - Q^4)^2, so the backward sees H Diag((I - Q_P^4)^2)
 * instead of H, which changes dq_P (dX and dq_R do not use H).  The caller
 * passes Y to the backward.
 */
typedef enum { POETX_XFAST = 0, POETX_XMEM = 1, POETX_XOUT = 2 } poetx_mode;

/* Operation selector for poetx_workspace_size. */
typedef enum { POETX_OP_CNP = 0, POETX_OP_FWD = 1, POETX_OP_BWD = 2, POETX_OP_MERGE = 3 } poetx_op;

/*
 * One linear layer.  act_dtype is the dtype of X, Y, dZ, dX, the saved
 * activation and the G blocks; the block products and contractions run on MFMA
 * in that dtype with fp32 accumulation.  w_dtype is the storage of the
 * pre-merged weight: POETX_F32 (with act F32), POETX_BF16 or POETX_I8 (with act
 * BF16).  POETX_I8 stores symmetric codes with one fp32 scale per output column
 * (POET-XQ, wispaper.ai POET-X blog, "Quantized Training"): W = code * scale[col].
 * Limits: 1 <= m, n <= 1 << 20; 2 <= b <= 1024.
 */
typedef struct {
  int32_t m;
  int32_t n;
  int32_t b;
  int32_t act_dtype;
  int32_t w_dtype;
  int32_t mode; /* poetx_mode: what the forward saves for the backward */
} poetx_layer_desc;

/* ---------------------------------------------------------------- helpers -- */

/* Library version string (static storage). */
const char* poetx_version(void);

/* Message of the last failing call on this thread ("" if none; static per thread). */
const char* poetx_last_error(void);

/* Number of packed values per b x b block: b (b - 1) / 2. */
int64_t poetx_packed_len(int32_t b);

/* Bytes of a side's G buffer: [2][nb][b][b] elements of `dtype`.  Slice 0 holds
 * Delta = G - I of every block, slice 1 holds Delta^T (the layout the forward's
 * block products read).  Entries outside a partial block's r x r corner are 0. */
size_t poetx_g_bytes(int32_t d, int32_t b, int32_t dtype);

/* Bytes of the pre-merged weight buffer: values [m][ldw] of w_dtype, ldw =
 * round_up(n, 64) (columns n and up zero), followed at offset
 * round_up(m*ldw*size(w_dtype), 256) by
 *  - POETX_I8: the fp32 column scales [ldw] in pre-merged column order;
 *  - POETX_BF16: the transposed copy [n][round_up(m, 64)] of the values
 *    (columns m and up zero), which the forward contraction reads so that
 *    both of its operands are contiguous along the summed index.
 * poetx_premerge, poetx_merge_reinit and poetx_store_weight write every part;
 * the contractions sum over the zero padding as well. */
size_t poetx_weight_bytes(const poetx_layer_desc* desc);

/* Bytes of the state the forward saves for the backward of the same T tokens.
 * POETX_XFAST: H = Xt Diag(G_R) W~ as [T][round_up(n, 64)] elements of
 * act_dtype, then, at the next 256-byte boundary, the gathered input
 * Xt = X[:, perm_R] as [T][round_up(m, 64)].  POETX_XMEM and POETX_XOUT: Xt
 * only, at offset 0.
 * The backward reads Xt from here instead of gathering X again, so a caller
 * need not keep X for the backward. */
size_t poetx_saved_bytes(const poetx_layer_desc* desc, int64_t T);

/* Workspace bytes for `op` (POETX_OP_CNP uses desc->m as the side length d and
 * ignores T; POETX_OP_MERGE ignores T).  Returns 0 for invalid arguments. */
size_t poetx_workspace_size(const poetx_layer_desc* desc, int64_t T, int32_t op);

/* Host helper: the permutation drawn from `seed` (used by poetx_merge_reinit).
 * SplitMix64 (Steele, Lea, Flood 2014) seeded with `seed` drives a Durstenfeld
 * shuffle of the identity: for i = d-1 down to 1, j = floor(u * (i+1) / 2^64)
 * for the next 64-bit output u, swap p[i] and p[j].  host_out: [d] host memory.
 * Errors: POETX_E_NULL, POETX_E_SHAPE (d < 1). */
poetx_status poetx_perm_from_seed(uint64_t seed, int32_t d, int32_t* host_out);

/* Kernel classes for the measurement timer. */
typedef enum {
  POETX_KC_NONE = 0,
  POETX_KC_GEMM = 1,    /* the W~ contractions (forward and backward) */
  POETX_KC_APPLY = 2,   /* block-diagonal products over token rows */
  POETX_KC_DGRAD = 3,   /* block gradients summed over tokens */
  POETX_KC_CNP = 4,     /* CNP build and chain rule */
  POETX_KC_PERMUTE = 5, /* permutation gathers */
  POETX_KC_OPTIM = 6    /* optimiser steps on the packed parameters */
} poetx_kernel_class;

/* Measurement support (not for use on a hot path).  While a class is enabled,
 * every launch of that class, on any stream, is bracketed by two hipEvents
 * recorded on the launch's stream, and its algorithmic flop and byte counts
 * are noted.  poetx_timer_read waits for the recorded events, returns the
 * number of launches, their summed duration in milliseconds and the summed
 * algorithmic flops and bytes, and clears the record.  kernel_class 0
 * disables.  Errors: POETX_E_SHAPE (unknown class), POETX_E_NULL, POETX_E_HIP. */
poetx_status poetx_timer_enable(int32_t kernel_class);
poetx_status poetx_timer_read(int64_t* launches, double* total_ms, double* flops, double* bytes);

/* ------------------------------------------------------------- the calls -- */

/*
 * Build the CNP blocks of one side (zhichai.net blog, 第四斧: Q^2 computed once,
 * Q^3, Q^4 and G formed from it; POET notes, 关键设计 2, k = 3).
 *   q      [nb][b(b-1)/2] fp32, packed skew parameters, nb = ceil(d / b)
 *   d, b   side length (m for R, n for P) and block size
 *   dtype  POETX_F32 or POETX_BF16: dtype of g (must equal the layer's act_dtype)
 *   g      out, poetx_g_bytes(d, b, dtype) bytes: Delta = G - I and Delta^T
 *   ws     >= poetx_workspace_size(desc with m = d, 0, POETX_OP_CNP)
 */
poetx_status poetx_cnp_build(const float* q, int32_t d, int32_t b, int32_t dtype, void* g, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * poetx_cnp_build for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same result, bit for bit, with the workspace taken
 * from a fixed device array inside the library instead of a caller buffer.
 *   q, d, b, dtype, g  as for poetx_cnp_build
 *   stream   must belong to the current device
 * The array holds POETX_NOALLOC_SCRATCH_BYTES (60 MiB) on each GPU the call
 * runs on, from the first call on that GPU until the process ends; that is
 * room for poetx_workspace_size(desc with m = d, 0, POETX_OP_CNP) of any side
 * up to 40 blocks of 512 in bf16 (d <= 20480 at b = 512) or 20 in fp32.
 * Every call on one GPU uses the same array: calls that overlap in time on one
 * GPU (other streams, other threads) race and must be serialised by the caller.
 * The call allocates nothing (no hipMalloc or torch allocation).
 * Errors: POETX_E_NULL, POETX_E_SHAPE, POETX_E_DTYPE, POETX_E_WORKSPACE (the
 * side's workspace exceeds the array), POETX_E_HIP.
 */
#define POETX_NOALLOC_SCRATCH_BYTES (60u << 20)
poetx_status poetx_cnp_build_noalloc(const float* q, int32_t d, int32_t b, int32_t dtype, void* g, void* stream);

/*
 * Fold the two permutations adjacent to W0 into it (zhichai.net blog, 第二斧;
 * gist.science summary, 2. Metodologia: four permutations reduced to two):
 * Wt[i][j] = W0[perm_R[i]][perm_P[j]], and for POETX_I8 scale_t[j] = scale[perm_P[j]].
 *   W0     [m][ld_w0] of w_dtype (natural layout), ld_w0 >= n
 *   w0_scale [n] fp32 column scales (POETX_I8 only, else NULL)
 *   perm_R [m], perm_P [n] int32 device permutations of 0..m-1 / 0..n-1
 *   Wt     out, poetx_weight_bytes(desc) bytes (pre-merged layout, scales or
 *          transposed copy included)
 * Pure data movement: the result is bit-exact.
 */
poetx_status poetx_premerge(const poetx_layer_desc* desc, const void* W0, int64_t ld_w0, const float* w0_scale,
                            const int32_t* perm_R, const int32_t* perm_P, void* Wt, void* stream);

/*
 * Forward Y = X R W0 P (input-centric, wispaper.ai POET-X blog, section 1):
 *   Xt = X[:, perm_R];  A = Xt Diag(G_R);  H = A W~;  Zt = H Diag(G_P);
 *   Y[:, perm_P] = Zt.
 *   X      [T][m] act_dtype, leading dimension m
 *   perm_R [m], perm_P [n] int32 device
 *   Wt     pre-merged weight (poetx_premerge / poetx_merge_reinit layout)
 *   g_R, g_P  G buffers from poetx_cnp_build for the two sides
 *   Y      out [T][n] act_dtype, leading dimension n
 *   H_save out, poetx_saved_bytes(desc, T) bytes: the saved state (H, then Xt;
 *          Xt only for POETX_XMEM and POETX_XOUT)
 *          read by poetx_linear_bwd
 *   ws     >= poetx_workspace_size(desc, T, POETX_OP_FWD)
 * T = 0 is a valid no-op.
 */
poetx_status poetx_linear_fwd(const poetx_layer_desc* desc, int64_t T, const void* X, const int32_t* perm_R,
                              const int32_t* perm_P, const void* Wt, const void* g_R, const void* g_P, void* Y,
                              void* H_save, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of the forward above for upstream gradient dZ = dL/dY: the input
 * gradient dX and the gradients of both sides' packed parameters.  W0 is frozen
 * (POET notes, 整体框架), so no weight gradient is formed.  Block gradients are
 * dG_P = H_blk^T dZt_blk and dG_R = Xt_blk^T dA_blk summed over all T tokens in
 * a fixed order (deterministic), then taken through the CNP chain rule and
 * projected onto the packed slots: dq[p(i,j)] = dQ[i][j] - dQ[j][i].
 *   Y      the forward's output [T][n] act_dtype for the same tokens: read in
 *          the POETX_XOUT mode (H is taken back from it), not read in the
 *          others (the gathered input is in the saved state), where it may be
 *          NULL
 *   dZ     [T][n] act_dtype
 *   q_R, q_P  the packed parameters the G buffers were built from
 *   H_save the forward's saved state for the same T tokens
 *   dX     out [T][m] act_dtype
 *   dq_R, dq_P out [nb][b(b-1)/2] fp32, overwritten (dead slots of a partial block are 0)
 *   ws     >= poetx_workspace_size(desc, T, POETX_OP_BWD)
 */
poetx_status poetx_linear_bwd(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ,
                              const int32_t* perm_R, const int32_t* perm_P, const void* Wt, const void* g_R,
                              const void* g_P, const float* q_R, const float* q_P, const void* H_save, void* dX,
                              float* dq_R, float* dq_P, void* ws, size_t ws_bytes, void* stream);

/*
 * Merge-then-reinitialise (POET notes, 关键设计 3 and 训练策略): fold the current
 * factors into the weight, W' = R W P = Psi_R^T (Diag(G_R) W~ Diag(G_P)) Psi_P,
 * reset the factors to the identity (q_R = q_P = 0), draw new permutations from
 * the seeds (same generator as poetx_perm_from_seed) and store the new
 * pre-merged weight W'[perm_R'][:, perm_P'].  The products run in fp32 on MFMA.
 * bf16 storage rounds to nearest even; int8 storage is re-quantised per output
 * column: scale = max|w| / 127 (1 for an all-zero column), code =
 * clamp(round_half_even(w / scale), -127, 127), every step in fp32.
 *   Wt      in/out pre-merged weight
 *   perm_R, perm_P  in/out int32 device permutations
 *   g_R, g_P   G buffers built from the current q_R, q_P
 *   q_R, q_P   out: zeroed
 * After the call the first round_up(m*round_up(n,64)*4, 256) bytes of ws hold the
 * merged weight in fp32 before rounding, laid out [m][round_up(n, 64)] in the
 * new pre-merged order.
 *   ws      >= poetx_workspace_size(desc, 0, POETX_OP_MERGE)
 */
poetx_status poetx_merge_reinit(const poetx_layer_desc* desc, void* Wt, int32_t* perm_R, int32_t* perm_P,
                                const void* g_R, const void* g_P, float* q_R, float* q_P, uint64_t seed_R,
                                uint64_t seed_P, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------- batched CNP (one layer) -- */

/* Most sides one batched CNP call accepts. */
#define POETX_MAX_SIDES 64

/* Workspace bytes of poetx_cnp_build_batch for `count` sides of lengths d[i]
 * (host array) and block size b; 0 for invalid arguments. */
size_t poetx_cnp_batch_workspace_size(int32_t count, const int32_t* d, int32_t b, int32_t dtype);

/*
 * poetx_cnp_build for `count` sides at once (e.g. both sides of every linear of
 * a decoder layer, rebuilt after each optimiser step): the blocks of all sides
 * share each launch.  The result is bit-identical to `count` separate
 * poetx_cnp_build calls.  q, d and g are HOST arrays of length count holding
 * the per-side arguments of poetx_cnp_build (device pointers, side lengths).
 *   count  1 .. POETX_MAX_SIDES
 *   ws     >= poetx_cnp_batch_workspace_size(count, d, b, dtype)
 * Errors: POETX_E_NULL, POETX_E_SHAPE, POETX_E_DTYPE, POETX_E_WORKSPACE, POETX_E_HIP.
 */
poetx_status poetx_cnp_build_batch(int32_t count, const float* const* q, const int32_t* d, int32_t b, int32_t dtype,
                                   void* const* g, void* ws, size_t ws_bytes, void* stream);

/* Bytes of a gradient state holding `blocks` CNP blocks of size b: the summed
 * block gradients and the chain rule's intermediates.  Opaque layout. */
size_t poetx_cnp_grad_bytes(int64_t blocks, int32_t b, int32_t dtype);

/*
 * poetx_linear_bwd split in two, so that the CNP chain rule of many linears can
 * run as one batch.  This call computes dX exactly as poetx_linear_bwd does and
 * the block gradients dG_R, dG_P (same definition and summation order), which
 * it stores in the gradient state `dg` at blocks [dg_first, dg_first + nb_R +
 * nb_P) (R side first) of a state sized for dg_blocks blocks.
 *   dg        gradient state of poetx_cnp_grad_bytes(dg_blocks, b, act_dtype) bytes
 *   ws        >= poetx_workspace_size(desc, T, POETX_OP_BWD)
 * Other arguments as for poetx_linear_bwd.  Errors as for poetx_linear_bwd, and
 * POETX_E_SHAPE when the linear's blocks do not fit in [0, dg_blocks).
 */
poetx_status poetx_linear_bwd_dx(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ,
                                 const int32_t* perm_R, const int32_t* perm_P, const void* Wt, const void* g_R,
                                 const void* g_P, const float* q_R, const float* q_P, const void* H_save, void* dX,
                                 void* dg, int64_t dg_first, int64_t dg_blocks, void* ws, size_t ws_bytes,
                                 void* stream);

/* The operands of one side's block gradients (see poetx_linear_bwd): block k
 * of the side is dG_k = A[:, kb..kb+r)^T B[:, kb..kb+r) summed over the token
 * rows, kb = k b, r = min(b, d - kb).  A and B are device [rows][lda] and
 * [rows][ldb] matrices of the layer's act_dtype: for the R side the gathered
 * input Xt and dA = dZt Diag(G_P)^T W~^T, for the P side H and dZt. */
typedef struct poetx_grad_side {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  int32_t d;
} poetx_grad_side;

/*
 * poetx_linear_bwd_dx without the block gradients, so that those of many
 * linears run as one batch (poetx_block_grads_batch).  Computes dX exactly as
 * poetx_linear_bwd does and writes the operands of the two sides' block
 * gradients to sides[0] (R) and sides[1] (P) (a HOST array of 2).  They point
 * into H_save and ws and stay valid until either is written again.
 * Arguments and errors as for poetx_linear_bwd (q_R, q_P and dq are not taken).
 */
poetx_status poetx_linear_bwd_dx_sides(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ,
                                       const int32_t* perm_R, const int32_t* perm_P, const void* Wt, const void* g_R,
                                       const void* g_P, const void* H_save, void* dX, poetx_grad_side* sides,
                                       void* ws, size_t ws_bytes, void* stream);

/*
 * Group calls: the forwards, or the backwards to dX, of up to POETX_MAX_GROUP
 * linears over the same T token rows (for instance q, k and v of an attention
 * layer, or gate and up of an MLP), with the block products of all of them in
 * shared launches, and those W~ contractions of equal K that are too small to
 * fill the GPU alone in one launch where together they do (k and v of a
 * grouped-query attention layer).  Each linear's outputs are bit-identical to
 * its own poetx_linear_fwd / poetx_linear_bwd_dx_sides call (the same kernels
 * take the same operands in the same order; the launches only share
 * workgroups).  The linears must
 * share b; their inputs may be the same tensor, and every other buffer (ws,
 * H_save, outputs) must be their own.  Layers with act_dtype F32 run one call
 * per linear.
 */
#define POETX_MAX_GROUP 8

/* One linear of poetx_linear_fwd_group: the arguments of poetx_linear_fwd. */
typedef struct poetx_fwd_call {
  const poetx_layer_desc* desc;
  const void* X;
  const int32_t* perm_R;
  const int32_t* perm_P;
  const void* Wt;
  const void* g_R;
  const void* g_P;
  void* Y;
  void* H_save;
  void* ws;
  size_t ws_bytes;
} poetx_fwd_call;

/*
 * poetx_linear_fwd of calls[0 .. count) (a HOST array), T rows each.
 * Errors: POETX_E_NULL (calls, or a pointer poetx_linear_fwd requires),
 * POETX_E_SHAPE (count outside [1, POETX_MAX_GROUP], T outside [0, 2^31), b
 * not shared), and each call's errors as for poetx_linear_fwd; arguments are
 * all checked before the first launch.
 */
poetx_status poetx_linear_fwd_group(int32_t count, const poetx_fwd_call* calls, int64_t T, void* stream);

/* One linear of poetx_linear_bwd_dx_group: the arguments of
 * poetx_linear_bwd_dx_sides. */
typedef struct poetx_bwd_call {
  const poetx_layer_desc* desc;
  const void* Y;
  const void* dZ;
  const int32_t* perm_R;
  const int32_t* perm_P;
  const void* Wt;
  const void* g_R;
  const void* g_P;
  const void* H_save;
  void* dX;
  void* ws;
  size_t ws_bytes;
} poetx_bwd_call;

/*
 * poetx_linear_bwd_dx_sides of calls[0 .. count) (a HOST array), T rows each:
 * dX of every linear, and the operands of its block gradients in
 * sides[2 i] (R) and sides[2 i + 1] (P) (a HOST array of 2 count), valid
 * until that linear's H_save or ws is written again.  Calls that pass the same
 * dX (linears that read one input) receive the sum of their input gradients,
 * accumulated in fp32 in call order and rounded once to act_dtype; they must
 * share m (at most 16384) and act_dtype.  Errors as for
 * poetx_linear_fwd_group, with each call's errors as for
 * poetx_linear_bwd_dx_sides.
 */
poetx_status poetx_linear_bwd_dx_group(int32_t count, const poetx_bwd_call* calls, int64_t T, poetx_grad_side* sides,
                                       void* stream);

/* Workspace bytes of poetx_block_grads_batch (the fp32 partial sums of token
 * splits; 0 when no split is used or for invalid arguments). */
size_t poetx_block_grads_workspace_size(int32_t count, const int32_t* d, int64_t rows, int32_t b, int32_t dtype);

/*
 * The block gradients of `count` sides over the same `rows` token rows, as
 * poetx_linear_bwd defines them, into the gradient state `dg`: side i owns the
 * next ceil(d_i / b) blocks, as poetx_cnp_backward_batch then reads them.  The
 * sides share launches (up to 16 per launch), so the token range is split for
 * the whole batch: the sums are taken in a fixed order, but in other splits
 * than per-linear calls, so results match those to fp32 rounding, not bit for
 * bit.
 *   sides  HOST array of count operand descriptors (poetx_linear_bwd_dx_sides)
 *   count  1 .. POETX_MAX_SIDES;  dtype F32 or BF16 (the operands' act_dtype)
 *   dg     gradient state of at least poetx_cnp_grad_bytes(sum of blocks, b, dtype) bytes
 *   ws     >= poetx_block_grads_workspace_size(count, d, rows, b, dtype), 256-byte aligned
 * Errors: POETX_E_NULL, POETX_E_SHAPE, POETX_E_DTYPE, POETX_E_WORKSPACE, POETX_E_HIP.
 */
poetx_status poetx_block_grads_batch(int32_t count, const poetx_grad_side* sides, int64_t rows, int32_t b,
                                     int32_t dtype, void* dg, size_t dg_bytes, void* ws, size_t ws_bytes,
                                     void* stream);

/*
 * The CNP chain rule and skew projection (as in poetx_linear_bwd) for `count`
 * sides whose block gradients fill the gradient state `dg` in order: side i
 * owns the next ceil(d[i] / b) blocks.  q, d and dq are HOST arrays of length
 * count (device pointers, side lengths); dq[i] [nb_i][b(b-1)/2] fp32 is
 * overwritten, dead slots of a partial block with 0.  The result is
 * bit-identical to the chain rule inside poetx_linear_bwd.
 *   count  1 .. POETX_MAX_SIDES, with the sum of the sides' blocks equal to the
 *          state's block count
 *   dg     gradient state written by poetx_linear_bwd_dx or poetx_block_grads_batch;
 *          dg_bytes its size
 * Errors: POETX_E_NULL, POETX_E_SHAPE, POETX_E_DTYPE, POETX_E_WORKSPACE, POETX_E_HIP.
 */
poetx_status poetx_cnp_backward_batch(int32_t count, const float* const* q, const int32_t* d, int32_t b, int32_t dtype,
                                      void* dg, size_t dg_bytes, float* const* dq, void* stream);

/*
 * poetx_cnp_backward_batch reading the dense Q and S = Q^2 that the
 * poetx_cnp_build_batch call which built these sides' G left in its workspace
 * `build_ws`, instead of forming them again (one unpacking and one of the six
 * b x b products fewer).  The same sides in the same order, and build_ws not
 * written since that build; the chain rule is then taken at the q the G were
 * built from.  The result is bit-identical to poetx_cnp_backward_batch with
 * those q.
 *   build_ws  the build's workspace, build_ws_bytes >= poetx_cnp_batch_workspace_size
 * Other arguments and errors as for poetx_cnp_backward_batch.
 */
poetx_status poetx_cnp_backward_batch_reuse(int32_t count, const float* const* q, const int32_t* d, int32_t b,
                                            int32_t dtype, const void* build_ws, size_t build_ws_bytes, void* dg,
                                            size_t dg_bytes, float* const* dq, void* stream);

/* ---------------------------------- one SPO factor (c > 1, fully stochastic) -- */

/*
 * The layer calls above hold one block-stochastic factor per side.  The POET
 * notes ("Reparameterized LLM Training via Orthogonal Equivalence
 * Transformation", 关键设计 1) build R and P as products of c primitives, each
 * either block-stochastic, Psi^T Diag(G^1, ..., G^nb) Psi, or fully
 * stochastic, I + D(S) (G - I_b) D(S)^T for an ordered subset S of b of the d
 * coordinates (D(S)[S[j]][j] = 1).  The calls below apply one such factor to
 * token rows, Y = X F, and take its backward; a product of c factors is c
 * calls in order (Y = X R_1 ... R_c W0 P_1 ... P_c with the innermost R_c and
 * P_1 inside poetx_linear_fwd).
 */
typedef enum {
  POETX_SPO_BLOCK = 0, /* idx: a permutation of the d columns; ceil(d/b) blocks */
  POETX_SPO_FULL = 1   /* idx: b distinct columns in [0, d), in the order of G's rows; one block */
} poetx_spo_kind;

typedef struct {
  int32_t d;         /* columns of the activation, 1 .. 2^20 */
  int32_t b;         /* block size, 2 .. 1024; FULL: also the subset size, b <= d */
  int32_t kind;      /* poetx_spo_kind */
  int32_t act_dtype; /* POETX_F32 or POETX_BF16 (X, Y, dY, dX and G) */
} poetx_spo_desc;

/* Bytes of the state poetx_spo_fwd saves for the backward: the gathered input
 * X[:, idx], [T][round_up(d_eff, 64)] with d_eff = d (BLOCK) or b (FULL);
 * 0 for invalid arguments. */
size_t poetx_spo_saved_bytes(const poetx_spo_desc* desc, int64_t T);
/* Workspace bytes of poetx_spo_fwd (op = POETX_OP_FWD) or poetx_spo_bwd
 * (POETX_OP_BWD); 0 for invalid arguments. */
size_t poetx_spo_workspace_size(const poetx_spo_desc* desc, int64_t T, int32_t op);

/*
 * Y = X F for one factor, row form:
 *   BLOCK: Xt = X[:, idx], Y[:, idx] = Xt Diag(G)
 *   FULL:  Xt = X[:, idx], Y = X except Y[:, idx] = Xt G
 *   X, Y   [T][d] contiguous, act_dtype; Y may be X (in place)
 *   idx    device int32: [d] permutation (BLOCK) or [b] distinct columns (FULL)
 *   G      the blocks from poetx_cnp_build(q, d_eff, b, act_dtype, G, ...)
 *   saved  >= poetx_spo_saved_bytes(desc, T); keeps Xt for poetx_spo_bwd
 *   ws     >= poetx_spo_workspace_size(desc, T, POETX_OP_FWD)
 * Errors: POETX_E_NULL, POETX_E_SHAPE, POETX_E_DTYPE, POETX_E_WORKSPACE, POETX_E_HIP.
 */
poetx_status poetx_spo_fwd(const poetx_spo_desc* desc, int64_t T, const void* X, const int32_t* idx, const void* G,
                           void* Y, void* saved, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of poetx_spo_fwd: dX = dY F^T, and the packed gradient of the
 * factor's q (the block gradients Xt_k^T dY[:, idx]_k summed over all T rows,
 * then the CNP chain rule and skew projection as in poetx_linear_bwd).
 *   dY, dX  [T][d] contiguous, act_dtype; dX may be dY (in place)
 *   q       fp32 [nb_eff][b(b-1)/2], the parameters G was built from
 *   saved   the state written by the forward of the same rows
 *   dq      fp32 [nb_eff][b(b-1)/2], overwritten (dead slots of a partial block: 0)
 *   ws      >= poetx_spo_workspace_size(desc, T, POETX_OP_BWD)
 * Errors: as for poetx_spo_fwd.
 */
poetx_status poetx_spo_bwd(const poetx_spo_desc* desc, int64_t T, const void* dY, const int32_t* idx, const void* G,
                           const float* q, const void* saved, void* dX, float* dq, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Merging a chain's outer factors into the weight (POET notes, 关键设计 1 and
 * 3: merge-then-reinitialise of R = R_1 ... R_c and P = P_1 ... P_c).  After
 * poetx_merge_reinit has folded the linear's own R_c and P_1, its workspace
 * holds the merged weight in fp32, [m][round_up(n, 64)] in the new pre-merged
 * order.  Each outer factor F is folded into that matrix W:
 *   side 1 (F one of P_2 .. P_c, acting on the n output columns):  W <- W F~
 *   side 0 (F one of R_1 .. R_{c-1}, acting on the m input rows): W <- F~ W
 * with F~ = Psi F Psi^T the factor in the pre-merged order (Psi the linear's
 * permutation on that side, Psi[i][perm[i]] = 1): a factor of the same kind
 * whose index array is perm^-1 o idx.  Fold P_2, ..., P_c in that order and
 * R_{c-1}, ..., R_1 in that order; then poetx_store_weight writes the result in
 * the layer's weight format.  The products run in fp32 on MFMA with the
 * factor's G blocks (its activation dtype), the same blocks its forward uses.
 *   f      the factor (f->d = n for side 1, m for side 0)
 *   idx, G the factor's index array and G buffer (poetx_spo_fwd's arguments)
 *   perm   the linear's permutation on that side after the merge
 *   W      in/out fp32 [m][ldw], ldw >= n; columns n .. ldw - 1 may be zeroed
 *   ws     >= poetx_fold_workspace_size(desc, side, f)
 * Errors: POETX_E_NULL, POETX_E_SHAPE, POETX_E_DTYPE, POETX_E_WORKSPACE, POETX_E_HIP.
 */
size_t poetx_fold_workspace_size(const poetx_layer_desc* desc, int32_t side, const poetx_spo_desc* f);
poetx_status poetx_fold_factor(const poetx_layer_desc* desc, int32_t side, const poetx_spo_desc* f, const int32_t* idx,
                               const void* G, const int32_t* perm, float* W, int64_t ldw, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * Write an fp32 pre-merged weight W [m][ldw] into the layer's weight buffer Wt
 * (poetx_weight_bytes layout), as poetx_merge_reinit stores its result: fp32
 * copied, bf16 rounded to nearest even (and the transposed copy written), int8
 * requantised per output column (scale = max|w| / 127, 1 for an all-zero
 * column; code = clamp(round_half_even(w / scale), -127, 127), in fp32).
 *   ws  >= poetx_store_workspace_size(desc)
 * Errors: POETX_E_NULL, POETX_E_SHAPE, POETX_E_DTYPE, POETX_E_WORKSPACE, POETX_E_HIP.
 */
size_t poetx_store_workspace_size(const poetx_layer_desc* desc);
poetx_status poetx_store_weight(const poetx_layer_desc* desc, const float* W, int64_t ldw, void* Wt, void* ws,
                                size_t ws_bytes, void* stream);

/* ------------------------------------------ optimiser step on packed q -- */

/* Hyper-parameters of one Adam step with decoupled weight decay. */
typedef struct {
  float lr;           /* step size, finite and >= 0 */
  float beta1;        /* decay of the first moment, in [0, 1) */
  float beta2;        /* decay of the second moment, in [0, 1) */
  float eps;          /* added to the root of the corrected second moment, > 0 */
  float weight_decay; /* decoupled decay rate, finite (0 disables it) */
  int64_t t;          /* 1-based number of steps since the moments were zero */
} poetx_adam_params;

/*
 * One optimiser step on the packed parameters of `count` sides, in place, in
 * as few launches as the sides allow (one per 32 sides).  The optimiser keeps
 * state only for the packed half of each skew Q (zhichai.net POET-X blog,
 * 第四斧 item 1); the pages do not name it, and the update is Adam (Kingma &
 * Ba 2015) with decoupled weight decay (Loshchilov & Hutter 2019).  For every
 * slot, in fp32, with g = dq[i][slot]:
 *     m1 = beta1 m1 + (1 - beta1) g
 *     m2 = beta2 m2 + (1 - beta2) g^2
 *     q  = q - lr ( (m1 / (1 - beta1^t)) / (sqrt(m2 / (1 - beta2^t)) + eps) + weight_decay q )
 * The bias corrections are formed in double on the host and rounded to fp32.
 * Slots with g = 0 and zero moments change only by the decay term, so the
 * dead slots of a partial block (dq = 0 there) stay 0 when q starts 0 there.
 *   len          HOST array [count]: slots of side i (0 skips the side); for a
 *                side of length d and block size b, ceil(d/b) * b(b-1)/2
 *   q, m1, m2    HOST arrays [count] of device pointers to fp32 [len[i]],
 *                read and overwritten (m1, m2: first and second moments)
 *   dq           HOST array [count] of device pointers to fp32 [len[i]], read
 *                only (e.g. written by poetx_linear_bwd)
 * The four arrays of one side, and the arrays of different sides, must not
 * overlap.  No workspace; 16-byte aligned pointers take the vector path.
 *   count  1 .. POETX_MAX_SIDES; len[i] in [0, 2^36]
 * Errors: POETX_E_NULL, POETX_E_SHAPE (count, len or a hyper-parameter out of
 * range), POETX_E_HIP.
 */
poetx_status poetx_adam_step_batch(int32_t count, const int64_t* len, float* const* q, const float* const* dq,
                                   float* const* m1, float* const* m2, const poetx_adam_params* hp, void* stream);

/* ----------------------------------- weight-centric baseline (comparison) -- */

/*
 * The same layer computed in the order original POET uses, for comparison with
 * the input-centric calls above (zhichai.net POET-X blog, 第一斧; wispaper.ai
 * POET-X blog, "The 'Weight-Centric' Wall"): the factors are applied to the
 * weight first, M = Diag(G_R) W~ Diag(G_P) (so that R W0 P = Psi_R^T M Psi_P),
 * and each direction is then one dense contraction with M.  The backward forms
 * the full weight gradient dM = Xt^T dZt and takes the block gradients from it:
 * dG_R = diagonal blocks of dM (W~ Diag(G_P))^T, dG_P = diagonal blocks of
 * (Diag(G_R) W~)^T dM.  The results are the same function and gradients as
 * poetx_linear_fwd / poetx_linear_bwd (up to rounding: M, the weight-side
 * products and dM are stored in act_dtype).
 * Supported layers: (act, weight) = (F32, F32) or (BF16, BF16); others get
 * POETX_E_UNSUPPORTED.
 */

/* Bytes of the state poetx_wc_fwd leaves for poetx_wc_bwd of the same T rows:
 * M and U = Diag(G_R) W~ as [m][round_up(n, 64)], (W~ Diag(G_P))^T as
 * [n][round_up(m, 64)], and Xt = X[:, perm_R] as [T][round_up(m, 64)], each at
 * a 256-byte boundary, in act_dtype; 0 for invalid arguments. */
size_t poetx_wc_state_bytes(const poetx_layer_desc* desc, int64_t T);

/* Workspace bytes of poetx_wc_fwd (op = POETX_OP_FWD) or poetx_wc_bwd
 * (POETX_OP_BWD); 0 for invalid arguments. */
size_t poetx_wc_workspace_size(const poetx_layer_desc* desc, int64_t T, int32_t op);

/*
 * Weight-centric forward: build M (three block products over the weight and
 * their transposes), then Y[:, perm_P] = X[:, perm_R] M.
 *   X, perm_R, perm_P, Wt, g_R, g_P, Y  as for poetx_linear_fwd
 *   state  out, poetx_wc_state_bytes(desc, T) bytes, 256-byte aligned
 *   ws     >= poetx_wc_workspace_size(desc, T, POETX_OP_FWD)
 * T = 0 builds M only.
 * Errors: POETX_E_NULL, POETX_E_SHAPE, POETX_E_DTYPE, POETX_E_UNSUPPORTED,
 * POETX_E_WORKSPACE, POETX_E_HIP.
 */
poetx_status poetx_wc_fwd(const poetx_layer_desc* desc, int64_t T, const void* X, const int32_t* perm_R,
                          const int32_t* perm_P, const void* Wt, const void* g_R, const void* g_P, void* Y, void* state,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Weight-centric backward for upstream gradient dZ: dX = dZ[:, perm_P] M^T
 * scattered by perm_R, and dq_R, dq_P through the weight gradient dM (see
 * above), the CNP chain rule and the skew projection, as in poetx_linear_bwd.
 *   dZ [T][n], dX out [T][m], q_R, q_P, dq_R, dq_P  as for poetx_linear_bwd
 *   state  written by poetx_wc_fwd for the same T rows
 *   ws     >= poetx_wc_workspace_size(desc, T, POETX_OP_BWD)
 * Errors: as for poetx_wc_fwd.
 */
poetx_status poetx_wc_bwd(const poetx_layer_desc* desc, int64_t T, const void* dZ, const int32_t* perm_R,
                          const int32_t* perm_P, const void* g_R, const void* g_P, const float* q_R, const float* q_P,
                          const void* state, void* dX, float* dq_R, float* dq_P, void* ws, size_t ws_bytes,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* POETX_H */
