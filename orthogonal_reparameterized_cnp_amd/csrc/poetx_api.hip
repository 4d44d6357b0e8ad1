// C ABI of libpoetx: argument validation, workspace planning and the order of
// kernel launches for each call.  All arithmetic happens in the kernels of
// poetx_kernels.hip.
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/poetx.h"
#include "poetx_internal.h"

using namespace pxk;

namespace {

thread_local std::string g_err;

// ---------------------------------------------------------------------------
// measurement timer: hipEvents around the launches of one kernel class
// ---------------------------------------------------------------------------
struct TimerRec {
  hipEvent_t a, b;
  double flops, bytes;
};
struct Timer {
  std::mutex mu;
  int cls = 0;
  std::vector<TimerRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Timer& timer() {
  static Timer t;
  return t;
}

struct Timed {
  bool on = false;
  hipStream_t s;
  TimerRec rec{};
  Timed(int cls, hipStream_t s_, double flops, double bytes) : s(s_) {
    Timer& t = timer();
    std::lock_guard<std::mutex> g(t.mu);
    if (t.cls == 0 || t.cls != cls) return;
    rec.a = t.get();
    rec.b = t.get();
    if (!rec.a || !rec.b) return;
    rec.flops = flops;
    rec.bytes = bytes;
    on = hipEventRecord(rec.a, s) == hipSuccess;
  }
  ~Timed() {
    if (!on) return;
    Timer& t = timer();
    std::lock_guard<std::mutex> g(t.mu);
    if (hipEventRecord(rec.b, s) == hipSuccess) t.recs.push_back(rec);
  }
};

poetx_status fail(poetx_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

#define PX_TIMED(cls, flops, bytes, expr)       \
  do {                                          \
    Timed t_((cls), s, (double)(flops), (double)(bytes)); \
    PX_HIP(expr);                               \
  } while (0)

#define PX_HIP(expr)                                                                         \
  do {                                                                                       \
    hipError_t e_ = (expr);                                                                  \
    if (e_ != hipSuccess) return fail(POETX_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxT = (int64_t(1) << 31) - 1;

poetx_status check_desc(const poetx_layer_desc* d) {
  if (!d) return fail(POETX_E_NULL, "desc is NULL");
  if (d->m < 1 || d->n < 1 || d->m > kMaxDim || d->n > kMaxDim)
    return fail(POETX_E_SHAPE, "m and n must be in [1, 2^20]");
  if (d->b < 2 || d->b > 1024) return fail(POETX_E_SHAPE, "b must be in [2, 1024]");
  if (nblocks(d->m, d->b) > 65535 || nblocks(d->n, d->b) > 65535)
    return fail(POETX_E_SHAPE, "at most 65535 blocks per side");
  if (d->mode != POETX_XFAST && d->mode != POETX_XMEM && d->mode != POETX_XOUT)
    return fail(POETX_E_SHAPE, "mode must be XFAST, XMEM or XOUT");
  const bool ok = (d->act_dtype == POETX_F32 && d->w_dtype == POETX_F32) ||
                  (d->act_dtype == POETX_BF16 && (d->w_dtype == POETX_BF16 || d->w_dtype == POETX_I8));
  if (!ok) return fail(POETX_E_DTYPE, "supported (act, weight) dtypes: (F32, F32), (BF16, BF16), (BF16, I8)");
  return POETX_OK;
}

// Bump allocator over the caller's workspace (256-byte aligned regions).
struct Plan {
  size_t off = 0;
  char* base = nullptr;
  template <typename T> T* take(size_t bytes) {
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += (size_t)round_up((int64_t)bytes, 256);
    return p;
  }
};

size_t g_slice(int d, int b, int dt) { return (size_t)nblocks(d, b) * b * b * dt_size(dt); }

// sum over a side's blocks of r^2 and r^3 (algorithmic flop counts)
double sum_r2(int d, int b) {
  const double r = d - (double)(nblocks(d, b) - 1) * b;
  return (nblocks(d, b) - 1) * (double)b * b + r * r;
}
double sum_r3(int d, int b) {
  const double r = d - (double)(nblocks(d, b) - 1) * b;
  return (nblocks(d, b) - 1) * (double)b * b * b + r * r * r;
}

size_t weight_scale_offset(const poetx_layer_desc* d) {
  return (size_t)round_up((int64_t)d->m * lead(d->n) * (int64_t)dt_size(d->w_dtype), 256);
}

// bf16 weights also keep W~^T [n][lead(m)] at the same offset (they have no
// scales): the forward reads it as a K-contiguous operand
bool has_weight_t(const poetx_layer_desc* d) { return d->w_dtype == POETX_BF16; }
size_t weight_t_offset(const poetx_layer_desc* d) { return weight_scale_offset(d); }

// The forward's saved state: H [T][lead(n)], then (256-byte aligned) the
// gathered input Xt [T][lead(m)], both in act_dtype; Xt alone for Xmem and Xout.
bool saves_h(const poetx_layer_desc* d) { return d->mode == POETX_XFAST; }
size_t saved_xt_offset(const poetx_layer_desc* d, int64_t T) {
  if (!saves_h(d)) return 0;
  return (size_t)round_up(T * lead(d->n) * (int64_t)dt_size(d->act_dtype), 256);
}

struct FwdWs {
  void *A, *Zt, *H;  // H: Xmem and Xout (Xfast writes it to the saved state)
};
template <class P> FwdWs plan_fwd(P& p, const poetx_layer_desc* d, int64_t T) {
  const size_t es = dt_size(d->act_dtype);
  FwdWs w;
  w.A = p.template take<char>(T * lead(d->m) * es);
  w.Zt = p.template take<char>(T * lead(d->n) * es);
  w.H = saves_h(d) ? nullptr : p.template take<char>(T * lead(d->n) * es);
  return w;
}

struct BwdWs {
  void *dZt, *dH, *dA, *dXt, *cnp;
  void* Hr;  // Xout: H taken back from the output
  float* part;
};
template <class P> BwdWs plan_bwd(P& p, const poetx_layer_desc* d, int64_t T) {
  const size_t es = dt_size(d->act_dtype);
  BwdWs w;
  w.dZt = p.template take<char>(T * lead(d->n) * es);
  w.dH = p.template take<char>(T * lead(d->n) * es);
  w.dA = p.template take<char>(T * lead(d->m) * es);
  w.dXt = p.template take<char>(T * lead(d->m) * es);
  w.cnp = p.template take<char>(cnp_grad_bytes(d->act_dtype, (int64_t)nblocks(d->m, d->b) + nblocks(d->n, d->b), d->b));
  w.part = p.template take<float>(
      block_grads_part_bytes(d->act_dtype, (int)T, nblocks(d->m, d->b) + nblocks(d->n, d->b), d->b));
  w.Hr = d->mode == POETX_XOUT ? p.template take<char>(T * lead(d->n) * es) : nullptr;
  return w;
}

struct MergeWs {
  float *Mq, *M;
  int32_t *newR, *newP, *invR, *invP, *rhoR, *rhoP, *fy;
  uint32_t* amax;
};
template <class P> MergeWs plan_merge(P& p, const poetx_layer_desc* d) {
  const size_t mat = (size_t)d->m * lead(d->n) * 4;
  MergeWs w;
  w.Mq = p.template take<float>(mat);  // first M1 (left product), finally the re-permuted fp32 weight
  w.M = p.template take<float>(mat);
  w.newR = p.template take<int32_t>((size_t)d->m * 4);
  w.newP = p.template take<int32_t>((size_t)d->n * 4);
  w.invR = p.template take<int32_t>((size_t)d->m * 4);
  w.invP = p.template take<int32_t>((size_t)d->n * 4);
  w.rhoR = p.template take<int32_t>((size_t)d->m * 4);
  w.rhoP = p.template take<int32_t>((size_t)d->n * 4);
  w.fy = p.template take<int32_t>((size_t)std::max(d->m, d->n) * 4);
  w.amax = p.template take<uint32_t>((size_t)d->n * 4);
  return w;
}

poetx_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return POETX_OK;
  if (!ws) return fail(POETX_E_NULL, "ws is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(POETX_E_WORKSPACE, "ws must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(POETX_E_WORKSPACE, "ws too small: need " + std::to_string(need) + " bytes, got " + std::to_string(ws_bytes));
  return POETX_OK;
}

constexpr int64_t kMaxBlocks = 65535;  // CNP blocks per launch (one grid dimension)
static_assert(POETX_MAX_SIDES == kMaxSides, "side table size");

// count sides of lengths d[i] with block size b: validity and total block count
poetx_status check_sides(int32_t count, const int32_t* d, int32_t b, int32_t dtype, int64_t* blocks) {
  if (count < 1 || count > POETX_MAX_SIDES) return fail(POETX_E_SHAPE, "count must be in [1, POETX_MAX_SIDES]");
  if (!d) return fail(POETX_E_NULL, "d is NULL");
  if (b < 2 || b > 1024) return fail(POETX_E_SHAPE, "b must be in [2, 1024]");
  if (dtype != POETX_F32 && dtype != POETX_BF16) return fail(POETX_E_DTYPE, "dtype must be F32 or BF16");
  int64_t nb = 0;
  for (int i = 0; i < count; ++i) {
    if (d[i] < 1 || d[i] > kMaxDim) return fail(POETX_E_SHAPE, "d[i] must be in [1, 2^20]");
    nb += nblocks(d[i], b);
  }
  if (nb > kMaxBlocks) return fail(POETX_E_SHAPE, "more than 65535 blocks in one batch");
  *blocks = nb;
  return POETX_OK;
}

}  // namespace

extern "C" {

const char* poetx_version(void) { return "libpoetx 0.1 (gfx950)"; }

const char* poetx_last_error(void) { return g_err.c_str(); }

int64_t poetx_packed_len(int32_t b) { return b < 2 ? 0 : packed_len(b); }

size_t poetx_g_bytes(int32_t d, int32_t b, int32_t dtype) {
  if (d < 1 || b < 2 || (dtype != POETX_F32 && dtype != POETX_BF16)) return 0;
  return 2 * g_slice(d, b, dtype);
}

size_t poetx_weight_bytes(const poetx_layer_desc* desc) {
  if (check_desc(desc) != POETX_OK) return 0;
  size_t bytes = weight_scale_offset(desc);
  if (desc->w_dtype == POETX_I8) bytes += (size_t)lead(desc->n) * 4;
  if (has_weight_t(desc)) bytes += (size_t)desc->n * lead(desc->m) * dt_size(desc->w_dtype);
  return bytes;
}

size_t poetx_saved_bytes(const poetx_layer_desc* desc, int64_t T) {
  if (check_desc(desc) != POETX_OK || T < 0) return 0;
  return saved_xt_offset(desc, T) + (size_t)T * lead(desc->m) * dt_size(desc->act_dtype);
}

size_t poetx_workspace_size(const poetx_layer_desc* desc, int64_t T, int32_t op) {
  if (!desc || T < 0 || T > kMaxT) return 0;
  if (op == POETX_OP_CNP) {
    if (desc->m < 1 || desc->b < 2 || (desc->act_dtype != POETX_F32 && desc->act_dtype != POETX_BF16)) return 0;
    return cnp_build_ws_bytes(desc->act_dtype, nblocks(desc->m, desc->b), desc->b);
  }
  if (check_desc(desc) != POETX_OK) return 0;
  Plan p;
  if (op == POETX_OP_FWD) plan_fwd(p, desc, T);
  else if (op == POETX_OP_BWD) plan_bwd(p, desc, T);
  else if (op == POETX_OP_MERGE) plan_merge(p, desc);
  else return 0;
  return p.off;
}

poetx_status poetx_perm_from_seed(uint64_t seed, int32_t d, int32_t* out) {
  if (!out) return fail(POETX_E_NULL, "host_out is NULL");
  if (d < 1) return fail(POETX_E_SHAPE, "d must be >= 1");
  for (int32_t i = 0; i < d; ++i) out[i] = i;
  uint64_t state = seed;
  for (int32_t i = d - 1; i >= 1; --i) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    const int32_t j = (int32_t)(((unsigned __int128)z * (uint64_t)(i + 1)) >> 64);
    const int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
  return POETX_OK;
}

poetx_status poetx_timer_enable(int32_t kernel_class) {
  if (kernel_class < POETX_KC_NONE || kernel_class > POETX_KC_OPTIM) return fail(POETX_E_SHAPE, "unknown kernel class");
  Timer& t = timer();
  std::lock_guard<std::mutex> g(t.mu);
  t.cls = kernel_class;
  return POETX_OK;
}

poetx_status poetx_timer_read(int64_t* launches, double* total_ms, double* flops, double* bytes) {
  if (!launches || !total_ms || !flops || !bytes) return fail(POETX_E_NULL, "output pointers must be non-NULL");
  Timer& t = timer();
  std::lock_guard<std::mutex> g(t.mu);
  double ms = 0, fl = 0, by = 0;
  poetx_status st = POETX_OK;
  for (const TimerRec& r : t.recs) {
    float e = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&e, r.a, r.b) != hipSuccess)
      st = fail(POETX_E_HIP, "event timing failed");
    ms += e;
    fl += r.flops;
    by += r.bytes;
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  *launches = (int64_t)t.recs.size();
  *total_ms = ms;
  *flops = fl;
  *bytes = by;
  t.recs.clear();
  return st;
}

poetx_status poetx_cnp_build(const float* q, int32_t d, int32_t b, int32_t dtype, void* g, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!q || !g) return fail(POETX_E_NULL, "q and g must be non-NULL");
  return poetx_cnp_build_batch(1, &q, &d, b, dtype, &g, ws, ws_bytes, stream);
}

size_t poetx_cnp_batch_workspace_size(int32_t count, const int32_t* d, int32_t b, int32_t dtype) {
  int64_t blocks = 0;
  if (check_sides(count, d, b, dtype, &blocks) != POETX_OK) return 0;
  return cnp_build_ws_bytes(dtype, blocks, b);
}

poetx_status poetx_cnp_build_batch(int32_t count, const float* const* q, const int32_t* d, int32_t b, int32_t dtype,
                                   void* const* g, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !g) return fail(POETX_E_NULL, "q and g must be non-NULL");
  int64_t blocks = 0;
  poetx_status st = check_sides(count, d, b, dtype, &blocks);
  if (st != POETX_OK) return st;
  double flops = 0, bytes = 0;
  for (int i = 0; i < count; ++i) {
    if (!q[i] || !g[i]) return fail(POETX_E_NULL, "q[i] and g[i] must be non-NULL");
    flops += 4 * sum_r3(d[i], b);
    bytes += 2.0 * g_slice(d[i], b, dtype) + 2.0 * nblocks(d[i], b) * b * b * 4;
  }
  st = check_ws(ws, ws_bytes, cnp_build_ws_bytes(dtype, blocks, b));
  if (st != POETX_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PX_TIMED(POETX_KC_CNP, flops, bytes, cnp_build_batch(dtype, count, q, d, b, g, ws, s));
  return POETX_OK;
}

size_t poetx_cnp_grad_bytes(int64_t blocks, int32_t b, int32_t dtype) {
  if (blocks < 1 || blocks > kMaxBlocks || b < 2 || b > 1024 || (dtype != POETX_F32 && dtype != POETX_BF16)) return 0;
  return cnp_grad_bytes(dtype, blocks, b);
}

poetx_status poetx_premerge(const poetx_layer_desc* desc, const void* W0, int64_t ld_w0, const float* w0_scale,
                            const int32_t* perm_R, const int32_t* perm_P, void* Wt, void* stream) {
  poetx_status st = check_desc(desc);
  if (st != POETX_OK) return st;
  if (!W0 || !perm_R || !perm_P || !Wt) return fail(POETX_E_NULL, "W0, perm_R, perm_P and Wt must be non-NULL");
  if (desc->w_dtype == POETX_I8 && !w0_scale) return fail(POETX_E_NULL, "w0_scale is required for I8 weights");
  if (ld_w0 < desc->n) return fail(POETX_E_SHAPE, "ld_w0 < n");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int m = desc->m, n = desc->n;
  PX_HIP(permute(desc->w_dtype, W0, ld_w0, perm_R, perm_P, Wt, lead(n), m, n, n, s));
  if (has_weight_t(desc))
    PX_HIP(transpose(desc->w_dtype, Wt, lead(n), m, n, reinterpret_cast<char*>(Wt) + weight_t_offset(desc), lead(m), s));
  if (desc->w_dtype == POETX_I8) {
    float* scale_t = reinterpret_cast<float*>(reinterpret_cast<char*>(Wt) + weight_scale_offset(desc));
    PX_HIP(permute(F32, w0_scale, 0, nullptr, perm_P, scale_t, 0, 1, n, n, s));
  }
  return POETX_OK;
}

}  // extern "C"

namespace {

// H = (Xt Diag(G_R)) W~ with A as the intermediate: the forward's first block
// product and its W~ contraction, also used by the Xmem backward to recompute
// H (same kernels on the same inputs, so the same bits).
poetx_status xt_to_h(const poetx_layer_desc* desc, int64_t T, const void* Xt, const void* Wt, const void* g_R, void* A,
                     void* H, hipStream_t s) {
  const int m = desc->m, n = desc->n, b = desc->b, at = desc->act_dtype, wt = desc->w_dtype;
  const int rows = (int)T;
  const int64_t ldm = lead(m), ldn = lead(n);
  const char* gR1 = reinterpret_cast<const char*>(g_R) + g_slice(m, b, at);  // Delta_R^T
  const float* scale_t =
      wt == POETX_I8 ? reinterpret_cast<const float*>(reinterpret_cast<const char*>(Wt) + weight_scale_offset(desc))
                     : nullptr;
  const double es = (double)dt_size(at), wes = (double)dt_size(wt);
  // A = Xt Diag(G_R)
  PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(m, b), 2.0 * rows * m * es + g_slice(m, b, at),
           apply(at, at, Xt, ldm, rows, m, b, at, gR1, nullptr, at, A, ldm, s));
  // H = A W~ (int8: codes times the column scale); bf16 weights are read from the W~^T copy
  if (has_weight_t(desc)) {
    const void* Wtt = reinterpret_cast<const char*>(Wt) + weight_t_offset(desc);
    PX_TIMED(POETX_KC_GEMM, 2.0 * rows * m * n, es * rows * m + wes * m * n + es * rows * n,
             gemm(at, at, A, ldm, wt, Wtt, ldm, false, rows, n, m, nullptr, at, H, ldn, s));
  } else {
    PX_TIMED(POETX_KC_GEMM, 2.0 * rows * m * n, es * rows * m + wes * m * n + es * rows * n,
             gemm(at, at, A, ldm, wt, Wt, lead(n), true, rows, n, m, scale_t, at, H, ldn, s));
  }
  return POETX_OK;
}

}  // namespace

extern "C" {

poetx_status poetx_linear_fwd(const poetx_layer_desc* desc, int64_t T, const void* X, const int32_t* perm_R,
                              const int32_t* perm_P, const void* Wt, const void* g_R, const void* g_P, void* Y,
                              void* H_save, void* ws, size_t ws_bytes, void* stream) {
  poetx_status st = check_desc(desc);
  if (st != POETX_OK) return st;
  if (T < 0 || T > kMaxT) return fail(POETX_E_SHAPE, "T must be in [0, 2^31)");
  if (T == 0) return POETX_OK;
  if (!X || !perm_R || !perm_P || !Wt || !g_R || !g_P || !Y || !H_save)
    return fail(POETX_E_NULL, "a required pointer is NULL");
  Plan p;
  plan_fwd(p, desc, T);
  st = check_ws(ws, ws_bytes, p.off);
  if (st != POETX_OK) return st;
  Plan q;
  q.base = reinterpret_cast<char*>(ws);
  const FwdWs w = plan_fwd(q, desc, T);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int m = desc->m, n = desc->n, b = desc->b, at = desc->act_dtype;
  const int rows = (int)T;
  const int64_t ldm = lead(m), ldn = lead(n);
  const char* gP1 = reinterpret_cast<const char*>(g_P) + g_slice(n, b, at);  // Delta_P^T
  const double es = (double)dt_size(at);
  // Xt = X[:, perm_R], kept in the saved state for the backward
  void* Xt = reinterpret_cast<char*>(H_save) + saved_xt_offset(desc, T);
  PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * m * es, permute(at, X, m, nullptr, perm_R, Xt, ldm, rows, m, m, s));
  // A = Xt Diag(G_R), H = A W~: H saved (Xfast) or kept in the workspace (Xmem)
  void* H = saves_h(desc) ? H_save : w.H;
  st = xt_to_h(desc, T, Xt, Wt, g_R, w.A, H, s);
  if (st != POETX_OK) return st;
  // Zt = H Diag(G_P)
  PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(n, b), 2.0 * rows * n * es + g_slice(n, b, at),
           apply(at, at, H, ldn, rows, n, b, at, gP1, nullptr, at, w.Zt, ldn, s));
  // Y[:, perm_P] = Zt
  PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * n * es, scatter(at, w.Zt, ldn, perm_P, Y, n, rows, n, s));
  return POETX_OK;
}

}  // extern "C"

namespace {

// dX and the block gradients of both sides into blocks [first, first + nb_R + nb_P)
// of the gradient state dg (total blocks); shared by both backward entry points.
poetx_status bwd_dx_core(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ,
                         const int32_t* perm_R, const int32_t* perm_P, const void* Wt, const void* g_R,
                         const void* g_P, const float* q_R, const float* q_P, const void* H_save, void* dX, void* dg,
                         int64_t first, int64_t total, const BwdWs& w, hipStream_t s) {
  const int m = desc->m, n = desc->n, b = desc->b, at = desc->act_dtype, wt = desc->w_dtype;
  const int rows = (int)T;
  const int64_t ldm = lead(m), ldn = lead(n);
  const float* scale_t =
      wt == POETX_I8 ? reinterpret_cast<const float*>(reinterpret_cast<const char*>(Wt) + weight_scale_offset(desc))
                     : nullptr;
  const double es = (double)dt_size(at), wes = (double)dt_size(wt);
  // dZt = dZ[:, perm_P]
  PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * n * es, permute(at, dZ, n, nullptr, perm_P, w.dZt, ldn, rows, n, n, s));
  // dH = dZt Diag(G_P)^T (int8: times the column scale, ready for the code contraction)
  PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(n, b), 2.0 * rows * n * es + g_slice(n, b, at),
           apply(at, at, w.dZt, ldn, rows, n, b, at, g_P, scale_t, at, w.dH, ldn, s));
  // dA = dH W~^T
  PX_TIMED(POETX_KC_GEMM, 2.0 * rows * m * n, es * rows * n + wes * m * n + es * rows * m,
           gemm(at, at, w.dH, ldn, wt, Wt, lead(n), false, rows, m, n, nullptr, at, w.dA, ldm, s));
  // block gradients of both sides over all tokens: dG_R = Xt^T dA, dG_P = H^T dZt, with Xt and H
  // from the forward's saved state.  Xmem recomputes H from Xt, into the buffers that dH (consumed
  // by the contraction above) and dXt (written below) occupy.  Xout takes H back from the output:
  // Zt = Y[:, perm_P] into dH's buffer, then H = Zt Diag(G_P)^T.
  const void* Xt = reinterpret_cast<const char*>(H_save) + saved_xt_offset(desc, T);
  const void* H = H_save;
  if (desc->mode == POETX_XMEM) {
    const poetx_status st = xt_to_h(desc, T, Xt, Wt, g_R, w.dXt, w.dH, s);
    if (st != POETX_OK) return st;
    H = w.dH;
  } else if (desc->mode == POETX_XOUT) {
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * n * es, permute(at, Y, n, nullptr, perm_P, w.dH, ldn, rows, n, n, s));
    PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(n, b), 2.0 * rows * n * es + g_slice(n, b, at),
             apply(at, at, w.dH, ldn, rows, n, b, at, g_P, nullptr, at, w.Hr, ldn, s));
    H = w.Hr;
  }
  const CnpSide sides[2] = {{q_R, m, Xt, ldm, w.dA, ldm}, {q_P, n, H, ldn, w.dZt, ldn}};
  PX_TIMED(POETX_KC_DGRAD, 2.0 * rows * (sum_r2(m, b) + sum_r2(n, b)),
           2.0 * rows * (m + n) * es + (4 + 2 * es) * (sum_r2(m, b) + sum_r2(n, b)),
           block_grads(at, sides, rows, b, dg, first, total, w.part, s));
  // dXt = dA Diag(G_R)^T;  dX[:, perm_R] = dXt
  PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(m, b), 2.0 * rows * m * es + g_slice(m, b, at),
           apply(at, at, w.dA, ldm, rows, m, b, at, g_R, nullptr, at, w.dXt, ldm, s));
  if (rows > 0)
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * m * es, scatter(at, w.dXt, ldm, perm_R, dX, m, rows, m, s));
  return POETX_OK;
}

poetx_status check_bwd(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ, const int32_t* perm_R,
                       const int32_t* perm_P, const void* Wt, const void* g_R, const void* g_P, const float* q_R,
                       const float* q_P, const void* H_save, void* dX, void* ws, size_t ws_bytes) {
  poetx_status st = check_desc(desc);
  if (st != POETX_OK) return st;
  if (T < 0 || T > kMaxT) return fail(POETX_E_SHAPE, "T must be in [0, 2^31)");
  if (!perm_R || !perm_P || !Wt || !g_R || !g_P || !q_R || !q_P) return fail(POETX_E_NULL, "a required pointer is NULL");
  if (T > 0 && (!dZ || !H_save || !dX)) return fail(POETX_E_NULL, "a required pointer is NULL");
  if (T > 0 && desc->mode == POETX_XOUT && !Y) return fail(POETX_E_NULL, "Y is NULL (POETX_XOUT reads it)");
  Plan p;
  plan_bwd(p, desc, T);
  return check_ws(ws, ws_bytes, p.off);
}

}  // namespace

extern "C" {

poetx_status poetx_linear_bwd(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ,
                              const int32_t* perm_R, const int32_t* perm_P, const void* Wt, const void* g_R,
                              const void* g_P, const float* q_R, const float* q_P, const void* H_save, void* dX,
                              float* dq_R, float* dq_P, void* ws, size_t ws_bytes, void* stream) {
  poetx_status st = check_bwd(desc, T, Y, dZ, perm_R, perm_P, Wt, g_R, g_P, q_R, q_P, H_save, dX, ws, ws_bytes);
  if (st != POETX_OK) return st;
  if (!dq_R || !dq_P) return fail(POETX_E_NULL, "a required pointer is NULL");
  Plan pq;
  pq.base = reinterpret_cast<char*>(ws);
  const BwdWs w = plan_bwd(pq, desc, T);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int m = desc->m, n = desc->n, b = desc->b, at = desc->act_dtype;
  const int64_t blocks = (int64_t)nblocks(m, b) + nblocks(n, b);
  st = bwd_dx_core(desc, T, Y, dZ, perm_R, perm_P, Wt, g_R, g_P, q_R, q_P, H_save, dX, w.cnp, 0, blocks, w, s);
  if (st != POETX_OK) return st;
  // CNP chain rule and skew projection of both sides
  const float* qs[2] = {q_R, q_P};
  const int ds[2] = {m, n};
  float* dqs[2] = {dq_R, dq_P};
  PX_TIMED(POETX_KC_CNP, 12 * (sum_r3(m, b) + sum_r3(n, b)), cnp_grad_bytes(at, blocks, b),
           cnp_chain_batch(at, 2, qs, ds, b, w.cnp, dqs, s));
  return POETX_OK;
}

poetx_status poetx_linear_bwd_dx(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ,
                                 const int32_t* perm_R, const int32_t* perm_P, const void* Wt, const void* g_R,
                                 const void* g_P, const float* q_R, const float* q_P, const void* H_save, void* dX,
                                 void* dg, int64_t dg_first, int64_t dg_blocks, void* ws, size_t ws_bytes,
                                 void* stream) {
  poetx_status st = check_bwd(desc, T, Y, dZ, perm_R, perm_P, Wt, g_R, g_P, q_R, q_P, H_save, dX, ws, ws_bytes);
  if (st != POETX_OK) return st;
  if (!dg) return fail(POETX_E_NULL, "dg is NULL");
  if (reinterpret_cast<uintptr_t>(dg) % 256) return fail(POETX_E_WORKSPACE, "dg must be 256-byte aligned");
  const int64_t blocks = (int64_t)nblocks(desc->m, desc->b) + nblocks(desc->n, desc->b);
  if (dg_blocks < 1 || dg_blocks > kMaxBlocks || dg_first < 0 || dg_first + blocks > dg_blocks)
    return fail(POETX_E_SHAPE, "the linear's blocks must fit in [0, dg_blocks) of the gradient state");
  Plan pq;
  pq.base = reinterpret_cast<char*>(ws);
  const BwdWs w = plan_bwd(pq, desc, T);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return bwd_dx_core(desc, T, Y, dZ, perm_R, perm_P, Wt, g_R, g_P, q_R, q_P, H_save, dX, dg, dg_first, dg_blocks, w, s);
}

poetx_status poetx_cnp_backward_batch(int32_t count, const float* const* q, const int32_t* d, int32_t b, int32_t dtype,
                                      void* dg, size_t dg_bytes, float* const* dq, void* stream) {
  if (!q || !dq || !dg) return fail(POETX_E_NULL, "q, dq and dg must be non-NULL");
  int64_t blocks = 0;
  poetx_status st = check_sides(count, d, b, dtype, &blocks);
  if (st != POETX_OK) return st;
  double flops = 0;
  for (int i = 0; i < count; ++i) {
    if (!q[i] || !dq[i]) return fail(POETX_E_NULL, "q[i] and dq[i] must be non-NULL");
    flops += 12 * sum_r3(d[i], b);
  }
  if (dg_bytes < cnp_grad_bytes(dtype, blocks, b))
    return fail(POETX_E_WORKSPACE, "dg smaller than poetx_cnp_grad_bytes of the sides' block count");
  if (reinterpret_cast<uintptr_t>(dg) % 256) return fail(POETX_E_WORKSPACE, "dg must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PX_TIMED(POETX_KC_CNP, flops, cnp_grad_bytes(dtype, blocks, b), cnp_chain_batch(dtype, count, q, d, b, dg, dq, s));
  return POETX_OK;
}

poetx_status poetx_merge_reinit(const poetx_layer_desc* desc, void* Wt, int32_t* perm_R, int32_t* perm_P,
                                const void* g_R, const void* g_P, float* q_R, float* q_P, uint64_t seed_R,
                                uint64_t seed_P, void* ws, size_t ws_bytes, void* stream) {
  poetx_status st = check_desc(desc);
  if (st != POETX_OK) return st;
  if (!Wt || !perm_R || !perm_P || !g_R || !g_P || !q_R || !q_P) return fail(POETX_E_NULL, "a required pointer is NULL");
  Plan p;
  plan_merge(p, desc);
  st = check_ws(ws, ws_bytes, p.off);
  if (st != POETX_OK) return st;
  Plan pq;
  pq.base = reinterpret_cast<char*>(ws);
  const MergeWs w = plan_merge(pq, desc);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int m = desc->m, n = desc->n, b = desc->b, at = desc->act_dtype, wt = desc->w_dtype;
  const int64_t ldw = lead(n);
  float* scale_t =
      wt == POETX_I8 ? reinterpret_cast<float*>(reinterpret_cast<char*>(Wt) + weight_scale_offset(desc)) : nullptr;
  const char* gP1 = reinterpret_cast<const char*>(g_P) + g_slice(n, b, at);
  // M1 = Diag(G_R) W~ (dequantised), then M = M1 Diag(G_P)
  PX_HIP(merge_left(at, g_R, wt, Wt, ldw, scale_t, m, n, b, w.Mq, ldw, s));
  PX_HIP(apply(F32, F32, w.Mq, ldw, m, n, b, at, gP1, nullptr, F32, w.M, ldw, s));
  // new permutations; rho = old^{-1} o new maps new pre-merged positions to old ones
  PX_HIP(perm_from_seed_device(seed_R, m, w.newR, w.fy, s));
  PX_HIP(perm_from_seed_device(seed_P, n, w.newP, w.fy, s));
  PX_HIP(inverse_perm(perm_R, m, w.invR, s));
  PX_HIP(inverse_perm(perm_P, n, w.invP, s));
  PX_HIP(compose_perm(w.invR, w.newR, m, w.rhoR, s));
  PX_HIP(compose_perm(w.invP, w.newP, n, w.rhoP, s));
  PX_HIP(permute(F32, w.M, ldw, w.rhoR, w.rhoP, w.Mq, ldw, m, n, n, s));
  if (wt == POETX_I8) {
    PX_HIP(fill_zero(w.amax, (size_t)n * 4, s));
    PX_HIP(col_absmax(w.Mq, ldw, m, n, w.amax, s));
  }
  PX_HIP(store_weight(w.Mq, ldw, m, n, wt, Wt, ldw, w.amax, scale_t, s));
  if (has_weight_t(desc))
    PX_HIP(transpose(wt, Wt, ldw, m, n, reinterpret_cast<char*>(Wt) + weight_t_offset(desc), lead(m), s));
  PX_HIP(hipMemcpyAsync(perm_R, w.newR, (size_t)m * 4, hipMemcpyDeviceToDevice, s));
  PX_HIP(hipMemcpyAsync(perm_P, w.newP, (size_t)n * 4, hipMemcpyDeviceToDevice, s));
  PX_HIP(fill_zero(q_R, (size_t)nblocks(m, b) * packed_len(b) * 4, s));
  PX_HIP(fill_zero(q_P, (size_t)nblocks(n, b) * packed_len(b) * 4, s));
  return POETX_OK;
}

}  // extern "C"

namespace {

int spo_d_eff(const poetx_spo_desc* d) { return d->kind == POETX_SPO_BLOCK ? d->d : d->b; }

poetx_status check_spo(const poetx_spo_desc* d, int64_t T) {
  if (!d) return fail(POETX_E_NULL, "desc is NULL");
  if (d->d < 1 || d->d > kMaxDim) return fail(POETX_E_SHAPE, "d must be in [1, 2^20]");
  if (d->b < 2 || d->b > 1024) return fail(POETX_E_SHAPE, "b must be in [2, 1024]");
  if (d->kind != POETX_SPO_BLOCK && d->kind != POETX_SPO_FULL) return fail(POETX_E_SHAPE, "kind must be BLOCK or FULL");
  if (d->kind == POETX_SPO_FULL && d->b > d->d) return fail(POETX_E_SHAPE, "a FULL factor needs b <= d");
  if (nblocks(spo_d_eff(d), d->b) > 65535) return fail(POETX_E_SHAPE, "at most 65535 blocks");
  if (d->act_dtype != POETX_F32 && d->act_dtype != POETX_BF16) return fail(POETX_E_DTYPE, "act_dtype must be F32 or BF16");
  if (T < 0 || T > kMaxT) return fail(POETX_E_SHAPE, "T must be in [0, 2^31)");
  return POETX_OK;
}

struct SpoWs {
  void *A, *B;  // fwd: A = Xt Diag(G); bwd: A = dY[:, idx], B = dXt
  void* cnp;
  float* part;
};
template <class P> SpoWs plan_spo(P& p, const poetx_spo_desc* d, int64_t T, bool bwd) {
  const int de = spo_d_eff(d), nb = nblocks(de, d->b);
  const size_t mat = (size_t)T * lead(de) * dt_size(d->act_dtype);
  SpoWs w{};
  w.A = p.template take<char>(mat);
  if (bwd) {
    w.B = p.template take<char>(mat);
    w.cnp = p.template take<char>(cnp_grad_bytes(d->act_dtype, nb, d->b));
    w.part = p.template take<float>(block_grads_part_bytes(d->act_dtype, (int)T, nb, d->b));
  }
  return w;
}

// out = in except out[:, idx] = src (FULL), or out = src[:, idx^-1] (BLOCK)
poetx_status spo_place(const poetx_spo_desc* d, int rows, const void* in, const void* src, const int32_t* idx,
                       const SpoWs& w, void* out, hipStream_t s) {
  const int at = d->act_dtype, de = spo_d_eff(d);
  const double es = (double)dt_size(at);
  if (rows <= 0) return POETX_OK;
  if (d->kind == POETX_SPO_BLOCK) {
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * d->d * es, scatter(at, src, lead(de), idx, out, d->d, rows, d->d, s));
    return POETX_OK;
  }
  if (out != in)
    PX_TIMED(POETX_KC_PERMUTE, 0, (2.0 * d->d + de) * rows * es,
             replace_cols(at, in, d->d, src, lead(de), de, idx, out, d->d, rows, d->d, s));
  else
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * de * es,
             scatter_cols(at, src, lead(de), rows, de, idx, out, d->d, d->d, s));
  return POETX_OK;
}

}  // namespace

extern "C" {

size_t poetx_spo_saved_bytes(const poetx_spo_desc* desc, int64_t T) {
  if (check_spo(desc, T) != POETX_OK) return 0;
  return (size_t)T * lead(spo_d_eff(desc)) * dt_size(desc->act_dtype);
}

size_t poetx_spo_workspace_size(const poetx_spo_desc* desc, int64_t T, int32_t op) {
  if (check_spo(desc, T) != POETX_OK || (op != POETX_OP_FWD && op != POETX_OP_BWD)) return 0;
  Plan p;
  plan_spo(p, desc, T, op == POETX_OP_BWD);
  return p.off;
}

poetx_status poetx_spo_fwd(const poetx_spo_desc* desc, int64_t T, const void* X, const int32_t* idx, const void* G,
                           void* Y, void* saved, void* ws, size_t ws_bytes, void* stream) {
  poetx_status st = check_spo(desc, T);
  if (st != POETX_OK) return st;
  if (T == 0) return POETX_OK;
  if (!X || !idx || !G || !Y || !saved) return fail(POETX_E_NULL, "a required pointer is NULL");
  Plan p;
  plan_spo(p, desc, T, false);
  st = check_ws(ws, ws_bytes, p.off);
  if (st != POETX_OK) return st;
  Plan pq;
  pq.base = reinterpret_cast<char*>(ws);
  const SpoWs w = plan_spo(pq, desc, T, false);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int at = desc->act_dtype, de = spo_d_eff(desc), b = desc->b, rows = (int)T;
  const int64_t ld = lead(de);
  const double es = (double)dt_size(at);
  const char* g1 = reinterpret_cast<const char*>(G) + g_slice(de, b, at);  // (G - I)^T
  // Xt = X[:, idx] (saved), A = Xt Diag(G), then placed back into Y
  PX_TIMED(POETX_KC_PERMUTE, 0, (double)rows * (desc->d + de) * es,
           permute(at, X, desc->d, nullptr, idx, saved, ld, rows, desc->d, de, s));
  PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(de, b), 2.0 * rows * de * es + g_slice(de, b, at),
           apply(at, at, saved, ld, rows, de, b, at, g1, nullptr, at, w.A, ld, s));
  return spo_place(desc, rows, X, w.A, idx, w, Y, s);
}

poetx_status poetx_spo_bwd(const poetx_spo_desc* desc, int64_t T, const void* dY, const int32_t* idx, const void* G,
                           const float* q, const void* saved, void* dX, float* dq, void* ws, size_t ws_bytes,
                           void* stream) {
  poetx_status st = check_spo(desc, T);
  if (st != POETX_OK) return st;
  if (!idx || !G || !q || !dq) return fail(POETX_E_NULL, "a required pointer is NULL");
  if (T > 0 && (!dY || !saved || !dX)) return fail(POETX_E_NULL, "a required pointer is NULL");
  Plan p;
  plan_spo(p, desc, T, true);
  st = check_ws(ws, ws_bytes, p.off);
  if (st != POETX_OK) return st;
  Plan pq;
  pq.base = reinterpret_cast<char*>(ws);
  const SpoWs w = plan_spo(pq, desc, T, true);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int at = desc->act_dtype, de = spo_d_eff(desc), b = desc->b, rows = (int)T;
  const int64_t ld = lead(de), nb = nblocks(de, b);
  const double es = (double)dt_size(at);
  // dA = dY[:, idx]
  if (rows > 0)
    PX_TIMED(POETX_KC_PERMUTE, 0, (double)rows * (desc->d + de) * es,
             permute(at, dY, desc->d, nullptr, idx, w.A, ld, rows, desc->d, de, s));
  // dG_k = Xt_k^T dA_k over all rows (the second side of the pair has no blocks)
  const CnpSide sides[2] = {{q, de, saved, ld, w.A, ld}, {q, 0, nullptr, ld, nullptr, ld}};
  PX_TIMED(POETX_KC_DGRAD, 2.0 * rows * sum_r2(de, b), 2.0 * rows * de * es + (4 + 2 * es) * sum_r2(de, b),
           block_grads(at, sides, rows, b, w.cnp, 0, nb, w.part, s));
  // dXt = dA Diag(G)^T, placed back into dX (FULL: the other columns of dY pass through)
  PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(de, b), 2.0 * rows * de * es + g_slice(de, b, at),
           apply(at, at, w.A, ld, rows, de, b, at, G, nullptr, at, w.B, ld, s));
  st = spo_place(desc, rows, dY, w.B, idx, w, dX, s);
  if (st != POETX_OK) return st;
  const float* qs[1] = {q};
  const int ds[1] = {de};
  float* dqs[1] = {dq};
  PX_TIMED(POETX_KC_CNP, 12 * sum_r3(de, b), cnp_grad_bytes(at, nb, b), cnp_chain_batch(at, 1, qs, ds, b, w.cnp, dqs, s));
  return POETX_OK;
}

poetx_status poetx_adam_step_batch(int32_t count, const int64_t* len, float* const* q, const float* const* dq,
                                   float* const* m1, float* const* m2, const poetx_adam_params* hp, void* stream) {
  if (count < 1 || count > POETX_MAX_SIDES) return fail(POETX_E_SHAPE, "count must be in [1, POETX_MAX_SIDES]");
  if (!len || !q || !dq || !m1 || !m2 || !hp) return fail(POETX_E_NULL, "len, q, dq, m1, m2 and hp must be non-NULL");
  if (!(std::isfinite(hp->lr) && hp->lr >= 0.f)) return fail(POETX_E_SHAPE, "lr must be finite and >= 0");
  if (!(hp->beta1 >= 0.f && hp->beta1 < 1.f && hp->beta2 >= 0.f && hp->beta2 < 1.f))
    return fail(POETX_E_SHAPE, "beta1 and beta2 must be in [0, 1)");
  if (!(std::isfinite(hp->eps) && hp->eps > 0.f)) return fail(POETX_E_SHAPE, "eps must be finite and > 0");
  if (!std::isfinite(hp->weight_decay)) return fail(POETX_E_SHAPE, "weight_decay must be finite");
  if (hp->t < 1) return fail(POETX_E_SHAPE, "t must be >= 1");
  double slots = 0;
  for (int i = 0; i < count; ++i) {
    if (len[i] < 0 || len[i] > (int64_t(1) << 36)) return fail(POETX_E_SHAPE, "len[i] must be in [0, 2^36]");
    if (len[i] > 0 && (!q[i] || !dq[i] || !m1[i] || !m2[i]))
      return fail(POETX_E_NULL, "q[i], dq[i], m1[i] and m2[i] must be non-NULL when len[i] > 0");
    slots += (double)len[i];
  }
  AdamHyper h{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->t};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PX_TIMED(POETX_KC_OPTIM, 0, 28.0 * slots, adam_batch(count, len, q, dq, m1, m2, h, s));
  return POETX_OK;
}

}  // extern "C"
