// C ABI of libpoetx: argument validation, workspace planning and the order of
// kernel launches for each call.  All arithmetic happens in the kernels of
// poetx_kernels.hip.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/poetx.h"
#include "poetx_internal.h"

using namespace pxk;

// Workspace of poetx_cnp_build_noalloc: a fixed device array of the library.
// Each GPU the library runs on holds its own copy for the life of the process.
// Host code never uses the name as an address (on the host it is a stand-in
// symbol); the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[POETX_NOALLOC_SCRATCH_BYTES];

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

// The K of a bf16 W~ contraction: lead(K), a multiple of 64, so that the
// direct-to-LDS loop serves ragged K too.  Both operands hold zeros in their
// pitch padding [K, lead(K)) (the library writes them: the weight formats
// and zero_pad below), so the extra products are exact zeros.
int k_padded(int K, int act_dtype) { return act_dtype == POETX_BF16 ? (int)lead(K) : K; }

// zeros in the pitch padding [d, lead(d)) of a [rows][lead(d)] activation operand that a W~
// contraction reads over k_padded(d)
hipError_t zero_pad(int act_dtype, void* p, int rows, int d, hipStream_t s) {
  if (act_dtype != POETX_BF16 || lead(d) == d) return hipSuccess;
  return zero_cols(act_dtype, p, lead(d), rows, d, (int)lead(d), s);
}

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
  void* Wb;          // int8 weights: W~^T widened to bf16
};
template <class P> FwdWs plan_fwd(P& p, const poetx_layer_desc* d, int64_t T) {
  const size_t es = dt_size(d->act_dtype);
  FwdWs w;
  w.A = p.template take<char>(T * lead(d->m) * es);
  w.Zt = p.template take<char>(T * lead(d->n) * es);
  w.H = saves_h(d) ? nullptr : p.template take<char>(T * lead(d->n) * es);
  // int8 weights: the transposed codes widened to bf16 for the W~ contraction
  w.Wb = d->w_dtype == POETX_I8 ? p.template take<char>((size_t)d->n * lead(d->m) * 2) : nullptr;
  return w;
}

struct BwdWs {
  void *dZt, *dH, *dA, *dXt, *cnp, *Wb;
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
  // int8 weights: the codes widened to bf16 for the W~^T contraction (and transposed for the Xmem recompute)
  w.Wb = d->w_dtype == POETX_I8
             ? p.template take<char>(std::max((size_t)d->m * lead(d->n), (size_t)d->n * lead(d->m)) * 2)
             : nullptr;
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

// Device address of `scratch` on the current device, looked up the first time
// the device is seen and kept per device ordinal.
struct ScratchTable {
  std::mutex mu;
  std::vector<void*> ptr;
};
ScratchTable& scratch_table() {
  static ScratchTable t;
  return t;
}
poetx_status scratch_ptr(void** out) {
  int dev = -1;
  PX_HIP(hipGetDevice(&dev));
  if (dev < 0) return fail(POETX_E_HIP, "no current device");
  ScratchTable& t = scratch_table();
  std::lock_guard<std::mutex> g(t.mu);
  if ((int)t.ptr.size() <= dev) t.ptr.resize(dev + 1, nullptr);
  if (!t.ptr[dev]) {
    void* p = nullptr;
    PX_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(POETX_E_HIP, "hipGetSymbolAddress returned NULL for the scratch array");
    t.ptr[dev] = p;
  }
  *out = t.ptr[dev];
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

poetx_status poetx_cnp_build_noalloc(const float* q, int32_t d, int32_t b, int32_t dtype, void* g, void* stream) {
  if (!q || !g) return fail(POETX_E_NULL, "q and g must be non-NULL");
  int64_t blocks = 0;
  poetx_status st = check_sides(1, &d, b, dtype, &blocks);
  if (st != POETX_OK) return st;
  const size_t need = cnp_build_ws_bytes(dtype, blocks, b);
  if (need > (size_t)POETX_NOALLOC_SCRATCH_BYTES)
    return fail(POETX_E_WORKSPACE, "side needs " + std::to_string(need) + " bytes of scratch; the fixed array holds " +
                                       std::to_string((size_t)POETX_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != POETX_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const double flops = 4 * sum_r3(d, b), bytes = 2.0 * g_slice(d, b, dtype) + 2.0 * nblocks(d, b) * b * b * 4;
  PX_TIMED(POETX_KC_CNP, flops, bytes, cnp_build_batch(dtype, 1, &q, &d, b, &g, ws, s));
  return POETX_OK;
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
  PX_HIP(zero_cols(desc->w_dtype, Wt, lead(n), m, n, (int)lead(n), s));  // the pitch padding of the format
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
                     void* H, void* Wb, hipStream_t s) {
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
  PX_HIP(zero_pad(at, A, rows, m, s));
  // H = A W~ (int8: codes times the column scale); bf16 weights are read from the W~^T copy, int8 codes
  // from their transpose widened to bf16 in the workspace (exact), so both take the same loop
  if (has_weight_t(desc)) {
    const void* Wtt = reinterpret_cast<const char*>(Wt) + weight_t_offset(desc);
    PX_TIMED(POETX_KC_GEMM, 2.0 * rows * m * n, es * rows * m + wes * m * n + es * rows * n,
             gemm(at, at, A, ldm, wt, Wtt, ldm, false, rows, n, k_padded(m, at), nullptr, at, H, ldn, s));
  } else if (wt == POETX_I8 && at == POETX_BF16 && Wb) {
    PX_TIMED(POETX_KC_GEMM, 0, 3.0 * m * n,
             widen_i8(reinterpret_cast<const int8_t*>(Wt), lead(n), m, n, true, reinterpret_cast<uint16_t*>(Wb), ldm, s));
    PX_TIMED(POETX_KC_GEMM, 2.0 * rows * m * n, es * rows * m + 2.0 * m * n + es * rows * n,
             gemm(at, at, A, ldm, POETX_BF16, Wb, ldm, false, rows, n, k_padded(m, at), scale_t, at, H, ldn, s));
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
  st = xt_to_h(desc, T, Xt, Wt, g_R, w.A, H, w.Wb, s);
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
// of the gradient state dg (total blocks); shared by the backward entry points.
// With `defer` the block gradients are not formed: defer[0] (R) and defer[1] (P)
// receive their operands instead.
poetx_status bwd_dx_core(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ,
                         const int32_t* perm_R, const int32_t* perm_P, const void* Wt, const void* g_R,
                         const void* g_P, const float* q_R, const float* q_P, const void* H_save, void* dX, void* dg,
                         int64_t first, int64_t total, const BwdWs& w, hipStream_t s, CnpSide* defer = nullptr,
                         bool scatter_dx = true) {
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
  PX_HIP(zero_pad(at, w.dH, rows, n, s));
  // dA = dH W~^T (int8: the codes widened to bf16 in the workspace first, exact)
  if (wt == POETX_I8 && at == POETX_BF16 && w.Wb) {
    PX_TIMED(POETX_KC_GEMM, 0, 3.0 * m * n,
             widen_i8(reinterpret_cast<const int8_t*>(Wt), lead(n), m, n, false, reinterpret_cast<uint16_t*>(w.Wb), ldn,
                      s));
    PX_TIMED(POETX_KC_GEMM, 2.0 * rows * m * n, es * rows * n + 2.0 * m * n + es * rows * m,
             gemm(at, at, w.dH, ldn, POETX_BF16, w.Wb, ldn, false, rows, m, k_padded(n, at), nullptr, at, w.dA, ldm, s));
  } else {
    PX_TIMED(POETX_KC_GEMM, 2.0 * rows * m * n, es * rows * n + wes * m * n + es * rows * m,
             gemm(at, at, w.dH, ldn, wt, Wt, lead(n), false, rows, m, k_padded(n, at), nullptr, at, w.dA, ldm, s));
  }
  // block gradients of both sides over all tokens: dG_R = Xt^T dA, dG_P = H^T dZt, with Xt and H
  // from the forward's saved state.  Xmem recomputes H from Xt, into the buffers that dH (consumed
  // by the contraction above) and dXt (written below) occupy.  Xout takes H back from the output:
  // Zt = Y[:, perm_P] into dH's buffer, then H = Zt Diag(G_P)^T.
  const void* Xt = reinterpret_cast<const char*>(H_save) + saved_xt_offset(desc, T);
  const void* H = H_save;
  if (desc->mode == POETX_XMEM) {
    const poetx_status st = xt_to_h(desc, T, Xt, Wt, g_R, w.dXt, w.dH, w.Wb, s);
    if (st != POETX_OK) return st;
    H = w.dH;
  } else if (desc->mode == POETX_XOUT) {
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * n * es, permute(at, Y, n, nullptr, perm_P, w.dH, ldn, rows, n, n, s));
    PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(n, b), 2.0 * rows * n * es + g_slice(n, b, at),
             apply(at, at, w.dH, ldn, rows, n, b, at, g_P, nullptr, at, w.Hr, ldn, s));
    H = w.Hr;
  }
  const CnpSide sides[2] = {{q_R, m, Xt, ldm, w.dA, ldm}, {q_P, n, H, ldn, w.dZt, ldn}};
  if (defer) {
    defer[0] = sides[0];
    defer[1] = sides[1];
  } else {
    PX_TIMED(POETX_KC_DGRAD, 2.0 * rows * (sum_r2(m, b) + sum_r2(n, b)),
             2.0 * rows * (m + n) * es + (4 + 2 * es) * (sum_r2(m, b) + sum_r2(n, b)),
             block_grads(at, sides, rows, b, dg, first, total, w.part, s));
  }
  // dXt = dA Diag(G_R)^T;  dX[:, perm_R] = dXt
  PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(m, b), 2.0 * rows * m * es + g_slice(m, b, at),
           apply(at, at, w.dA, ldm, rows, m, b, at, g_R, nullptr, at, w.dXt, ldm, s));
  if (rows > 0 && scatter_dx)
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * m * es, scatter(at, w.dXt, ldm, perm_R, dX, m, rows, m, s));
  return POETX_OK;
}

// dX[:, perm_R] = dXt of every call of a backward group; the calls that pass one dX tensor (they
// read one input) write the sum of their input gradients, accumulated in fp32 and rounded once
poetx_status scatter_group_dx(int count, const poetx_bwd_call* calls, const BwdWs* w, int rows, hipStream_t s) {
  bool done[POETX_MAX_GROUP] = {};
  for (int i = 0; i < count; ++i) {
    if (done[i]) continue;
    const int m = calls[i].desc->m, at = calls[i].desc->act_dtype;
    const void* in[POETX_MAX_GROUP];
    int64_t ld[POETX_MAX_GROUP];
    const int32_t* pm[POETX_MAX_GROUP];
    int nm = 0;
    for (int j = i; j < count; ++j) {
      if (done[j] || calls[j].dX != calls[i].dX) continue;
      done[j] = true;
      in[nm] = w[j].dXt;
      ld[nm] = lead(m);
      pm[nm++] = calls[j].perm_R;
    }
    PX_TIMED(POETX_KC_PERMUTE, 0, (double)dt_size(at) * rows * m * (nm + 1),
             scatter_sum(at, nm, in, ld, pm, calls[i].dX, m, rows, m, s));
  }
  return POETX_OK;
}

// need_q: the call reads q_R and q_P (not when the block gradients are left to the caller)
poetx_status check_bwd(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ, const int32_t* perm_R,
                       const int32_t* perm_P, const void* Wt, const void* g_R, const void* g_P, const float* q_R,
                       const float* q_P, const void* H_save, void* dX, void* ws, size_t ws_bytes,
                       bool need_q = true) {
  poetx_status st = check_desc(desc);
  if (st != POETX_OK) return st;
  if (T < 0 || T > kMaxT) return fail(POETX_E_SHAPE, "T must be in [0, 2^31)");
  if (!perm_R || !perm_P || !Wt || !g_R || !g_P || (need_q && (!q_R || !q_P)))
    return fail(POETX_E_NULL, "a required pointer is NULL");
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

poetx_status poetx_linear_bwd_dx_sides(const poetx_layer_desc* desc, int64_t T, const void* Y, const void* dZ,
                                       const int32_t* perm_R, const int32_t* perm_P, const void* Wt, const void* g_R,
                                       const void* g_P, const void* H_save, void* dX, poetx_grad_side* sides,
                                       void* ws, size_t ws_bytes, void* stream) {
  poetx_status st =
      check_bwd(desc, T, Y, dZ, perm_R, perm_P, Wt, g_R, g_P, nullptr, nullptr, H_save, dX, ws, ws_bytes, false);
  if (st != POETX_OK) return st;
  if (!sides) return fail(POETX_E_NULL, "sides is NULL");
  Plan pq;
  pq.base = reinterpret_cast<char*>(ws);
  const BwdWs w = plan_bwd(pq, desc, T);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  CnpSide cs[2];
  st = bwd_dx_core(desc, T, Y, dZ, perm_R, perm_P, Wt, g_R, g_P, nullptr, nullptr, H_save, dX, nullptr, 0, 0, w, s,
                   cs);
  if (st != POETX_OK) return st;
  for (int k = 0; k < 2; ++k) sides[k] = poetx_grad_side{cs[k].A, cs[k].lda, cs[k].B, cs[k].ldb, cs[k].d};
  return POETX_OK;
}

}  // extern "C"

namespace {

// gemm_batch, one launch at a time, so that the contraction timer sees every kernel launch
poetx_status gemm_batch_timed(int count, const GemmProblem* gp, const double* flops, const double* bytes,
                              hipStream_t s) {
  int launch_of[kGemmProblems];
  const int n = gemm_launches(count, gp, launch_of);
  for (int l = 0; l < n; ++l) {
    GemmProblem part[kGemmProblems];
    int np = 0;
    double fl = 0, by = 0;
    for (int i = 0; i < count; ++i)
      if (launch_of[i] == l) {
        part[np++] = gp[i];
        fl += flops[i];
        by += bytes[i];
      }
    PX_TIMED(POETX_KC_GEMM, fl, by, gemm_batch(np, part, s));
  }
  return POETX_OK;
}

}  // namespace

extern "C" {

poetx_status poetx_linear_fwd_group(int32_t count, const poetx_fwd_call* calls, int64_t T, void* stream) {
  if (!calls) return fail(POETX_E_NULL, "calls is NULL");
  if (count < 1 || count > POETX_MAX_GROUP) return fail(POETX_E_SHAPE, "count must be in [1, POETX_MAX_GROUP]");
  if (T < 0 || T > kMaxT) return fail(POETX_E_SHAPE, "T must be in [0, 2^31)");
  bool bf16 = true;
  for (int i = 0; i < count; ++i) {
    const poetx_fwd_call& c = calls[i];
    poetx_status st = check_desc(c.desc);
    if (st != POETX_OK) return st;
    if (c.desc->b != calls[0].desc->b) return fail(POETX_E_SHAPE, "the linears of a group must share b");
    if (T > 0 && (!c.X || !c.perm_R || !c.perm_P || !c.Wt || !c.g_R || !c.g_P || !c.Y || !c.H_save))
      return fail(POETX_E_NULL, "a required pointer is NULL");
    Plan p;
    plan_fwd(p, c.desc, T);
    st = check_ws(c.ws, c.ws_bytes, p.off);
    if (st != POETX_OK) return st;
    bf16 = bf16 && c.desc->act_dtype == POETX_BF16;
  }
  if (T == 0) return POETX_OK;
  if (!bf16) {
    // fp32 layers: one forward per linear
    for (int i = 0; i < count; ++i) {
      const poetx_fwd_call& c = calls[i];
      const poetx_status st = poetx_linear_fwd(c.desc, T, c.X, c.perm_R, c.perm_P, c.Wt, c.g_R, c.g_P, c.Y, c.H_save,
                                               c.ws, c.ws_bytes, stream);
      if (st != POETX_OK) return st;
    }
    return POETX_OK;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int rows = (int)T, b = calls[0].desc->b;
  FwdWs w[POETX_MAX_GROUP];
  void *Xt[POETX_MAX_GROUP], *H[POETX_MAX_GROUP];
  ApplySide sr[POETX_MAX_GROUP], sp[POETX_MAX_GROUP];
  GemmProblem gp[POETX_MAX_GROUP];
  double fl_g[POETX_MAX_GROUP], by_g[POETX_MAX_GROUP];
  double fl_r = 0, by_r = 0, fl_p = 0, by_p = 0;
  for (int i = 0; i < count; ++i) {
    const poetx_fwd_call& c = calls[i];
    const poetx_layer_desc* d = c.desc;
    const int m = d->m, n = d->n;
    const int64_t ldm = lead(m), ldn = lead(n);
    Plan q;
    q.base = reinterpret_cast<char*>(c.ws);
    w[i] = plan_fwd(q, d, T);
    Xt[i] = reinterpret_cast<char*>(c.H_save) + saved_xt_offset(d, T);
    H[i] = saves_h(d) ? c.H_save : w[i].H;
    const char* gR1 = reinterpret_cast<const char*>(c.g_R) + g_slice(m, b, BF16);  // Delta_R^T
    const char* gP1 = reinterpret_cast<const char*>(c.g_P) + g_slice(n, b, BF16);  // Delta_P^T
    sr[i] = ApplySide{Xt[i], ldm, m, gR1, nullptr, w[i].A, ldm};
    sp[i] = ApplySide{H[i], ldn, n, gP1, nullptr, w[i].Zt, ldn};
    fl_r += 2.0 * rows * sum_r2(m, b);
    by_r += 4.0 * rows * m + g_slice(m, b, BF16);
    fl_p += 2.0 * rows * sum_r2(n, b);
    by_p += 4.0 * rows * n + g_slice(n, b, BF16);
    // H = A W~: bf16 weights from the stored W~^T, int8 codes from their transpose widened to bf16 (exact)
    const float* scale_t = nullptr;
    const void* Bw = nullptr;
    if (has_weight_t(d)) {
      Bw = reinterpret_cast<const char*>(c.Wt) + weight_t_offset(d);
    } else {
      scale_t = reinterpret_cast<const float*>(reinterpret_cast<const char*>(c.Wt) + weight_scale_offset(d));
      Bw = w[i].Wb;
    }
    gp[i] = GemmProblem{w[i].A, ldm, Bw, ldm, rows, n, k_padded(m, BF16), scale_t, H[i], ldn};
    fl_g[i] = 2.0 * rows * m * n;
    by_g[i] = 2.0 * rows * m + 2.0 * m * n + 2.0 * rows * n;
  }
  // Xt = X[:, perm_R], kept in the saved state for the backward; the linears that read one input
  // tensor gather from it in one pass (each row of X read once)
  bool gathered[POETX_MAX_GROUP] = {};
  for (int i = 0; i < count; ++i) {
    if (gathered[i]) continue;
    const int m = calls[i].desc->m;
    const int32_t* cm[POETX_MAX_GROUP];
    void* xo[POETX_MAX_GROUP];
    int64_t ld[POETX_MAX_GROUP];
    int dd[POETX_MAX_GROUP], nm = 0;
    for (int j = i; j < count; ++j) {
      if (gathered[j] || calls[j].X != calls[i].X || calls[j].desc->m != m) continue;
      gathered[j] = true;
      cm[nm] = calls[j].perm_R;
      xo[nm] = Xt[j];
      ld[nm] = lead(m);
      dd[nm++] = m;
    }
    if (nm == 1)
      PX_TIMED(POETX_KC_PERMUTE, 0, 4.0 * rows * m,
               permute(BF16, calls[i].X, m, nullptr, cm[0], xo[0], ld[0], rows, m, m, s));
    else
      PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * m * (1 + nm),
               permute_multi(BF16, calls[i].X, m, nm, cm, xo, ld, dd, rows, m, s));
  }
  // A = Xt Diag(G_R) for every linear
  PX_TIMED(POETX_KC_APPLY, fl_r, by_r, apply_batch(count, sr, rows, b, s));
  for (int i = 0; i < count; ++i) PX_HIP(zero_pad(BF16, w[i].A, rows, calls[i].desc->m, s));
  for (int i = 0; i < count; ++i) {
    const poetx_layer_desc* d = calls[i].desc;
    if (d->w_dtype == POETX_I8)
      PX_TIMED(POETX_KC_GEMM, 0, 3.0 * d->m * d->n,
               widen_i8(reinterpret_cast<const int8_t*>(calls[i].Wt), lead(d->n), d->m, d->n, true,
                        reinterpret_cast<uint16_t*>(w[i].Wb), lead(d->m), s));
  }
  poetx_status st = gemm_batch_timed(count, gp, fl_g, by_g, s);
  if (st != POETX_OK) return st;
  // Zt = H Diag(G_P), then Y[:, perm_P] = Zt
  PX_TIMED(POETX_KC_APPLY, fl_p, by_p, apply_batch(count, sp, rows, b, s));
  for (int i = 0; i < count; ++i) {
    const int n = calls[i].desc->n;
    PX_TIMED(POETX_KC_PERMUTE, 0, 4.0 * rows * n,
             scatter(BF16, w[i].Zt, lead(n), calls[i].perm_P, calls[i].Y, n, rows, n, s));
  }
  return POETX_OK;
}

poetx_status poetx_linear_bwd_dx_group(int32_t count, const poetx_bwd_call* calls, int64_t T, poetx_grad_side* sides,
                                       void* stream) {
  if (!calls || !sides) return fail(POETX_E_NULL, "calls and sides must be non-NULL");
  if (count < 1 || count > POETX_MAX_GROUP) return fail(POETX_E_SHAPE, "count must be in [1, POETX_MAX_GROUP]");
  if (T < 0 || T > kMaxT) return fail(POETX_E_SHAPE, "T must be in [0, 2^31)");
  bool bf16 = true;
  for (int i = 0; i < count; ++i) {
    const poetx_bwd_call& c = calls[i];
    const poetx_status st = check_bwd(c.desc, T, c.Y, c.dZ, c.perm_R, c.perm_P, c.Wt, c.g_R, c.g_P, nullptr, nullptr,
                                      c.H_save, c.dX, c.ws, c.ws_bytes, false);
    if (st != POETX_OK) return st;
    if (c.desc->b != calls[0].desc->b) return fail(POETX_E_SHAPE, "the linears of a group must share b");
    for (int j = 0; j < i; ++j)
      if (T > 0 && calls[j].dX == c.dX &&
          (calls[j].desc->m != c.desc->m || calls[j].desc->act_dtype != c.desc->act_dtype || c.desc->m > 16384))
        return fail(POETX_E_SHAPE, "calls that share dX must share m (at most 16384) and act_dtype");
    bf16 = bf16 && c.desc->act_dtype == POETX_BF16;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  BwdWs w[POETX_MAX_GROUP];
  for (int i = 0; i < count; ++i) {
    Plan q;
    q.base = reinterpret_cast<char*>(calls[i].ws);
    w[i] = plan_bwd(q, calls[i].desc, T);
  }
  if (!bf16 || T == 0) {
    // fp32 layers (and no tokens): one backward per linear, the scatters to dX as for the group
    for (int i = 0; i < count; ++i) {
      const poetx_bwd_call& c = calls[i];
      CnpSide cs[2];
      const poetx_status st = bwd_dx_core(c.desc, T, c.Y, c.dZ, c.perm_R, c.perm_P, c.Wt, c.g_R, c.g_P, nullptr,
                                          nullptr, c.H_save, c.dX, nullptr, 0, 0, w[i], s, cs, false);
      if (st != POETX_OK) return st;
      for (int k = 0; k < 2; ++k)
        sides[2 * i + k] = poetx_grad_side{cs[k].A, cs[k].lda, cs[k].B, cs[k].ldb, cs[k].d};
    }
    return T > 0 ? scatter_group_dx(count, calls, w, (int)T, s) : POETX_OK;
  }
  const int rows = (int)T, b = calls[0].desc->b;
  ApplySide sp[POETX_MAX_GROUP], sr[POETX_MAX_GROUP];
  GemmProblem gp[POETX_MAX_GROUP];
  double fl_g[POETX_MAX_GROUP], by_g[POETX_MAX_GROUP];
  double fl_r = 0, by_r = 0, fl_p = 0, by_p = 0;
  for (int i = 0; i < count; ++i) {
    const poetx_bwd_call& c = calls[i];
    const poetx_layer_desc* d = c.desc;
    const int m = d->m, n = d->n;
    const int64_t ldm = lead(m), ldn = lead(n);
    const float* scale_t =
        d->w_dtype == POETX_I8
            ? reinterpret_cast<const float*>(reinterpret_cast<const char*>(c.Wt) + weight_scale_offset(d))
            : nullptr;
    // dZt = dZ[:, perm_P]
    PX_TIMED(POETX_KC_PERMUTE, 0, 4.0 * rows * n,
             permute(BF16, c.dZ, n, nullptr, c.perm_P, w[i].dZt, ldn, rows, n, n, s));
    // dH = dZt Diag(G_P)^T (int8: times the column scale); dA = dH W~^T (int8: the codes widened to bf16)
    sp[i] = ApplySide{w[i].dZt, ldn, n, c.g_P, scale_t, w[i].dH, ldn};
    const void* Bw = d->w_dtype == POETX_I8 ? w[i].Wb : c.Wt;
    gp[i] = GemmProblem{w[i].dH, ldn, Bw, d->w_dtype == POETX_I8 ? ldn : lead(n), rows, m, k_padded(n, BF16), nullptr,
                        w[i].dA, ldm};
    // dXt = dA Diag(G_R)^T
    sr[i] = ApplySide{w[i].dA, ldm, m, c.g_R, nullptr, w[i].dXt, ldm};
    fl_p += 2.0 * rows * sum_r2(n, b);
    by_p += 4.0 * rows * n + g_slice(n, b, BF16);
    fl_r += 2.0 * rows * sum_r2(m, b);
    by_r += 4.0 * rows * m + g_slice(m, b, BF16);
    fl_g[i] = 2.0 * rows * m * n;
    by_g[i] = 2.0 * rows * n + (d->w_dtype == POETX_I8 ? 2.0 : (double)dt_size(d->w_dtype)) * m * n + 2.0 * rows * m;
  }
  PX_TIMED(POETX_KC_APPLY, fl_p, by_p, apply_batch(count, sp, rows, b, s));
  for (int i = 0; i < count; ++i) PX_HIP(zero_pad(BF16, w[i].dH, rows, calls[i].desc->n, s));
  for (int i = 0; i < count; ++i) {
    const poetx_layer_desc* d = calls[i].desc;
    if (d->w_dtype == POETX_I8)
      PX_TIMED(POETX_KC_GEMM, 0, 3.0 * d->m * d->n,
               widen_i8(reinterpret_cast<const int8_t*>(calls[i].Wt), lead(d->n), d->m, d->n, false,
                        reinterpret_cast<uint16_t*>(w[i].Wb), lead(d->n), s));
  }
  poetx_status st = gemm_batch_timed(count, gp, fl_g, by_g, s);
  if (st != POETX_OK) return st;
  // H for the P side's block gradients, as in poetx_linear_bwd_dx_sides: saved (Xfast), recomputed from Xt
  // into the buffers of dH and dXt (Xmem), or taken back from the output (Xout)
  for (int i = 0; i < count; ++i) {
    const poetx_bwd_call& c = calls[i];
    const poetx_layer_desc* d = c.desc;
    const int m = d->m, n = d->n;
    const int64_t ldm = lead(m), ldn = lead(n);
    const void* Xt = reinterpret_cast<const char*>(c.H_save) + saved_xt_offset(d, T);
    const void* H = c.H_save;
    if (d->mode == POETX_XMEM) {
      const poetx_status st = xt_to_h(d, T, Xt, c.Wt, c.g_R, w[i].dXt, w[i].dH, w[i].Wb, s);
      if (st != POETX_OK) return st;
      H = w[i].dH;
    } else if (d->mode == POETX_XOUT) {
      PX_TIMED(POETX_KC_PERMUTE, 0, 4.0 * rows * n,
               permute(BF16, c.Y, n, nullptr, c.perm_P, w[i].dH, ldn, rows, n, n, s));
      PX_TIMED(POETX_KC_APPLY, 2.0 * rows * sum_r2(n, b), 4.0 * rows * n + g_slice(n, b, BF16),
               apply(BF16, BF16, w[i].dH, ldn, rows, n, b, BF16, c.g_P, nullptr, BF16, w[i].Hr, ldn, s));
      H = w[i].Hr;
    }
    sides[2 * i] = poetx_grad_side{Xt, ldm, w[i].dA, ldm, m};
    sides[2 * i + 1] = poetx_grad_side{H, ldn, w[i].dZt, ldn, n};
  }
  PX_TIMED(POETX_KC_APPLY, fl_r, by_r, apply_batch(count, sr, rows, b, s));
  return scatter_group_dx(count, calls, w, rows, s);
}

size_t poetx_block_grads_workspace_size(int32_t count, const int32_t* d, int64_t rows, int32_t b, int32_t dtype) {
  int64_t blocks = 0;
  if (rows < 0 || rows > kMaxT || check_sides(count, d, b, dtype, &blocks) != POETX_OK) return 0;
  // one launch per kGradSides sides, one after the other on the stream: the partials buffer is shared
  size_t need = 0;
  for (int c0 = 0; c0 < count; c0 += kGradSides) {
    int64_t nb = 0;
    for (int i = c0; i < std::min<int>(count, c0 + kGradSides); ++i) nb += nblocks(d[i], b);
    need = std::max(need, block_grads_part_bytes(dtype, (int)rows, (int)nb, b));
  }
  return need;
}

poetx_status poetx_block_grads_batch(int32_t count, const poetx_grad_side* sides, int64_t rows, int32_t b,
                                     int32_t dtype, void* dg, size_t dg_bytes, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!sides || !dg) return fail(POETX_E_NULL, "sides and dg must be non-NULL");
  if (count < 1 || count > POETX_MAX_SIDES) return fail(POETX_E_SHAPE, "count must be in [1, POETX_MAX_SIDES]");
  if (rows < 0 || rows > kMaxT) return fail(POETX_E_SHAPE, "rows must be in [0, 2^31)");
  int32_t d[POETX_MAX_SIDES];
  for (int i = 0; i < count; ++i) d[i] = sides[i].d;
  int64_t blocks = 0;
  poetx_status st = check_sides(count, d, b, dtype, &blocks);
  if (st != POETX_OK) return st;
  const double es = dtype == POETX_BF16 ? 2.0 : 4.0;
  double flops = 0, bytes = 0;
  for (int i = 0; i < count; ++i) {
    if (rows > 0 && (!sides[i].A || !sides[i].B)) return fail(POETX_E_NULL, "sides[i].A and sides[i].B must be non-NULL");
    if (sides[i].lda < d[i] || sides[i].ldb < d[i]) return fail(POETX_E_SHAPE, "lda and ldb must be >= d");
    flops += 2.0 * rows * sum_r2(d[i], b);
    bytes += 2.0 * rows * d[i] * es + (4 + 2 * es) * sum_r2(d[i], b);
  }
  if (dg_bytes < cnp_grad_bytes(dtype, blocks, b))
    return fail(POETX_E_WORKSPACE, "dg smaller than poetx_cnp_grad_bytes of the sides' block count");
  if (reinterpret_cast<uintptr_t>(dg) % 256) return fail(POETX_E_WORKSPACE, "dg must be 256-byte aligned");
  const size_t need = poetx_block_grads_workspace_size(count, d, rows, b, dtype);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(POETX_E_WORKSPACE, "ws smaller than poetx_block_grads_workspace_size");
  if (need > 0 && reinterpret_cast<uintptr_t>(ws) % 256) return fail(POETX_E_WORKSPACE, "ws must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int64_t zoff = 0;
  for (int c0 = 0; c0 < count; c0 += kGradSides) {
    const int nc = std::min<int>(count - c0, kGradSides);
    CnpSide cs[kGradSides];
    int64_t nb = 0;
    for (int k = 0; k < nc; ++k) {
      const poetx_grad_side& g = sides[c0 + k];
      cs[k] = CnpSide{nullptr, g.d, g.A, g.lda, g.B, g.ldb};
      nb += nblocks(g.d, b);
    }
    PX_TIMED(POETX_KC_DGRAD, c0 == 0 ? flops : 0.0, c0 == 0 ? bytes : 0.0,
             block_grads_n(dtype, nc, cs, (int)rows, b, dg, zoff, blocks, reinterpret_cast<float*>(ws), s));
    zoff += nb;
  }
  return POETX_OK;
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

poetx_status poetx_cnp_backward_batch_reuse(int32_t count, const float* const* q, const int32_t* d, int32_t b,
                                            int32_t dtype, const void* build_ws, size_t build_ws_bytes, void* dg,
                                            size_t dg_bytes, float* const* dq, void* stream) {
  if (!q || !dq || !dg || !build_ws) return fail(POETX_E_NULL, "q, dq, dg and build_ws must be non-NULL");
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
  if (build_ws_bytes < cnp_build_ws_bytes(dtype, blocks, b))
    return fail(POETX_E_WORKSPACE, "build_ws smaller than poetx_cnp_batch_workspace_size of the sides");
  if (reinterpret_cast<uintptr_t>(build_ws) % 256) return fail(POETX_E_WORKSPACE, "build_ws must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PX_TIMED(POETX_KC_CNP, flops, cnp_grad_bytes(dtype, blocks, b),
           cnp_chain_batch(dtype, count, q, d, b, dg, dq, s, build_ws));
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
  PX_HIP(zero_cols(wt, Wt, ldw, m, n, (int)ldw, s));
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

// ---------------------------------------------------------------------------
// weight-centric baseline: the factors applied to the weight, then one dense
// contraction per direction (the order original POET computes in)
// ---------------------------------------------------------------------------
namespace {

// What the forward leaves for the backward: M = Diag(G_R) W~ Diag(G_P) and
// U = Diag(G_R) W~ as [m][lead(n)], V^T = (W~ Diag(G_P))^T as [n][lead(m)],
// and Xt = X[:, perm_R] as [T][lead(m)], all in act_dtype.
struct WcState {
  void *M, *U, *Vt, *Xt;
};
template <class P> WcState plan_wc_state(P& p, const poetx_layer_desc* d, int64_t T) {
  const size_t es = dt_size(d->act_dtype), mn = (size_t)d->m * lead(d->n), nm = (size_t)d->n * lead(d->m);
  WcState w;
  w.M = p.template take<char>(mn * es);
  w.U = p.template take<char>(mn * es);
  w.Vt = p.template take<char>(nm * es);
  w.Xt = p.template take<char>((size_t)T * lead(d->m) * es);
  return w;
}
struct WcFwdWs {
  void *Wtt, *Ut, *V, *Mt, *Yt;
};
template <class P> WcFwdWs plan_wc_fwd(P& p, const poetx_layer_desc* d, int64_t T) {
  const size_t es = dt_size(d->act_dtype), mn = (size_t)d->m * lead(d->n), nm = (size_t)d->n * lead(d->m);
  WcFwdWs w;
  w.Wtt = has_weight_t(d) ? nullptr : p.template take<char>(nm * es);  // fp32 weights keep no transposed copy
  w.Ut = p.template take<char>(nm * es);
  w.V = p.template take<char>(mn * es);
  w.Mt = p.template take<char>(nm * es);
  w.Yt = p.template take<char>((size_t)T * lead(d->n) * es);
  return w;
}
struct WcBwdWs {
  void *dZt, *dXt, *Xtt, *dZtt, *dM, *dMt, *cnp;
  float* part;
};
template <class P> WcBwdWs plan_wc_bwd(P& p, const poetx_layer_desc* d, int64_t T) {
  const int at = d->act_dtype, b = d->b, nbR = nblocks(d->m, b), nbP = nblocks(d->n, b);
  const size_t es = dt_size(at), mn = (size_t)d->m * lead(d->n), nm = (size_t)d->n * lead(d->m);
  const int64_t ldT = round_up(T, 64);
  WcBwdWs w;
  w.dZt = p.template take<char>((size_t)T * lead(d->n) * es);
  w.dXt = p.template take<char>((size_t)T * lead(d->m) * es);
  w.Xtt = p.template take<char>((size_t)d->m * ldT * es);
  w.dZtt = p.template take<char>((size_t)d->n * ldT * es);
  w.dM = p.template take<char>(mn * es);
  w.dMt = p.template take<char>(nm * es);
  w.cnp = p.template take<char>(cnp_grad_bytes(at, (int64_t)nbR + nbP, b));
  w.part = p.template take<float>(
      std::max(block_grads_part_bytes(at, d->n, nbR, b), block_grads_part_bytes(at, d->m, nbP, b)));
  return w;
}

poetx_status check_wc(const poetx_layer_desc* desc, int64_t T) {
  poetx_status st = check_desc(desc);
  if (st != POETX_OK) return st;
  if (desc->w_dtype != desc->act_dtype)
    return fail(POETX_E_UNSUPPORTED, "the weight-centric path takes (F32, F32) or (BF16, BF16) layers");
  if (T < 0 || T > kMaxT) return fail(POETX_E_SHAPE, "T must be in [0, 2^31)");
  return POETX_OK;
}

}  // namespace

extern "C" {

size_t poetx_wc_state_bytes(const poetx_layer_desc* desc, int64_t T) {
  if (check_wc(desc, T) != POETX_OK) return 0;
  Plan p;
  plan_wc_state(p, desc, T);
  return p.off;
}

size_t poetx_wc_workspace_size(const poetx_layer_desc* desc, int64_t T, int32_t op) {
  if (check_wc(desc, T) != POETX_OK) return 0;
  Plan p;
  if (op == POETX_OP_FWD) plan_wc_fwd(p, desc, T);
  else if (op == POETX_OP_BWD) plan_wc_bwd(p, desc, T);
  else return 0;
  return p.off;
}

poetx_status poetx_wc_fwd(const poetx_layer_desc* desc, int64_t T, const void* X, const int32_t* perm_R,
                          const int32_t* perm_P, const void* Wt, const void* g_R, const void* g_P, void* Y, void* state,
                          void* ws, size_t ws_bytes, void* stream) {
  poetx_status st = check_wc(desc, T);
  if (st != POETX_OK) return st;
  if (!perm_R || !perm_P || !Wt || !g_R || !g_P || !state) return fail(POETX_E_NULL, "a required pointer is NULL");
  if (T > 0 && (!X || !Y)) return fail(POETX_E_NULL, "X and Y must be non-NULL");
  if (reinterpret_cast<uintptr_t>(state) % 256) return fail(POETX_E_WORKSPACE, "state must be 256-byte aligned");
  Plan p;
  plan_wc_fwd(p, desc, T);
  st = check_ws(ws, ws_bytes, p.off);
  if (st != POETX_OK) return st;
  Plan ps, pw;
  ps.base = reinterpret_cast<char*>(state);
  pw.base = reinterpret_cast<char*>(ws);
  const WcState S = plan_wc_state(ps, desc, T);
  const WcFwdWs w = plan_wc_fwd(pw, desc, T);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int m = desc->m, n = desc->n, b = desc->b, at = desc->act_dtype, rows = (int)T;
  const int64_t ldm = lead(m), ldn = lead(n);
  const char* gR0 = reinterpret_cast<const char*>(g_R);                       // Delta_R
  const char* gP1 = reinterpret_cast<const char*>(g_P) + g_slice(n, b, at);  // Delta_P^T
  const double es = (double)dt_size(at), mn = (double)m * n;
  const void* Wtt = has_weight_t(desc) ? reinterpret_cast<const char*>(Wt) + weight_t_offset(desc) : w.Wtt;
  if (!has_weight_t(desc))
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * mn * es, transpose(at, Wt, ldn, m, n, w.Wtt, ldm, s));
  // U^T = W~^T Diag(G_R)^T, U = Diag(G_R) W~
  PX_TIMED(POETX_KC_APPLY, 2.0 * n * sum_r2(m, b), 2.0 * mn * es + g_slice(m, b, at),
           apply(at, at, Wtt, ldm, n, m, b, at, gR0, nullptr, at, w.Ut, ldm, s));
  PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * mn * es, transpose(at, w.Ut, ldm, n, m, S.U, ldn, s));
  // V = W~ Diag(G_P), kept transposed for the R-side gradient
  PX_TIMED(POETX_KC_APPLY, 2.0 * m * sum_r2(n, b), 2.0 * mn * es + g_slice(n, b, at),
           apply(at, at, Wt, ldn, m, n, b, at, gP1, nullptr, at, w.V, ldn, s));
  PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * mn * es, transpose(at, w.V, ldn, m, n, S.Vt, ldm, s));
  // M = U Diag(G_P) = Diag(G_R) W~ Diag(G_P), and M^T for the contraction
  PX_TIMED(POETX_KC_APPLY, 2.0 * m * sum_r2(n, b), 2.0 * mn * es + g_slice(n, b, at),
           apply(at, at, S.U, ldn, m, n, b, at, gP1, nullptr, at, S.M, ldn, s));
  PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * mn * es, transpose(at, S.M, ldn, m, n, w.Mt, ldm, s));
  if (rows == 0) return POETX_OK;
  // Xt = X[:, perm_R] (kept for the weight gradient), Yt = Xt M, Y[:, perm_P] = Yt
  PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * m * es, permute(at, X, m, nullptr, perm_R, S.Xt, ldm, rows, m, m, s));
  PX_TIMED(POETX_KC_GEMM, 2.0 * rows * mn, es * (rows * (double)(m + n) + mn),
           gemm(at, at, S.Xt, ldm, at, w.Mt, ldm, false, rows, n, m, nullptr, at, w.Yt, ldn, s));
  PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * n * es, scatter(at, w.Yt, ldn, perm_P, Y, n, rows, n, s));
  return POETX_OK;
}

poetx_status poetx_wc_bwd(const poetx_layer_desc* desc, int64_t T, const void* dZ, const int32_t* perm_R,
                          const int32_t* perm_P, const void* g_R, const void* g_P, const float* q_R, const float* q_P,
                          const void* state, void* dX, float* dq_R, float* dq_P, void* ws, size_t ws_bytes,
                          void* stream) {
  poetx_status st = check_wc(desc, T);
  if (st != POETX_OK) return st;
  if (!perm_R || !perm_P || !g_R || !g_P || !q_R || !q_P || !state || !dq_R || !dq_P)
    return fail(POETX_E_NULL, "a required pointer is NULL");
  if (T > 0 && (!dZ || !dX)) return fail(POETX_E_NULL, "dZ and dX must be non-NULL");
  if (reinterpret_cast<uintptr_t>(state) % 256) return fail(POETX_E_WORKSPACE, "state must be 256-byte aligned");
  Plan p;
  plan_wc_bwd(p, desc, T);
  st = check_ws(ws, ws_bytes, p.off);
  if (st != POETX_OK) return st;
  Plan ps, pw;
  ps.base = reinterpret_cast<char*>(const_cast<void*>(state));
  pw.base = reinterpret_cast<char*>(ws);
  const WcState S = plan_wc_state(ps, desc, T);
  const WcBwdWs w = plan_wc_bwd(pw, desc, T);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int m = desc->m, n = desc->n, b = desc->b, at = desc->act_dtype, rows = (int)T;
  const int64_t ldm = lead(m), ldn = lead(n), ldT = round_up(T, 64);
  const int nbR = nblocks(m, b), nbP = nblocks(n, b);
  const double es = (double)dt_size(at), mn = (double)m * n;
  if (rows > 0) {
    // dZt = dZ[:, perm_P];  dXt = dZt M^T;  dX[:, perm_R] = dXt
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * n * es, permute(at, dZ, n, nullptr, perm_P, w.dZt, ldn, rows, n, n, s));
    PX_TIMED(POETX_KC_GEMM, 2.0 * rows * mn, es * (rows * (double)(m + n) + mn),
             gemm(at, at, w.dZt, ldn, at, S.M, ldn, false, rows, m, n, nullptr, at, w.dXt, ldm, s));
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * m * es, scatter(at, w.dXt, ldm, perm_R, dX, m, rows, m, s));
    // the weight gradient dM = Xt^T dZt, both operands transposed so that the tokens are contiguous
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * m * es, transpose(at, S.Xt, ldm, rows, m, w.Xtt, ldT, s));
    PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * rows * n * es, transpose(at, w.dZt, ldn, rows, n, w.dZtt, ldT, s));
    PX_TIMED(POETX_KC_GEMM, 2.0 * rows * mn, es * (rows * (double)(m + n) + mn),
             gemm(at, at, w.Xtt, ldT, at, w.dZtt, ldT, false, m, n, rows, nullptr, at, w.dM, ldn, s));
  } else {
    PX_HIP(fill_zero(w.dM, (size_t)m * ldn * dt_size(at), s));
  }
  PX_TIMED(POETX_KC_PERMUTE, 0, 2.0 * mn * es, transpose(at, w.dM, ldn, m, n, w.dMt, ldm, s));
  // block gradients: M = Diag(G_R) V gives dG_R = (dM V^T) on R's diagonal blocks, a sum over the n
  // columns; M = U Diag(G_P) gives dG_P = (U^T dM) on P's diagonal blocks, a sum over the m rows
  const CnpSide sR[2] = {{q_R, m, w.dMt, ldm, S.Vt, ldm}, {q_R, 0, nullptr, ldm, nullptr, ldm}};
  PX_TIMED(POETX_KC_DGRAD, 2.0 * n * sum_r2(m, b), 2.0 * mn * es + (4 + 2 * es) * sum_r2(m, b),
           block_grads(at, sR, n, b, w.cnp, 0, (int64_t)nbR + nbP, w.part, s));
  const CnpSide sP[2] = {{q_P, n, S.U, ldn, w.dM, ldn}, {q_P, 0, nullptr, ldn, nullptr, ldn}};
  PX_TIMED(POETX_KC_DGRAD, 2.0 * m * sum_r2(n, b), 2.0 * mn * es + (4 + 2 * es) * sum_r2(n, b),
           block_grads(at, sP, m, b, w.cnp, nbR, (int64_t)nbR + nbP, w.part, s));
  // CNP chain rule and skew projection, as in poetx_linear_bwd
  const float* qs[2] = {q_R, q_P};
  const int ds[2] = {m, n};
  float* dqs[2] = {dq_R, dq_P};
  PX_TIMED(POETX_KC_CNP, 12 * (sum_r3(m, b) + sum_r3(n, b)), cnp_grad_bytes(at, (int64_t)nbR + nbP, b),
           cnp_chain_batch(at, 2, qs, ds, b, w.cnp, dqs, s));
  return POETX_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// merging the outer factors of a chain into the weight
// ---------------------------------------------------------------------------
namespace {

struct FoldWs {
  int32_t *inv, *sigma;
  float *Xg, *Ag, *Wtr;
};
template <class P> FoldWs plan_fold(P& p, const poetx_layer_desc* d, int32_t side, const poetx_spo_desc* f) {
  const int de = spo_d_eff(f), dd = f->d, rows = side == 1 ? d->m : d->n;
  FoldWs w{};
  w.inv = p.template take<int32_t>((size_t)dd * 4);
  w.sigma = p.template take<int32_t>((size_t)de * 4);
  w.Xg = p.template take<float>((size_t)rows * lead(de) * 4);
  w.Ag = p.template take<float>((size_t)rows * lead(de) * 4);
  w.Wtr = side == 0 ? p.template take<float>((size_t)d->n * lead(d->m) * 4) : nullptr;
  return w;
}

poetx_status check_fold(const poetx_layer_desc* d, int32_t side, const poetx_spo_desc* f) {
  poetx_status st = check_desc(d);
  if (st != POETX_OK) return st;
  st = check_spo(f, 0);
  if (st != POETX_OK) return st;
  if (side != 0 && side != 1) return fail(POETX_E_SHAPE, "side must be 0 (R) or 1 (P)");
  if (f->d != (side == 1 ? d->n : d->m)) return fail(POETX_E_SHAPE, "the factor's d must be n (side 1) or m (side 0)");
  return POETX_OK;
}

}  // namespace

extern "C" {

size_t poetx_fold_workspace_size(const poetx_layer_desc* desc, int32_t side, const poetx_spo_desc* f) {
  if (check_fold(desc, side, f) != POETX_OK) return 0;
  Plan p;
  plan_fold(p, desc, side, f);
  return p.off;
}

poetx_status poetx_fold_factor(const poetx_layer_desc* desc, int32_t side, const poetx_spo_desc* f, const int32_t* idx,
                               const void* G, const int32_t* perm, float* W, int64_t ldw, void* ws, size_t ws_bytes,
                               void* stream) {
  poetx_status st = check_fold(desc, side, f);
  if (st != POETX_OK) return st;
  if (!idx || !G || !perm || !W) return fail(POETX_E_NULL, "idx, G, perm and W must be non-NULL");
  if (ldw < desc->n) return fail(POETX_E_SHAPE, "ldw < n");
  Plan p;
  plan_fold(p, desc, side, f);
  st = check_ws(ws, ws_bytes, p.off);
  if (st != POETX_OK) return st;
  Plan pq;
  pq.base = reinterpret_cast<char*>(ws);
  const FoldWs w = plan_fold(pq, desc, side, f);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int m = desc->m, n = desc->n, d = f->d, de = spo_d_eff(f), b = f->b, gt = f->act_dtype;
  // the factor in the weight's pre-merged order: index array sigma = perm^-1 o idx
  PX_HIP(inverse_perm(perm, d, w.inv, s));
  PX_HIP(compose_idx(w.inv, d, idx, de, w.sigma, s));
  // rows the factor acts on from the right: W's m rows (P side), or the n rows of W^T (R side, the
  // factor transposed: W <- F W is W^T <- W^T F^T)
  float* Rm = W;
  int64_t ldr = ldw;
  int rows = m;
  if (side == 0) {
    PX_HIP(transpose(F32, W, ldw, m, n, w.Wtr, lead(m), s));
    Rm = w.Wtr;
    ldr = lead(m);
    rows = n;
  }
  const char* gsl = reinterpret_cast<const char*>(G) + (side == 1 ? g_slice(de, b, gt) : 0);  // G (P) or G^T (R)
  PX_HIP(permute(F32, Rm, ldr, nullptr, w.sigma, w.Xg, lead(de), rows, d, de, s));
  PX_HIP(apply(F32, F32, w.Xg, lead(de), rows, de, b, gt, gsl, nullptr, F32, w.Ag, lead(de), s));
  if (f->kind == POETX_SPO_BLOCK)
    PX_HIP(scatter(F32, w.Ag, lead(de), w.sigma, Rm, ldr, rows, d, s));
  else
    PX_HIP(scatter_cols(F32, w.Ag, lead(de), rows, de, w.sigma, Rm, ldr, d, s));
  if (side == 0) PX_HIP(transpose(F32, w.Wtr, lead(m), n, m, W, ldw, s));
  return POETX_OK;
}

size_t poetx_store_workspace_size(const poetx_layer_desc* desc) {
  if (check_desc(desc) != POETX_OK) return 0;
  return (size_t)round_up((int64_t)desc->n * 4, 256);
}

poetx_status poetx_store_weight(const poetx_layer_desc* desc, const float* W, int64_t ldw, void* Wt, void* ws,
                                size_t ws_bytes, void* stream) {
  poetx_status st = check_desc(desc);
  if (st != POETX_OK) return st;
  if (!W || !Wt) return fail(POETX_E_NULL, "W and Wt must be non-NULL");
  if (ldw < desc->n) return fail(POETX_E_SHAPE, "ldw < n");
  st = check_ws(ws, ws_bytes, poetx_store_workspace_size(desc));
  if (st != POETX_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int m = desc->m, n = desc->n, wt = desc->w_dtype;
  uint32_t* amax = reinterpret_cast<uint32_t*>(ws);
  float* scale_t =
      wt == POETX_I8 ? reinterpret_cast<float*>(reinterpret_cast<char*>(Wt) + weight_scale_offset(desc)) : nullptr;
  if (wt == POETX_I8) {
    PX_HIP(fill_zero(amax, (size_t)n * 4, s));
    PX_HIP(col_absmax(W, ldw, m, n, amax, s));
  }
  PX_HIP(store_weight(W, ldw, m, n, wt, Wt, lead(n), amax, scale_t, s));
  PX_HIP(zero_cols(wt, Wt, lead(n), m, n, (int)lead(n), s));
  if (has_weight_t(desc))
    PX_HIP(transpose(wt, Wt, lead(n), m, n, reinterpret_cast<char*>(Wt) + weight_t_offset(desc), lead(m), s));
  return POETX_OK;
}

}  // extern "C"
