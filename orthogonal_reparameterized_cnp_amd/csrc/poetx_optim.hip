// Optimiser step on the packed skew parameters of many sides in one launch.
//
// The optimiser keeps state only for the packed strict upper triangle of each
// block's Q (zhichai.net POET-X blog, 第四斧 item 1); its update is Adam
// (Kingma & Ba 2015, bias-corrected moments) with decoupled weight decay
// (Loshchilov & Hutter 2019).  The step is elementwise and streams q, dq and
// the two moments once: 16 bytes read and 12 written per slot, HBM-bound.
#include <algorithm>
#include <cmath>

#include "common.h"
#include "poetx_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;                              // slots per thread per pass
constexpr int kPasses = 4;                           // passes per workgroup
constexpr int64_t kChunk = kThreads * kVec * kPasses;  // slots per workgroup

struct AdamTable {
  float* q[pxk::kAdamSidesPerLaunch];
  const float* g[pxk::kAdamSidesPerLaunch];
  float* m1[pxk::kAdamSidesPerLaunch];
  float* m2[pxk::kAdamSidesPerLaunch];
  int64_t len[pxk::kAdamSidesPerLaunch];
  int64_t first[pxk::kAdamSidesPerLaunch + 1];  // first workgroup of each side
  int count;
};

struct AdamK {
  float lr, b1, omb1, b2, omb2, eps, wd, c1, c2;  // omb = 1 - beta, c = 1 / (1 - beta^t)
};

PX_DEV void adam_one(float& q, float g, float& m, float& v, const AdamK& k) {
  m = k.b1 * m + k.omb1 * g;
  v = k.b2 * v + k.omb2 * (g * g);
  const float u = (m * k.c1) / (__builtin_sqrtf(v * k.c2) + k.eps);
  q = q - k.lr * (u + k.wd * q);
}

// One workgroup per kChunk slots of one side; V = 4 needs every pointer of the
// launch 16-byte aligned (checked by the launcher), V = 1 has no requirement.
template <int V>
__global__ __launch_bounds__(kThreads) void k_adam(AdamTable tab, AdamK k) {
  int s = 0;
  while (s + 1 < tab.count && (int64_t)blockIdx.x >= tab.first[s + 1]) ++s;
  const int64_t base = ((int64_t)blockIdx.x - tab.first[s]) * kChunk;
  const int64_t end = std::min<int64_t>(tab.len[s], base + kChunk);
  float* __restrict__ q = tab.q[s];
  const float* __restrict__ g = tab.g[s];
  float* __restrict__ m1 = tab.m1[s];
  float* __restrict__ m2 = tab.m2[s];
  if (V == 4) {
    for (int64_t i = base + (int64_t)threadIdx.x * 4; i < end; i += kThreads * 4) {
      if (i + 4 <= end) {
        f32x4_v qv = *reinterpret_cast<const f32x4_v*>(q + i);
        const f32x4_v gv = *reinterpret_cast<const f32x4_v*>(g + i);
        f32x4_v mv = *reinterpret_cast<const f32x4_v*>(m1 + i);
        f32x4_v vv = *reinterpret_cast<const f32x4_v*>(m2 + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float qe = qv[e], me = mv[e], ve = vv[e];
          adam_one(qe, gv[e], me, ve, k);
          qv[e] = qe;
          mv[e] = me;
          vv[e] = ve;
        }
        *reinterpret_cast<f32x4_v*>(q + i) = qv;
        *reinterpret_cast<f32x4_v*>(m1 + i) = mv;
        *reinterpret_cast<f32x4_v*>(m2 + i) = vv;
      } else {
        for (int64_t j = i; j < end; ++j) adam_one(q[j], g[j], m1[j], m2[j], k);
      }
    }
  } else {
    for (int64_t i = base + threadIdx.x; i < end; i += kThreads) adam_one(q[i], g[i], m1[i], m2[i], k);
  }
}

}  // namespace

namespace pxk {

hipError_t adam_batch(int count, const int64_t* len, float* const* q, const float* const* g, float* const* m1,
                      float* const* m2, const AdamHyper& hp, hipStream_t s) {
  AdamK k;
  k.lr = (float)hp.lr;
  k.b1 = (float)hp.beta1;
  k.omb1 = (float)(1.0 - hp.beta1);
  k.b2 = (float)hp.beta2;
  k.omb2 = (float)(1.0 - hp.beta2);
  k.eps = (float)hp.eps;
  k.wd = (float)hp.weight_decay;
  k.c1 = (float)(1.0 / (1.0 - std::pow(hp.beta1, (double)hp.t)));
  k.c2 = (float)(1.0 / (1.0 - std::pow(hp.beta2, (double)hp.t)));
  for (int s0 = 0; s0 < count; s0 += kAdamSidesPerLaunch) {
    AdamTable tab{};
    bool aligned = true;
    int64_t wgs = 0;
    tab.count = 0;
    for (int i = s0; i < count && i < s0 + kAdamSidesPerLaunch; ++i) {
      if (len[i] == 0) continue;
      const int c = tab.count++;
      tab.q[c] = q[i];
      tab.g[c] = g[i];
      tab.m1[c] = m1[i];
      tab.m2[c] = m2[i];
      tab.len[c] = len[i];
      tab.first[c] = wgs;
      wgs += (len[i] + kChunk - 1) / kChunk;
      for (const void* p : {(const void*)q[i], (const void*)g[i], (const void*)m1[i], (const void*)m2[i]})
        aligned = aligned && reinterpret_cast<uintptr_t>(p) % 16 == 0;
    }
    if (tab.count == 0) continue;
    tab.first[tab.count] = wgs;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    if (aligned)
      k_adam<4><<<(unsigned)wgs, kThreads, 0, s>>>(tab, k);
    else
      k_adam<1><<<(unsigned)wgs, kThreads, 0, s>>>(tab, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pxk
