// Shared device helpers for libpoetx (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

#define PX_DEV __device__ __forceinline__

PX_DEV float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bfloat16, round to nearest, ties to even: the conversion
// instruction of gfx950 (v_cvt_pk_bf16_f32), one instruction per pair
PX_DEV bf16_t f2bf(float f) {
  const __bf16 h = (__bf16)f;
  bf16_t u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
// (a, b) -> bfloat16 pair, a in the low half
PX_DEV uint32_t f2bf2(float a, float b) {
  const bf16x2_v h = __builtin_convertvector((f32x2_v){a, b}, bf16x2_v);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// element conversions used by the operand loaders
template <typename D, typename S> struct Cvt;
template <> struct Cvt<bf16_t, bf16_t> { static PX_DEV bf16_t f(bf16_t x) { return x; } };
template <> struct Cvt<float, float> { static PX_DEV float f(float x) { return x; } };
template <> struct Cvt<float, bf16_t> { static PX_DEV float f(bf16_t x) { return bf2f(x); } };
template <> struct Cvt<bf16_t, float> { static PX_DEV bf16_t f(float x) { return f2bf(x); } };
// int8 codes are exact in bfloat16 (|code| <= 127)
template <> struct Cvt<bf16_t, int8_t> { static PX_DEV bf16_t f(int8_t x) { return f2bf((float)x); } };
template <> struct Cvt<float, int8_t> { static PX_DEV float f(int8_t x) { return (float)x; } };

template <typename T> PX_DEV float to_f32(T x);
template <> PX_DEV float to_f32<float>(float x) { return x; }
template <> PX_DEV float to_f32<bf16_t>(bf16_t x) { return bf2f(x); }
template <> PX_DEV float to_f32<int8_t>(int8_t x) { return (float)x; }

template <typename T> PX_DEV T from_f32(float x);
template <> PX_DEV float from_f32<float>(float x) { return x; }
template <> PX_DEV bf16_t from_f32<bf16_t>(float x) { return f2bf(x); }

PX_DEV int64_t packed_slot(int i, int j, int b) {
  // row-major strict upper triangle of a b x b block, i < j
  return (int64_t)i * b - ((int64_t)i * (i + 1)) / 2 + (j - i - 1);
}

// value of Q[i][j] of a block of size r (stride b) from its packed slots
PX_DEV float skew_at(const float* qk, int i, int j, int r, int b) {
  if (i >= r || j >= r || i == j) return 0.f;
  return i < j ? qk[packed_slot(i, j, b)] : -qk[packed_slot(j, i, b)];
}
