// Shared device/host definitions of the HIP encoder library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aenc {

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Element loads/stores for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// GELU in its exact form x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), with the
// complementary error function from Abramowitz & Stegun, Handbook of
// Mathematical Functions (1964), formula 7.1.26:
//   erfc(z) ~= (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
//   t = 1 / (1 + p z), z >= 0, absolute error <= 1.5e-7.
// For x >= 0, 1 + erf(x/sqrt2) = 2 - erfc(z); for x < 0 it is erfc(z), z = |x|/sqrt2.
__device__ __forceinline__ float gelu_erf(float x) {
  const float p = 0.3275911f;
  const float a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
              a4 = -1.453152027f, a5 = 1.061405429f;
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, z, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  // exp(-z^2) = 2^(-z^2 log2 e)
  const float e = __builtin_amdgcn_exp2f(-z * z * 1.44269504088896341f);
  const float q = poly * e;                       // erfc(z)
  const float one_plus_erf = x >= 0.0f ? 2.0f - q : q;
  return 0.5f * x * one_plus_erf;
}

// GELU for outputs rounded to bf16 (whose spacing is 2^-8 relative): no
// transcendental instructions. Phi(x) - 1/2 = x Q(x^2) on |x| <= 4.5, Q of
// degree 8 fitted to erf by iteratively reweighted least squares (towards the
// minimax fit); x is clamped to +-4.5 inside Phi. The GELU error is at most
// 1.1e-4 for |x| <= 8 and below 1.2e-5 |x| beyond.
__device__ __forceinline__ float gelu_bf16out(float x) {
  const float t = __builtin_amdgcn_fmed3f(x, -4.5f, 4.5f);
  const float u = t * t;
  float q = 3.805701934e-11f;
  q = fmaf(q, u, -4.002324250e-09f);
  q = fmaf(q, u, 1.846168800e-07f);
  q = fmaf(q, u, -4.959742000e-06f);
  q = fmaf(q, u, 8.727669774e-05f);
  q = fmaf(q, u, -1.076739514e-03f);
  q = fmaf(q, u, 9.729491547e-03f);
  q = fmaf(q, u, -6.624043733e-02f);
  q = fmaf(q, u, 3.988664746e-01f);
  return x * fmaf(t, q, 0.5f);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace aenc
