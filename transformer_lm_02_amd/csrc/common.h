// Internal helpers shared by the HIP kernels of libgpt_hip.so (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw bfloat16 storage
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- bf16 <-> fp32
// fp32 -> bf16 with round-to-nearest-even (NaN stays NaN): the gfx950
// conversion instruction v_cvt_pk_bf16_f32
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// two floats -> packed pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_convertvector((f32x2_cvt_t){lo, hi}, bf16x2_cvt_t));
}

// Activation storage: float (fp32 mode) or bf16_t (bf16 mode).
template <typename T> struct Act;
template <> struct Act<float> {
  __device__ __forceinline__ static float ld(const float* p) { return *p; }
  __device__ __forceinline__ static void st(float* p, float v) { *p = v; }
};
template <> struct Act<bf16_t> {
  __device__ __forceinline__ static float ld(const bf16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static void st(bf16_t* p, float v) { *p = f2bf(v); }
};
template <typename T> __device__ __forceinline__ float ldf(const T* p) { return Act<T>::ld(p); }
template <typename T> __device__ __forceinline__ void stf(T* p, float v) { Act<T>::st(p, v); }

// max that propagates NaN (IEEE maximum; v_maximum3_f32 on gfx950).  Unlike
// fmaxf it needs no canonicalisation of its inputs; for the finite and -inf
// values it is used on, both agree.
__device__ __forceinline__ float fmax_fast(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// tanh-approximate GELU and its derivative ("Let's Reproduce GPT-2 in One
// Read", the GELU check: GPT-2 uses the tanh form), c = sqrt(2/pi), a = 0.044715.
#define GELU_C 0.7978845608028654f
#define GELU_A 0.044715f
// Evaluated through the identity 0.5 (1 + tanh z) = 1 / (1 + e^(-2z)):
// gelu(u) = u s with s = 1 / (1 + 2^(-2 z log2 e)), z = c (u + a u^3), and
// gelu'(u) = s + 2 u s (1 - s) c (1 + 3 a u^2).  One hardware exponential and
// one hardware reciprocal (v_exp_f32, v_rcp_f32) per element; for u far
// below zero e^(-2z) overflows to inf and s to 0, the limits of both.
#define GELU_K0 (-2.0f * GELU_C * 1.4426950408889634f)
#define GELU_K1 (-2.0f * GELU_C * GELU_A * 1.4426950408889634f)
__device__ __forceinline__ float gelu_sig(float u, float u2) {
  const float e = __builtin_amdgcn_exp2f(u * fmaf(u2, GELU_K1, GELU_K0));
  return __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float gelu_f(float u) { return u * gelu_sig(u, u * u); }
__device__ __forceinline__ float gelu_grad_f(float u) {
  const float u2 = u * u;
  const float s = gelu_sig(u, u2);
  const float q = fmaf(u2, 6.0f * GELU_C * GELU_A, 2.0f * GELU_C);  // 2c (1 + 3 a u^2)
  return fmaf(u * s * (1.0f - s), q, s);
}
// both at once from one exponential: g = gelu(u), gp = gelu'(u)
__device__ __forceinline__ void gelu_both(float u, float& g, float& gp) {
  const float u2 = u * u;
  const float s = gelu_sig(u, u2);
  const float q = fmaf(u2, 6.0f * GELU_C * GELU_A, 2.0f * GELU_C);
  g = u * s;
  gp = fmaf(g * (1.0f - s), q, s);
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
