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
// Read", the GELU check: GPT-2 uses the tanh form).  tanh(y) is evaluated as
// 1 - 2/(exp(2y)+1), which is exact at both tails.
#define GELU_C 0.7978845608028654f
#define GELU_A 0.044715f
__device__ __forceinline__ float tanh_fast(float y) {
  float e = __expf(2.0f * y);
  return 1.0f - 2.0f / (e + 1.0f);
}
__device__ __forceinline__ float gelu_f(float u) {
  float t = tanh_fast(GELU_C * (u + GELU_A * u * u * u));
  return 0.5f * u * (1.0f + t);
}
__device__ __forceinline__ float gelu_grad_f(float u) {
  float t = tanh_fast(GELU_C * (u + GELU_A * u * u * u));
  return 0.5f * (1.0f + t) + 0.5f * u * (1.0f - t * t) * GELU_C * (1.0f + 3.0f * GELU_A * u * u);
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
