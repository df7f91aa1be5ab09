// Internal helpers shared by the HIP kernels of libgpt_hip.so (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// The 16-bit activation format is fixed per compilation: every kernel source
// and the host orchestration are compiled twice, once for bfloat16 (namespace
// b16) and once, with GPT_HALF_FP16 defined, for IEEE binary16 (namespace
// f16).  Kernels name the format only through h16_t and the helpers below.
#ifdef GPT_HALF_FP16
#define HALF_NS f16
typedef _Float16 h16_el;
#define H16_NEG_INF 0xfc00u  // binary16 -inf
#else
#define HALF_NS b16
typedef __bf16 h16_el;
#define H16_NEG_INF 0xff80u  // bfloat16 -inf
#endif

namespace HALF_NS {

typedef uint16_t h16_t;  // raw 16-bit storage of the build's format
typedef h16_el h16x8_t __attribute__((ext_vector_type(8)));
typedef h16_el h16x4_t __attribute__((ext_vector_type(4)));
typedef h16_el h16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- 16-bit <-> fp32
// fp32 -> 16-bit with round-to-nearest-even; NaN stays NaN, and in binary16 a
// value beyond the largest finite one becomes inf (so that an overflow shows
// up in the gradient norm instead of saturating silently).
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h16_t f2h(float f) { return __builtin_bit_cast(h16_t, (h16_el)f); }
// two floats -> packed pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_cvt_t){lo, hi}, h16x2_t));
}
#ifdef GPT_HALF_FP16
__device__ __forceinline__ float h2f(h16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ float h_lo(uint32_t w) { return h2f((h16_t)(w & 0xffffu)); }
__device__ __forceinline__ float h_hi(uint32_t w) { return h2f((h16_t)(w >> 16)); }
// the binary16 builtins take __fp16 vectors
typedef __fp16 fp16v8_t __attribute__((__vector_size__(8 * sizeof(__fp16))));
typedef __fp16 fp16v4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __fp16 fp16v2_t __attribute__((__vector_size__(2 * sizeof(__fp16))));
#define MFMA_32X32X16(a, b, c)                                                          \
  __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(fp16v8_t, (a)),             \
                                         __builtin_bit_cast(fp16v8_t, (b)), (c), 0, 0, 0)
#define DS_READ_TR16_B64(p)                                                             \
  __builtin_bit_cast(h16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16(                  \
                                  (__attribute__((address_space(3))) fp16v4_t*)(p)))
#define FDOT2(a, b, c)                                                                  \
  __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16v2_t, (a)), __builtin_bit_cast(fp16v2_t, (b)), \
                         (c), false)
#else
// a bfloat16 is the top half of an fp32
__device__ __forceinline__ float h2f(h16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ float h_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float h_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
#define MFMA_32X32X16(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_bf16((a), (b), (c), 0, 0, 0)
#define DS_READ_TR16_B64(p) __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p)
#define FDOT2(a, b, c) __builtin_amdgcn_fdot2_f32_bf16((a), (b), (c), false)
#endif

// Activation storage: float (fp32 mode) or h16_t (16-bit modes).
template <typename T> struct Act;
template <> struct Act<float> {
  __device__ __forceinline__ static float ld(const float* p) { return *p; }
  __device__ __forceinline__ static void st(float* p, float v) { *p = v; }
};
template <> struct Act<h16_t> {
  __device__ __forceinline__ static float ld(const h16_t* p) { return h2f(*p); }
  __device__ __forceinline__ static void st(h16_t* p, float v) { *p = f2h(v); }
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
// Sum over the 64 lanes without LDS: rotations by 8, 4, 2 and 1 inside each
// row of 16 lanes (DPP), then row pairs and half-waves exchanged with the
// gfx950 permlane16/permlane32 swaps.  Every step adds a lane's partial to
// one that covers the same lanes as its partner's, so all 64 lanes end with
// the same value, bit for bit.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0x128>(v);  // row_ror:8
  v += dpp_f32<0x124>(v);  // row_ror:4
  v += dpp_f32<0x122>(v);  // row_ror:2
  v += dpp_f32<0x121>(v);  // row_ror:1
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
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

// ---------------------------------------------------------------- dropout
// Masks from Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11): ten rounds of the bijection that
// multiplies words 0 and 2 by two constants and mixes the halves of the
// products with words 1 and 3 and the key; the key grows by two Weyl
// increments between rounds.  Counter-based, so a backward kernel regenerates
// the forward's mask from the element's coordinates alone.
//
// Element (row, col) of a site's matrix (for attention, query row and key
// column of head bh = b * n_head + h) is kept when word col % 4 of
// philox(counter = {col / 4, row, site_word + bh, step}, key = seed) is at
// least thresh; a kept value is multiplied by scale = 1 / (1 - p).
struct Drop {
  uint32_t k0 = 0, k1 = 0;  // the 64-bit seed
  uint32_t step = 0;        // counter word 3: tells forward calls apart
  uint32_t site = 0;        // counter word 2: site * 2^24 (attention adds bh)
  uint32_t thresh = 0;      // 0: no dropout
  float scale = 1.f;
};
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // each 32 x 32 -> 64-bit product is one v_mad_u64_u32 giving both halves
    // (1.4x the rate of separate v_mul_hi_u32 / v_mul_lo_u32, measured)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    c0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    c1 = (uint32_t)p1;
    c2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c3 = (uint32_t)p0;
  }
  return make_uint4(c0, c1, c2, c3);
}
// multipliers (0 or scale) of columns 4g .. 4g+3 of one row
__device__ __forceinline__ float4 drop4(const Drop& d, uint32_t g, uint32_t row, uint32_t bh) {
  const uint4 w = philox4x32_10(g, row, d.site + bh, d.step, d.k0, d.k1);
  return make_float4(w.x >= d.thresh ? d.scale : 0.f, w.y >= d.thresh ? d.scale : 0.f,
                     w.z >= d.thresh ? d.scale : 0.f, w.w >= d.thresh ? d.scale : 0.f);
}
// multiplier of one element
__device__ __forceinline__ float drop1(const Drop& d, uint32_t col, uint32_t row, uint32_t bh) {
  const uint4 w = philox4x32_10(col >> 2, row, d.site + bh, d.step, d.k0, d.k1);
  const uint32_t x = (col & 2) ? ((col & 1) ? w.w : w.z) : ((col & 1) ? w.y : w.x);
  return x >= d.thresh ? d.scale : 0.f;
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Non-temporal stores, for outputs no kernel reads soon: written through L2
// without keeping the lines, they leave L2 to data that is read again.
typedef unsigned int ntu4_t __attribute__((ext_vector_type(4)));
typedef unsigned int ntu2_t __attribute__((ext_vector_type(2)));
typedef float ntf4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt(void* p, uint4 v) {
  const ntu4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (ntu4_t*)p);
}
__device__ __forceinline__ void st_nt(void* p, uint2 v) {
  const ntu2_t w = {v.x, v.y};
  __builtin_nontemporal_store(w, (ntu2_t*)p);
}
__device__ __forceinline__ void st_nt(float4* p, float4 v) {
  const ntf4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (ntf4_t*)p);
}

}  // namespace HALF_NS
