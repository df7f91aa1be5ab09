// Causal multi-head self-attention, forward and backward.
//
// What is computed is the manual path of "nanoGPT" (stanleyjacob.dev), Part V
// Deep dive 1: per head, softmax(q k^T / sqrt(hs)) with the entries above the
// diagonal at -inf, times v; q, k, v are the column blocks of the fused
// c_attn output, head h at columns h*hs.  The 16-bit kernels reach the same
// result tile by tile with an online softmax and never store the T x T
// matrix ("Let's reproduce GPT-2 (124M)", chapter "Flash Attention, 96ms"):
// the forward keeps the row logsumexp, the backward recomputes the
// probabilities from it.
//
// 16-bit kernels (head width 64) use v_mfma_f32_32x32x16_bf16 (_f16 for binary16).  The forward
// computes S^T = K Q^T so that one lane owns one query row: its running max
// and sum stay in the lane, and the probabilities in the accumulator
// registers are directly the B operand of O^T = V^T P^T.  The backward is two
// kernels: dK/dV per key block (iterating over query blocks) and dQ per
// query block (iterating over key blocks), so no atomics are needed.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace HALF_NS {

#define LOG2E 1.4426950408889634f
#define LN2 0.6931471805599453f

// ================================================================ generic (fp32 mode)
template <typename T>
__global__ void attn_fwd_generic(const T* __restrict__ qkv, T* __restrict__ out,
                                 float* __restrict__ lse, int B, int Tn, int H, int C, Drop dr) {
  const int hs = C / H;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= Tn) return;
  const int64_t ld = 3 * (int64_t)C;
  const T* Q = qkv + ((int64_t)b * Tn + q) * ld + h * hs;
  const float scale = 1.0f / sqrtf((float)hs);
  float o[128];
  for (int c = 0; c < hs; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= q; ++j) {
    const T* K = qkv + ((int64_t)b * Tn + j) * ld + C + h * hs;
    const T* V = K + C;
    float s = 0.f;
    for (int c = 0; c < hs; ++c) s += ldf(Q + c) * ldf(K + c);
    s *= scale;
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn), p = expf(s - mn);
    l = l * alpha + p;  // the normaliser sums the probabilities before dropout
    const float pz = dr.thresh ? p * drop1(dr, (uint32_t)j, (uint32_t)q, (uint32_t)bh) : p;
    for (int c = 0; c < hs; ++c) o[c] = o[c] * alpha + pz * ldf(V + c);
    m = mn;
  }
  T* O = out + ((int64_t)b * Tn + q) * C + h * hs;
  for (int c = 0; c < hs; ++c) stf(O + c, o[c] / l);
  lse[(int64_t)bh * Tn + q] = m + logf(l);
}

// D[bh][q] = sum_c dO[q][c] * O[q][c]  (= rowsum(P * dP)); with L2 given,
// also L2[bh][q] = lse[bh][q] * log2(e) (the exponent offset of the 16-bit
// backward kernels)
template <typename T>
__global__ void attn_bwd_dot(const T* __restrict__ out, const T* __restrict__ dout,
                             const float* __restrict__ lse, float* __restrict__ D,
                             float* __restrict__ L2, int B, int Tn, int H, int C) {
  const int hs = C / H;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)B * H * Tn) return;
  const int q = row % Tn, bh = row / Tn, b = bh / H, h = bh % H;
  const T* O = out + ((int64_t)b * Tn + q) * C + h * hs;
  const T* dO = dout + ((int64_t)b * Tn + q) * C + h * hs;
  float s = 0.f;
  for (int c = lane; c < hs; c += 64) s += ldf(O + c) * ldf(dO + c);
  s = wave_sum(s);
  if (lane == 0) {
    D[row] = s;
    if (L2) L2[row] = lse[row] * LOG2E;
  }
}

template <typename T>
__global__ void attn_bwd_dq_generic(const T* __restrict__ qkv, const float* __restrict__ lse,
                                    const float* __restrict__ D, const T* __restrict__ dout,
                                    T* __restrict__ dqkv, int B, int Tn, int H, int C, Drop dr) {
  const int hs = C / H;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= Tn) return;
  const int64_t ld = 3 * (int64_t)C;
  const T* Q = qkv + ((int64_t)b * Tn + q) * ld + h * hs;
  const T* dO = dout + ((int64_t)b * Tn + q) * C + h * hs;
  const float scale = 1.0f / sqrtf((float)hs);
  const float L = lse[(int64_t)bh * Tn + q], Dq = D[(int64_t)bh * Tn + q];
  float dq[128];
  for (int c = 0; c < hs; ++c) dq[c] = 0.f;
  for (int j = 0; j <= q; ++j) {
    const T* K = qkv + ((int64_t)b * Tn + j) * ld + C + h * hs;
    const T* V = K + C;
    float s = 0.f, dp = 0.f;
    for (int c = 0; c < hs; ++c) {
      s += ldf(Q + c) * ldf(K + c);
      dp += ldf(dO + c) * ldf(V + c);
    }
    const float p = expf(s * scale - L);
    if (dr.thresh) dp *= drop1(dr, (uint32_t)j, (uint32_t)q, (uint32_t)bh);
    const float ds = p * (dp - Dq);
    for (int c = 0; c < hs; ++c) dq[c] += ds * ldf(K + c);
  }
  T* dQ = dqkv + ((int64_t)b * Tn + q) * ld + h * hs;
  for (int c = 0; c < hs; ++c) stf(dQ + c, dq[c] * scale);
}

template <typename T>
__global__ void attn_bwd_dkdv_generic(const T* __restrict__ qkv, const float* __restrict__ lse,
                                      const float* __restrict__ D, const T* __restrict__ dout,
                                      T* __restrict__ dqkv, int B, int Tn, int H, int C, Drop dr) {
  const int hs = C / H;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= Tn) return;
  const int64_t ld = 3 * (int64_t)C;
  const T* K = qkv + ((int64_t)b * Tn + j) * ld + C + h * hs;
  const T* V = K + C;
  const float scale = 1.0f / sqrtf((float)hs);
  float dk[128], dv[128];
  for (int c = 0; c < hs; ++c) dk[c] = dv[c] = 0.f;
  for (int q = j; q < Tn; ++q) {
    const T* Q = qkv + ((int64_t)b * Tn + q) * ld + h * hs;
    const T* dO = dout + ((int64_t)b * Tn + q) * C + h * hs;
    float s = 0.f, dp = 0.f;
    for (int c = 0; c < hs; ++c) {
      s += ldf(Q + c) * ldf(K + c);
      dp += ldf(dO + c) * ldf(V + c);
    }
    const float p = expf(s * scale - lse[(int64_t)bh * Tn + q]);
    const float z = dr.thresh ? drop1(dr, (uint32_t)j, (uint32_t)q, (uint32_t)bh) : 1.f;
    const float ds = p * (z * dp - D[(int64_t)bh * Tn + q]);
    for (int c = 0; c < hs; ++c) {
      dv[c] += p * z * ldf(dO + c);
      dk[c] += ds * ldf(Q + c);
    }
  }
  T* dK = dqkv + ((int64_t)b * Tn + j) * ld + C + h * hs;
  T* dV = dK + C;
  for (int c = 0; c < hs; ++c) {
    stf(dK + c, dk[c] * scale);
    stf(dV + c, dv[c]);
  }
}

// ================================================================ 16-bit flash kernels (hs = 64)
// Tiles of 64 rows x 64 16-bit (one row per key or query, head dims
// contiguous) go from HBM into LDS with buffer loads in LDS mode, through a
// ring of NS stages.  A tile keeps its memory layout; the 16-byte chunk c of
// row r is stored at position c ^ f(r), f(r) = 4*((r>>1)&1) + ((r>>2)&3),
// which makes both access patterns conflict-free: plain 16-byte reads of 16
// consecutive rows (an MFMA operand whose k index is the head dimension) and
// the gfx950 transposing read ds_read_b64_tr_b16 of 4 rows x 32 columns (an
// operand whose k index is the key or query).
#define AS3(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ int tsw(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// This wave's share (2 of 8 loads of 1 KB) of a 64 x 64 tile whose row 0 is
// global row `row0` of a buffer with row pitch `ld` elements (rows past the
// buffer's end read as zero).
__device__ __forceinline__ void tile_dma(__amdgpu_buffer_rsrc_t rs, h16_t* lds, int row0, int ld,
                                         int col0, int lane, int wave) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = 2 * wave + i;
    const int r = 8 * q + (lane >> 3), c = (lane & 7) ^ tsw(r);
    const uint32_t off = (uint32_t)(((int64_t)(row0 + r) * ld + col0 + 8 * c) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, AS3(lds + q * 512), 16, off, 0, 0, 0);
  }
}
// 32x32x16 MFMA operand with rows = tile rows base..base+31 and k = head dims
// 16ks + 8(lane/32) + 0..7 (plain read)
__device__ __forceinline__ h16x8_t frag_hd(const h16_t* t, int base, int ks, int lane) {
  const int r = base + (lane & 31), c = 2 * ks + (lane >> 5);
  return *(const h16x8_t*)(t + r * 64 + ((c ^ tsw(r)) << 3));
}
// 32x32x16 MFMA operand with rows = head dims col0..col0+31 and k = tile rows
// 16ks + 8(j/4) + 4(lane/32) + j%4 (j = 0..7), the order in which a 32x32
// accumulator holds its rows (transposing read)
__device__ __forceinline__ h16x8_t frag_rows(const h16_t* __restrict__ t, int col0, int ks, int lane) {
  const int G = lane >> 4, u = lane & 15;
  const int col = col0 + 16 * (G & 1) + 4 * (u & 3);
  const int r0 = 16 * ks + 4 * (G >> 1) + (u >> 2);
  const int c = col >> 3;
  const h16_t* pa = t + r0 * 64 + ((c ^ tsw(r0)) << 3) + (col & 7);
  const h16_t* pb = t + (r0 + 8) * 64 + ((c ^ tsw(r0 + 8)) << 3) + (col & 7);
  const h16x4_t lo = DS_READ_TR16_B64((__attribute__((address_space(3))) h16x4_t*)pa);
  const h16x4_t hi = DS_READ_TR16_B64((__attribute__((address_space(3))) h16x4_t*)pb);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// 8 accumulator values (registers 8s..8s+7 of a 32x32 tile) -> 16-bit operand
__device__ __forceinline__ h16x8_t pack_acc(const f32x16_t& a, int s) {
  uint4 v;
  v.x = pack2h(a[8 * s + 0], a[8 * s + 1]);
  v.y = pack2h(a[8 * s + 2], a[8 * s + 3]);
  v.z = pack2h(a[8 * s + 4], a[8 * s + 5]);
  v.w = pack2h(a[8 * s + 6], a[8 * s + 7]);
  return *(h16x8_t*)&v;
}
__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// 2^x by the hardware instruction; every argument here is <= 0 or -inf, so
// no range reduction is needed (results below 2^-126 flush to zero)
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
#define MFMA32(a, b, c) MFMA_32X32X16(a, b, c)
// row offset inside a 32x32 accumulator tile for register r of this lane
#define ACC_ROW(r, lane) (8 * ((r) >> 2) + 4 * ((lane) >> 5) + ((r) & 3))
// ring depths (stages of 64 rows in LDS) of the three kernels
#ifndef FLASH_FWD_NS
#define FLASH_FWD_NS 3
#endif
#ifndef FLASH_DKDV_NS
#define FLASH_DKDV_NS 3
#endif
#ifndef FLASH_DQ_NS
#define FLASH_DQ_NS 3
#endif
#define TILE_ELEMS 4096

template <int N>
using Slot = std::integral_constant<int, N>;
// f(i + S, Slot<S>) for S = S0 .. NS-1 while i + S < n: the ring loop
// unrolled by its depth, so every slot index is a compile-time constant
template <int S, int NS, typename F>
__device__ __forceinline__ void slot_steps(int i, int n, F& f) {
  if constexpr (S < NS) {
    if (i + S < n) {
      f(i + S, Slot<S>());
      slot_steps<S + 1, NS>(i, n, f);
    }
  }
}

// ---------------------------------------------------------------- forward
// grid: (T/128 query blocks, heaviest first) x (B*H); 4 waves x 32 query
// rows.  S^T = K Q^T puts one query per lane, so the running max and sum are
// the lane's own; P^T in the accumulator registers is directly the B operand
// of O^T = V^T P^T.  The key loop is unrolled by the ring depth so that every
// LDS address is a per-lane base plus an immediate offset.
// DROP: dropout of the probabilities (Philox words of 4 consecutive keys per
// call); the kept/dropped bits are written to dmask for the backward, one
// 32-bit word per (query, 64-key block, lane half): bit 16t + r is register
// r of accumulator tile t, i.e. key kv0 + 32t + 8(r/4) + 4(lane/32) + r%4,
// at dmask[((bh * nkb + kb) * 2 + lane/32) * T + query].
template <int FLASH_NS, bool DROP>
__global__ __launch_bounds__(256, 2) void flash_fwd_kernel(const h16_t* __restrict__ qkv,
                                                           h16_t* __restrict__ out,
                                                           float* __restrict__ lse, int B, int Tn,
                                                           int H, int C, Drop dr,
                                                           uint32_t* __restrict__ dmask) {
  __shared__ __attribute__((aligned(1024))) h16_t ring[FLASH_NS][2][TILE_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int nqb = (Tn + 127) / 128;
  const int qb = nqb - 1 - (int)(blockIdx.x / (B * H));
  const int bh = blockIdx.x % (B * H), b = bh / H, h = bh % H;
  const int q0 = qb * 128, qw = q0 + 32 * wave;
  const int ld = 3 * C;
  const h16_t* base = qkv + (int64_t)b * Tn * ld;
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(base, (uint32_t)((int64_t)Tn * ld * 2));
  const int my_q = qw + (lane & 31);

  h16x8_t fq[4];  // Q^T operand: lane holds Q[my_q][16ks + 8(lane/32) + 0..7]
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (my_q < Tn) v = *(const uint4*)(base + (int64_t)my_q * ld + h * 64 + 16 * ks + 8 * (lane >> 5));
    fq[ks] = *(h16x8_t*)&v;
  }
  const float sc = LOG2E * 0.125f;  // log2(e) / sqrt(64)
  const h16x2_t ones = {(h16_el)1.0f, (h16_el)1.0f};
  float m = -INFINITY, l = 0.f;     // m in log2 units of the scaled scores
  f32x16_t o[2] = {zero16(), zero16()};
  const int nkv = (min(Tn, q0 + 128) + 63) / 64;
#pragma unroll
  for (int st = 0; st < FLASH_NS - 1; ++st)
    if (st < nkv) {
      tile_dma(rs, ring[st][0], 64 * st, ld, C + h * 64, lane, wave);
      tile_dma(rs, ring[st][1], 64 * st, ld, 2 * C + h * 64, lane, wave);
    }
  auto step = [&](int kb, auto slot) {
    constexpr int SL = decltype(slot)::value;
    if (kb + FLASH_NS - 2 < nkv) vm_wait_barrier<(FLASH_NS - 2) * 4>();
    else vm_wait_barrier<0>();
    if (kb + FLASH_NS - 1 < nkv) {
      constexpr int NX = (SL + FLASH_NS - 1) % FLASH_NS;
      const int r0 = 64 * (kb + FLASH_NS - 1);
      tile_dma(rs, ring[NX][0], r0, ld, C + h * 64, lane, wave);
      tile_dma(rs, ring[NX][1], r0, ld, 2 * C + h * 64, lane, wave);
    }
    const h16_t* tK = ring[SL][0];
    const h16_t* tV = ring[SL][1];
    const int kv0 = kb * 64;
    if (kv0 > qw + 31) return;  // every key of the block is after this wave's queries
    f32x16_t s[2] = {zero16(), zero16()};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) s[t] = MFMA32(frag_hd(tK, 32 * t, ks, lane), fq[ks], s[t]);
    if (kv0 + 63 > qw || kv0 + 64 > Tn) {
      // keys kv0 + 32t + ACC_ROW(r) past the lane's query or the sequence end
      const int lim = min(my_q, Tn - 1) - kv0 - 4 * (lane >> 5);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[t][r] = (32 * t + 8 * (r >> 2) + (r & 3)) > lim ? -INFINITY : s[t][r];
    }
    float mb = fmax_fast(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mb = fmax_fast(fmax_fast(mb, s[0][r]), s[1][r]);
    {
      // the other half-wave's value: lanes l and l^32 hold one query's two
      // halves of the keys; the swap leaves lane l's pair in both results
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mb), __float_as_uint(mb), false, false);
      mb = fmax_fast(__uint_as_float(pr[0]), __uint_as_float(pr[1])) * sc;
    }
    // The reference point m of the exponentials moves only when some
    // query's block maximum exceeds it by more than 8 (log2 units): the
    // probabilities then stay below 2^8 and the accumulator is rescaled
    // rarely.  Every lane that moves takes its exact new maximum.
    if (__builtin_amdgcn_ballot_w64(mb > m + 8.0f)) {
      const float mn = fmaxf(m, mb);
      const float alpha = fexp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ht][r] *= alpha;
      m = mn;
    }
    const float nm = -m;
    uint32_t mw = 0;  // DROP: this block's kept bits
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        uint32_t w[4];
        float pe[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pe[2 * j] = fexp2(fmaf(s[t][8 * ss + 2 * j], sc, nm));
          pe[2 * j + 1] = fexp2(fmaf(s[t][8 * ss + 2 * j + 1], sc, nm));
          w[j] = pack2h(pe[2 * j], pe[2 * j + 1]);
          // the row sum adds the probabilities as rounded for the product
          // (before dropout: the normaliser is the softmax's)
          l = FDOT2(__builtin_bit_cast(h16x2_t, w[j]), ones, l);
        }
        if constexpr (DROP) {
          // keys kv0 + 32t + 16ss + 4(lane/32) + 0..3 (registers 8ss..8ss+3),
          // then + 8 (registers 8ss+4..8ss+7)
          const uint32_t g = (uint32_t)(kv0 + 32 * t + 16 * ss + 4 * (lane >> 5)) >> 2;
          const float4 za = drop4(dr, g, (uint32_t)my_q, (uint32_t)bh);
          const float4 zb = drop4(dr, g + 2, (uint32_t)my_q, (uint32_t)bh);
          w[0] = pack2h(pe[0] * za.x, pe[1] * za.y);
          w[1] = pack2h(pe[2] * za.z, pe[3] * za.w);
          w[2] = pack2h(pe[4] * zb.x, pe[5] * zb.y);
          w[3] = pack2h(pe[6] * zb.z, pe[7] * zb.w);
          const uint32_t bits = (za.x > 0.f ? 1u : 0u) | (za.y > 0.f ? 2u : 0u) |
                                (za.z > 0.f ? 4u : 0u) | (za.w > 0.f ? 8u : 0u) |
                                (zb.x > 0.f ? 16u : 0u) | (zb.y > 0.f ? 32u : 0u) |
                                (zb.z > 0.f ? 64u : 0u) | (zb.w > 0.f ? 128u : 0u);
          mw |= bits << (16 * t + 8 * ss);
        }
        const uint4 wv = make_uint4(w[0], w[1], w[2], w[3]);
        const h16x8_t pb = __builtin_bit_cast(h16x8_t, wv);
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
          o[ht] = MFMA32(frag_rows(tV, 32 * ht, 2 * t + ss, lane), pb, o[ht]);
      }
    if constexpr (DROP) {
      if (my_q < Tn) {
        const int nkb = (Tn + 63) / 64;
        dmask[((int64_t)(bh * nkb + kb) * 2 + (lane >> 5)) * Tn + my_q] = mw;
      }
    }
  };
  for (int kb = 0; kb < nkv; kb += FLASH_NS) slot_steps<0, FLASH_NS>(kb, nkv, step);
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = 1.0f / lt;
  if (my_q < Tn) {
    h16_t* O = out + ((int64_t)b * Tn + my_q) * C + h * 64;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int hd = 32 * ht + 8 * rg + 4 * (lane >> 5);
        uint2 v;
        v.x = pack2h(o[ht][4 * rg + 0] * inv, o[ht][4 * rg + 1] * inv);
        v.y = pack2h(o[ht][4 * rg + 2] * inv, o[ht][4 * rg + 3] * inv);
        *(uint2*)(O + hd) = v;
      }
    if (lane < 32) lse[(int64_t)bh * Tn + my_q] = (m + __log2f(lt)) * LN2;
  }
}

// ---------------------------------------------------------------- backward: dK, dV
// grid: (T/128 key blocks) x (B*H); 4 waves x 32 keys; query blocks of 64 from
// the diagonal on.  S = Q K^T and dP = dO V^T put one key per lane; P^T and
// dS^T are then the A operands of dV += P^T dO and dK += dS^T Q, whose B
// operands are transposing reads of the dO and Q tiles.  Dg holds
// -rowsum(dO * O) at [0, B*H*T) and the row logsumexp times log2(e) at
// [B*H*T, 2*B*H*T).
// DROP: each stage also brings the forward's kept bits of its 64 queries for
// this workgroup's 128 keys (4 runs of 64 words: key block 0/1 x lane half
// 0/1), one run per wave, into the second quarter of that wave's small slot.
template <int FLASH_NS, bool DROP>
__global__ __launch_bounds__(256, 2) void flash_bwd_dkdv_kernel(
    const h16_t* __restrict__ qkv, const float* __restrict__ Dg, const h16_t* __restrict__ dout,
    h16_t* __restrict__ dqkv, float* __restrict__ cs_part, int B, int Tn, int H, int C, Drop dr,
    const uint32_t* __restrict__ dmask) {
  // per stage: Q tile, dO tile, 4 small slots (wave 0: scaled logsumexp, wave 1: D)
  __shared__ __attribute__((aligned(1024))) h16_t ring[FLASH_NS][2 * TILE_ELEMS + 4 * 512];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int bh = blockIdx.x % (B * H), b = bh / H, h = bh % H;
  const int kblk = blockIdx.x / (B * H);
  const int k0 = kblk * 128, kw = k0 + 32 * wave;
  const int ld = 3 * C;
  const int64_t bht = (int64_t)B * H * Tn;
  const h16_t* base = qkv + (int64_t)b * Tn * ld;
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(base, (uint32_t)((int64_t)Tn * ld * 2));
  const __amdgpu_buffer_rsrc_t rdo = rsrc_of(dout + (int64_t)b * Tn * C, (uint32_t)((int64_t)Tn * C * 2));
  const float* small_src = Dg + (wave == 0 ? bht : 0) + (int64_t)bh * Tn;
  const __amdgpu_buffer_rsrc_t rsm = rsrc_of(small_src, (uint32_t)(Tn * 4));

  const int my_kv = kw + (lane & 31);
  h16x8_t fk[4], fv[4];  // K^T, V^T operands: lane holds row my_kv
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0);
    if (my_kv < Tn) {
      a = *(const uint4*)(base + (int64_t)my_kv * ld + C + h * 64 + 16 * ks + 8 * (lane >> 5));
      c = *(const uint4*)(base + (int64_t)my_kv * ld + 2 * C + h * 64 + 16 * ks + 8 * (lane >> 5));
    }
    fk[ks] = *(h16x8_t*)&a;
    fv[ks] = *(h16x8_t*)&c;
  }
  const float sc = LOG2E * 0.125f;
  f32x16_t dv[2] = {zero16(), zero16()}, dk[2] = {zero16(), zero16()};
  const int qstart = k0;
  const int nq = (Tn - qstart + 63) / 64;
  // the kept bits: run (key block k0/64 + wave/2, lane half wave%2) of this head
  const int nkb = (Tn + 63) / 64;
  const __amdgpu_buffer_rsrc_t rmk =
      rsrc_of(dmask, DROP ? (uint32_t)((int64_t)B * H * nkb * 2 * Tn * 4) : 0u);
  const int64_t mrun = ((int64_t)(bh * nkb + (k0 >> 6) + (wave >> 1)) * 2 + (wave & 1)) * Tn;
  // 5 loads per wave per stage (6 with DROP): 2 + 2 tile loads, one small load
  constexpr int LOADS = DROP ? 6 : 5;
  auto stage = [&](h16_t* dst, int qs) {
    tile_dma(rq, dst, qs, ld, h * 64, lane, wave);
    tile_dma(rdo, dst + TILE_ELEMS, qs, C, h * 64, lane, wave);
    // wave 0 fetches the 64 scaled logsumexp values of the block, wave 1
    // the 64 D values (rows past the end read as zero); waves 2 and 3 issue
    // a load that reads nothing so that every wave counts the same loads
    const uint32_t off = wave < 2 ? (uint32_t)((qs + lane) * 4) : 0xFFFFFF00u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsm, AS3(dst + 2 * TILE_ELEMS + wave * 512), 4, off,
                                             0, 0, 0);
    if constexpr (DROP) {
      // words of queries qs + lane; a run's end may read the next run's
      // words (queries >= T, whose probabilities are zero) or, at the
      // buffer's end, nothing
      const int64_t wi = mrun + qs + lane;
      const uint32_t moff = wi < (int64_t)B * H * nkb * 2 * Tn ? (uint32_t)(wi * 4) : 0xFFFFFF00u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rmk, AS3(dst + 2 * TILE_ELEMS + wave * 512 + 128), 4,
                                               moff, 0, 0, 0);
    }
  };
#pragma unroll
  for (int st = 0; st < FLASH_NS - 1; ++st)
    if (st < nq) stage(ring[st], qstart + 64 * st);
  // this lane's key in the forward's word layout: run (key block, half) and bit
  const int kloc = my_kv - k0;  // 0..127
  const int krun = 2 * (kloc >> 6) + ((kloc >> 2) & 1);
  const int kbit = 16 * ((kloc >> 5) & 1) + 4 * ((kloc >> 3) & 3) + (kloc & 3);
  auto step = [&](int qi, auto slot) {
    constexpr int SL = decltype(slot)::value;
    if (qi + FLASH_NS - 2 < nq) vm_wait_barrier<(FLASH_NS - 2) * LOADS>();
    else vm_wait_barrier<0>();
    if (qi + FLASH_NS - 1 < nq)
      stage(ring[(SL + FLASH_NS - 1) % FLASH_NS], qstart + 64 * (qi + FLASH_NS - 1));
    const h16_t* tQ = ring[SL];
    const h16_t* tdO = tQ + TILE_ELEMS;
    const float* sL = (const float*)(tQ + 2 * TILE_ELEMS);
    const float* sD = (const float*)(tQ + 2 * TILE_ELEMS + 512);
    const uint32_t* sM = (const uint32_t*)(tQ + 2 * TILE_ELEMS + krun * 512 + 128);
    const int qs = qstart + 64 * qi;
    if (qs + 63 < kw || kw >= Tn) return;  // no query of this block sees these keys
    // query qs + 32t + ACC_ROW(r) is kept when it lies in [my_kv, Tn);
    // c = 32t + 8(r/4) + r%4 is kept when (unsigned)(c - lo) < span
    const bool diag = qs < kw + 31 || qs + 64 > Tn;
    const int lo = my_kv - qs - 4 * (lane >> 5);
    const unsigned span = (unsigned)(Tn - my_kv);
    // the two 32-query halves of the block one after the other keeps the
    // live accumulators (S, dP, dK, dV) within 256 registers
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // dP starts from -D of its query rows (read from LDS into the
      // accumulator), so the products leave dP - D
      f32x16_t sa = zero16(), dpa = zero16();
      if constexpr (!DROP) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dpa[r] = sD[32 * t + ACC_ROW(r, lane)];
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        sa = MFMA32(frag_hd(tQ, 32 * t, ks, lane), fk[ks], sa);
        dpa = MFMA32(frag_hd(tdO, 32 * t, ks, lane), fv[ks], dpa);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qq = 32 * t + ACC_ROW(r, lane);
        sa[r] = fexp2(fmaf(sa[r], sc, -sL[qq]));
      }
      if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * t + 8 * (r >> 2) + (r & 3);
          sa[r] = (unsigned)(c - lo) < span ? sa[r] : 0.f;
        }
      }
      if constexpr (DROP) {
        // dropout: dS = P (z dP~ - D) and dV += (P z)^T dO, z from the
        // forward's bit for (query, this lane's key)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qq = 32 * t + ACC_ROW(r, lane);
          const float z = (sM[qq] >> kbit) & 1u ? dr.scale : 0.f;
          dpa[r] = sa[r] * (z * dpa[r] + sD[qq]);
          sa[r] *= z;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dpa[r] = sa[r] * dpa[r];
        }
      }
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const h16x8_t pa = pack_acc(sa, ss);
        const h16x8_t da = pack_acc(dpa, ss);
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          dv[ht] = MFMA32(pa, frag_rows(tdO, 32 * ht, 2 * t + ss, lane), dv[ht]);
          dk[ht] = MFMA32(da, frag_rows(tQ, 32 * ht, 2 * t + ss, lane), dk[ht]);
        }
      }
    }
  };
  for (int qi = 0; qi < nq; qi += FLASH_NS) slot_steps<0, FLASH_NS>(qi, nq, step);
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = kw + ACC_ROW(r, lane);
      if (kv < Tn) {
        h16_t* row = dqkv + ((int64_t)b * Tn + kv) * ld + h * 64 + 32 * ht + (lane & 31);
        row[C] = f2h(dk[ht][r] * 0.125f);
        row[2 * C] = f2h(dv[ht][r]);
      }
    }
  if (cs_part) {
    // column sums of this block's dK and dV over its valid keys (the bias
    // gradient of the fused projection): per wave over its 32 keys, then the
    // 4 waves in a fixed order; one partial row per (batch, key block)
    __shared__ float red[4][128];
    float sk[2] = {0.f, 0.f}, sv[2] = {0.f, 0.f};
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kw + ACC_ROW(r, lane) < Tn) {
          sk[ht] += dk[ht][r];
          sv[ht] += dv[ht][r];
        }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      sk[ht] += __shfl_xor(sk[ht], 32, 64);
      sv[ht] += __shfl_xor(sv[ht], 32, 64);
    }
    if (lane < 32) {
      red[wave][32 * 0 + lane] = sk[0];
      red[wave][32 * 1 + lane] = sk[1];
      red[wave][64 + lane] = sv[0];
      red[wave][96 + lane] = sv[1];
    }
    __syncthreads();
    if (tid < 128) {
      const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
      const int kind = tid >> 6, c = tid & 63;  // kind 0: k, 1: v
      const int nblk = (Tn + 127) / 128;
      cs_part[((int64_t)b * nblk + kblk) * 3 * C + (1 + kind) * C + h * 64 + c] =
          kind == 0 ? v * 0.125f : v;
    }
  }
}

// ---------------------------------------------------------------- backward: dQ
// grid: (T/128 query blocks, heaviest first) x (B*H); 4 waves x 32 queries.
// S^T = K Q^T and dP^T = V dO^T put one query per lane; dS^T is the B
// operand of dQ^T += K^T dS^T, whose A operand is a transposing read of K.
// DROP: the forward's kept bits (same lane layout) from dmask.
template <int FLASH_NS, bool DROP>
__global__ __launch_bounds__(256, 2) void flash_bwd_dq_kernel(
    const h16_t* __restrict__ qkv, const h16_t* __restrict__ outp, const float* __restrict__ lse,
    float* __restrict__ Dg, const h16_t* __restrict__ dout, h16_t* __restrict__ dqkv,
    float* __restrict__ cs_part, int B, int Tn, int H, int C, Drop dr,
    const uint32_t* __restrict__ dmask) {
  __shared__ __attribute__((aligned(1024))) h16_t ring[FLASH_NS][2][TILE_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int nqb = (Tn + 127) / 128;
  const int qb = nqb - 1 - (int)(blockIdx.x / (B * H));
  const int bh = blockIdx.x % (B * H), b = bh / H, h = bh % H;
  const int q0 = qb * 128, qw = q0 + 32 * wave;
  const int ld = 3 * C;
  const int64_t bht = (int64_t)B * H * Tn;
  const h16_t* base = qkv + (int64_t)b * Tn * ld;
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(base, (uint32_t)((int64_t)Tn * ld * 2));
  const int my_q = qw + (lane & 31);

  // lanes l and l+32 hold the two halves of query row my_q: Q and dO as MFMA
  // operands, and the attention output O to form D = rowsum(dO * O)
  h16x8_t fq[4], fdo[4];
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0), o = make_uint4(0, 0, 0, 0);
    if (my_q < Tn) {
      const int64_t ro = ((int64_t)b * Tn + my_q) * C + h * 64 + 16 * ks + 8 * (lane >> 5);
      a = *(const uint4*)(base + (int64_t)my_q * ld + h * 64 + 16 * ks + 8 * (lane >> 5));
      c = *(const uint4*)(dout + ro);
      o = *(const uint4*)(outp + ro);
    }
    fq[ks] = *(h16x8_t*)&a;
    fdo[ks] = *(h16x8_t*)&c;
    const uint32_t ov[4] = {o.x, o.y, o.z, o.w}, gv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dsum = fmaf(h_lo(ov[j]), h_lo(gv[j]), dsum);
      dsum = fmaf(h_hi(ov[j]), h_hi(gv[j]), dsum);
    }
  }
  const float Dq = dsum + __shfl_xor(dsum, 32, 64);
  const float sc = LOG2E * 0.125f;
  const float L2q = my_q < Tn ? lse[(int64_t)bh * Tn + my_q] * LOG2E : 0.f;
  const float nL2 = -L2q;
  // -D and the scaled logsumexp of every query row, for the key-side kernel
  // that runs next
  if (lane < 32 && my_q < Tn) {
    Dg[(int64_t)bh * Tn + my_q] = -Dq;
    Dg[bht + (int64_t)bh * Tn + my_q] = L2q;
  }
  f32x16_t dq[2] = {zero16(), zero16()};
  // without dropout every dP accumulation starts from -D of the lane's query
  // (a loop-invariant accumulator input), so the products leave dP - D
  f32x16_t dp0 = zero16();
  if constexpr (!DROP) {
#pragma unroll
    for (int r = 0; r < 16; ++r) dp0[r] = -Dq;
  }
  const int nkv = (min(Tn, q0 + 128) + 63) / 64;
#pragma unroll
  for (int st = 0; st < FLASH_NS - 1; ++st)
    if (st < nkv) {
      tile_dma(rs, ring[st][0], 64 * st, ld, C + h * 64, lane, wave);
      tile_dma(rs, ring[st][1], 64 * st, ld, 2 * C + h * 64, lane, wave);
    }
  auto step = [&](int kb, auto slot) {
    constexpr int SL = decltype(slot)::value;
    if (kb + FLASH_NS - 2 < nkv) vm_wait_barrier<(FLASH_NS - 2) * 4>();
    else vm_wait_barrier<0>();
    if (kb + FLASH_NS - 1 < nkv) {
      constexpr int NX = (SL + FLASH_NS - 1) % FLASH_NS;
      const int r0 = 64 * (kb + FLASH_NS - 1);
      tile_dma(rs, ring[NX][0], r0, ld, C + h * 64, lane, wave);
      tile_dma(rs, ring[NX][1], r0, ld, 2 * C + h * 64, lane, wave);
    }
    const h16_t* tK = ring[SL][0];
    const h16_t* tV = ring[SL][1];
    const int kv0 = kb * 64;
    if (kv0 > qw + 31) return;
    uint32_t mw = 0;
    if constexpr (DROP) {
      if (my_q < Tn) {
        const int nkb = (Tn + 63) / 64;
        mw = dmask[((int64_t)(bh * nkb + kb) * 2 + (lane >> 5)) * Tn + my_q];
      }
    }
    f32x16_t s[2] = {zero16(), zero16()}, dp[2] = {dp0, dp0};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = MFMA32(frag_hd(tK, 32 * t, ks, lane), fq[ks], s[t]);
        dp[t] = MFMA32(frag_hd(tV, 32 * t, ks, lane), fdo[ks], dp[t]);
      }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = fexp2(fmaf(s[t][r], sc, nL2));
    if (kv0 + 63 > qw || kv0 + 64 > Tn) {
      const int lim = min(my_q, Tn - 1) - kv0 - 4 * (lane >> 5);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[t][r] = (32 * t + 8 * (r >> 2) + (r & 3)) > lim ? 0.f : s[t][r];
    }
    if constexpr (DROP) {
      // dS = P (z dP~ - D), z = scale where the forward kept the element
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float z = (mw >> (16 * t + r)) & 1u ? dr.scale : 0.f;
          dp[t][r] = s[t][r] * (z * dp[t][r] - Dq);
        }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[t][r] = s[t][r] * dp[t][r];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const h16x8_t db = pack_acc(dp[t], ss);
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
          dq[ht] = MFMA32(frag_rows(tK, 32 * ht, 2 * t + ss, lane), db, dq[ht]);
      }
  };
  for (int kb = 0; kb < nkv; kb += FLASH_NS) slot_steps<0, FLASH_NS>(kb, nkv, step);
  if (my_q < Tn) {
    h16_t* dQ = dqkv + ((int64_t)b * Tn + my_q) * ld + h * 64;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int hd = 32 * ht + 8 * rg + 4 * (lane >> 5);
        uint2 v;
        v.x = pack2h(dq[ht][4 * rg + 0] * 0.125f, dq[ht][4 * rg + 1] * 0.125f);
        v.y = pack2h(dq[ht][4 * rg + 2] * 0.125f, dq[ht][4 * rg + 3] * 0.125f);
        *(uint2*)(dQ + hd) = v;
      }
  }
  if (cs_part) {
    // column sums of this block's dQ over its valid queries: the tile goes
    // to LDS as [head dim][query] (the ring is free once every wave is past
    // its last key block), then each head dimension is summed in a fixed order
    __syncthreads();
    constexpr int TP = 129;  // pitch: rows of consecutive dims fall in distinct banks
    float* tq = (float*)&ring[0][0][0];  // 64 x TP floats
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tq[(32 * ht + ACC_ROW(r, lane)) * TP + 32 * wave + (lane & 31)] =
            my_q < Tn ? dq[ht][r] : 0.f;
    __syncthreads();
    float* part4 = tq + 64 * TP;  // [4][64]
    {
      const int dcol = tid & 63, quarter = tid >> 6;
      float v = 0.f;
      for (int q = 0; q < 32; ++q) v += tq[dcol * TP + 32 * quarter + q];
      part4[quarter * 64 + dcol] = v;
    }
    __syncthreads();
    if (tid < 64) {
      const float v = ((part4[tid] + part4[64 + tid]) + part4[128 + tid]) + part4[192 + tid];
      cs_part[((int64_t)b * nqb + qb) * 3 * C + h * 64 + tid] = v * 0.125f;
    }
  }
}

// ================================================================ launchers
int attention_fwd_launch(bool h16, const void* qkv, void* out, float* lse, int B, int Tn, int H,
                         int C, hipStream_t s, Drop dr, uint32_t* dmask) {
  const int hs = C / H;
  if (hs * H != C || hs > 128) return -5;
  if (h16 && hs == 64) {
    const int nqb = (Tn + 127) / 128;
    if (dr.thresh && !dmask) return -5;
    if (dr.thresh)
      hipLaunchKernelGGL((flash_fwd_kernel<FLASH_FWD_NS, true>), dim3(nqb * B * H), dim3(256), 0,
                         s, (const h16_t*)qkv, (h16_t*)out, lse, B, Tn, H, C, dr, dmask);
    else
      hipLaunchKernelGGL((flash_fwd_kernel<FLASH_FWD_NS, false>), dim3(nqb * B * H), dim3(256), 0,
                         s, (const h16_t*)qkv, (h16_t*)out, lse, B, Tn, H, C, dr, dmask);
  } else if (h16) {
    hipLaunchKernelGGL(attn_fwd_generic<h16_t>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                       (const h16_t*)qkv, (h16_t*)out, lse, B, Tn, H, C, dr);
  } else {
    hipLaunchKernelGGL(attn_fwd_generic<float>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                       (const float*)qkv, (float*)out, lse, B, Tn, H, C, dr);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// D: fp32 scratch of 2*B*H*T elements (rowsum(dout * out), negated by the
// 16-bit head-width-64 kernels, then the row logsumexp times log2(e) for
// those kernels).  dr: the forward's dropout of the probabilities
// (rowsum(dout * out) is still the row's D with dropout: it equals
// rowsum(P * dP) for dP = z dP~); the head-width-64 16-bit kernels read the
// forward's kept bits from dmask, the others regenerate them.
// cs_part / cs_out (optional): cs_out[n] (+)= column sums of dqkv (the bias
// gradient of the fused q|k|v projection); cs_part is fp32 scratch of at
// least max(B * cdiv(Tn, 128), colsum_part_rows(B * Tn)) x 3C elements.
int attention_bwd_launch(bool h16, const void* qkv, const void* out, const float* lse,
                         const void* dout, void* dqkv, float* D, int B, int Tn, int H, int C,
                         float* cs_part, float* cs_out, int cs_beta, hipStream_t s,
                         ColsumJob* defer, Drop dr, const uint32_t* dmask) {
  const int hs = C / H;
  if (hs * H != C || hs > 128) return -5;
  const int64_t rows = (int64_t)B * H * Tn;
  if (h16) {
    const bool flash = hs == 64;
    if (!flash)
      hipLaunchKernelGGL(attn_bwd_dot<h16_t>, dim3(cdiv(rows, 4)), dim3(256), 0, s,
                         (const h16_t*)out, (const h16_t*)dout, lse, D, nullptr, B, Tn, H, C);
    if (flash) {
      // the query-side kernel forms D and the scaled logsumexp of its rows,
      // so it runs first
      const int nb = (Tn + 127) / 128;
      float* cp = cs_out ? cs_part : nullptr;
      if (dr.thresh && !dmask) return -5;
#define FLASH_BWD(DROP)                                                                            \
  hipLaunchKernelGGL((flash_bwd_dq_kernel<FLASH_DQ_NS, DROP>), dim3(nb * B * H), dim3(256), 0, s, \
                     (const h16_t*)qkv, (const h16_t*)out, lse, D, (const h16_t*)dout,             \
                     (h16_t*)dqkv, cp, B, Tn, H, C, dr, dmask);                                    \
  hipLaunchKernelGGL((flash_bwd_dkdv_kernel<FLASH_DKDV_NS, DROP>), dim3(nb * B * H), dim3(256), 0, \
                     s, (const h16_t*)qkv, D, (const h16_t*)dout, (h16_t*)dqkv, cp, B, Tn, H, C,   \
                     dr, dmask);
      if (dr.thresh) {
        FLASH_BWD(true)
      } else {
        FLASH_BWD(false)
      }
#undef FLASH_BWD
      if (cs_out) {
        if (hipGetLastError() != hipSuccess) return -4;
        if (defer) {
          *defer = ColsumJob();
          defer->part = cs_part;
          defer->out[0] = cs_out;
          defer->nrow = B * nb;
          defer->ncol = defer->seg = 3 * C;
          return 0;
        }
        return colsum_finalize_launch(cs_part, B * nb, 3 * C, cs_out, cs_beta, s);
      }
    } else {
      hipLaunchKernelGGL(attn_bwd_dq_generic<h16_t>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                         (const h16_t*)qkv, lse, D, (const h16_t*)dout, (h16_t*)dqkv, B, Tn, H, C,
                         dr);
      hipLaunchKernelGGL(attn_bwd_dkdv_generic<h16_t>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                         (const h16_t*)qkv, lse, D, (const h16_t*)dout, (h16_t*)dqkv, B, Tn, H, C,
                         dr);
    }
    if (cs_out && !flash) {
      if (hipGetLastError() != hipSuccess) return -4;
      return colsum_launch(true, dqkv, B * Tn, 3 * C, cs_part, cs_out, cs_beta, s);
    }
  } else {
    hipLaunchKernelGGL(attn_bwd_dot<float>, dim3(cdiv(rows, 4)), dim3(256), 0, s,
                       (const float*)out, (const float*)dout, lse, D, nullptr, B, Tn, H, C);
    hipLaunchKernelGGL(attn_bwd_dq_generic<float>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                       (const float*)qkv, lse, D, (const float*)dout, (float*)dqkv, B, Tn, H, C, dr);
    hipLaunchKernelGGL(attn_bwd_dkdv_generic<float>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                       (const float*)qkv, lse, D, (const float*)dout, (float*)dqkv, B, Tn, H, C, dr);
    if (cs_out) {
      if (hipGetLastError() != hipSuccess) return -4;
      return colsum_launch(false, dqkv, B * Tn, 3 * C, cs_part, cs_out, cs_beta, s);
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace HALF_NS
