// Causal multi-head self-attention, forward and backward.
//
// What is computed is the manual path of "nanoGPT" (stanleyjacob.dev), Part V
// Deep dive 1: per head, softmax(q k^T / sqrt(hs)) with the entries above the
// diagonal at -inf, times v; q, k, v are the column blocks of the fused
// c_attn output, head h at columns h*hs.  The bf16 kernels reach the same
// result tile by tile with an online softmax and never store the T x T
// matrix ("Let's reproduce GPT-2 (124M)", chapter "Flash Attention, 96ms"):
// the forward keeps the row logsumexp, the backward recomputes the
// probabilities from it.
//
// bf16 kernels (head width 64) use v_mfma_f32_32x32x16_bf16.  The forward
// computes S^T = K Q^T so that one lane owns one query row: its running max
// and sum stay in the lane, and the probabilities in the accumulator
// registers are directly the B operand of O^T = V^T P^T.  The backward is two
// kernels: dK/dV per key block (iterating over query blocks) and dQ per
// query block (iterating over key blocks), so no atomics are needed.
#include "common.h"

#define LOG2E 1.4426950408889634f
#define LN2 0.6931471805599453f

// ================================================================ generic (fp32 mode)
template <typename T>
__global__ void attn_fwd_generic(const T* __restrict__ qkv, T* __restrict__ out,
                                 float* __restrict__ lse, int B, int Tn, int H, int C) {
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
    l = l * alpha + p;
    for (int c = 0; c < hs; ++c) o[c] = o[c] * alpha + p * ldf(V + c);
    m = mn;
  }
  T* O = out + ((int64_t)b * Tn + q) * C + h * hs;
  for (int c = 0; c < hs; ++c) stf(O + c, o[c] / l);
  lse[(int64_t)bh * Tn + q] = m + logf(l);
}

// D[bh][q] = sum_c dO[q][c] * O[q][c]  (= rowsum(P * dP))
template <typename T>
__global__ void attn_bwd_dot(const T* __restrict__ out, const T* __restrict__ dout,
                             float* __restrict__ D, int B, int Tn, int H, int C) {
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
  if (lane == 0) D[row] = s;
}

template <typename T>
__global__ void attn_bwd_dq_generic(const T* __restrict__ qkv, const float* __restrict__ lse,
                                    const float* __restrict__ D, const T* __restrict__ dout,
                                    T* __restrict__ dqkv, int B, int Tn, int H, int C) {
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
    const float ds = p * (dp - Dq);
    for (int c = 0; c < hs; ++c) dq[c] += ds * ldf(K + c);
  }
  T* dQ = dqkv + ((int64_t)b * Tn + q) * ld + h * hs;
  for (int c = 0; c < hs; ++c) stf(dQ + c, dq[c] * scale);
}

template <typename T>
__global__ void attn_bwd_dkdv_generic(const T* __restrict__ qkv, const float* __restrict__ lse,
                                      const float* __restrict__ D, const T* __restrict__ dout,
                                      T* __restrict__ dqkv, int B, int Tn, int H, int C) {
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
    const float ds = p * (dp - D[(int64_t)bh * Tn + q]);
    for (int c = 0; c < hs; ++c) {
      dv[c] += p * ldf(dO + c);
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

// ================================================================ bf16 flash kernels (hs = 64)
// LDS tiles of 64 rows x 64 bf16:
//  "row" layout  [row][64], 16-byte chunk c of row r at chunk position c ^ (r & 7);
//  "tr" layout   [col][64] holding the transpose (element (row, col) at
//                [col][row]), 8-byte unit u (4 rows) of line col at u ^ (col & 15).
__device__ __forceinline__ int row_off(int r, int c) { return r * 64 + ((c ^ (r & 7)) << 3); }
__device__ __forceinline__ int tr_off(int col, int u) { return col * 64 + ((u ^ (col & 15)) << 2); }

// Stage a 64 x 64 bf16 tile (global rows r0.., row pitch ld, columns at col0)
// into LDS in "row" layout; rows >= nrows are zero.  256 threads, 2 chunks each.
__device__ __forceinline__ void stage_row(bf16_t* lds, const bf16_t* __restrict__ g, int64_t ld,
                                          int r0, int nrows, int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i, r = idx >> 3, c = idx & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < nrows) v = *(const uint4*)(g + (int64_t)(r0 + r) * ld + 8 * c);
    *(uint4*)(lds + row_off(r, c)) = v;
  }
}
// Same tile into the "tr" layout (transposed).  Each thread reads 2 rows x 8
// columns and writes 8 packed pairs.
__device__ __forceinline__ void stage_tr(bf16_t* lds, const bf16_t* __restrict__ g, int64_t ld,
                                         int r0, int nrows, int tid) {
  const int cc = tid & 7, rp = tid >> 3;  // column chunk, row pair (0..31)
  const int r = 2 * rp;
  uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
  if (r0 + r < nrows) a = *(const uint4*)(g + (int64_t)(r0 + r) * ld + 8 * cc);
  if (r0 + r + 1 < nrows) b = *(const uint4*)(g + (int64_t)(r0 + r + 1) * ld + 8 * cc);
  const uint32_t* pa = (const uint32_t*)&a;
  const uint32_t* pb = (const uint32_t*)&b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
    const uint32_t v = (j & 1) ? ((pa[w] >> 16) | (pb[w] & 0xffff0000u))
                               : ((pa[w] & 0xffffu) | (pb[w] << 16));
    const int col = 8 * cc + j;
    // rows r, r+1 live in unit r/4 at half (r % 4) / 2
    *(uint32_t*)(lds + tr_off(col, r >> 2) + (r & 3)) = v;
  }
}

// A/B operand of a 32x32x16 MFMA from the "row" layout: row base+lane%32,
// k-chunk (2*ks + lane/32).
__device__ __forceinline__ bf16x8_t frag_row(const bf16_t* lds, int base, int ks, int lane) {
  return *(const bf16x8_t*)(lds + row_off(base + (lane & 31), 2 * ks + (lane >> 5)));
}
// Operand whose k index runs over the rows of a "tr" tile, in the order of
// the 32x32 accumulator layout: line `col`, rows 16*ks + 8*(j/4) + 4*g + j%4.
__device__ __forceinline__ bf16x8_t frag_tr(const bf16_t* lds, int col, int ks, int lane) {
  const int g = lane >> 5;
  const uint2 lo = *(const uint2*)(lds + tr_off(col, 4 * ks + g));
  const uint2 hi = *(const uint2*)(lds + tr_off(col, 4 * ks + 2 + g));
  uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return *(bf16x8_t*)&v;
}
// 8 accumulator values (registers 8s..8s+7 of a 32x32 tile) -> bf16 operand.
__device__ __forceinline__ bf16x8_t pack_acc(const f32x16_t& a, int s, float mul) {
  uint4 v;
  v.x = pack2bf(a[8 * s + 0] * mul, a[8 * s + 1] * mul);
  v.y = pack2bf(a[8 * s + 2] * mul, a[8 * s + 3] * mul);
  v.z = pack2bf(a[8 * s + 4] * mul, a[8 * s + 5] * mul);
  v.w = pack2bf(a[8 * s + 6] * mul, a[8 * s + 7] * mul);
  return *(bf16x8_t*)&v;
}
__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}
#define MFMA32(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_bf16((a), (b), (c), 0, 0, 0)
// row offset inside a 32x32 accumulator tile for register r of this lane
#define ACC_ROW(r, lane) (8 * ((r) >> 2) + 4 * ((lane) >> 5) + ((r) & 3))

// ---------------------------------------------------------------- forward
// grid: (T/128 query blocks, heaviest first) x (B*H); 4 waves x 32 query rows.
__global__ __launch_bounds__(256) void flash_fwd_kernel(const bf16_t* __restrict__ qkv,
                                                        bf16_t* __restrict__ out,
                                                        float* __restrict__ lse, int B, int Tn,
                                                        int H, int C) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][64 * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[2][64 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nqb = (Tn + 127) / 128;
  const int qb = nqb - 1 - (int)(blockIdx.x / (B * H));
  const int bh = blockIdx.x % (B * H), b = bh / H, h = bh % H;
  const int q0 = qb * 128, qw = q0 + 32 * wave;
  const int64_t ld = 3 * (int64_t)C;
  const bf16_t* base = qkv + (int64_t)b * Tn * ld;
  const bf16_t* Kg = base + C + h * 64;
  const bf16_t* Vg = base + 2 * C + h * 64;

  // Q^T operand (B of S^T = K Q^T): lane holds Q[qw + lane%32][16ks + 8g + j]
  bf16x8_t fq[4];
  {
    const int q = qw + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (q < Tn) v = *(const uint4*)(base + (int64_t)q * ld + h * 64 + 16 * ks + 8 * (lane >> 5));
      fq[ks] = *(bf16x8_t*)&v;
    }
  }
  const float sc = LOG2E * 0.125f;  // log2(e) / sqrt(64)
  float m = -INFINITY, l = 0.f;
  f32x16_t o[2] = {zero16(), zero16()};
  const int my_q = qw + (lane & 31);

  const int kv_end = min(Tn, q0 + 128);
  const int nkv = (kv_end + 63) / 64;
  stage_row(sK[0], Kg, ld, 0, Tn, tid);
  stage_tr(sVt[0], Vg, ld, 0, Tn, tid);
  __syncthreads();
  for (int kb = 0; kb < nkv; ++kb) {
    const int cur = kb & 1, kv0 = kb * 64;
    if (kb + 1 < nkv) {
      stage_row(sK[cur ^ 1], Kg, ld, kv0 + 64, Tn, tid);
      stage_tr(sVt[cur ^ 1], Vg, ld, kv0 + 64, Tn, tid);
    }
    if (kv0 <= qw + 31) {  // some key of this block is visible to this wave
      f32x16_t s[2] = {zero16(), zero16()};
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) s[t] = MFMA32(frag_row(sK[cur], 32 * t, ks, lane), fq[ks], s[t]);
      const bool diag = kv0 + 63 > qw || kv0 + 64 > Tn;
      float mb = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[t][r] * sc;
          if (diag) {
            const int kv = kv0 + 32 * t + ACC_ROW(r, lane);
            if (kv > my_q || kv >= Tn) v = -INFINITY;
          }
          s[t][r] = v;
          mb = fmaxf(mb, v);
        }
      mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
      const float mn = fmaxf(m, mb);
      const float alpha = exp2f(m - mn);
      float ls = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[t][r] - mn);
          s[t][r] = p;
          ls += p;
        }
      l = l * alpha + ls;
      m = mn;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ht][r] *= alpha;
      // O^T += V^T P^T over the 64 keys (4 steps of 16)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const bf16x8_t pb = pack_acc(s[t], ss, 1.0f);
#pragma unroll
          for (int ht = 0; ht < 2; ++ht)
            o[ht] = MFMA32(frag_tr(sVt[cur], 32 * ht + (lane & 31), 2 * t + ss, lane), pb, o[ht]);
        }
    }
    __syncthreads();
  }
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = 1.0f / lt;
  if (my_q < Tn) {
    bf16_t* O = out + ((int64_t)b * Tn + my_q) * C + h * 64;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int hd = 32 * ht + 8 * rg + 4 * (lane >> 5);
        uint2 v;
        v.x = pack2bf(o[ht][4 * rg + 0] * inv, o[ht][4 * rg + 1] * inv);
        v.y = pack2bf(o[ht][4 * rg + 2] * inv, o[ht][4 * rg + 3] * inv);
        *(uint2*)(O + hd) = v;
      }
    if (lane < 32) lse[(int64_t)bh * Tn + my_q] = (m + __log2f(lt)) * LN2;
  }
}

// ---------------------------------------------------------------- backward: dK, dV
// grid: (T/128 key blocks) x (B*H); 4 waves x 32 key rows; query blocks of 64.
__global__ __launch_bounds__(256) void flash_bwd_dkdv_kernel(
    const bf16_t* __restrict__ qkv, const float* __restrict__ lse, const float* __restrict__ Dg,
    const bf16_t* __restrict__ dout, bf16_t* __restrict__ dqkv, int B, int Tn, int H, int C) {
  __shared__ __attribute__((aligned(16))) bf16_t sQ[2][64 * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sQt[2][64 * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sdO[2][64 * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sdOt[2][64 * 64];
  __shared__ float sL[2][64], sD[2][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x % (B * H), b = bh / H, h = bh % H;
  const int kb = blockIdx.x / (B * H);
  const int k0 = kb * 128, kw = k0 + 32 * wave;
  const int64_t ld = 3 * (int64_t)C;
  const bf16_t* base = qkv + (int64_t)b * Tn * ld;
  const bf16_t* Qg = base + h * 64;
  const bf16_t* dOg = dout + (int64_t)b * Tn * C + h * 64;
  const float* Lg = lse + (int64_t)bh * Tn;
  const float* DDg = Dg + (int64_t)bh * Tn;

  // K and V rows of this wave as B operands (K^T, V^T): lane holds row kw+lane%32
  bf16x8_t fk[4], fv[4];
  {
    const int kv = kw + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0);
      if (kv < Tn) {
        a = *(const uint4*)(base + (int64_t)kv * ld + C + h * 64 + 16 * ks + 8 * (lane >> 5));
        c = *(const uint4*)(base + (int64_t)kv * ld + 2 * C + h * 64 + 16 * ks + 8 * (lane >> 5));
      }
      fk[ks] = *(bf16x8_t*)&a;
      fv[ks] = *(bf16x8_t*)&c;
    }
  }
  const float sc = LOG2E * 0.125f;
  const int my_kv = kw + (lane & 31);
  f32x16_t dv[2] = {zero16(), zero16()}, dk[2] = {zero16(), zero16()};

  const int qstart = (k0 / 64) * 64;
  const int nq = (Tn - qstart + 63) / 64;
  auto stage = [&](int buf, int qs) {
    stage_row(sQ[buf], Qg, ld, qs, Tn, tid);
    stage_tr(sQt[buf], Qg, ld, qs, Tn, tid);
    stage_row(sdO[buf], dOg, C, qs, Tn, tid);
    stage_tr(sdOt[buf], dOg, C, qs, Tn, tid);
    if (tid < 64) {
      const int q = qs + tid;
      sL[buf][tid] = q < Tn ? Lg[q] * LOG2E : 0.f;
      sD[buf][tid] = q < Tn ? DDg[q] : 0.f;
    }
  };
  if (nq > 0) stage(0, qstart);
  __syncthreads();
  for (int qi = 0; qi < nq; ++qi) {
    const int cur = qi & 1, qs = qstart + 64 * qi;
    if (qi + 1 < nq) stage(cur ^ 1, qs + 64);
    if (qs + 63 >= kw && kw < Tn) {  // some query of this block sees these keys
      // S = Q K^T and dP = dO V^T for 2 query tiles of 32: rows q, columns kv
      f32x16_t s[2] = {zero16(), zero16()}, dp[2] = {zero16(), zero16()};
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          s[t] = MFMA32(frag_row(sQ[cur], 32 * t, ks, lane), fk[ks], s[t]);
          dp[t] = MFMA32(frag_row(sdO[cur], 32 * t, ks, lane), fv[ks], dp[t]);
        }
      const bool diag = qs < kw + 31 || qs + 64 > Tn;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qq = 32 * t + ACC_ROW(r, lane);
          float p = exp2f(s[t][r] * sc - sL[cur][qq]);
          if (diag && (qs + qq < my_kv || qs + qq >= Tn)) p = 0.f;
          s[t][r] = p;
          dp[t][r] = p * (dp[t][r] - sD[cur][qq]);
        }
      // dV += P^T dO, dK += dS^T Q (k index = query, 4 steps of 16)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const bf16x8_t pa = pack_acc(s[t], ss, 1.0f);
          const bf16x8_t da = pack_acc(dp[t], ss, 1.0f);
#pragma unroll
          for (int ht = 0; ht < 2; ++ht) {
            dv[ht] = MFMA32(pa, frag_tr(sdOt[cur], 32 * ht + (lane & 31), 2 * t + ss, lane), dv[ht]);
            dk[ht] = MFMA32(da, frag_tr(sQt[cur], 32 * ht + (lane & 31), 2 * t + ss, lane), dk[ht]);
          }
        }
    }
    __syncthreads();
  }
  // dk/dv tiles: rows = key (ACC_ROW), columns = head dim lane%32
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = kw + ACC_ROW(r, lane);
      if (kv < Tn) {
        bf16_t* row = dqkv + ((int64_t)b * Tn + kv) * ld + h * 64 + 32 * ht + (lane & 31);
        row[C] = f2bf(dk[ht][r] * 0.125f);
        row[2 * C] = f2bf(dv[ht][r]);
      }
    }
}

// ---------------------------------------------------------------- backward: dQ
// grid: (T/128 query blocks, heaviest first) x (B*H); 4 waves x 32 query rows.
__global__ __launch_bounds__(256) void flash_bwd_dq_kernel(
    const bf16_t* __restrict__ qkv, const float* __restrict__ lse, const float* __restrict__ Dg,
    const bf16_t* __restrict__ dout, bf16_t* __restrict__ dqkv, int B, int Tn, int H, int C) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][64 * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sKt[2][64 * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][64 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nqb = (Tn + 127) / 128;
  const int qb = nqb - 1 - (int)(blockIdx.x / (B * H));
  const int bh = blockIdx.x % (B * H), b = bh / H, h = bh % H;
  const int q0 = qb * 128, qw = q0 + 32 * wave;
  const int64_t ld = 3 * (int64_t)C;
  const bf16_t* base = qkv + (int64_t)b * Tn * ld;
  const bf16_t* Kg = base + C + h * 64;
  const bf16_t* Vg = base + 2 * C + h * 64;
  const int my_q = qw + (lane & 31);

  bf16x8_t fq[4], fdo[4];
  {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0);
      if (my_q < Tn) {
        a = *(const uint4*)(base + (int64_t)my_q * ld + h * 64 + 16 * ks + 8 * (lane >> 5));
        c = *(const uint4*)(dout + ((int64_t)b * Tn + my_q) * C + h * 64 + 16 * ks + 8 * (lane >> 5));
      }
      fq[ks] = *(bf16x8_t*)&a;
      fdo[ks] = *(bf16x8_t*)&c;
    }
  }
  const float sc = LOG2E * 0.125f;
  const float L2 = my_q < Tn ? lse[(int64_t)bh * Tn + my_q] * LOG2E : 0.f;
  const float Dq = my_q < Tn ? Dg[(int64_t)bh * Tn + my_q] : 0.f;
  f32x16_t dq[2] = {zero16(), zero16()};

  const int kv_end = min(Tn, q0 + 128);
  const int nkv = (kv_end + 63) / 64;
  stage_row(sK[0], Kg, ld, 0, Tn, tid);
  stage_tr(sKt[0], Kg, ld, 0, Tn, tid);
  stage_row(sV[0], Vg, ld, 0, Tn, tid);
  __syncthreads();
  for (int kb = 0; kb < nkv; ++kb) {
    const int cur = kb & 1, kv0 = kb * 64;
    if (kb + 1 < nkv) {
      stage_row(sK[cur ^ 1], Kg, ld, kv0 + 64, Tn, tid);
      stage_tr(sKt[cur ^ 1], Kg, ld, kv0 + 64, Tn, tid);
      stage_row(sV[cur ^ 1], Vg, ld, kv0 + 64, Tn, tid);
    }
    if (kv0 <= qw + 31) {
      // S^T = K Q^T, dP^T = V dO^T: rows kv, columns q (= this lane's query)
      f32x16_t s[2] = {zero16(), zero16()}, dp[2] = {zero16(), zero16()};
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          s[t] = MFMA32(frag_row(sK[cur], 32 * t, ks, lane), fq[ks], s[t]);
          dp[t] = MFMA32(frag_row(sV[cur], 32 * t, ks, lane), fdo[ks], dp[t]);
        }
      const bool diag = kv0 + 63 > qw || kv0 + 64 > Tn;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = kv0 + 32 * t + ACC_ROW(r, lane);
          float p = exp2f(s[t][r] * sc - L2);
          if (diag && (kv > my_q || kv >= Tn)) p = 0.f;
          dp[t][r] = p * (dp[t][r] - Dq);
        }
      // dQ^T += K^T dS^T (k index = key)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const bf16x8_t db = pack_acc(dp[t], ss, 1.0f);
#pragma unroll
          for (int ht = 0; ht < 2; ++ht)
            dq[ht] = MFMA32(frag_tr(sKt[cur], 32 * ht + (lane & 31), 2 * t + ss, lane), db, dq[ht]);
        }
    }
    __syncthreads();
  }
  if (my_q < Tn) {
    bf16_t* dQ = dqkv + ((int64_t)b * Tn + my_q) * ld + h * 64;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int hd = 32 * ht + 8 * rg + 4 * (lane >> 5);
        uint2 v;
        v.x = pack2bf(dq[ht][4 * rg + 0] * 0.125f, dq[ht][4 * rg + 1] * 0.125f);
        v.y = pack2bf(dq[ht][4 * rg + 2] * 0.125f, dq[ht][4 * rg + 3] * 0.125f);
        *(uint2*)(dQ + hd) = v;
      }
  }
}

// ================================================================ launchers
int attention_fwd_launch(bool bf16, const void* qkv, void* out, float* lse, int B, int Tn, int H,
                         int C, hipStream_t s) {
  const int hs = C / H;
  if (hs * H != C || hs > 128) return -5;
  if (bf16 && hs == 64) {
    const int nqb = (Tn + 127) / 128;
    hipLaunchKernelGGL(flash_fwd_kernel, dim3(nqb * B * H), dim3(256), 0, s,
                       (const bf16_t*)qkv, (bf16_t*)out, lse, B, Tn, H, C);
  } else if (bf16) {
    hipLaunchKernelGGL(attn_fwd_generic<bf16_t>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                       (const bf16_t*)qkv, (bf16_t*)out, lse, B, Tn, H, C);
  } else {
    hipLaunchKernelGGL(attn_fwd_generic<float>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                       (const float*)qkv, (float*)out, lse, B, Tn, H, C);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// D: fp32 scratch of B*H*T elements.
int attention_bwd_launch(bool bf16, const void* qkv, const void* out, const float* lse,
                         const void* dout, void* dqkv, float* D, int B, int Tn, int H, int C,
                         hipStream_t s) {
  const int hs = C / H;
  if (hs * H != C || hs > 128) return -5;
  const int64_t rows = (int64_t)B * H * Tn;
  if (bf16) {
    hipLaunchKernelGGL(attn_bwd_dot<bf16_t>, dim3(cdiv(rows, 4)), dim3(256), 0, s,
                       (const bf16_t*)out, (const bf16_t*)dout, D, B, Tn, H, C);
    if (hs == 64) {
      const int nb = (Tn + 127) / 128;
      hipLaunchKernelGGL(flash_bwd_dkdv_kernel, dim3(nb * B * H), dim3(256), 0, s,
                         (const bf16_t*)qkv, lse, D, (const bf16_t*)dout, (bf16_t*)dqkv, B, Tn, H, C);
      hipLaunchKernelGGL(flash_bwd_dq_kernel, dim3(nb * B * H), dim3(256), 0, s,
                         (const bf16_t*)qkv, lse, D, (const bf16_t*)dout, (bf16_t*)dqkv, B, Tn, H, C);
    } else {
      hipLaunchKernelGGL(attn_bwd_dq_generic<bf16_t>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                         (const bf16_t*)qkv, lse, D, (const bf16_t*)dout, (bf16_t*)dqkv, B, Tn, H, C);
      hipLaunchKernelGGL(attn_bwd_dkdv_generic<bf16_t>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                         (const bf16_t*)qkv, lse, D, (const bf16_t*)dout, (bf16_t*)dqkv, B, Tn, H, C);
    }
  } else {
    hipLaunchKernelGGL(attn_bwd_dot<float>, dim3(cdiv(rows, 4)), dim3(256), 0, s,
                       (const float*)out, (const float*)dout, D, B, Tn, H, C);
    hipLaunchKernelGGL(attn_bwd_dq_generic<float>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                       (const float*)qkv, lse, D, (const float*)dout, (float*)dqkv, B, Tn, H, C);
    hipLaunchKernelGGL(attn_bwd_dkdv_generic<float>, dim3(cdiv(Tn, 64), B * H), dim3(64), 0, s,
                       (const float*)qkv, lse, D, (const float*)dout, (float*)dqkv, B, Tn, H, C);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
