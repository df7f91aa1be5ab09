// LayerNorm forward and backward, one wavefront per row.
//
// "nanoGPT" (stanleyjacob.dev), Part V Deep dive 1: LayerNorm with bias;
// "Let's reproduce GPT-2 (124M)", chapter "Float16, Gradient Scalers, BF16":
// layer norms stay in fp32 under mixed precision.  Reading of the pages
// (silent on it): biased variance and eps = 1e-5, PyTorch's defaults.
//   y = (x - mean) * rstd * w + b,  rstd = 1/sqrt(var + eps)
//   dx = rstd * (g - mean(g) - xhat * mean(g * xhat)),  g = dy * w
// The backward also adds dx into the residual-stream gradient, writes its
// bf16/fp32 copy for the next matrix product, and produces per-block column
// partial sums of dy*xhat (dw), dy (db) and of the updated residual gradient
// (the bias gradient of the projection whose output is that residual).
#include "common.h"

#define LN_EPS 1e-5f
#define LN_MAXV 8  // float4 per lane: C <= 2048

template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) { *(float4*)p = v; }
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float4 v) {
  *(uint2*)p = make_uint2(pack2bf(v.x, v.y), pack2bf(v.z, v.w));
}

template <typename T>
__global__ __launch_bounds__(256) void ln_fwd_kernel(const float* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ b, T* __restrict__ y,
                                                     float* __restrict__ mean_out,
                                                     float* __restrict__ rstd_out, int M, int C) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int nv = C >> 2;
  const float4* xr = (const float4*)(x + row * C);
  float4 v[LN_MAXV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int j = lane + 64 * i;
    v[i] = j < nv ? xr[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    s += v[i].x + v[i].y + v[i].z + v[i].w;
  }
  const float mean = wave_sum(s) / C;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int j = lane + 64 * i;
    if (j < nv) {
      const float a = v[i].x - mean, bb = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      q += a * a + bb * bb + c * c + d * d;
    }
  }
  const float var = wave_sum(q) / C;
  const float rstd = 1.0f / sqrtf(var + LN_EPS);
  T* yr = y + row * C;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int j = lane + 64 * i;
    if (j < nv) {
      const float4 ww = ((const float4*)w)[j], bb = ((const float4*)b)[j];
      float4 o;
      o.x = (v[i].x - mean) * rstd * ww.x + bb.x;
      o.y = (v[i].y - mean) * rstd * ww.y + bb.y;
      o.z = (v[i].z - mean) * rstd * ww.z + bb.z;
      o.w = (v[i].w - mean) * rstd * ww.w + bb.w;
      store4<T>(yr + 4 * j, o);
    }
  }
  if (lane == 0) {
    mean_out[row] = mean;
    rstd_out[row] = rstd;
  }
}

// Rows are split into blocks of LN_BWD_ROWS; each block writes partial column
// sums part[blk][3][C] (dw, db, residual-gradient column sum).
#define LN_BWD_ROWS 64
template <typename T>
__global__ __launch_bounds__(256) void ln_bwd_kernel(
    const float* __restrict__ dy, const float* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const float* __restrict__ w, float* __restrict__ dres,
    T* __restrict__ dres_act, int accumulate, float* __restrict__ part, int M, int C) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nv = C >> 2;
  float4 pw[LN_MAXV], pb[LN_MAXV], pr[LN_MAXV], ww[LN_MAXV];
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    pw[i] = pb[i] = pr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int j = lane + 64 * i;
    ww[i] = j < nv ? ((const float4*)w)[j] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int64_t r0 = (int64_t)blockIdx.x * LN_BWD_ROWS;
  for (int rr = wave; rr < LN_BWD_ROWS; rr += 4) {
    const int64_t row = r0 + rr;
    if (row >= M) break;
    const float mu = mean[row], rs = rstd[row];
    const float4* dyr = (const float4*)(dy + row * C);
    const float4* xr = (const float4*)(x + row * C);
    float4 xh[LN_MAXV], g[LN_MAXV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const int j = lane + 64 * i;
      if (j < nv) {
        const float4 d = dyr[j], xv = xr[j];
        xh[i] = make_float4((xv.x - mu) * rs, (xv.y - mu) * rs, (xv.z - mu) * rs, (xv.w - mu) * rs);
        g[i] = make_float4(d.x * ww[i].x, d.y * ww[i].y, d.z * ww[i].z, d.w * ww[i].w);
        s1 += g[i].x + g[i].y + g[i].z + g[i].w;
        s2 += g[i].x * xh[i].x + g[i].y * xh[i].y + g[i].z * xh[i].z + g[i].w * xh[i].w;
        pw[i].x += d.x * xh[i].x; pw[i].y += d.y * xh[i].y;
        pw[i].z += d.z * xh[i].z; pw[i].w += d.w * xh[i].w;
        pb[i].x += d.x; pb[i].y += d.y; pb[i].z += d.z; pb[i].w += d.w;
      }
    }
    const float m1 = wave_sum(s1) / C, m2 = wave_sum(s2) / C;
    float4* dr = (float4*)(dres + row * C);
    T* da = dres_act + row * C;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const int j = lane + 64 * i;
      if (j < nv) {
        float4 o;
        o.x = rs * (g[i].x - m1 - xh[i].x * m2);
        o.y = rs * (g[i].y - m1 - xh[i].y * m2);
        o.z = rs * (g[i].z - m1 - xh[i].z * m2);
        o.w = rs * (g[i].w - m1 - xh[i].w * m2);
        if (accumulate) {
          const float4 p = dr[j];
          o.x += p.x; o.y += p.y; o.z += p.z; o.w += p.w;
        }
        dr[j] = o;
        store4<T>(da + 4 * j, o);
        pr[i].x += o.x; pr[i].y += o.y; pr[i].z += o.z; pr[i].w += o.w;
      }
    }
  }
  // reduce the 4 waves' partials through LDS (one wave at a time) and write
  // one partial row per block: part[blk][3][C]
  __shared__ float red[3 * LN_MAXV * 256];
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int i = 0; i < LN_MAXV; ++i) {
        const int j = lane + 64 * i;
        if (j < nv) {
          float4* r0 = (float4*)red + j;
          float4* r1 = (float4*)(red + C) + j;
          float4* r2 = (float4*)(red + 2 * C) + j;
          if (w == 0) {
            *r0 = pw[i]; *r1 = pb[i]; *r2 = pr[i];
          } else {
            float4 a = *r0, b = *r1, c = *r2;
            a.x += pw[i].x; a.y += pw[i].y; a.z += pw[i].z; a.w += pw[i].w;
            b.x += pb[i].x; b.y += pb[i].y; b.z += pb[i].z; b.w += pb[i].w;
            c.x += pr[i].x; c.y += pr[i].y; c.z += pr[i].z; c.w += pr[i].w;
            *r0 = a; *r1 = b; *r2 = c;
          }
        }
      }
    }
    __syncthreads();
  }
  float* out = part + (int64_t)blockIdx.x * 3 * C;
  for (int c = threadIdx.x; c < 3 * C; c += 256) out[c] = red[c];
}

// Column sums of a partial matrix part[nrow][ncol] into up to three outputs:
// column j goes to out[j / seg][j % seg] = (beta ? old : 0) + sum over rows.
// 64 columns per block; the 4 waves split the rows, then combine in LDS in a
// fixed order.
__global__ __launch_bounds__(256) void colsum_finalize_kernel(const float* __restrict__ part,
                                                              int nrow, int ncol, int seg,
                                                              float* out0, float* out1,
                                                              float* out2, int beta) {
  __shared__ float red[4][64];
  const int c = blockIdx.x * 64 + (threadIdx.x & 63), rg = threadIdx.x >> 6;
  float s = 0.f;
  if (c < ncol)
    for (int r = rg; r < nrow; r += 4) s += part[(int64_t)r * ncol + c];
  red[rg][threadIdx.x & 63] = s;
  __syncthreads();
  if (rg == 0 && c < ncol) {
    const float t = red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
    const int k = c / seg, i = c % seg;
    float* o = k == 0 ? out0 : (k == 1 ? out1 : out2);
    if (o) o[i] = (beta ? o[i] : 0.f) + t;
  }
}

int layernorm_fwd_launch(bool bf16, const float* x, const float* w, const float* b, void* y,
                         float* mean, float* rstd, int M, int C, hipStream_t s) {
  if (C % 4 || C > LN_MAXV * 256) return -5;
  if (bf16)
    hipLaunchKernelGGL(ln_fwd_kernel<bf16_t>, dim3(cdiv(M, 4)), dim3(256), 0, s, x, w, b,
                       (bf16_t*)y, mean, rstd, M, C);
  else
    hipLaunchKernelGGL(ln_fwd_kernel<float>, dim3(cdiv(M, 4)), dim3(256), 0, s, x, w, b,
                       (float*)y, mean, rstd, M, C);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// partial rows written by one backward call (4 per block)
int layernorm_bwd_part_rows(int M) { return (int)cdiv(M, LN_BWD_ROWS); }

// dres = (accumulate ? dres : 0) + LN'(dy); dres_act = copy; then
// dw, db (beta-accumulated) and bias_grad (+)= column sum of dres, if non-null.
int layernorm_bwd_launch(bool bf16, const float* dy, const float* x, const float* mean,
                         const float* rstd, const float* w, float* dres, void* dres_act,
                         int accumulate, float* part, float* dw, float* db, float* bias_grad,
                         int beta, int M, int C, hipStream_t s) {
  if (C % 4 || C > LN_MAXV * 256) return -5;
  const int nb = (int)cdiv(M, LN_BWD_ROWS);
  if (bf16)
    hipLaunchKernelGGL(ln_bwd_kernel<bf16_t>, dim3(nb), dim3(256), 0, s, dy, x, mean, rstd, w,
                       dres, (bf16_t*)dres_act, accumulate, part, M, C);
  else
    hipLaunchKernelGGL(ln_bwd_kernel<float>, dim3(nb), dim3(256), 0, s, dy, x, mean, rstd, w, dres,
                       (float*)dres_act, accumulate, part, M, C);
  hipLaunchKernelGGL(colsum_finalize_kernel, dim3(cdiv(3 * C, 64)), dim3(256), 0, s, part, nb,
                     3 * C, C, dw, db, bias_grad, beta);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int colsum_finalize_launch(const float* part, int nrow, int ncol, float* out, int beta,
                           hipStream_t s) {
  hipLaunchKernelGGL(colsum_finalize_kernel, dim3(cdiv(ncol, 64)), dim3(256), 0, s, part, nrow,
                     ncol, ncol, out, nullptr, nullptr, beta);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
