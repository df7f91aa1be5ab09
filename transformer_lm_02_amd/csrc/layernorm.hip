// LayerNorm forward and backward, one wavefront per row.
//
// "nanoGPT" (stanleyjacob.dev), Part V Deep dive 1: LayerNorm with bias;
// "Let's reproduce GPT-2 (124M)", chapter "Float16, Gradient Scalers, BF16":
// layer norms stay in fp32 under mixed precision.  Reading of the pages
// (silent on it): biased variance and eps = 1e-5, PyTorch's defaults.
//   y = (x - mean) * rstd * w + b,  rstd = 1/sqrt(var + eps)
//   dx = rstd * (g - mean(g) - xhat * mean(g * xhat)),  g = dy * w
// The backward also adds dx into the residual-stream gradient, writes its
// 16-bit/fp32 copy for the next matrix product, and produces per-block column
// partial sums of dy*xhat (dw), dy (db) and of the updated residual gradient
// (the bias gradient of the projection whose output is that residual).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace HALF_NS {

#define LN_EPS 1e-5f
#define LN_MAXV_MAX 8  // float4 per lane: C <= 2048

// 4 consecutive values of T as loaded (raw) and as fp32
template <typename T> struct Raw4;
template <> struct Raw4<float> {
  typedef float4 type;
  __device__ __forceinline__ static float4 load(const float* p) { return *(const float4*)p; }
  __device__ __forceinline__ static float4 zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ static float4 f32(float4 v) { return v; }
};
template <> struct Raw4<h16_t> {
  typedef uint2 type;
  __device__ __forceinline__ static uint2 load(const h16_t* p) { return *(const uint2*)p; }
  __device__ __forceinline__ static uint2 zero() { return make_uint2(0u, 0u); }
  __device__ __forceinline__ static float4 f32(uint2 u) {
    return make_float4(h_lo(u.x), h_hi(u.x),
                       h_lo(u.y), h_hi(u.y));
  }
};
template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) { *(float4*)p = v; }
template <>
__device__ __forceinline__ void store4<h16_t>(h16_t* p, float4 v) {
  *(uint2*)p = make_uint2(pack2h(v.x, v.y), pack2h(v.z, v.w));
}

template <typename T, int LN_MAXV>
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
  const float mean = wave_sum_dpp(s) / C;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int j = lane + 64 * i;
    if (j < nv) {
      const float a = v[i].x - mean, bb = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      q += a * a + bb * bb + c * c + d * d;
    }
  }
  const float var = wave_sum_dpp(q) / C;
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
// sums part[blk][3][C] (dw, db, residual-gradient column sum).  Each wave
// takes every 4th row of its block and loads its next row (dy, x and, when
// accumulating, the old residual gradient) while it works on the current one.
#define LN_BWD_ROWS 32
template <typename T, int LN_MAXV>
__global__ __launch_bounds__(256) void ln_bwd_kernel(
    const T* __restrict__ dy, const float* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const float* __restrict__ w, float* __restrict__ dres,
    T* __restrict__ dres_act, int accumulate, float* __restrict__ part, int M, int C, Drop dr) {
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
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  typedef typename Raw4<T>::type RawT;
  RawT dc[LN_MAXV];  // current row: dy (as stored), x
  float4 xc[LN_MAXV];
  {
    const int64_t row = r0 + wave;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const int j = lane + 64 * i;
      const bool ok = j < nv && row < M;
      dc[i] = ok ? Raw4<T>::load(dy + row * C + 4 * j) : Raw4<T>::zero();
      xc[i] = ok ? ((const float4*)(x + row * C))[j] : z4;
    }
  }
  for (int rr = wave; rr < LN_BWD_ROWS; rr += 4) {
    const int64_t row = r0 + rr;
    if (row >= M) break;
    float4 pc[LN_MAXV], xn[LN_MAXV];
    RawT dn[LN_MAXV];
    const int64_t nrow = row + 4;
    const bool more = rr + 4 < LN_BWD_ROWS && nrow < M;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const int j = lane + 64 * i;
      pc[i] = j < nv && accumulate ? ((const float4*)(dres + row * C))[j] : z4;
      dn[i] = j < nv && more ? Raw4<T>::load(dy + nrow * C + 4 * j) : Raw4<T>::zero();
      xn[i] = j < nv && more ? ((const float4*)(x + nrow * C))[j] : z4;
    }
    const float mu = mean[row], rs = rstd[row];
    float4 xh[LN_MAXV], g[LN_MAXV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const float4 d = Raw4<T>::f32(dc[i]), xv = xc[i];
      xh[i] = make_float4((xv.x - mu) * rs, (xv.y - mu) * rs, (xv.z - mu) * rs, (xv.w - mu) * rs);
      g[i] = make_float4(d.x * ww[i].x, d.y * ww[i].y, d.z * ww[i].z, d.w * ww[i].w);
      s1 += g[i].x + g[i].y + g[i].z + g[i].w;
      s2 += g[i].x * xh[i].x + g[i].y * xh[i].y + g[i].z * xh[i].z + g[i].w * xh[i].w;
      pw[i].x += d.x * xh[i].x; pw[i].y += d.y * xh[i].y;
      pw[i].z += d.z * xh[i].z; pw[i].w += d.w * xh[i].w;
      pb[i].x += d.x; pb[i].y += d.y; pb[i].z += d.z; pb[i].w += d.w;
    }
    const float m1 = wave_sum_dpp(s1) / C, m2 = wave_sum_dpp(s2) / C;
    float4* dres4 = (float4*)(dres + row * C);
    T* da = dres_act + row * C;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const int j = lane + 64 * i;
      if (j < nv) {
        float4 o;
        o.x = rs * (g[i].x - m1 - xh[i].x * m2) + pc[i].x;
        o.y = rs * (g[i].y - m1 - xh[i].y * m2) + pc[i].y;
        o.z = rs * (g[i].z - m1 - xh[i].z * m2) + pc[i].z;
        o.w = rs * (g[i].w - m1 - xh[i].w * m2) + pc[i].w;
        dres4[j] = o;
        if (dr.thresh) {
          // the gradient reaching the dropped-out branch output
          const float4 z = drop4(dr, (uint32_t)j, (uint32_t)row, 0);
          o.x *= z.x; o.y *= z.y; o.z *= z.z; o.w *= z.w;
        }
        store4<T>(da + 4 * j, o);
        pr[i].x += o.x; pr[i].y += o.y; pr[i].z += o.z; pr[i].w += o.w;
      }
    }
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      dc[i] = dn[i];
      xc[i] = xn[i];
    }
  }
  // reduce the 4 waves' partials through LDS (one wave at a time) and write
  // one partial row per block: part[blk][3][C]
  __shared__ float red[3 * LN_MAXV * 256];  // 3 x C floats
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

// Column sums of part [nrow][ncol] (ncol % 4 == 0, 16-byte aligned rows):
// each block takes 32 columns; its 256 threads are 8 float4 columns x 32 row
// groups, each with 4 independent loads in flight, then an LDS reduction.
// Column c goes to out_k[c % seg] with k = c / seg (seg % 4 == 0); with beta
// the sum is added to the output, else it replaces it.
__device__ __forceinline__ void colsum_finalize_block(const float* __restrict__ part, int nrow,
                                                      int ncol, int seg, float* out0, float* out1,
                                                      float* out2, int beta, int bx,
                                                      float4 (*red)[8]) {
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;
  const int c = bx * 32 + 4 * tx;
  float4 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < ncol) {
    int r = ty;
    for (; r + 96 < nrow; r += 128) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 v = *(const float4*)(part + (int64_t)(r + 32 * u) * ncol + c);
        acc[u].x += v.x; acc[u].y += v.y; acc[u].z += v.z; acc[u].w += v.w;
      }
    }
    for (; r < nrow; r += 32) {
      const float4 v = *(const float4*)(part + (int64_t)r * ncol + c);
      acc[0].x += v.x; acc[0].y += v.y; acc[0].z += v.z; acc[0].w += v.w;
    }
  }
  float4 t;
  t.x = (acc[0].x + acc[1].x) + (acc[2].x + acc[3].x);
  t.y = (acc[0].y + acc[1].y) + (acc[2].y + acc[3].y);
  t.z = (acc[0].z + acc[1].z) + (acc[2].z + acc[3].z);
  t.w = (acc[0].w + acc[1].w) + (acc[2].w + acc[3].w);
  red[ty][tx] = t;
  __syncthreads();
  if (threadIdx.x < 32) {
    // thread j sums column bx * 32 + j over the 32 row groups
    const int j = threadIdx.x, cc = bx * 32 + j;
    const float* rf = (const float*)red;
    float v = 0.f;
#pragma unroll 8
    for (int g = 0; g < 32; ++g) v += rf[g * 32 + j];
    if (cc < ncol) {
      const int k = cc / seg, i = cc % seg;
      float* o = k == 0 ? out0 : (k == 1 ? out1 : out2);
      if (o) o[i] = (beta ? o[i] : 0.f) + v;
    }
  }
}

__global__ __launch_bounds__(256) void colsum_finalize_kernel(const float* __restrict__ part,
                                                              int nrow, int ncol, int seg,
                                                              float* out0, float* out1,
                                                              float* out2, int beta) {
  __shared__ float4 red[32][8];
  colsum_finalize_block(part, nrow, ncol, seg, out0, out1, out2, beta, blockIdx.x, red);
}

// Several finalizes in one launch: job j owns blocks [blk0[j], blk0[j+1]).
// The table travels in the kernel arguments.
struct ColsumGroupArgs {
  ColsumJob job[COLSUM_GROUP_MAX];
  int blk0[COLSUM_GROUP_MAX + 1];
  int n, beta;
};
__global__ __launch_bounds__(256) void colsum_finalize_group_kernel(ColsumGroupArgs a) {
  __shared__ float4 red[32][8];
  const int bx = blockIdx.x;
  int j = 0;
  while (j + 1 < a.n && a.blk0[j + 1] <= bx) ++j;
  const ColsumJob& jb = a.job[j];
  colsum_finalize_block(jb.part, jb.nrow, jb.ncol, jb.seg, jb.out[0], jb.out[1], jb.out[2], a.beta,
                        bx - a.blk0[j], red);
}

// per-lane float4 count: C / 4 / 64 rounded up, so registers track the width
#define LN_DISPATCH(MACRO) \
  switch ((C / 4 + 63) / 64) {  \
    case 1: MACRO(1); break;    \
    case 2: MACRO(2); break;    \
    case 3: MACRO(3); break;    \
    case 4: MACRO(4); break;    \
    case 5: MACRO(5); break;    \
    case 6: MACRO(6); break;    \
    case 7: MACRO(7); break;    \
    default: MACRO(8); break;   \
  }

int layernorm_fwd_launch(bool h16, const float* x, const float* w, const float* b, void* y,
                         float* mean, float* rstd, int M, int C, hipStream_t s) {
  if (C % 4 || C > LN_MAXV_MAX * 256) return -5;
#define LNF(V)                                                                                  \
  if (h16)                                                                                      \
    hipLaunchKernelGGL((ln_fwd_kernel<h16_t, V>), dim3(cdiv(M, 4)), dim3(256), 0, s, x, w, b,  \
                       (h16_t*)y, mean, rstd, M, C);                                            \
  else                                                                                           \
    hipLaunchKernelGGL((ln_fwd_kernel<float, V>), dim3(cdiv(M, 4)), dim3(256), 0, s, x, w, b,   \
                       (float*)y, mean, rstd, M, C);
  LN_DISPATCH(LNF)
#undef LNF
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// partial rows written by one backward call (one per block)
int layernorm_bwd_part_rows(int M) { return (int)cdiv(M, LN_BWD_ROWS); }

// dres = (accumulate ? dres : 0) + LN'(dy); dres_act = z dres (z the dropout
// multipliers of dr, 1 without it: the output gradient of the dropped-out
// branch that feeds the residual); then dw, db (beta-accumulated) and
// bias_grad (+)= column sum of dres_act, if non-null.
int layernorm_bwd_launch(bool h16, const void* dy, const float* x, const float* mean,
                         const float* rstd, const float* w, float* dres, void* dres_act,
                         int accumulate, float* part, float* dw, float* db, float* bias_grad,
                         int beta, int M, int C, hipStream_t s, ColsumJob* defer, Drop dr) {
  if (C % 4 || C > LN_MAXV_MAX * 256) return -5;
  const int nb = (int)cdiv(M, LN_BWD_ROWS);
#define LNB(V)                                                                                   \
  if (h16)                                                                                       \
    hipLaunchKernelGGL((ln_bwd_kernel<h16_t, V>), dim3(nb), dim3(256), 0, s, (const h16_t*)dy, \
                       x, mean, rstd, w, dres, (h16_t*)dres_act, accumulate, part, M, C, dr);   \
  else                                                                                            \
    hipLaunchKernelGGL((ln_bwd_kernel<float, V>), dim3(nb), dim3(256), 0, s, (const float*)dy, x, \
                       mean, rstd, w, dres, (float*)dres_act, accumulate, part, M, C, dr);
  LN_DISPATCH(LNB)
#undef LNB
  if (defer) {
    defer->part = part;
    defer->out[0] = dw;
    defer->out[1] = db;
    defer->out[2] = bias_grad;
    defer->nrow = nb;
    defer->ncol = 3 * C;
    defer->seg = C;
  } else {
    hipLaunchKernelGGL(colsum_finalize_kernel, dim3(cdiv(3 * C, 32)), dim3(256), 0, s, part, nb,
                       3 * C, C, dw, db, bias_grad, beta);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int colsum_finalize_group_launch(const ColsumJob* jobs, int n, int beta, hipStream_t s) {
  for (int j0 = 0; j0 < n; j0 += COLSUM_GROUP_MAX) {
    ColsumGroupArgs a;
    a.n = std::min(n - j0, COLSUM_GROUP_MAX);
    a.beta = beta;
    int nblk = 0;
    for (int j = 0; j < a.n; ++j) {
      const ColsumJob& jb = jobs[j0 + j];
      if (!jb.part || jb.ncol % 4 || jb.seg < 1) return -5;
      a.job[j] = jb;
      a.blk0[j] = nblk;
      nblk += (int)cdiv(jb.ncol, 32);
    }
    a.blk0[a.n] = nblk;
    if (nblk > 0)
      hipLaunchKernelGGL(colsum_finalize_group_kernel, dim3(nblk), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return -4;
  }
  return 0;
}

int colsum_finalize_launch(const float* part, int nrow, int ncol, float* out, int beta,
                           hipStream_t s) {
  if (ncol % 4) return -5;
  hipLaunchKernelGGL(colsum_finalize_kernel, dim3(cdiv(ncol, 32)), dim3(256), 0, s, part, nrow,
                     ncol, ncol, out, nullptr, nullptr, beta);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace HALF_NS
