// Global-norm gradient clipping and one multi-tensor AdamW update.
//
// "andrej-karpathy-lets-reproduce-gpt-2" (youtube.nixfred.com), the
// optimization recipe: AdamW with betas (0.9, 0.95) and eps 1e-8, gradients
// clipped at a global norm of 1.0, weight decay 0.1 on the 2-D parameters
// only, one fused kernel rather than one launch per tensor.  Readings where
// the pages give no formula: coef = min(1, max_norm / (norm + 1e-6)); decay
// is decoupled, p <- p (1 - lr wd) before the Adam step; eps is added
// outside the square root; bias correction uses the 1-based step t.
#include "common.h"
#include "kernels.h"  // AdamChunk: {first element, count (multiple of 4), decay flag}

namespace HALF_NS {

// sum of squares, fp64 partial per block
__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ g, int64_t n,
                                                    double* __restrict__ part) {
  __shared__ double red[4];
  double s = 0.0;
  const int64_t nv = n >> 2;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += (int64_t)gridDim.x * 256) {
    const float4 v = ((const float4*)g)[i];
    // squared in fp64: a finite fp32 value squares to a finite fp64 one, so
    // the sum is non-finite exactly when some element is inf or NaN
    const double x = v.x, y = v.y, z = v.z, w = v.w;
    s += x * x + y * y + z * z + w * w;
  }
  if (blockIdx.x == 0)
    for (int64_t i = 4 * nv + threadIdx.x; i < n; i += 256) s += (double)g[i] * g[i];
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// scal[0] = clip coefficient, scal[1] = 1 if the norm is not finite
__global__ void norm_finalize_kernel(const double* __restrict__ part, int nblk, float max_norm,
                                     float* __restrict__ norm_out, float* __restrict__ scal) {
  __shared__ double red[4];
  double s = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 256) s += part[i];
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double norm = sqrt(red[0] + red[1] + red[2] + red[3]);
    const bool finite = isfinite(norm);
    double coef = 1.0;
    if (max_norm > 0.f && finite) coef = fmin(1.0, (double)max_norm / (norm + 1e-6));
    scal[0] = (float)coef;
    scal[1] = finite ? 0.f : 1.f;
    if (norm_out) *norm_out = (float)norm;
  }
}

// Dynamic loss scaling ("nanoGPT", Part IV Stage 5 and Part V Deep dive 2;
// "Let's reproduce GPT-2 (124M)", chapter "Float16, Gradient Scalers, BF16"):
// the gradients hold the true gradient times the scale S.  From the norm of
// the scaled gradients: norm = norm_s / S (the norm of the unscaled ones),
// found_inf = norm_s not finite (an inf or NaN element; a sum of squares of
// finite fp32 values cannot overflow fp64), coef = min(1, max_norm /
// (norm + 1e-6)); scal[0] = coef / S (the factor the update applies to the
// stored gradient), scal[1] = found_inf, scal[2..3] = the bias corrections
// 1 - beta^t at t = steps + 1.  Then the scale update: an overflow multiplies
// S by the backoff factor and restarts the count of clean steps; a clean step
// counts an update and, when the count reaches the interval, multiplies S by
// the growth factor (kept only if finite) and restarts the count.
struct ScalerState {
  float scale;
  int32_t growth_tracker, steps, found_inf;
};
__global__ void amp_finalize_kernel(const double* __restrict__ part, int nblk, float max_norm,
                                    float beta1, float beta2, ScalerState* __restrict__ st,
                                    float growth, float backoff, int interval,
                                    float* __restrict__ norm_out, float* __restrict__ scal) {
  __shared__ double red[4];
  double s = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 256) s += part[i];
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    ScalerState q = *st;
    const double inv = 1.0 / (double)q.scale;
    const double norm = sqrt(red[0] + red[1] + red[2] + red[3]) * inv;
    const bool found_inf = !isfinite(norm);
    double coef = 1.0;
    if (max_norm > 0.f && !found_inf) coef = fmin(1.0, (double)max_norm / (norm + 1e-6));
    const double t = (double)(q.steps + 1);
    scal[0] = (float)(coef * inv);
    scal[1] = found_inf ? 1.f : 0.f;
    scal[2] = (float)(1.0 - pow((double)beta1, t));
    scal[3] = (float)(1.0 - pow((double)beta2, t));
    if (norm_out) *norm_out = (float)norm;
    if (found_inf) {
      q.scale *= backoff;
      q.growth_tracker = 0;
    } else {
      q.steps += 1;
      if (++q.growth_tracker == interval) {
        const float grown = q.scale * growth;
        if (isfinite(grown)) q.scale = grown;
        q.growth_tracker = 0;
      }
    }
    q.found_inf = found_inf ? 1 : 0;
    *st = q;
  }
}

// The AdamW update of one element ("Let's reproduce GPT-2 (124M)", chapter
// "AdamW, Gradient Clipping"; PyTorch's order: decoupled decay first, then
// the bias-corrected step with eps outside the square root).  coef: the clip
// (and unscale) factor; decay = 1 - lr * wd for decayed tensors, else 1.
__device__ __forceinline__ void adamw_elem(float& pk, float gk_raw, float& mk, float& vk,
                                           float coef, float beta1, float beta2, float eps,
                                           float decay, float step, float rbc2) {
  // no multiply-add contraction: every kernel that applies the update (flat
  // chunks or matrix tiles, vector or scalar code) rounds the same way
#pragma clang fp contract(off)
  const float gk = gk_raw * coef;
  mk = beta1 * mk + (1.0f - beta1) * gk;
  vk = beta2 * vk + (1.0f - beta2) * gk * gk;
  const float denom = sqrtf(vk) * rbc2 + eps;  // sqrt(v / bc2) + eps
  pk = pk * decay - step * mk / denom;
}

// One chunk per workgroup.  16-bit copy of the updated weights written when
// shadow != nullptr.  bc_in_scal: the bias corrections come from scal[2..3]
// (the loss-scaled step, whose step count lives on the device).
__global__ __launch_bounds__(256) void adamw_kernel(
    float* __restrict__ p, const float* __restrict__ g, float* __restrict__ m,
    float* __restrict__ v, h16_t* __restrict__ shadow, const AdamChunk* __restrict__ chunks,
    const float* __restrict__ scal, float lr, float beta1, float beta2, float eps, float wd,
    float bc1, float bc2, int skip_nonfinite, int bc_in_scal) {
  if (skip_nonfinite && scal[1] != 0.f) return;
  if (bc_in_scal) {
    bc1 = scal[2];
    bc2 = scal[3];
  }
  const AdamChunk ch = chunks[blockIdx.x];
  const float coef = scal[0];
  const float decay = ch.decay ? 1.0f - lr * wd : 1.0f;
  const float step = lr / bc1;
  const float rbc2 = 1.0f / sqrtf(bc2);
  for (int i = threadIdx.x; i < ch.count / 4; i += 256) {
    const int64_t e = ch.offset / 4 + i;
    float4 pp = ((float4*)p)[e], gg = ((const float4*)g)[e];
    float4 mm = ((float4*)m)[e], vv = ((float4*)v)[e];
    float* pa = &pp.x;
    float* ga = &gg.x;
    float* ma = &mm.x;
    float* va = &vv.x;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      adamw_elem(pa[k], ga[k], ma[k], va[k], coef, beta1, beta2, eps, decay, step, rbc2);
    ((float4*)p)[e] = pp;
    ((float4*)m)[e] = mm;
    ((float4*)v)[e] = vv;
    if (shadow) *(uint2*)(shadow + 4 * e) = make_uint2(pack2h(pp.x, pp.y), pack2h(pp.z, pp.w));
  }
}

// AdamW over the weight matrices that have transposed 16-bit copies (every
// one of them 2-D, so decayed), one 64 x 64 tile per workgroup: the update of
// adamw_kernel, the 16-bit copy in the parameters' layout, and the same
// 16-bit values transposed through LDS into the copy that the input-gradient
// products read, so no separate transpose pass follows the step.  A job is a
// matrix [rows][cols] at element offset src of the parameters (and of the
// copy), transposed to dstT + dst with leading dimension ld.
__global__ __launch_bounds__(256) void adamw_tile_kernel(
    float* __restrict__ p, const float* __restrict__ g, float* __restrict__ m,
    float* __restrict__ v, h16_t* __restrict__ shadow, h16_t* __restrict__ dstT,
    const TransposeJob* __restrict__ jobs, int njobs, const float* __restrict__ scal, float lr,
    float beta1, float beta2, float eps, float wd, float bc1, float bc2, int skip_nonfinite,
    int bc_in_scal) {
  if (skip_nonfinite && scal[1] != 0.f) return;
  if (bc_in_scal) {
    bc1 = scal[2];
    bc2 = scal[3];
  }
  __shared__ __attribute__((aligned(16))) h16_t tile[64][72];
  int j = 0;
  while (j + 1 < njobs && (int)blockIdx.x >= jobs[j + 1].tile_begin) ++j;
  const TransposeJob job = jobs[j];
  const int t = blockIdx.x - job.tile_begin;
  const int tiles_c = (job.cols + 63) / 64;
  const int r0 = (t / tiles_c) * 64, c0 = (t % tiles_c) * 64;
  const float coef = scal[0];
  const float decay = 1.0f - lr * wd;
  const float step = lr / bc1;
  const float rbc2 = 1.0f / sqrtf(bc2);
  h16_t* D = dstT + job.dst;
  const bool full = r0 + 64 <= job.rows && c0 + 64 <= job.cols && job.cols % 8 == 0 &&
                    job.ld % 8 == 0 && job.src % 8 == 0 && job.dst % 8 == 0;
  if (full) {
    // 16 threads x 4 values cover a 64-value tile row: four passes of 16
    // rows, every load of the four issued before any is used.  The outputs
    // are read again only by the next step: non-temporal stores.
    float4 P4[4], G4[4], M4[4], V4[4];
    int64_t E4[4];
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int r = (threadIdx.x >> 4) + 16 * pass, c4 = 4 * (threadIdx.x & 15);
      E4[pass] = (job.src + (int64_t)(r0 + r) * job.cols + c0 + c4) / 4;
      P4[pass] = ((float4*)p)[E4[pass]];
      G4[pass] = ((const float4*)g)[E4[pass]];
      M4[pass] = ((float4*)m)[E4[pass]];
      V4[pass] = ((float4*)v)[E4[pass]];
    }
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int r = (threadIdx.x >> 4) + 16 * pass, c4 = 4 * (threadIdx.x & 15);
      const int64_t e = E4[pass];
      float4 pp = P4[pass], gg = G4[pass];
      float4 mm = M4[pass], vv = V4[pass];
      float* pa = &pp.x;
      const float* ga = &gg.x;
      float* ma = &mm.x;
      float* va = &vv.x;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        adamw_elem(pa[k], ga[k], ma[k], va[k], coef, beta1, beta2, eps, decay, step, rbc2);
      st_nt((float4*)p + e, pp);
      st_nt((float4*)m + e, mm);
      st_nt((float4*)v + e, vv);
      const uint2 w = make_uint2(pack2h(pp.x, pp.y), pack2h(pp.z, pp.w));
      st_nt(shadow + 4 * e, w);
      *(uint2*)&tile[r][c4] = w;
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int oc = (threadIdx.x >> 3) + 32 * pass, r8 = 8 * (threadIdx.x & 7);
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = (uint32_t)tile[r8 + 2 * k][oc] | ((uint32_t)tile[r8 + 2 * k + 1][oc] << 16);
      st_nt(D + (int64_t)(c0 + oc) * job.ld + r0 + r8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  } else {
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
      const int r = i / 64, c = i % 64;
      if (r0 + r < job.rows && c0 + c < job.cols) {
        const int64_t e = job.src + (int64_t)(r0 + r) * job.cols + c0 + c;
        float pk = p[e], mk = m[e], vk = v[e];
        adamw_elem(pk, g[e], mk, vk, coef, beta1, beta2, eps, decay, step, rbc2);
        p[e] = pk;
        m[e] = mk;
        v[e] = vk;
        const h16_t hv = f2h(pk);
        shadow[e] = hv;
        tile[r][c] = hv;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
      const int c = i / 64, r = i % 64;  // output row c, column r
      if (r0 + r < job.rows && c0 + c < job.cols) D[(int64_t)(c0 + c) * job.ld + r0 + r] = tile[r][c];
    }
  }
}

// fp32 -> 16-bit copy of the weights
__global__ void to_h16_kernel(const float* __restrict__ p, h16_t* __restrict__ o, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    o[i] = f2h(p[i]);
}

#define NORM_BLOCKS 1024
int adamw_norm_blocks() { return NORM_BLOCKS; }

int adamw_launch(float* p, const float* g, float* m, float* v, h16_t* shadow, int64_t n,
                 const AdamChunk* chunks, int nchunks, const TileJobs& tj, double* norm_part,
                 float* scal, float* norm_out, float lr, float beta1, float beta2, float eps,
                 float wd, float max_norm, int t, int skip_nonfinite, hipStream_t s) {
  hipLaunchKernelGGL(sumsq_kernel, dim3(NORM_BLOCKS), dim3(256), 0, s, g, n, norm_part);
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(1), dim3(256), 0, s, norm_part, NORM_BLOCKS,
                     max_norm, norm_out, scal);
  const float bc1 = (float)(1.0 - pow((double)beta1, (double)t));
  const float bc2 = (float)(1.0 - pow((double)beta2, (double)t));
  if (nchunks > 0)
    hipLaunchKernelGGL(adamw_kernel, dim3(nchunks), dim3(256), 0, s, p, g, m, v, shadow, chunks,
                       scal, lr, beta1, beta2, eps, wd, bc1, bc2, skip_nonfinite, 0);
  if (tj.ntiles > 0)
    hipLaunchKernelGGL(adamw_tile_kernel, dim3(tj.ntiles), dim3(256), 0, s, p, g, m, v, shadow,
                       tj.dstT, tj.jobs, tj.njobs, scal, lr, beta1, beta2, eps, wd, bc1, bc2,
                       skip_nonfinite, 0);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int adamw_amp_launch(float* p, const float* g, float* m, float* v, h16_t* shadow, int64_t n,
                     const AdamChunk* chunks, int nchunks, const TileJobs& tj,
                     double* norm_part, float* scal,
                     float* norm_out, float lr, float beta1, float beta2, float eps, float wd,
                     float max_norm, float* scaler, float growth, float backoff, int interval,
                     hipStream_t s) {
  hipLaunchKernelGGL(sumsq_kernel, dim3(NORM_BLOCKS), dim3(256), 0, s, g, n, norm_part);
  hipLaunchKernelGGL(amp_finalize_kernel, dim3(1), dim3(256), 0, s, norm_part, NORM_BLOCKS,
                     max_norm, beta1, beta2, (ScalerState*)scaler, growth, backoff, interval,
                     norm_out, scal);
  if (nchunks > 0)
    hipLaunchKernelGGL(adamw_kernel, dim3(nchunks), dim3(256), 0, s, p, g, m, v, shadow, chunks,
                       scal, lr, beta1, beta2, eps, wd, 1.f, 1.f, 1, 1);
  if (tj.ntiles > 0)
    hipLaunchKernelGGL(adamw_tile_kernel, dim3(tj.ntiles), dim3(256), 0, s, p, g, m, v, shadow,
                       tj.dstT, tj.jobs, tj.njobs, scal, lr, beta1, beta2, eps, wd, 1.f, 1.f, 1, 1);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int to_h16_launch(const float* p, h16_t* o, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(to_h16_kernel, dim3(2048), dim3(256), 0, s, p, o, n);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Transposed 16-bit copies of the weight matrices, so that the input-gradient
// products dX = dY W read both operands along the reduction dimension.
// One launch over a table of matrices; 64 x 64 tiles through LDS, moved with
// 16-byte loads and stores (a tile that is partial or not 8-aligned goes
// element by element).
__global__ __launch_bounds__(256) void transpose_h16_kernel(const h16_t* __restrict__ src,
                                                             h16_t* __restrict__ dst,
                                                             const TransposeJob* __restrict__ jobs,
                                                             int njobs) {
  __shared__ __attribute__((aligned(16))) h16_t tile[64][72];
  int j = 0;
  while (j + 1 < njobs && (int)blockIdx.x >= jobs[j + 1].tile_begin) ++j;
  const TransposeJob job = jobs[j];
  const int t = blockIdx.x - job.tile_begin;
  const int tiles_c = (job.cols + 63) / 64;
  const int r0 = (t / tiles_c) * 64, c0 = (t % tiles_c) * 64;
  const h16_t* S = src + job.src;
  h16_t* D = dst + job.dst;
  const bool full = r0 + 64 <= job.rows && c0 + 64 <= job.cols && job.cols % 8 == 0 &&
                    job.ld % 8 == 0 && job.src % 8 == 0 && job.dst % 8 == 0;
  if (full) {
    // 256 threads x 16 bytes cover 32 rows: two passes in, two passes out
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int r = (threadIdx.x >> 3) + 32 * pass, c8 = 8 * (threadIdx.x & 7);
      *(uint4*)&tile[r][c8] = *(const uint4*)(S + (int64_t)(r0 + r) * job.cols + c0 + c8);
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int oc = (threadIdx.x >> 3) + 32 * pass, r8 = 8 * (threadIdx.x & 7);
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = (uint32_t)tile[r8 + 2 * k][oc] | ((uint32_t)tile[r8 + 2 * k + 1][oc] << 16);
      *(uint4*)(D + (int64_t)(c0 + oc) * job.ld + r0 + r8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
      const int r = i / 64, c = i % 64;
      if (r0 + r < job.rows && c0 + c < job.cols) tile[r][c] = S[(int64_t)(r0 + r) * job.cols + c0 + c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
      const int c = i / 64, r = i % 64;  // output row c, column r
      if (r0 + r < job.rows && c0 + c < job.cols) D[(int64_t)(c0 + c) * job.ld + r0 + r] = tile[r][c];
    }
  }
}

int transpose_h16_launch(const h16_t* src, h16_t* dst, const TransposeJob* jobs, int njobs,
                          int total_tiles, hipStream_t s) {
  hipLaunchKernelGGL(transpose_h16_kernel, dim3(total_tiles), dim3(256), 0, s, src, dst, jobs, njobs);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace HALF_NS
