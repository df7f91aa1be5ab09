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

// sum of squares, fp64 partial per block
__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ g, int64_t n,
                                                    double* __restrict__ part) {
  __shared__ double red[4];
  double s = 0.0;
  const int64_t nv = n >> 2;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += (int64_t)gridDim.x * 256) {
    const float4 v = ((const float4*)g)[i];
    s += (double)(v.x * v.x) + (double)(v.y * v.y) + (double)(v.z * v.z) + (double)(v.w * v.w);
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

// One chunk per workgroup.  bf16 copy of the updated weights written when
// shadow != nullptr.
__global__ __launch_bounds__(256) void adamw_kernel(
    float* __restrict__ p, const float* __restrict__ g, float* __restrict__ m,
    float* __restrict__ v, bf16_t* __restrict__ shadow, const AdamChunk* __restrict__ chunks,
    const float* __restrict__ scal, float lr, float beta1, float beta2, float eps, float wd,
    float bc1, float bc2, int skip_nonfinite) {
  if (skip_nonfinite && scal[1] != 0.f) return;
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
    for (int k = 0; k < 4; ++k) {
      const float gk = ga[k] * coef;
      ma[k] = beta1 * ma[k] + (1.0f - beta1) * gk;
      va[k] = beta2 * va[k] + (1.0f - beta2) * gk * gk;
      const float denom = sqrtf(va[k]) * rbc2 + eps;  // sqrt(v / bc2) + eps
      pa[k] = pa[k] * decay - step * ma[k] / denom;
    }
    ((float4*)p)[e] = pp;
    ((float4*)m)[e] = mm;
    ((float4*)v)[e] = vv;
    if (shadow) *(uint2*)(shadow + 4 * e) = make_uint2(pack2bf(pp.x, pp.y), pack2bf(pp.z, pp.w));
  }
}

// fp32 -> bf16 copy of the weights
__global__ void to_bf16_kernel(const float* __restrict__ p, bf16_t* __restrict__ o, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    o[i] = f2bf(p[i]);
}

#define NORM_BLOCKS 1024
int adamw_norm_blocks() { return NORM_BLOCKS; }

int adamw_launch(float* p, const float* g, float* m, float* v, bf16_t* shadow, int64_t n,
                 const AdamChunk* chunks, int nchunks, double* norm_part, float* scal,
                 float* norm_out, float lr, float beta1, float beta2, float eps, float wd,
                 float max_norm, int t, int skip_nonfinite, hipStream_t s) {
  hipLaunchKernelGGL(sumsq_kernel, dim3(NORM_BLOCKS), dim3(256), 0, s, g, n, norm_part);
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(1), dim3(256), 0, s, norm_part, NORM_BLOCKS,
                     max_norm, norm_out, scal);
  const float bc1 = (float)(1.0 - pow((double)beta1, (double)t));
  const float bc2 = (float)(1.0 - pow((double)beta2, (double)t));
  hipLaunchKernelGGL(adamw_kernel, dim3(nchunks), dim3(256), 0, s, p, g, m, v, shadow, chunks,
                     scal, lr, beta1, beta2, eps, wd, bc1, bc2, skip_nonfinite);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int to_bf16_launch(const float* p, bf16_t* o, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(to_bf16_kernel, dim3(2048), dim3(256), 0, s, p, o, n);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Transposed bf16 copies of the weight matrices, so that the input-gradient
// products dX = dY W read both operands along the reduction dimension.
// One launch over a table of matrices; 64 x 64 tiles through LDS, moved with
// 16-byte loads and stores (a tile that is partial or not 8-aligned goes
// element by element).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t* __restrict__ src,
                                                             bf16_t* __restrict__ dst,
                                                             const TransposeJob* __restrict__ jobs,
                                                             int njobs) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[64][72];
  int j = 0;
  while (j + 1 < njobs && (int)blockIdx.x >= jobs[j + 1].tile_begin) ++j;
  const TransposeJob job = jobs[j];
  const int t = blockIdx.x - job.tile_begin;
  const int tiles_c = (job.cols + 63) / 64;
  const int r0 = (t / tiles_c) * 64, c0 = (t % tiles_c) * 64;
  const bf16_t* S = src + job.src;
  bf16_t* D = dst + job.dst;
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

int transpose_bf16_launch(const bf16_t* src, bf16_t* dst, const TransposeJob* jobs, int njobs,
                          int total_tiles, hipStream_t s) {
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(total_tiles), dim3(256), 0, s, src, dst, jobs, njobs);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
