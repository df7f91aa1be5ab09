// Embedding, fused masked softmax cross-entropy, bias-gradient column sums,
// parameter initialisation from a seed.
#include "common.h"
#include "kernels.h"

namespace HALF_NS {

// ---------------------------------------------------------------- embedding
// x[b*T + t] = wte[idx] + wpe[t] ("nanoGPT" (stanleyjacob.dev), Part IV Stage
// 4: token embeddings plus learned position embeddings, then dropout).  An id
// outside [0, Vp) reads no memory: its token row is taken as zero and flag
// bit 1 set.
__global__ void embed_fwd_kernel(const int32_t* __restrict__ idx, const float* __restrict__ wte,
                                 const float* __restrict__ wpe, float* __restrict__ x, int M,
                                 int Tn, int C, int Vp, int* __restrict__ flags, Drop dr) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const int id = idx[row], t = row % Tn;
  const bool ok = id >= 0 && id < Vp;
  if (!ok && lane == 0) atomicOr(flags, 1);
  const float4* a = (const float4*)(wte + (int64_t)(ok ? id : 0) * C);
  const float4* p = (const float4*)(wpe + (int64_t)t * C);
  float4* o = (float4*)(x + row * C);
  for (int j = lane; j < C / 4; j += 64) {
    float4 v = p[j];
    if (ok) {
      const float4 w = a[j];
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    if (dr.thresh) {
      const float4 z = drop4(dr, (uint32_t)j, (uint32_t)row, 0);
      v.x *= z.x; v.y *= z.y; v.z *= z.z; v.w *= z.w;
    }
    o[j] = v;
  }
}

// y[m][c] = x[m][c] times the dropout multiplier of element (m, c)
// (C % 4 == 0; y may be x): for example the gradient that reaches a
// dropped-out value
__global__ void dropout_rows_kernel(const float* x, float* y, int64_t M, int C, Drop dr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nv = C >> 2;
  if (i >= M * nv) return;
  const int64_t row = i / nv;
  const int j = (int)(i % nv);
  float4 v = ((const float4*)x)[i];
  const float4 z = drop4(dr, (uint32_t)j, (uint32_t)row, 0);
  v.x *= z.x; v.y *= z.y; v.z *= z.z; v.w *= z.w;
  ((float4*)y)[i] = v;
}

// dwte[idx[m]] += dx[m], rows of one id added inside the workgroup first.
// A workgroup takes EMB_ROWS consecutive rows and sorts (id, row) in LDS
// (bitonic), so that equal ids form runs (cut every EMB_SUB sorted
// positions); a wave sums a run's rows in row order and makes one fp32
// atomic add per column.  A frequent id (Zipf-like
// text puts ~10 % of the tokens on one id) then costs one atomic per
// workgroup per column instead of one per row, which the memory side would
// serialise.  Runs of different workgroups still add in the order the
// hardware serves them, so the last bits can differ run to run.
#define EMB_ROWS 256
#define EMB_THREADS 1024  // 16 waves share a workgroup's runs (each run costs a load latency)
#define EMB_CPL 12        // columns a lane holds: C <= 64 * EMB_CPL
#define EMB_SUB 16        // longest run a wave sums
__global__ __launch_bounds__(EMB_THREADS) void embed_bwd_wte_runs_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ dx, float* __restrict__ dwte, int M,
    int C, int Vp) {
  __shared__ uint64_t key[EMB_ROWS];  // (id << 32) | local row; id 0xffffffff: no row
  __shared__ int runs[EMB_ROWS];      // sorted positions where a run starts
  __shared__ int nruns;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * EMB_ROWS;
  if (tid < EMB_ROWS) {
    uint32_t id = 0xffffffffu;
    if (r0 + tid < M) {
      const int v = idx[r0 + tid];
      if (v >= 0 && v < Vp) id = (uint32_t)v;
    }
    key[tid] = ((uint64_t)id << 32) | (uint32_t)tid;
  }
  if (tid == 0) nruns = 0;
  __syncthreads();
  for (int k = 2; k <= EMB_ROWS; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int q = tid ^ j;
      if (tid < EMB_ROWS && q > tid) {
        const uint64_t a = key[tid], b = key[q];
        if ((a > b) == ((tid & k) == 0)) {
          key[tid] = b;
          key[q] = a;
        }
      }
      __syncthreads();
    }
  // a run also restarts at every EMB_SUB-th sorted position, so that no wave
  // sums more than EMB_SUB rows one after another (a batch of one repeated
  // id would otherwise put all EMB_ROWS rows on one wave)
  if (tid < EMB_ROWS) {
    const uint32_t my = (uint32_t)(key[tid] >> 32);
    if (my != 0xffffffffu &&
        (tid % EMB_SUB == 0 || (uint32_t)(key[tid - 1] >> 32) != my))
      runs[atomicAdd(&nruns, 1)] = tid;
  }
  __syncthreads();
  const int n = nruns;
  for (int s = wave; s < n; s += EMB_THREADS / 64) {
    const int p0 = runs[s];
    const uint32_t rid = (uint32_t)(key[p0] >> 32);
    float acc[EMB_CPL];
#pragma unroll
    for (int i = 0; i < EMB_CPL; ++i) acc[i] = 0.f;
    for (int p = p0; p < EMB_ROWS && (uint32_t)(key[p] >> 32) == rid && (p == p0 || p % EMB_SUB);
         ++p) {
      const float* src = dx + (r0 + (int)(key[p] & 0xffffffffu)) * C;
      // every column of the row requested before any is added
      float v[EMB_CPL];
#pragma unroll
      for (int i = 0; i < EMB_CPL; ++i) v[i] = src[min(lane + 64 * i, C - 1)];
#pragma unroll
      for (int i = 0; i < EMB_CPL; ++i) acc[i] += v[i];
    }
    float* dst = dwte + (int64_t)rid * C;
#pragma unroll
    for (int i = 0; i < EMB_CPL; ++i)
      if (lane + 64 * i < C) unsafeAtomicAdd(dst + lane + 64 * i, acc[i]);
  }
}

// dwte[idx[m]] += dx[m] (fp32 atomics: rows of frequent ids add up in the
// order the hardware serves them, so the last bits can differ run to run).
__global__ void embed_bwd_wte_kernel(const int32_t* __restrict__ idx, const float* __restrict__ dx,
                                     float* __restrict__ dwte, int M, int C, int Vp) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const int id = idx[row];
  if (id < 0 || id >= Vp) return;
  const float* src = dx + row * C;
  float* dst = dwte + (int64_t)id * C;
  for (int j = lane; j < C; j += 64) unsafeAtomicAdd(dst + j, src[j]);
}

// dwpe[t] = (beta ? dwpe[t] : 0) + sum_b dx[b*T + t] for t < T; rows
// T..block_size-1 get (beta ? unchanged : 0).  Deterministic.
__global__ void embed_bwd_wpe_kernel(const float* __restrict__ dx, float* __restrict__ dwpe,
                                     int B, int Tn, int block_size, int C, int beta) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)block_size * C) return;
  const int t = i / C, c = i % C;
  float s = 0.f;
  if (t < Tn)
    for (int b = 0; b < B; ++b) s += dx[((int64_t)b * Tn + t) * C + c];
  dwpe[i] = (beta ? dwpe[i] : 0.f) + s;
}

// ---------------------------------------------------------------- cross-entropy
// count of targets in [0, V) (ignore_index = -1, "nanoGPT" Part IV Stage 4).
// A target outside [-1, V) names no class: it is counted as ignored (the
// cross-entropy kernels give its row zero loss and zero gradient too) and
// raises bit 2 of flags.
// One workgroup of 1024 threads: 16-byte loads where the targets are 16-byte
// aligned, so each thread has only a few loads in flight instead of a long
// chain of dependent round trips.
#define RED_THREADS 1024
__device__ __forceinline__ int valid_target(int y, int V, int& bad) {
  bad |= (y < -1) | (y >= V);
  return (y >= 0) & (y < V);
}
__global__ __launch_bounds__(RED_THREADS) void count_valid_kernel(const int32_t* __restrict__ tgt, int N,
                                                                  int V, int* __restrict__ out,
                                                                  int* __restrict__ flags) {
  __shared__ int red[RED_THREADS / 64];
  int c = 0, bad = 0;
  int done = 0;
  if (((uintptr_t)tgt & 15) == 0) {
    const int n4 = N >> 2;
#pragma unroll 4
    for (int i = threadIdx.x; i < n4; i += RED_THREADS) {
      const int4 v = ((const int4*)tgt)[i];
      c += valid_target(v.x, V, bad) + valid_target(v.y, V, bad) + valid_target(v.z, V, bad) +
           valid_target(v.w, V, bad);
    }
    done = n4 << 2;
  }
  for (int i = done + threadIdx.x; i < N; i += RED_THREADS) c += valid_target(tgt[i], V, bad);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if (bad && flags) atomicOr(flags, 2);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < RED_THREADS / 64; ++w) t += red[w];
    *out = t;
  }
}

// One row of logits per workgroup, read once into registers:
//   lse = log sum_{v < V} exp(z_v)  (padded columns v >= V are excluded),
//   row_loss = lse - z_y,
//   dz_v = scale * (exp(z_v - lse) - [v == y]) for v < V, 0 for V <= v < ldv,
// written over the logits ("Let's reproduce GPT-2 (124M)", chapter "Cross
// Entropy Loss"; scale = loss_scale / n_valid, zero for an ignored row).
#define CE_THREADS 1024    // fp32 kernel
#define CE_BF_THREADS 512  // 16-bit kernel: two rows in flight per compute unit
#define CE_BF_MAXU 13      // uint4 (8 16-bit) per thread: rows up to 53248 columns
template <int NT>
__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < NT / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One block per row; the row stays in registers.  Each thread takes the max
// m_t of its own columns and replaces every cached logit z by
// p = exp(z - m_t) (16-bit), adding the fp32 values into s_t.  The block then
// forms lse = M + log(sum_t s_t exp(m_t - M)) with M the row max, and the
// gradient is p * exp(m_t - lse) * scale; the thread holding the target
// column rewrites that one element as scale * (exp(z_y - lse) - 1).
// Columns >= V (padding) are cached as -inf, so every pass is branch-free.
__global__ __launch_bounds__(CE_BF_THREADS, 4) void ce_h16_kernel(
    h16_t* __restrict__ logits, const int32_t* __restrict__ tgt, float* __restrict__ row_loss,
    const int* __restrict__ n_valid, float loss_scale, const float* __restrict__ dscale, int V,
    int ldv, int write_grad) {
  __shared__ float red[CE_BF_THREADS / 64];
  const int64_t row = blockIdx.x;
  h16_t* z = logits + row * ldv;
  const int nvec = ldv >> 3;
  const int y = tgt[row];
  const bool has_y = y >= 0 && y < V;
  const float zy = has_y ? h2f(z[y]) : 0.f;
  const uint32_t NEG2 = H16_NEG_INF * 0x10001u;  // two 16-bit -inf
  // the row through one buffer descriptor (32-bit per-lane offsets, bounds
  // checked against the row length), so no per-slot 64-bit addresses
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(z, (short)0, ldv * 2, 0x00020000);
  const uint32_t voff = threadIdx.x * 16;
  uint4 cache[CE_BF_MAXU];
#pragma unroll
  for (int i = 0; i < CE_BF_MAXU; ++i) {
    const int vi = threadIdx.x + CE_BF_THREADS * i;
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + i * CE_BF_THREADS * 16, 0, 0);
    cache[i] = 8 * vi < V ? make_uint4(v.x, v.y, v.z, v.w) : make_uint4(NEG2, NEG2, NEG2, NEG2);
  }
  // when V % 8 != 0 one vector straddles V: its owner masks the columns >= V
  // (the slot index ip is the same for the whole block)
  const int vp = V >> 3, ip = vp / CE_BF_THREADS;
  if ((V & 7) && (int)threadIdx.x == vp % CE_BF_THREADS) {
#pragma unroll
    for (int k = 0; k < CE_BF_MAXU; ++k)
      if (k == ip) {
        uint32_t w[4] = {cache[k].x, cache[k].y, cache[k].z, cache[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = 8 * vp + 2 * j;
          if (col >= V) w[j] = (w[j] & 0xffff0000u) | H16_NEG_INF;
          if (col + 1 >= V) w[j] = (w[j] & 0x0000ffffu) | (H16_NEG_INF << 16);
        }
        cache[k] = make_uint4(w[0], w[1], w[2], w[3]);
      }
  }
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < CE_BF_MAXU; ++i) {
    mt = fmax_fast(fmax_fast(fmax_fast(mt, h_lo(cache[i].x)), h_hi(cache[i].x)), h_lo(cache[i].y));
    mt = fmax_fast(fmax_fast(fmax_fast(mt, h_hi(cache[i].y)), h_lo(cache[i].z)), h_hi(cache[i].z));
    mt = fmax_fast(fmax_fast(mt, h_lo(cache[i].w)), h_hi(cache[i].w));
  }
  // a thread without columns keeps mt = -inf and s_t = 0
  const float mref = mt == -INFINITY ? 0.f : mt;
  float st = 0.f;
#pragma unroll
  for (int i = 0; i < CE_BF_MAXU; ++i) {
    uint32_t w[4] = {cache[i].x, cache[i].y, cache[i].z, cache[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = __expf(h_lo(w[j]) - mref), b = __expf(h_hi(w[j]) - mref);
      st += a + b;
      w[j] = pack2h(a, b);
    }
    cache[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  const float M = block_reduce<CE_BF_THREADS>(mt, true, red);
  const float S = block_reduce<CE_BF_THREADS>(mt == -INFINITY ? 0.f : st * __expf(mt - M), false, red);
  const float lse = M + __logf(S);
  const int nv = *n_valid;
  const float scale =
      (has_y && nv > 0) ? loss_scale * (dscale ? *dscale : 1.f) / (float)nv : 0.f;
  if (!write_grad) {  // the loss alone (evaluation): the logits stay as they are
    if (threadIdx.x == 0) row_loss[row] = has_y ? lse - zy : 0.f;
    return;
  }
  const float c = scale * __expf(mref - lse);
#pragma unroll
  for (int i = 0; i < CE_BF_MAXU; ++i) {
    // slots past the row end lie outside the descriptor: the store is dropped
    const uint32_t w[4] = {cache[i].x, cache[i].y, cache[i].z, cache[i].w};
    const u32x4_t d = {pack2h(h_lo(w[0]) * c, h_hi(w[0]) * c),
                       pack2h(h_lo(w[1]) * c, h_hi(w[1]) * c),
                       pack2h(h_lo(w[2]) * c, h_hi(w[2]) * c),
                       pack2h(h_lo(w[3]) * c, h_hi(w[3]) * c)};
    __builtin_amdgcn_raw_buffer_store_b128(d, rs, voff + i * CE_BF_THREADS * 16, 0, 0);
  }
  // the same thread wrote the vector holding y just above, so this store
  // lands after it
  if (has_y && (int)threadIdx.x == (y >> 3) % CE_BF_THREADS)
    z[y] = f2h(scale * (__expf(zy - lse) - 1.0f));
  if (threadIdx.x == 0) row_loss[row] = has_y ? lse - zy : 0.f;
}

// Rows of at most 512 columns (the character-level vocabulary): one wave per
// row, four rows per workgroup, each lane holding 8 consecutive columns in
// registers; the same loss and gradient as above, the gradient formed
// directly as scale * (exp(z - lse) - [v == y]).
#define CE_SMALL_MAXV 512
__global__ __launch_bounds__(256) void ce_h16_small_kernel(
    h16_t* __restrict__ logits, const int32_t* __restrict__ tgt, float* __restrict__ row_loss,
    const int* __restrict__ n_valid, float loss_scale, const float* __restrict__ dscale, int N,
    int V, int ldv, int write_grad) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;  // uniform per wave
  h16_t* z = logits + row * ldv;
  const int y = tgt[row];
  const bool has_y = y >= 0 && y < V;
  const int c0 = 8 * lane;
  const bool mine = c0 < ldv;
  const uint4 raw = mine ? *(const uint4*)(z + c0) : make_uint4(0, 0, 0, 0);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
  float m = -INFINITY, zyl = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x = (j & 1) ? h_hi(w[j >> 1]) : h_lo(w[j >> 1]);
    v[j] = (c0 + j < V) ? x : -INFINITY;  // padding and lanes past the row: excluded
    m = fmax_fast(m, v[j]);
    zyl = (c0 + j == y) ? x : zyl;
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += __expf(v[j] - m);
  s = wave_sum(s);
  const float lse = m + __logf(s);
  const float zy = wave_sum(zyl);  // one lane holds z_y, the others add zero
  if (lane == 0) row_loss[row] = has_y ? lse - zy : 0.f;
  if (!write_grad || !mine) return;
  const int nv = *n_valid;
  const float scale =
      (has_y && nv > 0) ? loss_scale * (dscale ? *dscale : 1.f) / (float)nv : 0.f;
  float d[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    d[j] = (c0 + j < V) ? scale * (__expf(v[j] - lse) - (c0 + j == y ? 1.f : 0.f)) : 0.f;
  *(uint4*)(z + c0) =
      make_uint4(pack2h(d[0], d[1]), pack2h(d[2], d[3]), pack2h(d[4], d[5]), pack2h(d[6], d[7]));
}

// fp32 logits (fp32 mode): the same, reading the row from memory per pass.
__global__ __launch_bounds__(CE_THREADS) void ce_f32_kernel(
    float* __restrict__ logits, const int32_t* __restrict__ tgt, float* __restrict__ row_loss,
    const int* __restrict__ n_valid, float loss_scale, const float* __restrict__ dscale, int V,
    int ldv, int write_grad) {
  __shared__ float red[CE_THREADS / 64];
  const int64_t row = blockIdx.x;
  float* z = logits + row * ldv;
  float mx = -INFINITY;
  for (int c = threadIdx.x; c < V; c += CE_THREADS) mx = fmaxf(mx, z[c]);
  mx = block_reduce<CE_THREADS>(mx, true, red);
  float s = 0.f;
  for (int c = threadIdx.x; c < V; c += CE_THREADS) s += expf(z[c] - mx);
  s = block_reduce<CE_THREADS>(s, false, red);
  const float lse = mx + logf(s);
  const int y = tgt[row];
  const int nv = *n_valid;
  const bool has_y = y >= 0 && y < V;
  const float scale =
      (has_y && nv > 0) ? loss_scale * (dscale ? *dscale : 1.f) / (float)nv : 0.f;
  const float zy = has_y ? z[y] : 0.f;
  if (!write_grad) {
    if (threadIdx.x == 0) row_loss[row] = has_y ? lse - zy : 0.f;
    return;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < ldv; c += CE_THREADS)
    z[c] = c < V ? scale * (expf(z[c] - lse) - (c == y ? 1.f : 0.f)) : 0.f;
  if (threadIdx.x == 0) row_loss[row] = has_y ? lse - zy : 0.f;
}

// loss = sum(row_loss) / n_valid, single workgroup, fixed order.
// mean of the row losses over the valid rows, summed in fp64 in a fixed
// order (thread strides, then waves in order)
__global__ __launch_bounds__(RED_THREADS) void loss_finalize_kernel(const float* __restrict__ row_loss, int N,
                                                                    const int* __restrict__ n_valid,
                                                                    float* __restrict__ loss) {
  __shared__ double red[RED_THREADS / 64];
  double s = 0.0;
  int done = 0;
  if (((uintptr_t)row_loss & 15) == 0) {
    const int n4 = N >> 2;
#pragma unroll 4
    for (int i = threadIdx.x; i < n4; i += RED_THREADS) {
      const float4 v = ((const float4*)row_loss)[i];
      s += ((double)v.x + (double)v.y) + ((double)v.z + (double)v.w);
    }
    done = n4 << 2;
  }
  for (int i = done + threadIdx.x; i < N; i += RED_THREADS) s += row_loss[i];
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < RED_THREADS / 64; ++w) t += red[w];
    const int nv = *n_valid;
    *loss = nv > 0 ? (float)(t / nv) : 0.f;
  }
}

// out = mean of x[0..n), summed in fp64 in a fixed order (thread strides,
// then waves in order): the mean of evaluation batches' losses
__global__ __launch_bounds__(256) void mean_kernel(const float* __restrict__ x, int n,
                                                   float* __restrict__ out) {
  __shared__ double red[4];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += x[i];
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) *out = (float)((red[0] + red[1] + red[2] + red[3]) / n);
}

// ---------------------------------------------------------------- column sums
// part[rb][n] = sum of a[row][n] over the CS_ROWS rows of block-row rb
// (bias gradients: db = sum over tokens of dy).  Each thread owns 8
// consecutive columns (one 16-byte 16-bit load per row); the 4 waves split the
// rows and combine in LDS in a fixed order.
#define CS_ROWS 256
template <typename T>
__global__ __launch_bounds__(256) void colsum_part_kernel(const T* __restrict__ a, int M, int N,
                                                          float* __restrict__ part) {
  __shared__ float red[4][64 * 8];
  const int lane = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 64 + lane) * 8;
  const int r0 = blockIdx.y * CS_ROWS, r1 = min(M, r0 + CS_ROWS);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (n0 < N) {
    for (int r = r0 + rg; r < r1; r += 4) {
      const T* p = a + (int64_t)r * N + n0;
      if constexpr (sizeof(T) == 2) {
        const uint4 v = *(const uint4*)p;
        const uint32_t* w = (const uint32_t*)&v;
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += h2f((h16_t)(w[e >> 1] >> (16 * (e & 1))));
      } else {
        const float4 v0 = *(const float4*)p, v1 = *(const float4*)(p + 4);
        s[0] += v0.x; s[1] += v0.y; s[2] += v0.z; s[3] += v0.w;
        s[4] += v1.x; s[5] += v1.y; s[6] += v1.z; s[7] += v1.w;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][lane * 8 + e] = s[e];
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int n = blockIdx.x * 512 + i;
    if (n < N) part[(int64_t)blockIdx.y * N + n] = red[0][i] + red[1][i] + red[2][i] + red[3][i];
  }
}

// ---------------------------------------------------------------- initialisation
// Parameters drawn on the device from a seed ("Let's reproduce GPT-2 (124M)",
// chapter "Model Initialization"; "nanoGPT" Part V Deep dive 1): every
// Linear weight and both embedding tables N(0, 0.02^2), the two projections
// per block that write into the residual stream N(0, (0.02 / sqrt(2 L))^2),
// biases 0, LayerNorm gains 1 and shifts 0.  The table of pieces carries the
// standard deviation or the constant of each piece.
// Element i takes normal number i % 4 of Philox4x32-10 at counter
// {i / 4 (low, high words), 'INIT', 0} under the 64-bit seed: the two pairs of
// 32-bit words become two pairs of normals by the Box-Muller transform
// (Box and Muller, 1958): r = sqrt(-2 ln u1), (r cos 2 pi u2, r sin 2 pi u2)
// with u1 in (0, 1), u2 in [0, 1).  The values depend only on the element's
// position and the seed, not on how the table cuts the tensors.
__device__ __forceinline__ void box_muller(uint32_t a, uint32_t b, float& n0, float& n1) {
  const float u1 = ((float)(a >> 8) + 0.5f) * (1.0f / 16777216.0f);  // (0, 1)
  const float u2 = (float)(b >> 8) * (1.0f / 16777216.0f);           // [0, 1)
  const float r = sqrtf(-2.0f * logf(u1));
  float sn, cs;
  sincosf(6.283185307179586f * u2, &sn, &cs);
  n0 = r * cs;
  n1 = r * sn;
}

__global__ __launch_bounds__(256) void init_params_kernel(float* __restrict__ p,
                                                          const InitSeg* __restrict__ segs,
                                                          uint32_t k0, uint32_t k1) {
  const InitSeg sg = segs[blockIdx.x];
  for (int j = 4 * (int)threadIdx.x; j < sg.count; j += 4 * 256) {
    const int64_t i = sg.offset + j;
    float4 o;
    if (sg.std > 0.f) {
      const uint64_t q = (uint64_t)i >> 2;
      const uint4 w = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), 0x494E4954u, 0u, k0, k1);
      float n0, n1, n2, n3;
      box_muller(w.x, w.y, n0, n1);
      box_muller(w.z, w.w, n2, n3);
      o = make_float4(n0 * sg.std, n1 * sg.std, n2 * sg.std, n3 * sg.std);
    } else {
      o = make_float4(sg.value, sg.value, sg.value, sg.value);
    }
    *(float4*)(p + i) = o;
  }
}

// ---------------------------------------------------------------- fused head + cross-entropy
// The head's forward epilogue left p~ = exp(z) in the logits buffer,
// part[m][0..npart) (sums of p~ over blocks of 96 columns below V) and zy[m]
// (the target's logit).  Per row: S = sum of the parts (lane-strided, then a
// fixed-order wave sum), so log S = logsumexp_{v<V} z_v ("Let's reproduce
// GPT-2 (124M)", chapter "Cross Entropy Loss"); row_loss = log S - zy for a
// target in [0, V) (0 otherwise); sc = loss_scale * dscale / n_valid for such
// a row (0 otherwise) and r = sc / S.  The target's column of the buffer
// becomes exp(zy) - S, so that the logit gradient sc (softmax - onehot) is r
// times the stored row; h2[m] = r * h[m] in 16 bits (the weight gradient's
// token-side operand).  p~ overflows or vanishes for logits beyond about
// +-80: a valid row with S outside [1e-28, 1e28] raises flag bit 4.
#define HEAD_MAXP 9  // row-sum blocks per lane: npart <= 576 (rows of up to 55296 columns)
#define HEAD_MAXH 4  // 16-byte chunks of x per lane: C <= 2048
__global__ __launch_bounds__(256) void head_combine_kernel(
    const float* __restrict__ part, int npart, const float* __restrict__ zy,
    const int32_t* __restrict__ tgt, int V, const int* __restrict__ n_valid, float loss_scale,
    const float* __restrict__ dscale, const h16_t* __restrict__ h, int C,
    float* __restrict__ row_loss, float* __restrict__ r_out, h16_t* __restrict__ h2,
    h16_t* __restrict__ logits, int ldv, int M, int* __restrict__ flags) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;  // uniform per wave
  const float* pr = part + row * npart;
  // every load issued before any is used (indices clamped into the row, the
  // extra values masked to zero): the same per-lane order as a strided loop
  float pv[HEAD_MAXP];
#pragma unroll
  for (int i = 0; i < HEAD_MAXP; ++i) pv[i] = pr[min(lane + 64 * i, npart - 1)];
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < HEAD_MAXP; ++i) acc += lane + 64 * i < npart ? pv[i] : 0.f;
  const float S = wave_sum(acc);
  const int y = tgt[row];
  const bool valid = y >= 0 && y < V;
  const int nv = *n_valid;
  const float sc = (valid && nv > 0) ? loss_scale * (dscale ? *dscale : 1.f) / (float)nv : 0.f;
  const float r = sc / S;
  if (lane == 0) {
    const float z = valid ? zy[row] : 0.f;
    row_loss[row] = valid ? __logf(S) - z : 0.f;
    r_out[row] = r;
    if (valid) logits[row * ldv + y] = f2h(__expf(z) - S);
    if (valid && !(S >= 1e-28f && S <= 1e28f)) atomicOr(flags, 4);
  }
  const h16_t* hr = h + row * C;
  h16_t* o = h2 + row * C;
  uint4 hv[HEAD_MAXH];
#pragma unroll
  for (int i = 0; i < HEAD_MAXH; ++i) hv[i] = *(const uint4*)(hr + 8 * min(lane + 64 * i, C / 8 - 1));
#pragma unroll
  for (int i = 0; i < HEAD_MAXH; ++i) {
    const int j = lane + 64 * i;
    if (j < C / 8) {
      const uint32_t u[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
      uint32_t q[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) q[k] = pack2h(r * h_lo(u[k]), r * h_hi(u[k]));
      *(uint4*)(o + 8 * j) = make_uint4(q[0], q[1], q[2], q[3]);
    }
  }
}

// ---------------------------------------------------------------- launchers
int colsum_finalize_launch(const float* part, int nrow, int ncol, float* out, int beta,
                           hipStream_t s);

int head_combine_launch(const float* part, int npart, const float* zy, const int32_t* tgt, int V,
                        const int* n_valid, float loss_scale, const float* dscale, const h16_t* h,
                        int C, float* row_loss, float* r, h16_t* h2, h16_t* logits, int ldv, int M,
                        int* flags, hipStream_t s) {
  if (C % 8 || C > 8 * 64 * HEAD_MAXH || npart < 1 || npart > 64 * HEAD_MAXP) return -5;
  hipLaunchKernelGGL(head_combine_kernel, dim3(cdiv(M, 4)), dim3(256), 0, s, part, npart, zy, tgt, V,
                     n_valid, loss_scale, dscale, h, C, row_loss, r, h2, logits, ldv, M, flags);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mean_launch(const float* x, int n, float* out, hipStream_t s) {
  if (n < 1) return -5;
  hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(256), 0, s, x, n, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int init_params_launch(float* params, const InitSeg* segs, int nsegs, uint64_t seed,
                       hipStream_t s) {
  if (nsegs <= 0) return 0;
  hipLaunchKernelGGL(init_params_kernel, dim3(nsegs), dim3(256), 0, s, params, segs,
                     (uint32_t)seed, (uint32_t)(seed >> 32));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int embed_fwd_launch(const int32_t* idx, const float* wte, const float* wpe, float* x, int M,
                     int Tn, int C, int Vp, int* flags, hipStream_t s, Drop dr) {
  hipLaunchKernelGGL(embed_fwd_kernel, dim3(cdiv(M, 4)), dim3(256), 0, s, idx, wte, wpe, x, M, Tn,
                     C, Vp, flags, dr);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int dropout_rows_launch(const float* x, float* y, int64_t M, int C, Drop dr, hipStream_t s) {
  if (M <= 0) return 0;
  if (C % 4) return -5;
  if (!dr.thresh) {
    if (x == y) return 0;
    return hipMemcpyAsync(y, x, (size_t)M * C * 4, hipMemcpyDeviceToDevice, s) == hipSuccess ? 0
                                                                                           : -4;
  }
  hipLaunchKernelGGL(dropout_rows_kernel, dim3(cdiv(M * (C / 4), 256)), dim3(256), 0, s, x, y, M,
                     C, dr);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int embed_bwd_launch(const int32_t* idx, const float* dx, float* dwte, float* dwpe, int B, int Tn,
                     int block_size, int C, int Vp, int beta_wpe, hipStream_t s) {
  const int M = B * Tn;
  if (C <= 64 * EMB_CPL)
    hipLaunchKernelGGL(embed_bwd_wte_runs_kernel, dim3(cdiv(M, EMB_ROWS)), dim3(EMB_THREADS), 0, s, idx,
                       dx, dwte, M, C, Vp);
  else
    hipLaunchKernelGGL(embed_bwd_wte_kernel, dim3(cdiv(M, 4)), dim3(256), 0, s, idx, dx, dwte, M, C,
                       Vp);
  hipLaunchKernelGGL(embed_bwd_wpe_kernel, dim3(cdiv((int64_t)block_size * C, 256)), dim3(256), 0,
                     s, dx, dwpe, B, Tn, block_size, C, beta_wpe);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int count_valid_launch(const int32_t* tgt, int N, int V, int* out, int* flags, hipStream_t s) {
  hipLaunchKernelGGL(count_valid_kernel, dim3(1), dim3(RED_THREADS), 0, s, tgt, N, V, out, flags);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int cross_entropy_launch(bool h16, void* logits, const int32_t* tgt, float* row_loss,
                         const int* n_valid, float loss_scale, const float* dscale, int N, int V,
                         int ldv, hipStream_t s, int write_grad) {
  if (h16 && ldv % 8 == 0 && ldv <= CE_SMALL_MAXV) {
    hipLaunchKernelGGL(ce_h16_small_kernel, dim3(cdiv(N, 4)), dim3(256), 0, s, (h16_t*)logits,
                       tgt, row_loss, n_valid, loss_scale, dscale, N, V, ldv, write_grad);
  } else if (h16) {
    if (ldv % 8 || ldv > CE_BF_MAXU * CE_BF_THREADS * 8) return -5;
    hipLaunchKernelGGL(ce_h16_kernel, dim3(N), dim3(CE_BF_THREADS), 0, s, (h16_t*)logits, tgt,
                       row_loss, n_valid, loss_scale, dscale, V, ldv, write_grad);
  } else {
    hipLaunchKernelGGL(ce_f32_kernel, dim3(N), dim3(CE_THREADS), 0, s, (float*)logits, tgt,
                       row_loss, n_valid, loss_scale, dscale, V, ldv, write_grad);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int loss_finalize_launch(const float* row_loss, int N, const int* n_valid, float* loss,
                         hipStream_t s) {
  hipLaunchKernelGGL(loss_finalize_kernel, dim3(1), dim3(RED_THREADS), 0, s, row_loss, N, n_valid, loss);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int colsum_part_rows(int M) { return (int)cdiv(M, CS_ROWS); }

// out (+)= column sums of a [M][N] (N % 8 == 0); part: fp32 scratch
// [colsum_part_rows(M)][N].
int colsum_launch(bool h16, const void* a, int M, int N, float* part, float* out, int beta,
                  hipStream_t s) {
  if (N % 8) return -5;
  const int nb = colsum_part_rows(M);
  if (h16)
    hipLaunchKernelGGL(colsum_part_kernel<h16_t>, dim3(cdiv(N, 512), nb), dim3(256), 0, s,
                       (const h16_t*)a, M, N, part);
  else
    hipLaunchKernelGGL(colsum_part_kernel<float>, dim3(cdiv(N, 512), nb), dim3(256), 0, s,
                       (const float*)a, M, N, part);
  if (hipGetLastError() != hipSuccess) return -4;
  return colsum_finalize_launch(part, nb, N, out, beta, s);
}

}  // namespace HALF_NS
