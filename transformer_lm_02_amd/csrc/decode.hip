// Sampling from the model with a key/value cache.
//
// "nanoGPT" (stanleyjacob.dev), Part IV, one generation (sample.py +
// model.py, generate): per new token the context is cropped to block_size,
// the last position's logits are divided by the temperature, everything below
// the top-k cutoff is removed, and one token is drawn from the softmax.  "Build
// GPT from scratch" (learn.byteknotlabs.com), exercise "Add a KV cache": the
// keys and values of earlier positions are kept, so a step feeds one new token
// per sequence and its cost no longer grows with the whole forward.
//
// Cache layout (the mode's activation type): kv[layer][k|v][b][h][t][hs],
// t < max_len.  A sequence's keys for one head are contiguous, so the
// attention of one new query streams them in order.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace HALF_NS {

namespace {

// keys and values of rows [0, T) of every sequence (qkv [B*T][3C], head h at
// columns h*hs of the k and v blocks) into cache positions pos0 + t
template <typename T>
__global__ void kv_store_kernel(const T* __restrict__ qkv, T* __restrict__ kv, int B, int Tn,
                                int H, int hs, int max_len, int pos0) {
  const int C = H * hs;
  const int64_t n = (int64_t)B * Tn * 2 * C;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % (2 * C));  // column inside the k|v blocks
  const int64_t row = i / (2 * C);   // b * Tn + t
  const int b = (int)(row / Tn), t = (int)(row % Tn);
  const int which = c / C, h = (c % C) / hs, e = c % hs;
  const int64_t dst = ((((int64_t)which * B + b) * H + h) * max_len + pos0 + t) * hs + e;
  kv[dst] = qkv[row * 3 * C + C + c];
}

// One new query per sequence and head against cache positions [0, len).  A
// workgroup of DEC_WAVES waves takes one (sequence, head); wave w takes the
// 64-position chunks w, w + DEC_WAVES, ...: lanes are positions for the
// scores (each lane a whole key row), an online softmax over the chunks, then
// lanes are head dimensions for p . V (one coalesced value row per position).
// The waves' (max, sum, output) are merged through LDS in wave order.
#define DEC_WAVES 16
template <typename T>
__device__ __forceinline__ float dot_row(const float* __restrict__ q, const T* __restrict__ r, int hs) {
  float s = 0.f;
  if constexpr (sizeof(T) == 2) {
    if ((hs & 7) == 0) {
      for (int e = 0; e < hs; e += 8) {
        const uint4 v = *(const uint4*)(r + e);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s = fmaf(q[e + 2 * j], h_lo(w[j]), s);
          s = fmaf(q[e + 2 * j + 1], h_hi(w[j]), s);
        }
      }
      return s;
    }
  }
  for (int e = 0; e < hs; ++e) s = fmaf(q[e], ldf(r + e), s);
  return s;
}

template <typename T>
__global__ __launch_bounds__(64 * DEC_WAVES) void decode_attn_kernel(const T* __restrict__ qkv,
                                                                     const T* __restrict__ kv,
                                                                     T* __restrict__ out, int B, int H,
                                                                     int hs, int max_len, int len) {
  __shared__ float qs[128];
  __shared__ float pw[DEC_WAVES][64];          // a chunk's probabilities, per wave
  __shared__ float ml[DEC_WAVES][2];           // per-wave running max and sum
  __shared__ float ow[DEC_WAVES][128];         // per-wave output
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int C = H * hs;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float scale = 1.0f / sqrtf((float)hs);
  if (tid < hs) qs[tid] = ldf(qkv + (int64_t)b * 3 * C + h * hs + tid) * scale;
  __syncthreads();
  const T* K = kv + (((int64_t)0 * B + b) * H + h) * (int64_t)max_len * hs;
  const T* V = kv + (((int64_t)1 * B + b) * H + h) * (int64_t)max_len * hs;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;  // o: head dims lane, lane + 64
  for (int c0 = wave * 64; c0 < len; c0 += DEC_WAVES * 64) {
    const int t = c0 + lane;
    const float s = t < len ? dot_row(qs, K + (int64_t)t * hs, hs) : -INFINITY;
    const float mc = wave_max(s);
    const float mn = fmaxf(m, mc);
    const float alpha = __expf(m - mn);  // 0 on the first chunk (m = -inf)
    const float p = t < len ? __expf(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    o0 *= alpha;
    o1 *= alpha;
    m = mn;
    pw[wave][lane] = p;
    __builtin_amdgcn_wave_barrier();
    const int nt = min(64, len - c0);
    const T* vr = V + (int64_t)c0 * hs;
    // 8 value rows in flight at a time (the loads do not depend on o)
    const int e0 = min(lane, hs - 1), e1 = min(lane + 64, hs - 1);
    int j = 0;
    for (; j + 8 <= nt; j += 8) {
      float v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v0[u] = ldf(vr + (int64_t)(j + u) * hs + e0);
        v1[u] = hs > 64 ? ldf(vr + (int64_t)(j + u) * hs + e1) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float pj = pw[wave][j + u];
        o0 = fmaf(pj, v0[u], o0);
        o1 = fmaf(pj, v1[u], o1);
      }
    }
    for (; j < nt; ++j) {
      const float pj = pw[wave][j];
      o0 = fmaf(pj, ldf(vr + (int64_t)j * hs + e0), o0);
      if (hs > 64) o1 = fmaf(pj, ldf(vr + (int64_t)j * hs + e1), o1);
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (lane == 0) {
    ml[wave][0] = m;
    ml[wave][1] = l;
  }
  if (lane < hs) ow[wave][lane] = o0;
  if (lane + 64 < hs) ow[wave][lane + 64] = o1;
  __syncthreads();
  if (tid < hs) {
    float M = -INFINITY;
    for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, ml[w][0]);
    float L = 0.f, O = 0.f;
    for (int w = 0; w < DEC_WAVES; ++w) {
      if (ml[w][0] == -INFINITY) continue;  // a wave with no positions
      const float f = __expf(ml[w][0] - M);
      L += ml[w][1] * f;
      O += ow[w][tid] * f;
    }
    stf(out + (int64_t)b * C + h * hs + tid, O / L);
  }
}

// Head width 64 in a 16-bit type (the GPT-2 family), the same work and
// merge as above with every load of a chunk requested at once, so that a
// chunk costs one memory latency: lane t holds key row c0 + t (eight 16-byte
// loads), and for p . V lane l holds head dims 2(l % 32) and 2(l % 32) + 1 of
// value rows c0 + 32(l / 32) + i, i < 32 (32 four-byte loads, each
// instruction two 128-byte rows); the halves are added at the end.  Key rows
// past len are read at len - 1, value rows where they are (the cache's slack
// keeps them inside it), and both weigh 0.  The first
// chunk's loads are issued before the query is staged, the next chunk's after
// the current one is consumed.
#define DEC64_WAVES 8  // a chunk's rows in flight take 64 registers a lane
template <typename T>
__global__ __launch_bounds__(64 * DEC64_WAVES) void decode_attn64_kernel(const T* __restrict__ qkv,
                                                                       const T* __restrict__ kv,
                                                                       T* __restrict__ out, int B,
                                                                       int H, int max_len, int len) {
  static_assert(sizeof(T) == 2, "16-bit activations");
  constexpr int hs = 64;
  __shared__ float qs[hs];
  __shared__ float pw[DEC64_WAVES][64];
  __shared__ float ml[DEC64_WAVES][2];
  __shared__ float ow[DEC64_WAVES][hs];
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int C = H * hs;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const T* K = kv + ((int64_t)b * H + h) * (int64_t)max_len * hs;
  const T* V = kv + (((int64_t)B + b) * H + h) * (int64_t)max_len * hs;
  const int dp = lane & 31, hf = lane >> 5;
  // (a clamped index rather than a guarded load, which would be waited on
  // before the chunk's loads are issued)
  const float qv = ldf(qkv + (int64_t)b * 3 * C + h * hs + min(tid, hs - 1));
  uint4 kr[8];
  uint32_t vr[32];
  auto issue = [&](int c0) {
    const uint4* kp = (const uint4*)(K + (int64_t)min(c0 + lane, len - 1) * hs);
#pragma unroll
    for (int i = 0; i < 8; ++i) kr[i] = kp[i];
    // value rows at one address and immediate offsets, past len too: the
    // cache ends in 64 rows of slack, so even the last sequence and head
    // stay inside it; such rows are zeroed where they are used
    const T* vb = V + (int64_t)(c0 + 32 * hf) * hs + 2 * dp;
#pragma unroll
    for (int i = 0; i < 32; ++i) vr[i] = *(const uint32_t*)(vb + i * hs);
  };
  int c0 = wave * 64;
  if (c0 < len) issue(c0);
  if (tid < hs) qs[tid] = qv * 0.125f;  // 1 / sqrt(64)
  __syncthreads();
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (; c0 < len; c0 += DEC64_WAVES * 64) {
    float sc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc = fmaf(qs[8 * i + 2 * j], h_lo(w[j]), sc);
        sc = fmaf(qs[8 * i + 2 * j + 1], h_hi(w[j]), sc);
      }
    }
    const bool valid = c0 + lane < len;
    sc = valid ? sc : -INFINITY;
    const float mn = fmaxf(m, wave_max(sc));
    const float alpha = __expf(m - mn);  // 0 on the first chunk (m = -inf)
    const float p = valid ? __expf(sc - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    o0 *= alpha;
    o1 *= alpha;
    m = mn;
    pw[wave][lane] = p;
    __builtin_amdgcn_wave_barrier();
    // rows at or past len hold stale or uninitialised memory (0 x NaN would
    // not vanish): they read as zero
    const int vrow0 = c0 + 32 * hf;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float pj = pw[wave][32 * hf + i];
      const uint32_t vv = vrow0 + i < len ? vr[i] : 0u;
      o0 = fmaf(pj, h_lo(vv), o0);
      o1 = fmaf(pj, h_hi(vv), o1);
    }
    __builtin_amdgcn_wave_barrier();
    if (c0 + DEC64_WAVES * 64 < len) issue(c0 + DEC64_WAVES * 64);
  }
  o0 += __shfl_xor(o0, 32, 64);
  o1 += __shfl_xor(o1, 32, 64);
  if (lane == 0) {
    ml[wave][0] = m;
    ml[wave][1] = l;
  }
  if (lane < 32) {
    ow[wave][2 * dp] = o0;
    ow[wave][2 * dp + 1] = o1;
  }
  __syncthreads();
  if (tid < hs) {
    float M = -INFINITY;
    for (int w = 0; w < DEC64_WAVES; ++w) M = fmaxf(M, ml[w][0]);
    float L = 0.f, O = 0.f;
    for (int w = 0; w < DEC64_WAVES; ++w) {
      if (ml[w][0] == -INFINITY) continue;  // a wave with no positions
      const float f = __expf(ml[w][0] - M);
      L += ml[w][1] * f;
      O += ow[w][tid] * f;
    }
    stf(out + (int64_t)b * C + h * hs + tid, O / L);
  }
}

// ---------------------------------------------------------------- few-row products
// out[m][n] = epi(sum_k A[m][k] W[n][k]) for the M <= GEMV_MAX_M rows of a
// decode step (one per sequence), W [N][K] in the mode's activation type.
// Every workgroup stages the rows in LDS: rows given in the activation type
// are copied; with LN the rows are the LayerNorm of fp32 rows x, computed
// with the forward's formula (mean, biased variance, eps 1e-5) and rounded
// like its output.  Each wave takes NC
// consecutive columns, lanes split K in 8-element chunks (16-byte weight
// loads), and a wave reduction finishes every (column, row) sum.
// up to 4 rows (one per sequence): past that the tiled products are faster
// (measured: B = 8 and 16 decode steps take longer through this kernel)
#define GEMV_MAX_M 4
#define GEMV_MAX_K_LN 2048  // LayerNorm rows are held in registers: K / 256 per thread
#define GEMV_LDS_BYTES (64 * 1024)
#define GEMV_PRE 6     // chunks of 512 columns of K requested first: plain rows
#define GEMV_PRE_LN 2  // and rows that are normalised first
enum { GV_ACT = 0, GV_F32 = 1, GV_RESID = 2, GV_GELU = 3 };
struct GemvArgs {
  const void* A;  // act [M][K], or fp32 [M][K] with LN
  const float* lnw;
  const float* lnb;
  const void* W;
  const float* bias;
  const float* aux;  // GV_RESID: fp32 [M][ldo]
  void* out;         // act (GV_ACT, GV_GELU: gelu(u)) or fp32 (GV_F32, GV_RESID) [M][ldo]
  int M, N, K, ldo;
  // q|k|v projection: columns [C, 3C) also go to the cache at position pos
  void* kv;
  int H, hs, max_len, pos, C;
};

// 8 consecutive elements as they are loaded (16 bytes of a 16-bit type, 32
// of fp32), unpacked to floats only where they are used
template <typename T>
struct Raw8 {
  uint4 w[sizeof(T) / 2];
};
template <typename T>
__device__ __forceinline__ Raw8<T> raw8(const T* p) {
  Raw8<T> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.w[i] = ((const uint4*)p)[i];
  return r;
}
template <typename T>
__device__ __forceinline__ void unpack8(const Raw8<T>& r, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = h_lo(w[j]);
      v[2 * j + 1] = h_hi(w[j]);
    }
  } else {
    const uint32_t w[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w,
                           r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(w[j]);
  }
}
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  unpack8(raw8(p), v);
}

template <typename T, int EPI, bool LN, int NC>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char gv_lds[];
  T* As = (T*)gv_lds;  // [M][K]: the rows, or their LayerNorm, staged in LDS
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = a.M, K = a.K;
  const int n0 = (blockIdx.x * 4 + wave) * NC;
  const T* W = (const T*)a.W;
  // Chunk i of a lane is K columns [8 lane + 512 i, +8).  The weights of the
  // first PRE chunks are requested before the rows are staged, so that their
  // latency overlaps the staging.  Loads take no branch of their own (the
  // compiler would wait on each): a chunk past K reads columns K - 8.. and
  // is not used, a wave past the last column reads column N - 1 and stores
  // nothing.
  constexpr int PRE = LN ? GEMV_PRE_LN : GEMV_PRE;
  Raw8<T> wpre[NC][PRE];
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    if (512 * i < K) {
      const int k = min(8 * lane + 512 * i, K - 8);
#pragma unroll
      for (int c = 0; c < NC; ++c) wpre[c][i] = raw8(W + (int64_t)min(n0 + c, a.N - 1) * K + k);
    }
  }
  if constexpr (LN) {
    // the whole workgroup normalises the M rows: thread t holds elements
    // t + 256 j of every row; each row's sum, then its sum of centred
    // squares, goes through the waves' partials in LDS.  Rows past M repeat
    // row M - 1 and are not stored.
    constexpr int PT = GEMV_MAX_K_LN / 256;
    __shared__ float red[GEMV_MAX_M][4];
    const float* x = (const float*)a.A;
    float xv[GEMV_MAX_M][PT], gv[PT], bv[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int k = tid + 256 * j, kc = min(k, K - 1);
      const float gg = a.lnw[kc], bb = a.lnb[kc];
      gv[j] = k < K ? gg : 0.f;
      bv[j] = k < K ? bb : 0.f;
#pragma unroll
      for (int m = 0; m < GEMV_MAX_M; ++m) {
        const float xx = x[(int64_t)min(m, M - 1) * K + kc];
        xv[m][j] = k < K ? xx : 0.f;
      }
    }
    float mean[GEMV_MAX_M], rstd[GEMV_MAX_M];
    // (reductions only for the M rows: a uniform branch, no load inside)
#pragma unroll
    for (int m = 0; m < GEMV_MAX_M; ++m) {
      if (m >= M) break;
      float t = 0.f;
#pragma unroll
      for (int j = 0; j < PT; ++j) t += xv[m][j];
      t = wave_sum(t);
      if (lane == 0) red[m][wave] = t;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < GEMV_MAX_M; ++m) mean[m] = (red[m][0] + red[m][1] + red[m][2] + red[m][3]) / K;
    __syncthreads();  // red is reused
#pragma unroll
    for (int m = 0; m < GEMV_MAX_M; ++m) {
      if (m >= M) break;
      float t = 0.f;
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const float c = tid + 256 * j < K ? xv[m][j] - mean[m] : 0.f;
        t += c * c;
      }
      t = wave_sum(t);
      if (lane == 0) red[m][wave] = t;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < GEMV_MAX_M; ++m)
      rstd[m] = 1.0f / sqrtf((red[m][0] + red[m][1] + red[m][2] + red[m][3]) / K + 1e-5f);
#pragma unroll
    for (int m = 0; m < GEMV_MAX_M; ++m) {
      if (m < M) {
#pragma unroll
        for (int j = 0; j < PT; ++j) {
          const int k = tid + 256 * j;
          if (k < K) stf(As + m * K + k, (xv[m][j] - mean[m]) * rstd[m] * gv[j] + bv[j]);
        }
      }
    }
  } else {
    // a plain copy of the M rows, 8 elements a thread per pass, every load
    // issued before the first store
    constexpr int MAXP = GEMV_LDS_BYTES / (256 * 8 * (int)sizeof(T));
    const T* A = (const T*)a.A;
    const int total = M * K;  // a multiple of 8, at most MAXP passes
    Raw8<T> st[MAXP];
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (p * 2048 < total) st[p] = raw8(A + min(p * 2048 + 8 * tid, total - 8));
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
      const int e = p * 2048 + 8 * tid;
      if (p * 2048 < total && e < total) *(Raw8<T>*)(As + e) = st[p];
    }
  }
  __syncthreads();
  if (n0 >= a.N) return;
  float acc[NC][GEMV_MAX_M];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int m = 0; m < GEMV_MAX_M; ++m) acc[c][m] = 0.f;
  auto fma_chunk = [&](int i, const Raw8<T> (&wr)[NC]) {
    const int k = 8 * lane + 512 * i;
    if (k < K) {
      float w[NC][8];
#pragma unroll
      for (int c = 0; c < NC; ++c) unpack8(wr[c], w[c]);
#pragma unroll
      for (int m = 0; m < GEMV_MAX_M; ++m) {
        if (m < M) {
          float x[8];
          load8(As + m * K + k, x);
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[c][m] = fmaf(x[j], w[c][j], acc[c][m]);
        }
      }
    }
  };
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    if (512 * i < K) {
      Raw8<T> wr[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) wr[c] = wpre[c][i];
      fma_chunk(i, wr);
    }
  }
  for (int i = PRE; 512 * i < K; ++i) {
    const int k = min(8 * lane + 512 * i, K - 8);
    Raw8<T> wr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) wr[c] = raw8(W + (int64_t)min(n0 + c, a.N - 1) * K + k);
    fma_chunk(i, wr);
  }
  // lane c*M + m finishes (column n0 + c, row m)
  float v = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int m = 0; m < GEMV_MAX_M; ++m) {
      if (m < M) {
        const float t = wave_sum(acc[c][m]);
        if (lane == c * M + m) v = t;
      }
    }
  if (lane >= NC * M) return;
  const int c = lane / M, m = lane % M, n = n0 + c;
  if (n >= a.N) return;
  const float u = v + (a.bias ? a.bias[n] : 0.f);
  const int64_t o = (int64_t)m * a.ldo + n;
  if constexpr (EPI == GV_F32) {
    ((float*)a.out)[o] = u;
  } else if constexpr (EPI == GV_RESID) {
    ((float*)a.out)[o] = a.aux[o] + u;
  } else if constexpr (EPI == GV_GELU) {
    stf((T*)a.out + o, gelu_f(u));
  } else {
    stf((T*)a.out + o, u);
    if (a.kv && n >= a.C) {
      const int which = (n - a.C) / a.C, h = ((n - a.C) % a.C) / a.hs, e = n % a.hs;
      T* dst = (T*)a.kv + ((((int64_t)which * M + m) * a.H + h) * a.max_len + a.pos) * a.hs + e;
      stf(dst, u);
    }
  }
}

// ---------------------------------------------------------------- sampling
// One workgroup per row.  z = logits / temperature over the first V ids; the
// top-k cutoff is the k-th largest z, found by a radix select on the
// order-preserving 32-bit keys of the floats; ids with z >= cutoff are kept;
// e = exp(z - max); the token is the first id whose running sum of e exceeds
// u * sum(e).  Wave w owns the ids [w*SEG, (w+1)*SEG) and lane l the ids
// w*SEG + 64 j + l (coalesced loads, held in registers), so the search for
// the token goes by segments (a scan of the 16 wave sums), then by rows of 64
// consecutive ids inside the segment, then by lanes (a wave scan).
#define SAMP_THREADS 1024
#define SAMP_PER 56                    // rows of 64 ids per wave
#define SAMP_SEG (SAMP_PER * 64)       // ids per wave: rows of up to 16 x 3584 = 57344 ids
#define SAMP_BINS 4096
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// inclusive prefix sum across the 64 lanes
__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__global__ __launch_bounds__(SAMP_THREADS) void sample_kernel(const float* __restrict__ logits,
                                                               int V, int ldv, float inv_temp,
                                                               int top_k, const float* __restrict__ u,
                                                               int32_t* __restrict__ tok) {
  __shared__ uint32_t hist[SAMP_BINS];
  __shared__ uint32_t cscan[SAMP_THREADS];
  __shared__ float fred[SAMP_THREADS / 64];
  __shared__ float fsum[SAMP_THREADS / 64];  // apart from fred: no barrier between their uses
  __shared__ uint32_t sel[3];  // [0]: key prefix found so far, [1]: rank still to find,
                               // [2]: 1 once the prefix's bin holds exactly that rank
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float* z = logits + (int64_t)row * ldv;
  const int seg0 = wave * SAMP_SEG;
  // -1 unless a draw lands below: no kept mass to draw from (a NaN or +inf
  // logit makes the total NaN), or a uniform that is negative or NaN.  The
  // barriers of the reductions below order this store before the draw's.
  if (tid == 0) tok[row] = -1;
  // every load issued before any is used: a clamped index (masked
  // afterwards, so no load sits in a branch of its own) as a 32-bit byte
  // offset from the row (one address register each), and a scheduling
  // barrier that keeps the loads ahead of the arithmetic
  float zv[SAMP_PER];
#pragma unroll
  for (int j = 0; j < SAMP_PER; ++j) {
    const uint32_t off = (uint32_t)min(seg0 + 64 * j + lane, V - 1) * 4u;
    zv[j] = *(const float*)((const char*)z + off);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < SAMP_PER; ++j) zv[j] = seg0 + 64 * j + lane < V ? zv[j] * inv_temp : -INFINITY;

  // maximum (the softmax reference)
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < SAMP_PER; ++j) mx = fmaxf(mx, zv[j]);
  mx = wave_max(mx);
  if (lane == 0) fred[wave] = mx;
  __syncthreads();
  mx = fred[0];
  for (int w = 1; w < SAMP_THREADS / 64; ++w) mx = fmaxf(mx, fred[w]);
  // from here on an element is its order-preserving key, 0 past V (no
  // float has key 0 but one NaN pattern), so that no test of its id and no
  // second copy of the keys is held across the passes
  uint32_t kz[SAMP_PER];
#pragma unroll
  for (int j = 0; j < SAMP_PER; ++j) kz[j] = seg0 + 64 * j + lane < V ? order_key(zv[j]) : 0u;

  // cutoff: the key of the k-th largest value, by a radix select over the
  // key bits in passes of 12, 12 and 8 (a histogram of 4096 bins spreads the
  // clustered leading bits of similar logits, so few atomics collide); the
  // bin holding the rank is found by a block-wide suffix scan of the bins
  uint32_t cut_key = 0u;  // keeps everything
  if (top_k > 0 && top_k < V) {
    if (tid == 0) {
      sel[0] = 0u;
      sel[1] = (uint32_t)top_k;
      sel[2] = 0u;
    }
    for (int pass = 0; pass < 3; ++pass) {
      const int width = pass < 2 ? 12 : 8, shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
      const int nb = 1 << width;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (shift + width));
      for (int t = tid; t < SAMP_BINS; t += SAMP_THREADS) hist[t] = 0u;
      __syncthreads();
      const uint32_t prefix = sel[0];
#pragma unroll
      for (int j = 0; j < SAMP_PER; ++j) {
        const uint32_t k = kz[j];
        if (k != 0u && (k & hi_mask) == prefix)
          atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1u);
      }
      __syncthreads();
      // thread t owns bins [t*bpt, (t+1)*bpt); suffix sums over the lanes of
      // a wave (shuffles), then over the waves (one barrier)
      const int bpt = nb / SAMP_THREADS > 0 ? nb / SAMP_THREADS : 1;
      const int b0 = tid * bpt;
      uint32_t own = 0u;
      for (int b = b0; b < b0 + bpt && b < nb; ++b) own += hist[b];
      uint32_t suf = own;  // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += t;
      }
      if (lane == 0) cscan[wave] = suf;  // the wave's total
      __syncthreads();
      uint32_t later = 0u;  // bins of later waves (higher digits)
      for (int w = wave + 1; w < SAMP_THREADS / 64; ++w) later += cscan[w];
      const uint32_t rank = sel[1];
      const uint32_t incl = later + suf, above = incl - own;  // in higher bins than this thread's
      __syncthreads();
      if (b0 < nb && above < rank && rank <= incl) {
        uint32_t acc = above;
        int dgt = b0;
        for (int b = min(b0 + bpt, nb) - 1; b >= b0; --b) {
          if (acc + hist[b] >= rank) {
            dgt = b;
            break;
          }
          acc += hist[b];
        }
        sel[0] = prefix | ((uint32_t)dgt << shift);
        sel[1] = rank - acc;
        // every value of the bin is kept: the prefix with its lower bits 0
        // keeps exactly them and all above, so the later passes can go
        sel[2] = rank - acc == hist[dgt];
      }
      __syncthreads();
      if (sel[2]) break;
    }
    cut_key = sel[0];
  }

  // e of the kept ids (key >= cutoff; ids past V have key 0); the sum of
  // each wave's segment
  const uint32_t keep_k = max(cut_key, 1u);
  float wsum = 0.f;
#pragma unroll
  for (int j = 0; j < SAMP_PER; ++j) {
    zv[j] = kz[j] >= keep_k ? __expf(key_value(kz[j]) - mx) : 0.f;
    wsum += zv[j];
  }
  wsum = wave_sum(wsum);
  if (lane == 0) fsum[wave] = wsum;
  __syncthreads();
  float total = 0.f, before = 0.f;
  for (int w = 0; w < SAMP_THREADS / 64; ++w) {
    if (w < wave) before += fsum[w];
    total += fsum[w];
  }
  const float target = u[row] * total;
  // the wave whose segment crosses the target (a target at or past the total,
  // by rounding, goes to the last wave with a kept id) walks its rows, then
  // its lanes
  const float incl = before + fsum[wave];
  bool last_kept = true;
  for (int w = wave + 1; w < SAMP_THREADS / 64; ++w) last_kept = last_kept && fsum[w] == 0.f;
  const bool crosses = before <= target && target < incl;
  const bool overflow = target >= total && fsum[wave] > 0.f && last_kept;
  if (crosses || overflow) {
    // rows in groups of 8: group sums, then the rows of one group, then the
    // lanes of one row; the reductions of a level are independent of each
    // other.  In the overflow case the last kept id is taken instead.
    constexpr int RG = 8, NG = SAMP_PER / RG;
    static_assert(SAMP_PER % RG == 0, "whole row groups");
    float gs[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float t = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) t += zv[g * RG + r];
      gs[g] = wave_sum(t);
    }
    float acc = before;
    int gsel = -1, glast = -1;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (gs[g] > 0.f) glast = g;
      if (gsel < 0 && acc + gs[g] > target) gsel = g;
      if (gsel < 0) acc += gs[g];
    }
    if (gsel < 0) {  // overflow (rounding): the last group with a kept id
      gsel = glast;
      acc = -INFINITY;
    }
    float rz[RG], rsum[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      float v = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) v = g == gsel ? zv[g * RG + r] : v;
      rz[r] = v;
      rsum[r] = wave_sum(v);
    }
    int rsel = -1, rlast = -1;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      if (rsum[r] > 0.f) rlast = r;
      if (rsel < 0 && acc + rsum[r] > target) rsel = r;
      if (rsel < 0) acc += rsum[r];
    }
    if (rsel < 0) {
      rsel = rlast;
      acc = -INFINITY;
    }
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) v = r == rsel ? rz[r] : v;
    const float pre = acc + wave_incl_scan(v, lane);
    const uint64_t over = __ballot(v > 0.f && pre > target);
    const uint64_t kept = __ballot(v > 0.f);
    const int base = seg0 + 64 * (gsel * RG + rsel);
    const int pick = over ? base + (int)__builtin_ctzll(over)
                          : (kept ? base + 63 - (int)__builtin_clzll(kept) : -1);
    if (lane == 0 && pick >= 0) tok[row] = pick;
  }
}

}  // namespace

int kv_store_launch(bool h16, const void* qkv, void* kv, int B, int Tn, int H, int hs,
                    int max_len, int pos0, hipStream_t s) {
  if (pos0 < 0 || pos0 + Tn > max_len) return -5;
  const int64_t n = (int64_t)B * Tn * 2 * H * hs;
  const unsigned grid = (unsigned)cdiv(n, 256);
  if (h16)
    hipLaunchKernelGGL(kv_store_kernel<h16_t>, dim3(grid), dim3(256), 0, s, (const h16_t*)qkv,
                       (h16_t*)kv, B, Tn, H, hs, max_len, pos0);
  else
    hipLaunchKernelGGL(kv_store_kernel<float>, dim3(grid), dim3(256), 0, s, (const float*)qkv,
                       (float*)kv, B, Tn, H, hs, max_len, pos0);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int decode_attn_launch(bool h16, const void* qkv, const void* kv, void* out, int B, int H, int hs,
                       int max_len, int len, hipStream_t s) {
  if (hs < 1 || hs > 128 || len < 1 || len > max_len) return -5;
  if (h16 && hs == 64)
    hipLaunchKernelGGL(decode_attn64_kernel<h16_t>, dim3(B * H), dim3(64 * DEC64_WAVES), 0, s,
                       (const h16_t*)qkv, (const h16_t*)kv, (h16_t*)out, B, H, max_len, len);
  else if (h16)
    hipLaunchKernelGGL(decode_attn_kernel<h16_t>, dim3(B * H), dim3(64 * DEC_WAVES), 0, s,
                       (const h16_t*)qkv, (const h16_t*)kv, (h16_t*)out, B, H, hs, max_len, len);
  else
    hipLaunchKernelGGL(decode_attn_kernel<float>, dim3(B * H), dim3(64 * DEC_WAVES), 0, s,
                       (const float*)qkv, (const float*)kv, (float*)out, B, H, hs, max_len, len);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int sample_launch(const float* logits, int B, int V, int ldv, float temperature, int top_k,
                  const float* u, int32_t* tok, hipStream_t s) {
  if (B < 1 || V < 1 || V > (SAMP_THREADS / 64) * SAMP_SEG || ldv < V || !(temperature > 0.f))
    return -5;
  hipLaunchKernelGGL(sample_kernel, dim3(B), dim3(SAMP_THREADS), 0, s, logits, V, ldv,
                     1.0f / temperature, top_k, u, tok);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// the rows (normalised with ln) are staged in LDS, which bounds M * K
bool gemv_fits(bool h16, bool ln, int M, int K) {
  const int es = h16 ? 2 : 4;
  return M >= 1 && M <= GEMV_MAX_M && K % 8 == 0 && (int64_t)M * K * es <= GEMV_LDS_BYTES &&
         (!ln || K <= GEMV_MAX_K_LN);
}

// epi: 0 act, 1 fp32, 2 fp32 residual add, 3 gelu (act); ln_w set: A is fp32
// and is normalised first; kv set (act epilogue): cache store of columns [C, 3C)
int gemv_launch(bool h16, int epi, const void* A, const float* ln_w, const float* ln_b,
                const void* W, const float* bias, const float* aux, void* out, int M, int N, int K,
                int ldo, void* kv, int H, int hs, int max_len, int pos, hipStream_t s) {
  const bool ln = ln_w != nullptr;
  if (!gemv_fits(h16, ln, M, K) || N < 1 || epi < 0 || epi > 3) return -5;
  if (kv && epi != GV_ACT) return -5;
  if (((uintptr_t)A | (uintptr_t)W) & 15) return -5;
  GemvArgs a{A, ln_w, ln_b, W, bias, aux, out, M, N, K, ldo, kv, H, hs, max_len, pos, H * hs};
  const size_t lds = (size_t)M * K * (h16 ? 2 : 4);
  const int nc = N >= 8192 ? 4 : 2;
  const unsigned grid = (unsigned)cdiv(N, 4 * nc);
#define GV(T, E, L, NCV) hipLaunchKernelGGL((gemv_kernel<T, E, L, NCV>), dim3(grid), dim3(256), lds, s, a)
#define GV_EPI(T, L, NCV)                            \
  switch (epi) {                                     \
    case GV_ACT: GV(T, GV_ACT, L, NCV); break;       \
    case GV_F32: GV(T, GV_F32, L, NCV); break;       \
    case GV_RESID: GV(T, GV_RESID, L, NCV); break;   \
    default: GV(T, GV_GELU, L, NCV); break;          \
  }
  if (h16) {
    if (ln) {
      if (nc == 4) { GV_EPI(h16_t, true, 4) } else { GV_EPI(h16_t, true, 2) }
    } else {
      if (nc == 4) { GV_EPI(h16_t, false, 4) } else { GV_EPI(h16_t, false, 2) }
    }
  } else {
    if (ln) {
      if (nc == 4) { GV_EPI(float, true, 4) } else { GV_EPI(float, true, 2) }
    } else {
      if (nc == 4) { GV_EPI(float, false, 4) } else { GV_EPI(float, false, 2) }
    }
  }
#undef GV_EPI
#undef GV
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace HALF_NS
