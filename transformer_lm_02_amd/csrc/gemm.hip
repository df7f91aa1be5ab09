// Matrix products of the step: every Linear layer's forward, input gradient
// and weight gradient, and the tied LM head and its two transposes
// ("nanoGPT" (stanleyjacob.dev), Part V Deep dive 1: c_attn, c_proj, c_fc,
// the MLP projection and lm_head; their gradients are those of y = x W^T + b).
//
// 16-bit path: v_mfma_f32_32x32x16_bf16 (or _f16) on gfx950, 4 waves per workgroup in a
// 2x2 grid, BM x BN x 64 block tiles double-buffered in LDS, fp32
// accumulation, and the elementwise work of the step fused into the
// epilogue (bias, residual add, tanh-GELU and its derivative, fp32 gradient
// accumulation).  fp32 path: a plain LDS-tiled FMA kernel with the same
// epilogues, used in the fp32 correctness mode.
#include "common.h"
#include "gemm.h"
#include "kernels.h"

namespace HALF_NS {

// ---------------------------------------------------------------- epilogue
template <int EPI, typename T>
__device__ __forceinline__ void epi_apply(const GemmEpiArgs& e, int m, int n, float acc) {
  const int64_t i = (int64_t)m * e.ldc + n;
  if constexpr (EPI == EPI_ACT) {
    stf((T*)e.out + i, acc + (e.bias ? e.bias[n] : 0.f));
  } else if constexpr (EPI == EPI_F32) {
    ((float*)e.out)[i] = acc + (e.bias ? e.bias[n] : 0.f);
  } else if constexpr (EPI == EPI_RESID) {
    float y = acc + (e.bias ? e.bias[n] : 0.f);
    if (e.drop.thresh) y *= drop1(e.drop, (uint32_t)n, (uint32_t)m, 0);
    ((float*)e.out)[i] = ((const float*)e.aux)[i] + y;
  } else if constexpr (EPI == EPI_GELU) {
    float g, gp;
    gelu_both(acc + (e.bias ? e.bias[n] : 0.f), g, gp);
    stf((T*)e.out + i, gp);
    stf((T*)e.out2 + i, g);
  } else if constexpr (EPI == EPI_GELU_BWD) {
    stf((T*)e.out + i, acc * ldf((const T*)e.aux + i));
  } else {  // EPI_ACCUM
    float* o = (float*)e.out + i;
    *o = (e.beta ? *o : 0.f) + acc;
  }
}

// ---------------------------------------------------------------- tile order
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Give each XCD a contiguous range of tile ids, and walk tiles in
// groups of GROUP_M tile-rows so that neighbouring workgroups on one XCD
// share A row-blocks and B column-blocks in that XCD's L2.
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int n = tiles_m * tiles_n;
  const int xcd = wg & 7, local = wg >> 3;
  const int base = n >> 3, rem = n & 7;
  const int tile = xcd * base + min(xcd, rem) + local;
  constexpr int GROUP_M = 8;
  const int per_group = GROUP_M * tiles_n;
  const int g = tile / per_group;
  const int first_m = g * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int r = tile - g * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

struct GemmArgs {
  const h16_t* A;
  const h16_t* B;
  int lda, ldb, M, N, K, ka_rows, kb_rows, tiles_m, tiles_n;
  GemmEpiArgs e;
};

// ---------------------------------------------------------------- 16-bit MFMA kernel
// LDS layouts (16-bit elements, one k-tile of 64):
//  k-contiguous operand: [rows][64], the 16-byte chunk c of row r stored at
//    chunk position c ^ (r & 7);
//  m/n-contiguous operand (transposed while staging): [8 k-chunks][rows][8],
//    row r stored at position r ^ ((r >> 3) & 7) within its chunk plane.
// Both give conflict-free 16-byte reads for the MFMA operand pattern (lane l
// reads row l%32 of a 32-row slab, k-chunk l/32).
template <int ROWS, bool KC>
struct OperandTile {
  static constexpr int ELEMS = ROWS * 64;
  __device__ __forceinline__ static int off(int r, int c) {  // r row, c k-chunk (0..7)
    if constexpr (KC) return r * 64 + ((c ^ (r & 7)) << 3);
    else return c * ROWS * 8 + ((r ^ ((r >> 3) & 7)) << 3);
  }
  // staging registers per thread (uint4 each)
  static constexpr int NREG = ROWS / 32;

  // global -> registers for k-tile starting at k0
  __device__ __forceinline__ static void load(uint4 (&reg)[NREG], const h16_t* __restrict__ P,
                                              int ld, int row0, int nrows, int k0, int K,
                                              int krows, int tid) {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int r = (tid >> 3) + 32 * i, c = tid & 7;
        const int gr = row0 + r, gk = k0 + 8 * c;
        if (gr < nrows && gk < K)
          reg[i] = *(const uint4*)(P + (int64_t)gr * ld + gk);
        else
          reg[i] = make_uint4(0, 0, 0, 0);
      }
    } else {
      // NREG/4 sub-blocks of 4 k-rows x 8 columns per thread
#pragma unroll
      for (int s = 0; s < NREG / 4; ++s) {
        const int idx = tid + 256 * s;
        const int mc = idx % (ROWS / 8), kg = idx / (ROWS / 8);
        const int gm = row0 + 8 * mc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gk = k0 + 4 * kg + r;
          if (gk < krows && gm < ld)
            reg[4 * s + r] = *(const uint4*)(P + (int64_t)gk * ld + gm);
          else
            reg[4 * s + r] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ static void store(const uint4 (&reg)[NREG], h16_t* lds, int tid) {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int r = (tid >> 3) + 32 * i, c = tid & 7;
        *(uint4*)(lds + off(r, c)) = reg[i];
      }
    } else {
#pragma unroll
      for (int s = 0; s < NREG / 4; ++s) {
        const int idx = tid + 256 * s;
        const int mc = idx % (ROWS / 8), kg = idx / (ROWS / 8);
        const uint32_t* r0 = (const uint32_t*)&reg[4 * s + 0];
        const uint32_t* r1 = (const uint32_t*)&reg[4 * s + 1];
        const uint32_t* r2 = (const uint32_t*)&reg[4 * s + 2];
        const uint32_t* r3 = (const uint32_t*)&reg[4 * s + 3];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int w = j >> 1;
          uint32_t lo, hi;
          if (j & 1) {
            lo = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
            hi = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
          } else {
            lo = (r0[w] & 0xffffu) | (r1[w] << 16);
            hi = (r2[w] & 0xffffu) | (r3[w] << 16);
          }
          const int m = 8 * mc + j;
          *(uint2*)(lds + off(m, kg >> 1) + 4 * (kg & 1)) = make_uint2(lo, hi);
        }
      }
    }
  }
};

template <int BM, int BN, bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs p) {
  using TA = OperandTile<BM, AK>;
  using TB = OperandTile<BN, BKC>;
  __shared__ __attribute__((aligned(16))) h16_t lds_a[2][TA::ELEMS];
  __shared__ __attribute__((aligned(16))) h16_t lds_b[2][TB::ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int TM = BM / 64, TN = BN / 64;  // 32x32 MFMA tiles per wave

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // rows of A / B that may be read
  const int a_rows = AK ? p.M : p.lda, b_rows = BKC ? p.N : p.ldb;
  uint4 ra[TA::NREG], rb[TB::NREG];
  const int nk = (p.K + 63) / 64;

  TA::load(ra, p.A, p.lda, m0, a_rows, 0, p.K, p.ka_rows, tid);
  TB::load(rb, p.B, p.ldb, n0, b_rows, 0, p.K, p.kb_rows, tid);
  TA::store(ra, lds_a[0], tid);
  TB::store(rb, lds_b[0], tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      TA::load(ra, p.A, p.lda, m0, a_rows, (kt + 1) * 64, p.K, p.ka_rows, tid);
      TB::load(rb, p.B, p.ldb, n0, b_rows, (kt + 1) * 64, p.K, p.kb_rows, tid);
    }
    const h16_t* la = lds_a[cur];
    const h16_t* lb = lds_b[cur];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      h16x8_t fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *(const h16x8_t*)(la + TA::off(wm * (BM / 2) + 32 * i + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *(const h16x8_t*)(lb + TB::off(wn * (BN / 2) + 32 * j + (lane & 31), c));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = MFMA_32X32X16(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      TA::store(ra, lds_a[cur ^ 1], tid);
      TB::store(rb, lds_b[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // accumulator layout of a 32x32 tile: lane l, register r ->
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * (BN / 2) + 32 * j + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / 2) + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < p.M) epi_apply<EPI, h16_t>(p.e, row, col, acc[i][j][r]);
      }
    }
}

// ---------------------------------------------------------------- fp32 kernel
struct GemmArgsF {
  const float* A;
  const float* B;
  int lda, ldb, M, N, K, ka_rows, kb_rows, tiles_m, tiles_n;
  GemmEpiArgs e;
};

template <bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgsF p) {
  __shared__ float sa[16][65];
  __shared__ float sb[16][65];
  const int tid = threadIdx.x;
  const int tm = blockIdx.x % p.tiles_m, tn = blockIdx.x / p.tiles_m;
  const int m0 = tm * 64, n0 = tn * 64;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    for (int e = tid; e < 64 * 16; e += 256) {
      const int r = e / 16, k = e % 16;   // k fastest: k-contiguous reads
      const int r2 = e % 64, k2 = e / 64; // row fastest: row-contiguous reads
      {
        const int rr = AK ? r : r2, kk = AK ? k : k2;
        const int gm = m0 + rr, gk = k0 + kk;
        float v = 0.f;
        if (AK) { if (gm < p.M && gk < p.K) v = p.A[(int64_t)gm * p.lda + gk]; }
        else { if (gm < p.lda && gk < p.ka_rows && gk < p.K) v = p.A[(int64_t)gk * p.lda + gm]; }
        sa[kk][rr] = v;
      }
      {
        const int rr = BKC ? r : r2, kk = BKC ? k : k2;
        const int gn = n0 + rr, gk = k0 + kk;
        float v = 0.f;
        if (BKC) { if (gn < p.N && gk < p.K) v = p.B[(int64_t)gn * p.ldb + gk]; }
        else { if (gn < p.ldb && gk < p.kb_rows && gk < p.K) v = p.B[(int64_t)gk * p.ldb + gn]; }
        sb[kk][rr] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sa[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sb[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty + 16 * i, col = n0 + tx + 16 * j;
      if (row < p.M && col < p.N) epi_apply<EPI, float>(p.e, row, col, acc[i][j]);
    }
}

// ---------------------------------------------------------------- dispatch
template <int BM, int BN, bool AK, bool BKC, int EPI>
static void run_mfma(const GemmArgs& a, hipStream_t s) {
  GemmArgs p = a;
  p.tiles_m = (int)cdiv(p.M, BM);
  p.tiles_n = (int)cdiv(p.N, BN);
  hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, AK, BKC, EPI>), dim3(p.tiles_m * p.tiles_n),
                     dim3(256), 0, s, p);
}

template <bool AK, bool BKC, int EPI>
static void run_mfma_shape(const GemmArgs& a, hipStream_t s) {
  // 256x128 tiles when there are enough of them to fill 256 CUs, else 128x128
  const int64_t big = cdiv(a.M, 256) * cdiv(a.N, 128);
  if (big >= 512) run_mfma<256, 128, AK, BKC, EPI>(a, s);
  else run_mfma<128, 128, AK, BKC, EPI>(a, s);
}

template <bool AK, bool BKC, int EPI>
static void run_f32(const GemmArgsF& a, hipStream_t s) {
  GemmArgsF p = a;
  p.tiles_m = (int)cdiv(p.M, 64);
  p.tiles_n = (int)cdiv(p.N, 64);
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, EPI>), dim3(p.tiles_m * p.tiles_n), dim3(256), 0,
                     s, p);
}

#define GEMM_CASE(AKV, BKV, EPIV)                                                          \
  if (a_kcontig == AKV && b_kcontig == BKV && epi == EPIV) {                              \
    if (h16) run_mfma_shape<AKV, BKV, EPIV>(pa, stream);                                  \
    else run_f32<AKV, BKV, EPIV>(pf, stream);                                              \
    return hipGetLastError() == hipSuccess ? 0 : -4;                                       \
  }

int gemm2_launch(bool a_kcontig, bool b_kcontig, int epi, const void* A, int lda, const void* B,
                 int ldb, int M, int N, int K, int ka_rows, int kb_rows, const GemmEpiArgs& e,
                 float* ws, int64_t ws_bytes, hipStream_t s);

static int gemm_launch_plain(bool h16, bool a_kcontig, bool b_kcontig, int epi, const void* A,
                             int lda, const void* B, int ldb, int M, int N, int K, int ka_rows,
                             int kb_rows, const GemmEpiArgs& e, hipStream_t stream, float* ws,
                             int64_t ws_bytes);

int gemm_launch(bool h16, bool a_kcontig, bool b_kcontig, int epi, const void* A, int lda,
                const void* B, int ldb, int M, int N, int K, int ka_rows, int kb_rows,
                const GemmEpiArgs& e, hipStream_t stream, float* ws, int64_t ws_bytes) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (h16) {
    // the pipelined kernel when the shape allows it (column sums included)
    const int rc = gemm2_launch(a_kcontig, b_kcontig, epi, A, lda, B, ldb, M, N, K, ka_rows,
                                kb_rows, e, ws, ws_bytes, stream);
    if (rc != -5) return rc == 0 ? (hipGetLastError() == hipSuccess ? 0 : -4) : rc;
  }
  // the plain kernel may use the scratch: a pending chained reduction first
  if (e.chain)
    if (const int rc = splitk_chain_flush(e.chain, stream)) return rc;
  const int rc = gemm_launch_plain(h16, a_kcontig, b_kcontig, epi, A, lda, B, ldb, M, N, K,
                                   ka_rows, kb_rows, e, stream, ws, ws_bytes);
  if (rc != 0 || !e.cs_out) return rc;
  if (e.ldc != N) return -5;
  return colsum_launch(h16, e.out, M, N, e.cs_part, e.cs_out, e.cs_beta, stream);
}

static int gemm_launch_plain(bool h16, bool a_kcontig, bool b_kcontig, int epi, const void* A,
                             int lda, const void* B, int ldb, int M, int N, int K, int ka_rows,
                             int kb_rows, const GemmEpiArgs& e, hipStream_t stream, float* ws,
                             int64_t ws_bytes) {
  (void)ws;
  (void)ws_bytes;
  if (h16) {
    if ((a_kcontig && (K % 8 || lda % 8)) || (b_kcontig && (K % 8 || ldb % 8))) return -5;
    if ((!a_kcontig && lda % 8) || (!b_kcontig && ldb % 8)) return -5;
    if (((uintptr_t)A | (uintptr_t)B) & 15) return -5;
  }
  GemmArgs pa{(const h16_t*)A, (const h16_t*)B, lda, ldb, M, N, K, ka_rows, kb_rows, 0, 0, e};
  GemmArgsF pf{(const float*)A, (const float*)B, lda, ldb, M, N, K, ka_rows, kb_rows, 0, 0, e};
  // forward: y = x W^T (+ bias / residual / GELU)
  GEMM_CASE(true, true, EPI_ACT)
  GEMM_CASE(true, true, EPI_F32)
  GEMM_CASE(true, true, EPI_RESID)
  GEMM_CASE(true, true, EPI_GELU)
  GEMM_CASE(true, true, EPI_GELU_BWD)
  // input gradients: dx = dy W
  GEMM_CASE(true, false, EPI_ACT)
  GEMM_CASE(true, false, EPI_F32)
  GEMM_CASE(true, false, EPI_GELU_BWD)
  // weight gradients: dW (+)= dy^T x
  GEMM_CASE(false, false, EPI_ACCUM)
  return -5;
}

}  // namespace HALF_NS
