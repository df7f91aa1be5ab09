// Pipelined 16-bit MFMA GEMM for gfx950: C[m][n] = sum_k A(m,k) B(n,k).
//
// Same products and epilogues as gemm.hip (the Linear layers of "nanoGPT"
// (stanleyjacob.dev), Part V Deep dive 1, their input and weight gradients,
// and the tied LM head), arranged for CDNA4:
//  * operands go from HBM straight into LDS with buffer loads in LDS mode
//    (no VGPR staging) through an NS-stage ring, so NS-1 k-tiles are in
//    flight while one is multiplied; out-of-range reads return zero, which
//    handles ragged edges;
//  * a k-contiguous operand is stored [rows][64] with its 16-byte chunks
//    XOR-swizzled by row and read with ds_read_b128; an m/n-contiguous
//    operand (a transposed use: weight gradients, input gradients through
//    W) stays in its memory layout [64][rows] and is read with the gfx950
//    transposing LDS load ds_read_b64_tr_b16, so no register transpose;
//  * v_mfma_f32_32x32x16_bf16 (or _f16), 4 waves in a 2x2 grid, fp32 accumulators;
//  * the epilogue goes through LDS so every lane stores 8 contiguous outputs;
//  * weight gradients with few output tiles split K over workgroups into an
//    fp32 partial buffer that a second kernel sums in a fixed order.
#include <type_traits>
#include <utility>

#include "common.h"
#include "gemm.h"
#include "kernels.h"

namespace HALF_NS {

#define AS3(p) ((__attribute__((address_space(3))) void*)(p))

namespace {

constexpr uint32_t kOOB = 0xFFFFFF00u;  // byte offset beyond any buffer: loads return 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// One operand tile of ROWS x BK (k) 16-bit per stage.  Each wave issues
// ROWS*BK/2048 loads of 1 KB (64 lanes x 16 bytes, contiguous in LDS).
template <int ROWS, bool KC, int BK>
struct Stage {
  static constexpr int ELEMS = ROWS * BK;
  static constexpr int NLOAD = ELEMS / 512;  // 1 KB loads per stage
  static constexpr int LOADS = NLOAD / 4;    // per wave
  static_assert(NLOAD % 4 == 0, "tile must split into 4 waves of 1 KB loads");
  static constexpr int CPR = KC ? BK / 8 : ROWS / 8;  // 16-byte chunks per LDS row
  static constexpr int RPL = 64 / CPR;                // LDS rows per 1 KB load
  static_assert(64 % CPR == 0, "1 KB load must cover whole LDS rows");
  static_assert(KC || CPR % 16 == 0, "transposed tile needs whole 16-chunk bank groups");
  uint32_t voff[LOADS];
  int kofs[LOADS];
  int kfast;  // k-tiles ending at or before this k take the scalar-offset path

  // k-contiguous: LDS [ROWS][BK]; chunk c of row r at position c ^ sw(r)
  //   with sw(r) = (r>>1)&7 for BK 64, (r>>2)&3 for BK 32 (conflict-free
  //   16-byte reads of 16 consecutive rows)
  // m-contiguous: LDS [BK][ROWS]; chunk c of k-row k at position c ^ 4(k&3)
  //   (conflict-free transposing reads of 4 k-rows x 32 columns: two
  //   16-lane groups side by side)
  __device__ __forceinline__ static int swz(int r) {
    return BK == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3);
  }
  // krows: rows of an m/n-contiguous operand (reads at or past it return 0)
  __device__ __forceinline__ void init(int row0, int ld, int lane, int wave, int K, int krows) {
    // A k-contiguous tile's rows past the operand start beyond its buffer, so
    // their loads are out of range whatever k offset is added.  An
    // m/n-contiguous tile needs every column inside the row pitch for that.
    if constexpr (KC) kfast = K;
    else kfast = row0 + ROWS <= ld ? (K < krows ? K : krows) : 0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = i * 4 + wave;
      const int r = q * RPL + lane / CPR, pos = lane % CPR;
      if constexpr (KC) {
        const int c = pos ^ swz(r);
        voff[i] = (uint32_t)(((int64_t)(row0 + r) * ld + 8 * c) * 2);
        kofs[i] = 8 * c;
      } else {
        const int c = pos ^ (4 * (r & 3));
        voff[i] = (uint32_t)(((int64_t)r * ld + row0 + 8 * c) * 2);
        kofs[i] = 0;
      }
    }
  }
  // lds and wave are wave-uniform.  A k-tile wholly in range carries its k
  // offset in the scalar offset operand, so a load needs no vector ALU work;
  // a k-tile that crosses K (or the rows of an m/n-contiguous operand) sends
  // each lane's chunks past the end to an offset beyond the buffer instead.
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, h16_t* lds, int kt, int ld,
                                        int K, int wave) const {
    if ((kt + 1) * BK <= kfast) {
      const uint32_t soff =
          KC ? (uint32_t)kt * (uint32_t)(BK * 2) : (uint32_t)kt * (uint32_t)(BK * ld) * 2u;
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, AS3(lds + (i * 4 + wave) * 512), 16,
                                                 (int)voff[i], (int)soff, 0, 0);
      return;
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = i * 4 + wave;
      uint32_t off;
      if constexpr (KC) {
        off = (kt * BK + kofs[i] < K) ? voff[i] + (uint32_t)kt * (uint32_t)(BK * 2) : kOOB;
      } else {
        off = voff[i] + (uint32_t)kt * (uint32_t)(BK * ld * 2);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, AS3(lds + q * 512), 16, off, 0, 0, 0);
    }
  }
  // MFMA 32x32x16 operand: lane holds (row rbase + lane%32, k 16ks + 8(lane/32) + 0..7)
  __device__ __forceinline__ static h16x8_t frag(const h16_t* __restrict__ lds, int rbase, int ks,
                                                  int lane) {
    if constexpr (KC) {
      const int r = rbase + (lane & 31), c = 2 * ks + (lane >> 5);
      return *(const h16x8_t*)(lds + r * BK + ((c ^ swz(r)) << 3));
    } else {
      const int G = lane >> 4, t = lane & 15;
      const int m = rbase + 16 * (G & 1) + 4 * (t & 3);
      const int k0 = 16 * ks + 8 * (G >> 1) + (t >> 2);
      const int c = m >> 3;
      const int ka = k0, kb = k0 + 4;
      const h16_t* pa = lds + ka * ROWS + ((c ^ (4 * (ka & 3))) << 3) + (m & 7);
      const h16_t* pb = lds + kb * ROWS + ((c ^ (4 * (kb & 3))) << 3) + (m & 7);
      const h16x4_t lo = DS_READ_TR16_B64(
          (__attribute__((address_space(3))) h16x4_t*)(pa));
      const h16x4_t hi = DS_READ_TR16_B64(
          (__attribute__((address_space(3))) h16x4_t*)(pb));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
};

// f(std::integral_constant<int, i>()) for i = 0 .. N-1
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_from(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for_from<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_from<0, N>(f);
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Outputs no kernel reads soon go out with non-temporal stores (st_nt): the
// head's exp(z) (read by the backward), the weight gradients and their
// split-K partials, the stored GELU derivative.  They leave L2 to the
// operands the products re-read (the head's forward reads its activation
// rows from L2 across all 262 column tiles).  Outputs the next kernel reads
// keep ordinary stores.

// A previous launch's split-K reduction run by workgroups past the tiles:
// out[i] = (beta ? out[i] : 0) + sum over k < ks of part[k * 4 n4 + i]
struct SplitKRed {
  const float* part = nullptr;
  float* out = nullptr;
  int64_t n4 = 0;  // float4 groups
  int ks = 0, beta = 0, wgs = 0;
};

struct Gemm2Args {
  const h16_t* A;
  const h16_t* B;
  int lda, ldb, M, N, K, ka_rows, kb_rows, tiles_m, tiles_n;
  int ksplit, k_tiles_per_split;
  float* part;  // split-K partials [ksplit][M][N] (EPI_ACCUM with ksplit > 1)
  GemmEpiArgs e;
  SplitKRed red;  // EPI_ACCUM: wgs workgroups after the tiles
};

// Workgroup w of the reducers: float4 groups w * 256 * U + t + 256 j, then
// every wgs * 256 * U further; each thread keeps U groups in flight.  The
// partials are added in split order, as splitk_reduce_kernel adds them.
__device__ __forceinline__ void splitk_reduce_wg(const SplitKRed& r, int w) {
  constexpr int U = 8;
  const float4* part = (const float4*)r.part;
  float4* out = (float4*)r.out;
  const int64_t stride = (int64_t)r.wgs * 256 * U;
  for (int64_t i0 = (int64_t)w * 256 * U + threadIdx.x; i0 < r.n4; i0 += stride) {
    float4 s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + 256 * u;
      s[u] = r.beta && i < r.n4 ? out[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int k = 0; k < r.ks; ++k) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + 256 * u;
        v[u] = i < r.n4 ? part[(int64_t)k * r.n4 + i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u].x += v[u].x;
        s[u].y += v[u].y;
        s[u].z += v[u].z;
        s[u].w += v[u].w;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + 256 * u;
      if (i < r.n4) st_nt(&out[i], s[u]);
    }
  }
}

// Workgroup -> (output tile, k split).  Workgroups go to the 8 XCDs in
// turn (workgroup w to XCD w % 8), so the linear work index (split-major,
// then tiles in groups of 8 row tiles) is cut into 8 contiguous chunks, one
// per XCD: the workgroups resident on one XCD then share a split's k range
// and neighbouring tiles' operand rows in that XCD's L2.
__device__ __forceinline__ void tile_split_coords(int wg, int tiles_m, int tiles_n, int ksplit,
                                                  int& tm, int& tn, int& split) {
  const int tiles = tiles_m * tiles_n;
  const int n = tiles * ksplit;
  const int xcd = wg & 7, local = wg >> 3;
  const int base = n >> 3, rem = n & 7;
  const int w = xcd * base + min(xcd, rem) + local;
  split = w / tiles;
  const int tile = w - split * tiles;
  constexpr int GROUP_M = 8;
  const int per_group = GROUP_M * tiles_n;
  const int g = tile / per_group;
  const int first_m = g * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int r = tile - g * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// Operand an epilogue reads besides the accumulators (8 consecutive outputs
// of one row): the residual (fp32), the GELU pre-activation (16-bit) or the
// gradient being accumulated into (fp32).  Loaded for a whole slab of rows
// before any of them is stored, so the loads overlap.
struct Aux8 {
  float4 a, b;
};
template <int EPI>
__device__ __forceinline__ Aux8 aux8(const GemmEpiArgs& e, int splitk, int m, int n) {
  const int64_t i = (int64_t)m * e.ldc + n;
  Aux8 x;
  x.a = x.b = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (EPI == EPI_RESID) {
    const float4* s = (const float4*)((const float*)e.aux + i);
    x.a = s[0];
    x.b = s[1];
  } else if constexpr (EPI == EPI_GELU_BWD) {
    const uint4 u = *(const uint4*)((const h16_t*)e.aux + i);
    x.a = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                      __uint_as_float(u.w));
  } else if constexpr (EPI == EPI_ACCUM) {
    if (!splitk && e.beta) {
      const float4* s = (const float4*)((const float*)e.out + i);
      x.a = s[0];
      x.b = s[1];
    }
  } else if constexpr (EPI == EPI_HEAD_DX) {
    x.a.x = e.head.r[m];  // the row's softmax factor
  }
  return x;
}
template <int EPI>
constexpr bool epi_reads_aux() {
  return EPI == EPI_RESID || EPI == EPI_GELU_BWD || EPI == EPI_ACCUM || EPI == EPI_HEAD_DX;
}

// 8 consecutive outputs of one row: epilogue and 16/32-byte stores
template <int EPI>
__device__ __forceinline__ void epi8(const GemmEpiArgs& e, float* part, int splitk, int m, int n,
                                     const float* v, const float* bias8, const Aux8& x,
                                     float* csum) {
  const int64_t i = (int64_t)m * e.ldc + n;
  if constexpr (EPI == EPI_ACCUM) {
    if (splitk) {
      float4* o = (float4*)(part + i);
      st_nt(&o[0], make_float4(v[0], v[1], v[2], v[3]));
      st_nt(&o[1], make_float4(v[4], v[5], v[6], v[7]));
    } else {
      float4* o = (float4*)((float*)e.out + i);
      st_nt(&o[0], make_float4(x.a.x + v[0], x.a.y + v[1], x.a.z + v[2], x.a.w + v[3]));
      st_nt(&o[1], make_float4(x.b.x + v[4], x.b.y + v[5], x.b.z + v[6], x.b.w + v[7]));
    }
  } else if constexpr (EPI == EPI_F32) {
    float4* o = (float4*)((float*)e.out + i);
    o[0] = make_float4(v[0] + bias8[0], v[1] + bias8[1], v[2] + bias8[2], v[3] + bias8[3]);
    o[1] = make_float4(v[4] + bias8[4], v[5] + bias8[5], v[6] + bias8[6], v[7] + bias8[7]);
  } else if constexpr (EPI == EPI_RESID) {
    float4* o = (float4*)((float*)e.out + i);
    if (e.drop.thresh) {
      const float4 z0 = drop4(e.drop, (uint32_t)n >> 2, (uint32_t)m, 0);
      const float4 z1 = drop4(e.drop, ((uint32_t)n >> 2) + 1, (uint32_t)m, 0);
      o[0] = make_float4(x.a.x + z0.x * (v[0] + bias8[0]), x.a.y + z0.y * (v[1] + bias8[1]),
                         x.a.z + z0.z * (v[2] + bias8[2]), x.a.w + z0.w * (v[3] + bias8[3]));
      o[1] = make_float4(x.b.x + z1.x * (v[4] + bias8[4]), x.b.y + z1.y * (v[5] + bias8[5]),
                         x.b.z + z1.z * (v[6] + bias8[6]), x.b.w + z1.w * (v[7] + bias8[7]));
    } else {
      o[0] = make_float4(x.a.x + v[0] + bias8[0], x.a.y + v[1] + bias8[1], x.a.z + v[2] + bias8[2],
                         x.a.w + v[3] + bias8[3]);
      o[1] = make_float4(x.b.x + v[4] + bias8[4], x.b.y + v[5] + bias8[5], x.b.z + v[6] + bias8[6],
                         x.b.w + v[7] + bias8[7]);
    }
  } else if constexpr (EPI == EPI_ACT) {
    *(uint4*)((h16_t*)e.out + i) =
        make_uint4(pack2h(v[0] + bias8[0], v[1] + bias8[1]), pack2h(v[2] + bias8[2], v[3] + bias8[3]),
                   pack2h(v[4] + bias8[4], v[5] + bias8[5]), pack2h(v[6] + bias8[6], v[7] + bias8[7]));
  } else if constexpr (EPI == EPI_GELU) {
    // the backward needs only gelu'(u): it is stored in place of u
    float g[8], gp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) gelu_both(v[j] + bias8[j], g[j], gp[j]);
    st_nt((h16_t*)e.out + i, make_uint4(pack2h(gp[0], gp[1]), pack2h(gp[2], gp[3]),
                                        pack2h(gp[4], gp[5]), pack2h(gp[6], gp[7])));
    *(uint4*)((h16_t*)e.out2 + i) =
        make_uint4(pack2h(g[0], g[1]), pack2h(g[2], g[3]), pack2h(g[4], g[5]), pack2h(g[6], g[7]));
  } else if constexpr (EPI == EPI_HEAD_DX) {
    const float r = x.a.x;
    *(uint4*)((h16_t*)e.out + i) = make_uint4(pack2h(r * v[0], r * v[1]), pack2h(r * v[2], r * v[3]),
                                              pack2h(r * v[4], r * v[5]), pack2h(r * v[6], r * v[7]));
  } else {  // EPI_GELU_BWD: the 16-bit gelu'(u) values travel in x.a's bits
    const uint32_t w[4] = {__float_as_uint(x.a.x), __float_as_uint(x.a.y), __float_as_uint(x.a.z),
                           __float_as_uint(x.a.w)};
    float d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = v[j] * h2f((h16_t)(w[j >> 1] >> (16 * (j & 1))));
#pragma unroll
    for (int j = 0; j < 8; ++j) csum[j] += d[j];
    *(uint4*)((h16_t*)e.out + i) =
        make_uint4(pack2h(d[0], d[1]), pack2h(d[2], d[3]), pack2h(d[4], d[5]), pack2h(d[6], d[7]));
  }
}

template <int BM, int BN, bool AK, bool BKC, int EPI, int NS, int BK, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm2_kernel(Gemm2Args p) {
  using SA = Stage<BM, AK, BK>;
  using SB = Stage<BN, BKC, BK>;
  constexpr int STAGE_ELEMS = SA::ELEMS + SB::ELEMS;
  constexpr int WR = BM / 2, WC = BN / 2;   // wave tile
  constexpr int TM = WR / 32, TN = WC / 32; // 32x32 MFMA tiles per wave
  constexpr int KS = BK / 16;               // MFMA k-steps per k-tile
  constexpr int EP_PITCH = WC + 8;          // fp32 staging pitch: rows r, r+4 32 banks apart
  constexpr int LDS_ELEMS_RING = NS * STAGE_ELEMS;
  constexpr int LDS_ELEMS_EPI = 4 * 32 * EP_PITCH * 2;  // in 16-bit units
  // EPI_HEAD: after the main loop, the tile's target ids and each wave's
  // per-lane row sums of a 32-row slab ([32][12] fp32) follow the staging area
  constexpr int LDS_ELEMS_HEAD = EPI == EPI_HEAD ? LDS_ELEMS_EPI + 2 * BM + 4 * 32 * 12 * 2 : 0;
  constexpr int LDS_ELEMS_0 = LDS_ELEMS_RING > LDS_ELEMS_EPI ? LDS_ELEMS_RING : LDS_ELEMS_EPI;
  constexpr int LDS_ELEMS = LDS_ELEMS_0 > LDS_ELEMS_HEAD ? LDS_ELEMS_0 : LDS_ELEMS_HEAD;
  __shared__ __attribute__((aligned(1024))) h16_t lds[LDS_ELEMS];

  if constexpr (EPI == EPI_ACCUM) {
    // workgroups past the tiles run a previous launch's split-K reduction
    const int nwork = p.tiles_m * p.tiles_n * p.ksplit;
    if ((int)blockIdx.x >= nwork) {
      splitk_reduce_wg(p.red, (int)blockIdx.x - nwork);
      return;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn, split;
  tile_split_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.ksplit, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm = wave >> 1, wn = wave & 1;
  const int nk_total = (p.K + BK - 1) / BK;
  const int kt0 = split * p.k_tiles_per_split;
  const int nk = min(nk_total - kt0, p.k_tiles_per_split);
  // EPI_HEAD: thread t fetches the target id of row m0 + t now, so the load's
  // latency is spent under the main loop rather than in the epilogue
  int y_pref = -1;
  if constexpr (EPI == EPI_HEAD) {
    if (tid < BM && m0 + tid < p.M) y_pref = p.e.head.tgt[m0 + tid];
  }

  const uint32_t a_bytes = (uint32_t)((int64_t)(AK ? p.M : p.ka_rows) * p.lda * 2);
  const uint32_t b_bytes = (uint32_t)((int64_t)(BKC ? p.N : p.kb_rows) * p.ldb * 2);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, b_bytes);
  SA sa;
  SB sb;
  sa.init(m0, p.lda, lane, wave, p.K, p.ka_rows);
  sb.init(n0, p.ldb, lane, wave, p.K, p.kb_rows);

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  constexpr int L = SA::LOADS + SB::LOADS;  // loads per wave per stage
  constexpr int NF = (TM + TN) * (AK ? 1 : 2) / 1;  // LDS reads per k-step (tr reads count 2)
  (void)NF;
  // Epilogue lane layout: per 32-row slab of the wave tile, each lane takes 8
  // consecutive columns of one row, RPI rows per pass, NIT passes.
  constexpr int LPR = WC / 8;                // lanes per row
  constexpr int RPI = 64 / LPR;              // rows per pass (lanes >= RPI*LPR idle)
  constexpr int NIT = (32 + RPI - 1) / RPI;  // row passes per 32-row slab
  const int my_c = 8 * (lane % LPR), my_r = lane / LPR;
  const bool lane_on = my_r < RPI;
  const int gcol = n0 + wn * WC + my_c;
  // The residual epilogue on 128x192 tiles reads the residual of the wave's
  // first slab during the main loop: pass q's two 16-byte loads follow k-tile
  // q's operand loads, so those HBM reads overlap the products rather than
  // the epilogue's stores (the second slab is read as before; registers allow
  // one).  Buffer loads with out-of-range offsets (reading zero) for lanes
  // without a row keep every wave's load count, and so its waits, fixed.
  constexpr bool RPRE = EPI == EPI_RESID && OCC > 1 && BM == 128 && BN == 192;
  static_assert(!RPRE || NS == 2, "the waits below assume one k-tile in flight");
  // (taken when the main loop has a k-tile for every pass)
  const bool rpre_on = RPRE && nk >= NIT;
  Aux8 rpre[RPRE ? NIT : 1];
  __amdgpu_buffer_rsrc_t rres;
  if constexpr (RPRE) rres = make_rsrc(p.e.aux, (uint32_t)((int64_t)p.M * p.e.ldc * 4));
  // pass q's loads (q a compile-time index, so rpre stays in registers)
  auto res_issue = [&](auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    if constexpr (RPRE && q < NIT) {
      const int lr = q * RPI + my_r, grow = m0 + wm * WR + lr;
      const uint32_t off = lane_on && lr < 32 && grow < p.M && gcol < p.N
                               ? (uint32_t)(((int64_t)grow * p.e.ldc + gcol) * 4)
                               : kOOB;
      // after this k-tile's operand loads, in issue order: the waits count on it
      asm volatile("" ::: "memory");
      rpre[q].a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rres, (int)off, 0, 0));
      rpre[q].b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rres, (int)(off + 16), 0, 0));
    }
  };
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    if (s < nk) {
      sa.issue(ra, lds + s * STAGE_ELEMS, kt0 + s, p.lda, p.K, wave);
      sb.issue(rb, lds + s * STAGE_ELEMS + SA::ELEMS, kt0 + s, p.ldb, p.K, wave);
    }
  }
  if constexpr (OCC > 1) {
    // Two workgroups share the CU: the other one's MFMAs hide this one's
    // latencies, so fragments are single-buffered (registers stay within the
    // 256 per wave that two waves per SIMD allow).
    // One k-tile; res_prev: the previous k-tile issued two residual loads
    // after its operand loads, which may stay in flight
    auto ktile = [&](int kt, bool res_prev) __attribute__((always_inline)) {
      if (kt + NS - 2 < nk) {
        if (RPRE && res_prev) wait_vm_barrier<(NS - 2) * L + 2>();
        else wait_vm_barrier<(NS - 2) * L>();
      } else {
        wait_vm_barrier<0>();
      }
      if (kt + NS - 1 < nk) {
        const int s = (kt + NS - 1) % NS;
        sa.issue(ra, lds + s * STAGE_ELEMS, kt0 + kt + NS - 1, p.lda, p.K, wave);
        sb.issue(rb, lds + s * STAGE_ELEMS + SA::ELEMS, kt0 + kt + NS - 1, p.ldb, p.K, wave);
      }
      const h16_t* la = lds + (kt % NS) * STAGE_ELEMS;
      const h16_t* lb = la + SA::ELEMS;
      return std::make_pair(la, lb);
    };
    auto kmath = [&](const h16_t* la, const h16_t* lb) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        h16x8_t fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = SA::frag(la, wm * WR + 32 * i, ks, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = SB::frag(lb, wn * WC + 32 * j, ks, lane);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = MFMA_32X32X16(fa[i], fb[j], acc[i][j]);
      }
    };
    int kt = 0;
    if constexpr (RPRE) {
      // the first NIT k-tiles unrolled, each followed by one pass's residual loads
      if (rpre_on) {
        static_for<NIT>([&](auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value;
          const auto ab = ktile(q, q >= 1);
          res_issue(qc);
          kmath(ab.first, ab.second);
        });
        kt = NIT;
      }
    }
    for (; kt < nk; ++kt) {
      const auto ab = ktile(kt, rpre_on && kt == NIT);
      kmath(ab.first, ab.second);
    }
  } else {
    // Software pipeline.  Stage kt is known resident after a wait (own DMA
    // count) and a barrier (everyone's); that barrier sits before the last
    // k-step of tile kt-1, so the first fragments of tile kt are read while the
    // last MFMAs of tile kt-1 run, and fragments of k-step ks+1 while ks runs.
    // Before each such barrier the wave's LDS reads of the older stage have
    // completed (lgkmcnt 0), so the DMA that refills that slot cannot overtake
    // them.
    h16x8_t fa[2][TM], fb[2][TN];
    if (nk > 0) {
      if (NS - 2 < nk) wait_vm_barrier<(NS - 2) * L>();
      else wait_vm_barrier<0>();
      const h16_t* la = lds;
      const h16_t* lb = la + SA::ELEMS;
  #pragma unroll
      for (int i = 0; i < TM; ++i) fa[0][i] = SA::frag(la, wm * WR + 32 * i, 0, lane);
  #pragma unroll
      for (int j = 0; j < TN; ++j) fb[0][j] = SB::frag(lb, wn * WC + 32 * j, 0, lane);
    }
    // one k-tile; HAS_NEXT: another tile follows (the last one is peeled so
    // the pipelined body has no data-dependent branch around its waits)
    auto tile = [&](int kt, auto has_next) {
      constexpr bool HAS_NEXT = decltype(has_next)::value;
      if (kt + NS - 1 < nk) {
        const int s = (kt + NS - 1) % NS;
        sa.issue(ra, lds + s * STAGE_ELEMS, kt0 + kt + NS - 1, p.lda, p.K, wave);
        sb.issue(rb, lds + s * STAGE_ELEMS + SA::ELEMS, kt0 + kt + NS - 1, p.ldb, p.K, wave);
      }
      const h16_t* la = lds + (kt % NS) * STAGE_ELEMS;
      const h16_t* lb = la + SA::ELEMS;
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cur = ks & 1;  // KS is even: k-step 0 of every tile uses buffer 0
        if (ks + 1 < KS) {
  #pragma unroll
          for (int i = 0; i < TM; ++i) fa[cur ^ 1][i] = SA::frag(la, wm * WR + 32 * i, ks + 1, lane);
  #pragma unroll
          for (int j = 0; j < TN; ++j) fb[cur ^ 1][j] = SB::frag(lb, wn * WC + 32 * j, ks + 1, lane);
        } else if constexpr (HAS_NEXT) {
          // next stage: wait for it, then read its first fragments.  The
          // lgkmcnt(0) wait is the compiler-visible builtin (vmcnt 63, expcnt
          // 7, lgkmcnt 0) so its own wait accounting knows the older reads
          // have landed.
          __builtin_amdgcn_s_waitcnt(0xC07F);
          if (kt + NS - 1 < nk) wait_vm_barrier<(NS - 2) * L>();
          else wait_vm_barrier<0>();
          const h16_t* na = lds + ((kt + 1) % NS) * STAGE_ELEMS;
          const h16_t* nb = na + SA::ELEMS;
  #pragma unroll
          for (int i = 0; i < TM; ++i) fa[cur ^ 1][i] = SA::frag(na, wm * WR + 32 * i, 0, lane);
  #pragma unroll
          for (int j = 0; j < TN; ++j) fb[cur ^ 1][j] = SB::frag(nb, wn * WC + 32 * j, 0, lane);
        }
  #pragma unroll
        for (int i = 0; i < TM; ++i)
  #pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = MFMA_32X32X16(fa[cur][i], fb[cur][j], acc[i][j]);
        // interleave: LDS reads between MFMAs
  #pragma unroll
        for (int g = 0; g < TM + TN; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x100, AK && BKC ? 1 : 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, (TM * TN + TM + TN - 1) / (TM + TN), 0);
        }
      }
    };
    for (int kt = 0; kt + 1 < nk; ++kt) tile(kt, std::true_type());
    if (nk > 0) tile(nk - 1, std::false_type());
  }
  // every wave is done with the ring before it is reused for the epilogue
  wait_vm_barrier<0>();
  int* ys = (int*)(lds + LDS_ELEMS_EPI);
  if constexpr (EPI == EPI_HEAD) {
    if (tid < BM) ys[tid] = y_pref;
    __syncthreads();
  }

  // epilogue: per 32-row slab of the wave tile, stage fp32 in LDS, then each
  // lane handles 8 consecutive columns of one row
  float* ep = (float*)lds + wave * 32 * EP_PITCH;
  float bias8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (EPI != EPI_ACCUM && EPI != EPI_GELU_BWD && p.e.bias != nullptr && gcol < p.N) {
    const float4 b0 = *(const float4*)(p.e.bias + gcol), b1 = *(const float4*)(p.e.bias + gcol + 4);
    bias8[0] = b0.x; bias8[1] = b0.y; bias8[2] = b0.z; bias8[3] = b0.w;
    bias8[4] = b1.x; bias8[5] = b1.y; bias8[6] = b1.z; bias8[7] = b1.w;
  }
  float* part = p.part ? p.part + (int64_t)split * p.M * p.e.ldc : nullptr;
  const int splitk = p.ksplit > 1;
  // column sums of this lane's 8 columns over its rows (GELU-derivative
  // epilogue with cs_part set); zeros otherwise
  float csum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // prefetch group (register budget): a whole slab when the accumulators
  // leave room (or the operand is 16 bytes per pass), else two passes
  constexpr int PG =
      ((EPI == EPI_GELU_BWD && TM * TN <= 12) || TM * TN <= 6 || (OCC == 1 && TN <= 3)) ? NIT : 2;
  // unrolled in full: a runtime slab index would put the accumulators in scratch
#pragma clang loop unroll(full)
  for (int i = 0; i < TM; ++i) {
    const int grow0 = m0 + wm * WR + 32 * i + my_r;
    // accumulator layout of a 32x32 tile: lane l, register r -> row
    // 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ep[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EP_PITCH + 32 * j + (lane & 31)] = acc[i][j][r];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    auto row_pass = [&](int it, const Aux8& x) {
      const int lr = it * RPI + my_r;
      const int grow = grow0 + it * RPI;
      if (lane_on && lr < 32) {
        const float4 v0 = *(const float4*)(ep + lr * EP_PITCH + my_c);
        const float4 v1 = *(const float4*)(ep + lr * EP_PITCH + my_c + 4);
        const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        if (grow < p.M && gcol < p.N) epi8<EPI>(p.e, part, splitk, grow, gcol, v, bias8, x, csum);
      }
    };
    if constexpr (EPI == EPI_HEAD) {
      // p~ = exp(z) below V (0 above), the target's z, and the sum of p~ over
      // this wave's 96 columns of each row: each of the LPR lanes of a row
      // sums its 8 columns, and after the slab one lane per row adds the 12
      // sums in a fixed order
      static_assert(LPR == 12, "row sums assume 12 lanes a row");
      const int blk = (n0 + wn * WC) / 96;
      float* ps = (float*)(ys + BM) + wave * 32 * 12;
#pragma unroll 1
      for (int it = 0; it < NIT; ++it) {
        const int lr = it * RPI + my_r;
        const int grow = grow0 + it * RPI;
        float sum = 0.f;
        if (lane_on && lr < 32 && grow < p.M && gcol < p.N) {
          const float4 v0 = *(const float4*)(ep + lr * EP_PITCH + my_c);
          const float4 v1 = *(const float4*)(ep + lr * EP_PITCH + my_c + 4);
          const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          const int y = ys[grow - m0];
          float e8[8], zy = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            e8[j] = gcol + j < p.e.head.V ? __expf(v[j]) : 0.f;
            sum += e8[j];
            zy = (gcol + j == y) ? v[j] : zy;
          }
          st_nt((h16_t*)p.e.out + (int64_t)grow * p.e.ldc + gcol,
                make_uint4(pack2h(e8[0], e8[1]), pack2h(e8[2], e8[3]), pack2h(e8[4], e8[5]),
                           pack2h(e8[6], e8[7])));
          if (y >= gcol && y < gcol + 8 && y < p.e.head.V) p.e.head.zy[grow] = zy;
        }
        if (lane_on && lr < 32) ps[lr * 12 + my_c / 8] = sum;
      }
      // lane r adds the 12 lane sums of slab row r in a fixed order (the
      // wave's own LDS writes above, so no barrier)
      __builtin_amdgcn_s_waitcnt(0xC07F);
      const int grow = grow0 - my_r + lane;
      if (lane < 32 && grow < p.M && n0 + wn * WC < p.N) {
        const float4 a = *(const float4*)(ps + lane * 12);
        const float4 b4 = *(const float4*)(ps + lane * 12 + 4);
        const float4 c = *(const float4*)(ps + lane * 12 + 8);
        const float tot = ((a.x + a.y) + (a.z + a.w)) + ((b4.x + b4.y) + (b4.z + b4.w)) +
                          ((c.x + c.y) + (c.z + c.w));
        p.e.head.part[(int64_t)grow * p.e.head.npart + blk] = tot;
      }
    } else if constexpr (epi_reads_aux<EPI>()) {
      // the auxiliary operands of PG row passes are loaded together, then
      // those passes run (PG = the whole slab where registers allow); the
      // first slab's residual may already be in registers
      if (rpre_on && i == 0) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) row_pass(it, rpre[it]);
      } else {
#pragma unroll
      for (int g0 = 0; g0 < NIT; g0 += PG) {
        Aux8 ax[PG];
#pragma unroll
        for (int k = 0; k < PG; ++k) {
          const int it = g0 + k;
          const int lr = it * RPI + my_r;
          if (it < NIT && lane_on && lr < 32 && grow0 + it * RPI < p.M && gcol < p.N)
            ax[k] = aux8<EPI>(p.e, splitk, grow0 + it * RPI, gcol);
        }
#pragma unroll
        for (int k = 0; k < PG; ++k)
          if (g0 + k < NIT) row_pass(g0 + k, ax[k]);
      }
      }
    } else {
      // nothing to prefetch: a rolled loop keeps the code (and registers) small
#pragma unroll 1
      for (int it = 0; it < NIT; ++it) row_pass(it, Aux8{});
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if constexpr (EPI == EPI_GELU_BWD) {
    if (p.e.cs_part) {
      // this wave's staging area is free again (its last reads completed
      // above): lanes of one row pass put their sums side by side, then the
      // two waves sharing these columns are added in a fixed order, giving
      // one partial row per row tile: cs_part[tm][n]
      float* cw = (float*)lds + wave * 32 * EP_PITCH;
      if (lane_on) {
#pragma unroll
        for (int j = 0; j < 8; ++j) cw[my_r * WC + my_c + j] = csum[j];
      }
      __syncthreads();
      for (int t = tid; t < 2 * WC; t += 256) {
        const int wnn = t / WC, c = t % WC;
        float v = 0.f;
#pragma unroll
        for (int wmm = 0; wmm < 2; ++wmm) {
          const float* src = (const float*)lds + (wmm * 2 + wnn) * 32 * EP_PITCH;
          for (int r = 0; r < RPI; ++r) v += src[r * WC + c];
        }
        const int n = n0 + wnn * WC + c;
        if (n < p.N) p.e.cs_part[(int64_t)tm * p.N + n] = v;
      }
    }
  }
}

// out[i] = (beta ? out[i] : 0) + sum_s part[s][i], fixed order
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int ksplit, int64_t n,
                                     float* __restrict__ out, int beta) {
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i4 * 4 >= n) return;
  float4 s = beta ? ((const float4*)out)[i4] : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < ksplit; ++k) {
    const float4 v = ((const float4*)(part + (int64_t)k * n))[i4];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  st_nt((float4*)out + i4, s);
}

// launches one configuration; then, when column sums were asked for, adds
// the per-row-tile partials into cs_out
template <int BM, int BN, bool AK, bool BKC, int EPI, int NS, int BK, int OCC = 1>
int run2(Gemm2Args p, hipStream_t s) {
  p.tiles_m = (int)cdiv(p.M, BM);
  p.tiles_n = (int)cdiv(p.N, BN);
  hipLaunchKernelGGL((gemm2_kernel<BM, BN, AK, BKC, EPI, NS, BK, OCC>),
                     dim3(p.tiles_m * p.tiles_n * p.ksplit + p.red.wgs), dim3(256), 0, s, p);
  if (p.e.cs_part) {
    if (ColsumJob* d = p.e.cs_defer) {
      *d = ColsumJob();
      d->part = p.e.cs_part;
      d->out[0] = p.e.cs_out;
      d->nrow = p.tiles_m;
      d->ncol = d->seg = p.N;
      return hipGetLastError() == hipSuccess ? 0 : -4;
    }
    return colsum_finalize_launch(p.e.cs_part, p.tiles_m, p.N, p.e.cs_out, p.e.cs_beta, s);
  }
  return 0;
}

// rounds of 256 workgroups (one per CU) times the work of one tile
inline int64_t tile_cost(int64_t M, int64_t N, int BM, int BN) {
  const int64_t t = cdiv(M, BM) * cdiv(N, BN);
  return cdiv(t, 256) * BM * BN;
}

// Tile choice (measured on MI355X for the step's shapes):
//  * weight gradients (both operands m/n-contiguous): 128x128 tiles with
//    k-tiles of 64, two workgroups per CU, the token reduction split so that
//    about 400 workgroups run (partials summed in order afterwards); with
//    1024 such tiles or more (the head's gradient, never split) 128x256
//    tiles with k-tiles of 48 instead;
//  * k-contiguous products, two workgroups per CU (one's epilogue and waits
//    hide behind the other's MFMAs): with at least 1024 tiles of 256x192,
//    those tiles with 2 stages of 32 k; otherwise 128x192 tiles with 2 stages
//    of 64 k (half the barriers per k; deeper rings measured no faster);
//  * small problems: 128x128 tiles.
template <bool AK, bool BKC, int EPI>
int dispatch2(Gemm2Args p, float* ws, int64_t ws_bytes, hipStream_t s) {
  constexpr int BK = 32;
  p.ksplit = 1;
  p.k_tiles_per_split = (int)cdiv(p.K, BK);
  p.part = nullptr;
  if constexpr (EPI == EPI_ACCUM && !AK && !BKC) {
    // The head's product (a 50304-row gradient: thousands of tiles, no
    // split): 128x256 tiles with k-tiles of 48, so that two workgroups still
    // fit a CU, read a quarter fewer operand bytes per flop
    if (cdiv(p.M, 128) * cdiv(p.N, 128) >= 1024) {
      p.k_tiles_per_split = (int)cdiv(p.K, 48);
      SplitKChain* ch = p.e.chain;
      if (ch && ch->part) {
        p.red.part = ch->part;
        p.red.out = ch->out;
        p.red.n4 = ch->n / 4;
        p.red.ks = ch->ks;
        p.red.beta = ch->beta;
        p.red.wgs = 64;
        ch->part = nullptr;
      }
      return run2<128, 256, AK, BKC, EPI, 2, 48, 2>(p, s);
    }
    // 128x128 tiles, k-tiles of 64, two workgroups per CU; the token
    // reduction split so that about 400 workgroups run
    constexpr int BKW = 64;
    const int nk = (int)cdiv(p.K, BKW);
    p.k_tiles_per_split = nk;
    const int64_t tiles = cdiv(p.M, 128) * cdiv(p.N, 128);
    SplitKChain* ch = p.e.chain;
    if (ch) {
      ws = ch->ws[ch->next];
      ws_bytes = ch->ws_bytes;
    }
    int ks = 1;
    if (ws != nullptr && nk >= 8) {
      ks = (int)std::max<int64_t>(1, std::min<int64_t>(16, (400 + tiles / 2) / tiles));
      ks = std::min(ks, std::max(1, nk / 4));
      while (ks > 1 && (int64_t)ks * p.M * p.N * 4 > ws_bytes) --ks;
    }
    if (ks > 1) {
      p.k_tiles_per_split = (int)cdiv(nk, ks);
      ks = (int)cdiv(nk, p.k_tiles_per_split);
      p.ksplit = ks;
      p.part = ws;
    }
    if (ch && ch->part) {
      // the pending reduction in the slots the tiles leave free (two
      // workgroups per CU on 256 CUs), at least 64 workgroups
      p.red.part = ch->part;
      p.red.out = ch->out;
      p.red.n4 = ch->n / 4;
      p.red.ks = ch->ks;
      p.red.beta = ch->beta;
      p.red.wgs = (int)std::max<int64_t>(64, std::min<int64_t>(256, 512 - tiles * p.ksplit));
      ch->part = nullptr;
    }
    if (const int rc = run2<128, 128, AK, BKC, EPI, 2, BKW, 2>(p, s)) return rc;
    if (p.ksplit > 1) {
      const int64_t n = (int64_t)p.M * p.N;
      if (ch) {
        ch->part = ws;
        ch->out = (float*)p.e.out;
        ch->n = n;
        ch->ks = p.ksplit;
        ch->beta = p.e.beta;
        ch->next ^= 1;
      } else {
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(cdiv(n / 4, 256)), dim3(256), 0, s, ws,
                           p.ksplit, n, (float*)p.e.out, p.e.beta);
      }
    }
    return 0;
  } else {
    const int64_t t256 = cdiv(p.M, 256) * cdiv(p.N, 256);
    // the fused head's row sums are kept per 96 columns: tiles 192 wide
    if constexpr (EPI != EPI_HEAD) {
      if (t256 < 64) {  // small problem: smaller tiles keep more CUs busy
        return run2<128, 128, AK, BKC, EPI, 4, 64>(p, s);
      }
    }
    if constexpr (BKC) {
      if (cdiv(p.M, 256) * cdiv(p.N, 192) >= 1024) return run2<256, 192, AK, BKC, EPI, 2, BK, 2>(p, s);
      return run2<128, 192, AK, BKC, EPI, 2, 64, 2>(p, s);  // k-tiles of 64: half the barriers
    } else {
      return run2<256, 256, AK, BKC, EPI, 4, BK, 1>(p, s);
    }
  }
}

}  // namespace

int splitk_chain_flush(SplitKChain* ch, hipStream_t s) {
  if (!ch || !ch->part) return 0;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(cdiv(ch->n / 4, 256)), dim3(256), 0, s, ch->part,
                     ch->ks, ch->n, ch->out, ch->beta);
  ch->part = nullptr;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// The pipelined kernel covers 16-bit with k-contiguous K % 8 == 0, every
// leading dimension % 8 == 0, N % 8 == 0, ldc % 8 == 0 and operands below
// 4 GiB; otherwise returns -5 and the caller uses gemm.hip's kernel.
int gemm2_launch(bool a_kcontig, bool b_kcontig, int epi, const void* A, int lda, const void* B,
                 int ldb, int M, int N, int K, int ka_rows, int kb_rows, const GemmEpiArgs& e,
                 float* ws, int64_t ws_bytes, hipStream_t s) {
  if (K % 8 || lda % 8 || ldb % 8 || N % 8 || e.ldc % 8) return -5;
  if (e.cs_out && (epi != EPI_GELU_BWD || e.ldc != N || N % 4)) return -5;
  if (epi == EPI_HEAD &&
      (!e.head.tgt || !e.head.part || !e.head.zy || e.head.npart != (int)cdiv(N, 96)))
    return -5;
  if (epi == EPI_HEAD_DX && !e.head.r) return -5;
  if (epi == EPI_RESID && (int64_t)M * e.ldc * 4 >= (1ll << 32) - 4096) return -5;
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)e.out) & 15) return -5;
  if ((e.aux && ((uintptr_t)e.aux & 15)) || (e.out2 && ((uintptr_t)e.out2 & 15))) return -5;
  if (e.bias && ((uintptr_t)e.bias & 15)) return -5;
  const int64_t abytes = (int64_t)(a_kcontig ? M : ka_rows) * lda * 2;
  const int64_t bbytes = (int64_t)(b_kcontig ? N : kb_rows) * ldb * 2;
  if (abytes >= (1ll << 32) - 4096 || bbytes >= (1ll << 32) - 4096) return -5;
  Gemm2Args p{(const h16_t*)A, (const h16_t*)B, lda, ldb, M, N, K, ka_rows, kb_rows, 0, 0, 1, 0,
              nullptr, e};
#define G2(AKV, BKV, EPIV) \
  if (a_kcontig == AKV && b_kcontig == BKV && epi == EPIV) return dispatch2<AKV, BKV, EPIV>(p, ws, ws_bytes, s);
  G2(true, true, EPI_ACT)
  G2(true, true, EPI_F32)
  G2(true, true, EPI_RESID)
  G2(true, true, EPI_GELU)
  G2(true, true, EPI_GELU_BWD)
  G2(true, true, EPI_HEAD)
  G2(true, true, EPI_HEAD_DX)
  G2(true, false, EPI_ACT)
  G2(true, false, EPI_F32)
  G2(true, false, EPI_GELU_BWD)
  G2(false, false, EPI_ACCUM)
#undef G2
  return -5;
}

}  // namespace HALF_NS
