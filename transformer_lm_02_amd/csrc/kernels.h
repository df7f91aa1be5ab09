// Launchers of the HIP kernels (host side).  Each returns 0, -4 (HIP launch
// error) or -5 (shape the kernel does not cover).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "gemm.h"

namespace HALF_NS {


struct AdamChunk {
  int64_t offset;
  int32_t count;
  int32_t decay;
};

// One piece (at most 8192 elements, a multiple of 4, starting at a multiple
// of 4) of one parameter tensor for the initialisation from a seed:
// std > 0 draws N(0, std^2), otherwise every element is `value`.
struct InitSeg {
  int64_t offset;
  int32_t count;
  int32_t pad;
  float std;
  float value;
};
// The fused head + cross-entropy (see HeadEpi in gemm.h): per row the loss,
// the gradient factor r, h2 = r * h and the target column of the stored
// exp(z) minus the row's sum; flag bit 4 when a row's exp-sum leaves the
// range the 16-bit exp(z) can carry
int head_combine_launch(const float* part, int npart, const float* zy, const int32_t* tgt, int V,
                        const int* n_valid, float loss_scale, const float* dscale, const h16_t* h,
                        int C, float* row_loss, float* r, h16_t* h2, h16_t* logits, int ldv, int M,
                        int* flags, hipStream_t s);
// out = mean of x[0..n) (fp64 sum in a fixed order)
int mean_launch(const float* x, int n, float* out, hipStream_t s);
int init_params_launch(float* params, const InitSeg* segs, int nsegs, uint64_t seed,
                       hipStream_t s);

// one matrix of the transposed weight copy: src [rows][cols] (elements from
// the start of the 16-bit weights) -> dst [cols][ld] (ld >= rows)
struct TransposeJob {
  int64_t src, dst;
  int32_t rows, cols, ld, tile_begin;
};
int transpose_h16_launch(const h16_t* src, h16_t* dst, const TransposeJob* jobs, int njobs,
                          int total_tiles, hipStream_t s);

// dr: dropout of the attention probabilities (site word without bh; the
// kernels add b * H + h).  dmask: the kept bits, written by the forward and
// read by the backward of the head-width-64 16-bit kernels (required there
// with dropout: B * H * cdiv(T, 64) * 2 * T 32-bit words)
int attention_fwd_launch(bool h16, const void* qkv, void* out, float* lse, int B, int Tn, int H,
                         int C, hipStream_t s, Drop dr = Drop(), uint32_t* dmask = nullptr);
// defer (optional): see ColsumJob; honoured by the head-width-64 16-bit path
int attention_bwd_launch(bool h16, const void* qkv, const void* out, const float* lse,
                         const void* dout, void* dqkv, float* D, int B, int Tn, int H, int C,
                         float* cs_part, float* cs_out, int cs_beta, hipStream_t s,
                         ColsumJob* defer = nullptr, Drop dr = Drop(),
                         const uint32_t* dmask = nullptr);

int layernorm_fwd_launch(bool h16, const float* x, const float* w, const float* b, void* y,
                         float* mean, float* rstd, int M, int C, hipStream_t s);
int layernorm_bwd_part_rows(int M);
// dy: the mode's activation type (16-bit or fp32) [M][C]
// dres_act and bias_grad carry the dropout multipliers of dr (see layernorm.hip)
int layernorm_bwd_launch(bool h16, const void* dy, const float* x, const float* mean,
                         const float* rstd, const float* w, float* dres, void* dres_act,
                         int accumulate, float* part, float* dw, float* db, float* bias_grad,
                         int beta, int M, int C, hipStream_t s, ColsumJob* defer = nullptr,
                         Drop dr = Drop());

// dr: dropout of the embedding sum (Drop in common.h; default: none)
int embed_fwd_launch(const int32_t* idx, const float* wte, const float* wpe, float* x, int M,
                     int Tn, int C, int Vp, int* flags, hipStream_t s, Drop dr = Drop());
// y [M][C] fp32 = x times the dropout multipliers of dr (a copy when dr is
// off; y may be x); C % 4 == 0
int dropout_rows_launch(const float* x, float* y, int64_t M, int C, Drop dr, hipStream_t s);
int embed_bwd_launch(const int32_t* idx, const float* dx, float* dwte, float* dwpe, int B, int Tn,
                     int block_size, int C, int Vp, int beta_wpe, hipStream_t s);
// n_valid = count of targets in [0, V); a target outside [-1, V) sets bit 2
// of *flags (when flags is not null) and counts as ignored
int count_valid_launch(const int32_t* tgt, int N, int V, int* out, int* flags, hipStream_t s);
// dscale (optional, device): the gradient is further multiplied by *dscale;
// write_grad = 0: only the row losses (the logits are left as they are)
int cross_entropy_launch(bool h16, void* logits, const int32_t* tgt, float* row_loss,
                         const int* n_valid, float loss_scale, const float* dscale, int N, int V,
                         int ldv, hipStream_t s, int write_grad = 1);
int loss_finalize_launch(const float* row_loss, int N, const int* n_valid, float* loss,
                         hipStream_t s);
int colsum_part_rows(int M);
// out (+)= column sums of part [nrow][ncol] (ncol % 4 == 0)
int colsum_finalize_launch(const float* part, int nrow, int ncol, float* out, int beta,
                           hipStream_t s);
int colsum_launch(bool h16, const void* a, int M, int N, float* part, float* out, int beta,
                  hipStream_t s);
// finishes n ColsumJobs (each ncol % 4 == 0) in one launch per
// COLSUM_GROUP_MAX jobs
#define COLSUM_GROUP_MAX 56
int colsum_finalize_group_launch(const ColsumJob* jobs, int n, int beta, hipStream_t s);

// sampling with a key/value cache: cache kv[k|v][b][h][t][hs] of one layer
// (t < max_len), in the mode's activation type
int kv_store_launch(bool h16, const void* qkv, void* kv, int B, int Tn, int H, int hs,
                    int max_len, int pos0, hipStream_t s);
int decode_attn_launch(bool h16, const void* qkv, const void* kv, void* out, int B, int H, int hs,
                       int max_len, int len, hipStream_t s);
int sample_launch(const float* logits, int B, int V, int ldv, float temperature, int top_k,
                  const float* u, int32_t* tok, hipStream_t s);
// products of the few rows of a decode step: see decode.hip
bool gemv_fits(bool h16, bool ln, int M, int K);
int gemv_launch(bool h16, int epi, const void* A, const float* ln_w, const float* ln_b,
                const void* W, const float* bias, const float* aux, void* out, int M, int N, int K,
                int ldo, void* kv, int H, int hs, int max_len, int pos, hipStream_t s);

int adamw_norm_blocks();
// Weight matrices updated by 64 x 64 tiles, each also writing its transposed
// 16-bit copy (jobs as for transpose_h16_launch, dstT its destination base);
// ntiles = 0: none (every tensor in the flat chunks).
struct TileJobs {
  h16_t* dstT = nullptr;
  const TransposeJob* jobs = nullptr;
  int njobs = 0, ntiles = 0;
};
int adamw_launch(float* p, const float* g, float* m, float* v, h16_t* shadow, int64_t n,
                 const AdamChunk* chunks, int nchunks, const TileJobs& tj, double* norm_part,
                 float* scal, float* norm_out, float lr, float beta1, float beta2, float eps,
                 float wd, float max_norm, int t, int skip_nonfinite, hipStream_t s);
// the same with dynamic loss scaling; scaler: device {scale, growth_tracker,
// steps, found_inf} (float, int32 x3), read and updated in place
int adamw_amp_launch(float* p, const float* g, float* m, float* v, h16_t* shadow, int64_t n,
                     const AdamChunk* chunks, int nchunks, const TileJobs& tj,
                     double* norm_part, float* scal,
                     float* norm_out, float lr, float beta1, float beta2, float eps, float wd,
                     float max_norm, float* scaler, float growth, float backoff, int interval,
                     hipStream_t s);
int to_h16_launch(const float* p, h16_t* o, int64_t n, hipStream_t s);

}  // namespace HALF_NS
