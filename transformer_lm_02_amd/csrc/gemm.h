// GEMM launchers: C[m][n] = sum_k A(m,k) B(n,k), with fused epilogues.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace HALF_NS {

// Epilogues, applied per output element (m, n) to the fp32 accumulator:
enum GemmEpi {
  EPI_ACT = 0,      // out_act[m][n] = acc + bias[n]
  EPI_F32 = 1,      // out_f32[m][n] = acc + bias[n]
  EPI_RESID = 2,    // out_f32[m][n] = aux_f32[m][n] + z[m][n] (acc + bias[n])  (residual add;
                    // z the dropout multiplier of GemmEpiArgs::drop, 1 without dropout)
  EPI_GELU = 3,     // u = acc + bias[n]; out_act = gelu'(u); out2_act = gelu(u)
  EPI_GELU_BWD = 4, // out_act[m][n] = acc * aux_act[m][n]  (aux: the stored gelu'(u))
  EPI_ACCUM = 5,    // out_f32[m][n] = (beta ? out_f32[m][n] : 0) + acc
  EPI_HEAD = 6,     // tied head with the cross-entropy fused (see HeadEpi): out_act[m][n] =
                    // exp(acc) for n < V, 0 for n >= V; plus row sums and the target logit
  EPI_HEAD_DX = 7   // out_act[m][n] = r[m] acc  (see HeadEpi)
};

// Operands of the fused head + cross-entropy epilogues.  The forward stores
// p~ = exp(z) (shift 0) instead of the logits z, part[m][n / 96] = sum of p~
// over each block of 96 columns below V (fixed order, from the fp32 values)
// and zy[m] = z at n = tgt[m] (when 0 <= tgt[m] < V).  A later pass takes the
// row sum S, stores p~ - S at the target column and r[m] = sc[m] / S (sc the
// row's loss scale, zero for an ignored row): the logit gradient
// sc (softmax - onehot) is then r[m] times the stored row, which the
// input-gradient product applies in its epilogue.
struct HeadEpi {
  const int32_t* tgt = nullptr;
  float* part = nullptr;
  float* zy = nullptr;
  int V = 0;
  int npart = 0;  // blocks of 96 columns per row: ceil(N / 96)
  const float* r = nullptr;
};

// A column-sum finalize left for later: out[k][i] = (beta ? out[k][i] : 0)
// + sum over the nrow rows of part [nrow][ncol] at column k * seg + i
// (k = 0, 1, 2; a null out[k] skips its columns).  Producers fill one when
// handed a non-null ColsumJob*, so that one launch can finish many.
struct ColsumJob {
  const float* part = nullptr;
  float* out[3] = {nullptr, nullptr, nullptr};
  int nrow = 0, ncol = 0, seg = 0;
};

// Weight gradients launched one after another can pass their split-K
// reductions along: a launch handed a chain writes its partials into one
// half of the chain's scratch and leaves the reduction pending, and the next
// such launch runs the pending reduction in workgroups of its own beside its
// tiles (they use slots the tiles leave free) while its tiles write into the
// other half.  The reduction adds the partials in split order to the gradient
// (or to zero), as the standalone reduction does, so results are the same.
// splitk_chain_flush runs whatever is still pending.
struct SplitKChain {
  float* ws[2] = {nullptr, nullptr};  // the two halves of the scratch
  int64_t ws_bytes = 0;               // bytes of each half
  int next = 0;                       // the half the next launch writes
  // the pending reduction, if part is non-null: out[i] = (beta ? out[i] : 0)
  // + sum over k < ks of part[k * n + i]
  const float* part = nullptr;
  float* out = nullptr;
  int64_t n = 0;
  int ks = 0, beta = 0;
};

struct GemmEpiArgs {
  void* out = nullptr;
  void* out2 = nullptr;
  const void* aux = nullptr;
  const float* bias = nullptr;
  int ldc = 0;
  int beta = 0;
  // Optional column sums of the output (a bias gradient):
  // cs_out[n] = (cs_beta ? cs_out[n] : 0) + sum_m out[m][n].  cs_part is fp32
  // scratch of at least cdiv(M, 128) * N elements.  The GELU-derivative
  // epilogue of the pipelined kernel forms them from its fp32 values before
  // rounding; every other case sums the stored output afterwards.
  float* cs_part = nullptr;
  float* cs_out = nullptr;
  int cs_beta = 0;
  // non-null: the pipelined kernel's column sums are left in cs_part and
  // described here instead of finalized (part = nullptr if it finalized)
  ColsumJob* cs_defer = nullptr;
  // EPI_RESID: dropout of the branch output (element (m, n) of the site)
  Drop drop;
  // EPI_HEAD, EPI_HEAD_DX
  HeadEpi head;
  // EPI_ACCUM: non-null to take part in a chain of split-K reductions (host
  // side; the scratch then comes from the chain)
  SplitKChain* chain = nullptr;
};

// A(m,k) = a_kcontig ? A[m*lda + k] : A[k*lda + m]; likewise B(n,k).
// Loads of a k-contiguous operand require K % 8 == 0 (16-bit); an m- or
// n-contiguous operand reads rows k < ka_rows / kb_rows and columns below its
// leading dimension.  Outputs are written for m < M, n < N.
// ws / ws_bytes: optional fp32 scratch for split-K weight gradients.
int gemm_launch(bool h16, bool a_kcontig, bool b_kcontig, int epi,
                const void* A, int lda, const void* B, int ldb,
                int M, int N, int K, int ka_rows, int kb_rows,
                const GemmEpiArgs& e, hipStream_t stream,
                float* ws = nullptr, int64_t ws_bytes = 0);

// split-K scratch the launcher may use for an M x N weight gradient
inline int64_t gemm_splitk_bytes(int64_t M, int64_t N) { return 16 * M * N * 4; }

// runs the chain's pending reduction, if any, as a launch of its own
int splitk_chain_flush(SplitKChain* ch, hipStream_t stream);

}  // namespace HALF_NS
