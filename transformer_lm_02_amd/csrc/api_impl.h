// Declarations shared by the C ABI (api.cpp, compiled once) and the host
// orchestration (gpt_api.cpp), which is compiled twice: once per 16-bit
// activation format, into namespaces b16 (bfloat16) and f16 (IEEE binary16).
// The C ABI picks the build from the handle's mode: fp32 and bfloat16 modes
// run the b16 build, float16 mode the f16 build.
#pragma once
#include <stdint.h>

#include <string>

#include "gpt_hip.h"

// the calling thread's last error message (gpt_strerror appends it)
std::string& gpt_error_text();

#define GPT_IMPL_DECLS                                                                          \
  struct Model;                                                                                 \
  int gpt_query_sizes(const gpt_config* cfg, int64_t* n_params, int64_t* workspace_bytes);      \
  int gpt_init(Model** out, const gpt_config* cfg, float* params, float* grads, float* adam_m,  \
               float* adam_v, void* workspace, const float* init_params, uint64_t seed,         \
               void* stream);                                                                   \
  int gpt_forward_loss(Model* h, const int32_t* idx, const int32_t* targets, int32_t B,         \
                       int32_t T, float loss_scale, const float* dscale,                        \
                       const gpt_dropout* dropout, float* loss_out, void* logits_out,           \
                       void* stream);                                                           \
  int gpt_backward(Model* h, int32_t zero_first, void* stream);                                 \
  int gpt_eval_loss(Model* h, const int32_t* idx, const int32_t* targets, int32_t B, int32_t T, \
                    float* loss_out, void* stream);                                             \
  int gpt_estimate_loss(Model* h, const int32_t* idx, const int32_t* targets, int32_t n_batches, \
                        int32_t B, int32_t T, float* loss_out, void* stream);                   \
  int gpt_adamw_step(Model* h, float lr, float beta1, float beta2, float eps,                   \
                     float weight_decay, float max_norm, int32_t t, int32_t skip_nonfinite,     \
                     float* norm_out, void* stream);                                            \
  int gpt_amp_step(Model* h, float lr, float beta1, float beta2, float eps, float weight_decay, \
                   float max_norm, gpt_loss_scaler* scaler, float growth_factor,               \
                   float backoff_factor, int32_t growth_interval, float* norm_out,             \
                   void* stream);                                                               \
  int64_t gpt_kv_cache_bytes(const gpt_config* c, int32_t B, int32_t max_len);                  \
  int gpt_prefill(Model* h, const int32_t* idx, int32_t B, int32_t T0, void* kv,                \
                  int32_t max_len, float* logits_out, void* stream);                            \
  int gpt_decode_step(Model* h, const int32_t* tok, int32_t B, int32_t pos, void* kv,           \
                      int32_t max_len, float* logits_out, void* stream);                        \
  int gpt_sample(const float* logits, int32_t B, int32_t V, int32_t ldv, float temperature,     \
                 int32_t top_k, const float* u, int32_t* tok_out, void* stream);                \
  int gpt_read_flags(Model* h, int32_t* flags, void* stream);                                   \
  int gpt_set_option(Model* h, int32_t option, int32_t value);                                  \
  int gpt_get_option(Model* h, int32_t option, int32_t* value);                                 \
  int gpt_read_timing(Model* h, double* ms, int64_t* launches);                                 \
  void gpt_destroy(Model* h);                                                                   \
  int gpt_op_linear(int32_t h16, const void* A, const void* B, const float* bias, void* C,      \
                    int32_t out_f32, int32_t M, int32_t N, int32_t K, void* stream);            \
  int gpt_op_linear_gelu(int32_t h16, const void* A, const void* W, const float* bias,        \
                         void* dgelu, void* g, int32_t M, int32_t N, int32_t K, void* stream);   \
  int gpt_op_linear_gelu_bwd(int32_t h16, const void* dY, const void* Wt, const void* dgelu,    \
                             void* du, float* dbias, int32_t accumulate_bias, int32_t M,        \
                             int32_t N, int32_t K, float* workspace, int64_t workspace_bytes,   \
                             void* stream);                                                     \
  int gpt_op_linear_dw(int32_t h16, const void* dY, const void* X, float* dW,                   \
                       int32_t accumulate, int32_t M, int32_t N, int32_t K, float* workspace,   \
                       int64_t workspace_bytes, void* stream);                                  \
  int gpt_op_linear_dw_seq(int32_t h16, int32_t count, const void* const* dY,                  \
                           const void* const* X, float* const* dW, const int32_t* accumulate,   \
                           const int32_t* M, const int32_t* N, const int32_t* K,                \
                           float* workspace, int64_t workspace_bytes, void* stream);            \
  int gpt_op_linear_dx(int32_t h16, const void* dY, const void* W, float* dX, int32_t M,        \
                       int32_t N, int32_t K, void* stream);                                     \
  int gpt_op_attention_fwd(int32_t h16, const void* qkv, void* out, float* lse, int32_t B,      \
                           int32_t T, int32_t H, int32_t C, void* stream);                      \
  int gpt_op_attention_bwd(int32_t h16, const void* qkv, const void* out, const float* lse,     \
                           const void* dout, void* dqkv, float* D, int32_t B, int32_t T,        \
                           int32_t H, int32_t C, void* stream);                                 \
  int gpt_op_layernorm_fwd(int32_t h16, const float* x, const float* w, const float* b,         \
                           void* y, float* mean, float* rstd, int32_t M, int32_t C,             \
                           void* stream);                                                       \
  int gpt_op_dropout(const float* x, float* y, int64_t rows, int32_t cols, float p,             \
                     uint64_t seed, uint32_t step, uint32_t site_word, void* stream);           \
  int gpt_op_cross_entropy(int32_t h16, void* logits, const int32_t* targets, float* loss,      \
                           float* row_loss, int32_t* n_valid, float loss_scale, int32_t N,      \
                           int32_t V, int32_t ldv, void* stream);

namespace b16 {
GPT_IMPL_DECLS
}
namespace f16 {
GPT_IMPL_DECLS
}
