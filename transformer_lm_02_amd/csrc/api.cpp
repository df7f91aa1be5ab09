// C ABI of libgpt_hip.so.  Each entry point forwards to the build of the host
// orchestration for the handle's (or the call's) activation format: the b16
// build serves GPT_FP32 and GPT_BF16, the f16 build GPT_FP16.  The two builds
// share no state; a handle records which one created it.
#include "api_impl.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>
#include <string>

// Device scratch of gpt_op_linear_gelu_bwd_noalloc: the column-sum partials
// of its bias gradient, for callers that cannot allocate.  Each device holds
// its own copy until the process ends; its address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is handed to kernels.
static constexpr int64_t kNoAllocScratchBytes = 4 << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / 4];

std::string& gpt_error_text() {
  static thread_local std::string msg;
  return msg;
}

struct gpt_model {
  bool fp16;
  void* impl;  // b16::Model or f16::Model
};

namespace {
int null_handle() {
  gpt_error_text() = "null handle";
  return GPT_EINVAL;
}
// GPT_FP32 = 0 and GPT_BF16 = 1 pass a 0/1 flag to the b16 build; GPT_FP16
// passes 1 to the f16 build
bool op_fp16(int32_t dtype) { return dtype == GPT_FP16; }
int32_t op_h16(int32_t dtype) { return dtype != GPT_FP32; }
int bad_dtype() {
  gpt_error_text() = "dtype must be GPT_FP32, GPT_BF16 or GPT_FP16";
  return GPT_EINVAL;
}
bool dtype_ok(int32_t dtype) { return dtype == GPT_FP32 || dtype == GPT_BF16 || dtype == GPT_FP16; }

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// the scratch's device address on the calling thread's current device, which
// must be the device of `stream` (a null stream is the current device's)
int current_device_scratch(hipStream_t stream, float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    gpt_error_text() = hipGetErrorString(e);
    return GPT_EHIP;
  }
  if (stream) {
    hipDevice_t sdev = dev;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) {
      gpt_error_text() = hipGetErrorString(e);
      return GPT_EHIP;
    }
    if ((int)sdev != dev) {
      gpt_error_text() = "linear_gelu_bwd_noalloc: the stream belongs to another device than the "
                         "current one (make the stream's device current)";
      return GPT_EINVAL;
    }
  }
  if (dev < 0 || dev >= kMaxDevices) {
    gpt_error_text() = "device ordinal beyond the scratch table";
    return GPT_EUNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      gpt_error_text() = e != hipSuccess ? hipGetErrorString(e) : "null scratch address";
      return GPT_EHIP;
    }
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return GPT_OK;
}
}  // namespace

#define OP(name, dtype, ...)                                                            \
  (!dtype_ok(dtype) ? bad_dtype()                                                       \
                    : op_fp16(dtype) ? f16::name(op_h16(dtype), __VA_ARGS__)             \
                                     : b16::name(op_h16(dtype), __VA_ARGS__))

extern "C" {

int gpt_query_sizes(const gpt_config* cfg, int64_t* n_params, int64_t* workspace_bytes) {
  if (cfg && cfg->mode == GPT_FP16) return f16::gpt_query_sizes(cfg, n_params, workspace_bytes);
  return b16::gpt_query_sizes(cfg, n_params, workspace_bytes);
}

int gpt_init(gpt_model** out, const gpt_config* cfg, float* params, float* grads, float* adam_m,
             float* adam_v, void* workspace, const float* init_params, uint64_t seed,
             void* stream) {
  if (!out) {
    gpt_error_text() = "null output handle";
    return GPT_EINVAL;
  }
  *out = nullptr;
  const bool fp16 = cfg && cfg->mode == GPT_FP16;
  void* impl = nullptr;
  int rc;
  if (fp16) {
    f16::Model* m = nullptr;
    rc = f16::gpt_init(&m, cfg, params, grads, adam_m, adam_v, workspace, init_params, seed, stream);
    impl = m;
  } else {
    b16::Model* m = nullptr;
    rc = b16::gpt_init(&m, cfg, params, grads, adam_m, adam_v, workspace, init_params, seed, stream);
    impl = m;
  }
  if (rc != GPT_OK) return rc;  // the build's own init released what it made
  *out = new gpt_model{fp16, impl};
  return GPT_OK;
}

int gpt_forward_loss(gpt_model* h, const int32_t* idx, const int32_t* targets, int32_t B,
                     int32_t T, float loss_scale, float* loss_out, void* logits_out,
                     void* stream) {
  if (!h) return null_handle();
  return gpt_forward_loss_ex(h, idx, targets, B, T, loss_scale, nullptr, nullptr, loss_out,
                             logits_out, stream);
}

int gpt_forward_loss_scaled(gpt_model* h, const int32_t* idx, const int32_t* targets, int32_t B,
                            int32_t T, float loss_scale, const gpt_loss_scaler* scaler,
                            float* loss_out, void* logits_out, void* stream) {
  if (!h) return null_handle();
  if (!scaler) {
    gpt_error_text() = "null scaler";
    return GPT_EINVAL;
  }
  return gpt_forward_loss_ex(h, idx, targets, B, T, loss_scale, scaler, nullptr, loss_out,
                             logits_out, stream);
}

int gpt_forward_loss_ex(gpt_model* h, const int32_t* idx, const int32_t* targets, int32_t B,
                        int32_t T, float loss_scale, const gpt_loss_scaler* scaler,
                        const gpt_dropout* dropout, float* loss_out, void* logits_out,
                        void* stream) {
  if (!h) return null_handle();
  const float* ds = scaler ? &scaler->scale : nullptr;
  return h->fp16 ? f16::gpt_forward_loss((f16::Model*)h->impl, idx, targets, B, T, loss_scale, ds,
                                         dropout, loss_out, logits_out, stream)
                 : b16::gpt_forward_loss((b16::Model*)h->impl, idx, targets, B, T, loss_scale, ds,
                                         dropout, loss_out, logits_out, stream);
}

int gpt_eval_loss(gpt_model* h, const int32_t* idx, const int32_t* targets, int32_t B, int32_t T,
                  float* loss_out, void* stream) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_eval_loss((f16::Model*)h->impl, idx, targets, B, T, loss_out, stream)
                 : b16::gpt_eval_loss((b16::Model*)h->impl, idx, targets, B, T, loss_out, stream);
}

int gpt_estimate_loss(gpt_model* h, const int32_t* idx, const int32_t* targets, int32_t n_batches,
                      int32_t B, int32_t T, float* loss_out, void* stream) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_estimate_loss((f16::Model*)h->impl, idx, targets, n_batches, B, T,
                                          loss_out, stream)
                 : b16::gpt_estimate_loss((b16::Model*)h->impl, idx, targets, n_batches, B, T,
                                          loss_out, stream);
}

int gpt_backward(gpt_model* h, int32_t zero_first, void* stream) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_backward((f16::Model*)h->impl, zero_first, stream)
                 : b16::gpt_backward((b16::Model*)h->impl, zero_first, stream);
}

int gpt_adamw_step(gpt_model* h, float lr, float beta1, float beta2, float eps, float weight_decay,
                   float max_norm, int32_t t, int32_t skip_nonfinite, float* norm_out,
                   void* stream) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_adamw_step((f16::Model*)h->impl, lr, beta1, beta2, eps, weight_decay,
                                       max_norm, t, skip_nonfinite, norm_out, stream)
                 : b16::gpt_adamw_step((b16::Model*)h->impl, lr, beta1, beta2, eps, weight_decay,
                                       max_norm, t, skip_nonfinite, norm_out, stream);
}

int gpt_amp_step(gpt_model* h, float lr, float beta1, float beta2, float eps, float weight_decay,
                 float max_norm, gpt_loss_scaler* scaler, float growth_factor, float backoff_factor,
                 int32_t growth_interval, float* norm_out, void* stream) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_amp_step((f16::Model*)h->impl, lr, beta1, beta2, eps, weight_decay,
                                     max_norm, scaler, growth_factor, backoff_factor,
                                     growth_interval, norm_out, stream)
                 : b16::gpt_amp_step((b16::Model*)h->impl, lr, beta1, beta2, eps, weight_decay,
                                     max_norm, scaler, growth_factor, backoff_factor,
                                     growth_interval, norm_out, stream);
}

int64_t gpt_kv_cache_bytes(const gpt_config* cfg, int32_t B, int32_t max_len) {
  if (cfg && cfg->mode == GPT_FP16) return f16::gpt_kv_cache_bytes(cfg, B, max_len);
  return b16::gpt_kv_cache_bytes(cfg, B, max_len);
}

int gpt_prefill(gpt_model* h, const int32_t* idx, int32_t B, int32_t T0, void* kv,
                int32_t max_len, float* logits_out, void* stream) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_prefill((f16::Model*)h->impl, idx, B, T0, kv, max_len, logits_out,
                                    stream)
                 : b16::gpt_prefill((b16::Model*)h->impl, idx, B, T0, kv, max_len, logits_out,
                                    stream);
}

int gpt_decode_step(gpt_model* h, const int32_t* tok, int32_t B, int32_t pos, void* kv,
                    int32_t max_len, float* logits_out, void* stream) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_decode_step((f16::Model*)h->impl, tok, B, pos, kv, max_len,
                                        logits_out, stream)
                 : b16::gpt_decode_step((b16::Model*)h->impl, tok, B, pos, kv, max_len,
                                        logits_out, stream);
}

int gpt_sample(const float* logits, int32_t B, int32_t V, int32_t ldv, float temperature,
               int32_t top_k, const float* u, int32_t* tok_out, void* stream) {
  return b16::gpt_sample(logits, B, V, ldv, temperature, top_k, u, tok_out, stream);
}

int gpt_set_option(gpt_model* h, int32_t option, int32_t value) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_set_option((f16::Model*)h->impl, option, value)
                 : b16::gpt_set_option((b16::Model*)h->impl, option, value);
}

int gpt_get_option(gpt_model* h, int32_t option, int32_t* value) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_get_option((f16::Model*)h->impl, option, value)
                 : b16::gpt_get_option((b16::Model*)h->impl, option, value);
}

int gpt_read_timing(gpt_model* h, double* ms, int64_t* launches) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_read_timing((f16::Model*)h->impl, ms, launches)
                 : b16::gpt_read_timing((b16::Model*)h->impl, ms, launches);
}

int gpt_read_flags(gpt_model* h, int32_t* flags, void* stream) {
  if (!h) return null_handle();
  return h->fp16 ? f16::gpt_read_flags((f16::Model*)h->impl, flags, stream)
                 : b16::gpt_read_flags((b16::Model*)h->impl, flags, stream);
}

void gpt_destroy(gpt_model* h) {
  if (!h) return;
  if (h->fp16)
    f16::gpt_destroy((f16::Model*)h->impl);
  else
    b16::gpt_destroy((b16::Model*)h->impl);
  delete h;
}

// Learning rate at iteration it: linear warmup to max_lr, cosine decay to
// min_lr at decay_end, min_lr afterwards ("nanoGPT", Part IV Stage 1, get_lr)
double gpt_lr_at(int64_t it, double max_lr, double min_lr, int64_t warmup, int64_t decay_end) {
  if (it < 0 || warmup < 0 || decay_end <= warmup) return NAN;
  if (it < warmup) return max_lr * (double)(it + 1) / (double)warmup;
  if (it > decay_end) return min_lr;
  const double ratio = (double)(it - warmup) / (double)(decay_end - warmup);
  const double coeff = 0.5 * (1.0 + cos(M_PI * ratio));  // 1 at warmup, 0 at decay_end
  return min_lr + coeff * (max_lr - min_lr);
}

const char* gpt_strerror(int code) {
  static thread_local std::string msg;
  const char* base = "unknown error";
  switch (code) {
    case GPT_OK: return "ok";
    case GPT_EINVAL: base = "invalid argument"; break;
    case GPT_ESEQLEN: base = "sequence longer than block_size"; break;
    case GPT_ESTATE: base = "invalid call order"; break;
    case GPT_EHIP: base = "HIP error"; break;
    case GPT_EUNSUPPORTED: base = "unsupported shape"; break;
  }
  const std::string& e = gpt_error_text();
  msg = std::string(base) + (e.empty() ? "" : ": " + e);
  return msg.c_str();
}

int gpt_op_linear(int32_t dtype, const void* A, const void* B, const float* bias, void* C,
                  int32_t out_f32, int32_t M, int32_t N, int32_t K, void* stream) {
  return OP(gpt_op_linear, dtype, A, B, bias, C, out_f32, M, N, K, stream);
}

int gpt_op_linear_gelu(int32_t dtype, const void* A, const void* W, const float* bias,
                       void* dgelu, void* g, int32_t M, int32_t N, int32_t K, void* stream) {
  return OP(gpt_op_linear_gelu, dtype, A, W, bias, dgelu, g, M, N, K, stream);
}

int gpt_op_linear_gelu_bwd(int32_t dtype, const void* dY, const void* Wt, const void* dgelu,
                           void* du, float* dbias, int32_t accumulate_bias, int32_t M, int32_t N,
                           int32_t K, float* workspace, int64_t workspace_bytes, void* stream) {
  return OP(gpt_op_linear_gelu_bwd, dtype, dY, Wt, dgelu, du, dbias, accumulate_bias, M, N, K,
            workspace, workspace_bytes, stream);
}

int gpt_op_linear_gelu_bwd_noalloc(int32_t dtype, const void* dY, const void* Wt,
                                   const void* dgelu, void* du, float* dbias,
                                   int32_t accumulate_bias, int32_t M, int32_t N, int32_t K,
                                   void* stream) {
  if (!dtype_ok(dtype)) return bad_dtype();
  float* ws = nullptr;
  if (dbias && M > 0 && N > 0) {
    if (((int64_t)M + 127) / 128 * (int64_t)N * 4 > kNoAllocScratchBytes) {
      gpt_error_text() =
          "linear_gelu_bwd_noalloc: ceil(M/128) * N * 4 bytes of column sums exceed its 4 MiB "
          "scratch";
      return GPT_EINVAL;
    }
    if (int rc = current_device_scratch((hipStream_t)stream, &ws)) return rc;
  }
  return OP(gpt_op_linear_gelu_bwd, dtype, dY, Wt, dgelu, du, dbias, accumulate_bias, M, N, K, ws,
            ws ? kNoAllocScratchBytes : 0, stream);
}

int gpt_op_linear_dw(int32_t dtype, const void* dY, const void* X, float* dW, int32_t accumulate,
                     int32_t M, int32_t N, int32_t K, float* workspace, int64_t workspace_bytes,
                     void* stream) {
  return OP(gpt_op_linear_dw, dtype, dY, X, dW, accumulate, M, N, K, workspace, workspace_bytes,
            stream);
}

int gpt_op_linear_dw_seq(int32_t dtype, int32_t count, const void* const* dY, const void* const* X,
                         float* const* dW, const int32_t* accumulate, const int32_t* M,
                         const int32_t* N, const int32_t* K, float* workspace,
                         int64_t workspace_bytes, void* stream) {
  return OP(gpt_op_linear_dw_seq, dtype, count, dY, X, dW, accumulate, M, N, K, workspace,
            workspace_bytes, stream);
}

int gpt_op_linear_dx(int32_t dtype, const void* dY, const void* W, float* dX, int32_t M, int32_t N,
                     int32_t K, void* stream) {
  return OP(gpt_op_linear_dx, dtype, dY, W, dX, M, N, K, stream);
}

int gpt_op_attention_fwd(int32_t dtype, const void* qkv, void* out, float* lse, int32_t B,
                         int32_t T, int32_t H, int32_t C, void* stream) {
  return OP(gpt_op_attention_fwd, dtype, qkv, out, lse, B, T, H, C, stream);
}

int gpt_op_attention_bwd(int32_t dtype, const void* qkv, const void* out, const float* lse,
                         const void* dout, void* dqkv, float* D, int32_t B, int32_t T, int32_t H,
                         int32_t C, void* stream) {
  return OP(gpt_op_attention_bwd, dtype, qkv, out, lse, dout, dqkv, D, B, T, H, C, stream);
}

int gpt_op_layernorm_fwd(int32_t dtype, const float* x, const float* w, const float* b, void* y,
                         float* mean, float* rstd, int32_t M, int32_t C, void* stream) {
  return OP(gpt_op_layernorm_fwd, dtype, x, w, b, y, mean, rstd, M, C, stream);
}

int gpt_op_dropout(const float* x, float* y, int64_t rows, int32_t cols, float p, uint64_t seed,
                   uint32_t step, uint32_t site_word, void* stream) {
  return b16::gpt_op_dropout(x, y, rows, cols, p, seed, step, site_word, stream);
}

int gpt_op_cross_entropy(int32_t dtype, void* logits, const int32_t* targets, float* loss,
                         float* row_loss, int32_t* n_valid, float loss_scale, int32_t N, int32_t V,
                         int32_t ldv, void* stream) {
  return OP(gpt_op_cross_entropy, dtype, logits, targets, loss, row_loss, n_valid, loss_scale, N, V,
            ldv, stream);
}

}  // extern "C"
