/*
 * gpt_hip.h - C ABI of libgpt_hip.so: one GPT-2 training step (forward,
 * backward, fused AdamW) on an MI355X (gfx950), written in HIP.
 *
 * The model is the decoder-only pre-norm Transformer of "nanoGPT"
 * (stanleyjacob.dev), Part IV Stage 4 and Part V Deep dive 1: token plus
 * learned position embeddings, n_layer blocks of x += attn(ln_1(x)) and
 * x += mlp(ln_2(x)) with causal multi-head self-attention and a tanh-GELU MLP,
 * a final LayerNorm and an LM head tied to the token embedding, over a
 * vocabulary padded to a multiple of 64 ("Let's reproduce GPT-2 (124M)",
 * chapter "Nice/Ugly Numbers": 50257 -> 50304).
 *
 * Conventions shared by every entry point:
 *   - Device memory is owned by the caller.  The library never allocates or
 *     frees device memory; the handle holds host metadata only.
 *   - `stream` is a hipStream_t passed as void*.  Every call only enqueues
 *     work on it, except gpt_init (which waits once for its set-up work) and
 *     gpt_read_flags.  Scalars that the step produces (loss, gradient norm)
 *     are written to device memory.
 *   - Return value: 0 on success, a negative GPT_E* code on failure.  On
 *     failure nothing has been enqueued.  gpt_strerror names the code.
 *   - All float arguments and buffers are IEEE fp32 unless stated.
 *
 * Canonical flat parameter order (fp32, also used for grads, adam_m, adam_v):
 *   wte[Vp][d], wpe[block_size][d], then for each layer
 *   ln1.w[d] ln1.b[d] attn.w[3d][d] attn.b[3d] aproj.w[d][d] aproj.b[d]
 *   ln2.w[d] ln2.b[d] fc.w[4d][d] fc.b[4d] mproj.w[d][4d] mproj.b[d],
 *   then lnf.w[d] lnf.b[d].  Linear weights are [out][in].  The tied LM head
 *   is wte itself ("nanoGPT", Deep dive 1, weight tying).
 */
#ifndef GPT_HIP_H
#define GPT_HIP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  GPT_OK = 0,
  GPT_EINVAL = -1,   /* bad config or argument, null pointer, B > max_batch */
  GPT_ESEQLEN = -2,  /* T > block_size ("Let's reproduce GPT-2 (124M)",
                        chapter "Implementing the forward pass to get logits") */
  GPT_ESTATE = -3,   /* backward without a preceding forward with targets */
  GPT_EHIP = -4,     /* a HIP call failed; gpt_strerror adds its message */
  GPT_EUNSUPPORTED = -5 /* shape this build's kernels do not cover */
};

enum { GPT_FP32 = 0, GPT_BF16 = 1, GPT_FP16 = 2 };

/* Device flag bits reported by gpt_read_flags. */
enum {
  GPT_FLAG_BAD_TOKEN = 1,  /* an input id was outside [0, padded_vocab); its
                              embedding row was taken as zero */
  GPT_FLAG_BAD_TARGET = 2, /* a target was outside [-1, vocab_size); it was
                              treated as ignored (-1): left out of the count of
                              valid targets, zero loss and zero gradient */
  GPT_FLAG_HEAD_RANGE = 4  /* fused head + cross-entropy (GPT_OPT_FUSED_HEAD_CE):
                              a row's sum of exp(logit) left [1e-28, 1e28], the
                              range its 16-bit exp(logit) values carry exactly
                              (logits beyond about +-64); that step's loss and
                              gradients are not valid */
};

typedef struct {
  int32_t vocab_size;   /* real vocabulary V; logits columns >= V are masked */
  int32_t padded_vocab; /* Vp >= V: rows of wte */
  int32_t block_size;   /* maximum T: rows of wpe */
  int32_t n_layer;
  int32_t n_head;
  int32_t n_embd;       /* d; the MLP width is 4*d */
  int32_t mode;         /* GPT_FP32: fp32 everywhere; GPT_BF16: bf16 matrix
                           operands and stored activations with fp32
                           accumulation, fp32 residual stream, LayerNorm,
                           softmax, loss, master weights and optimizer state
                           ("Let's reproduce GPT-2 (124M)", chapter "Float16,
                           Gradient Scalers, BF16"); GPT_FP16: the same with
                           IEEE binary16 in place of bf16, trained with
                           dynamic loss scaling (gpt_forward_loss_scaled,
                           gpt_amp_step) */
  int32_t max_batch;    /* largest B the workspace is sized for */
} gpt_config;

typedef struct gpt_model gpt_model;

/* Sizes the caller must allocate: n_params fp32 elements for each of params,
 * grads, adam_m and adam_v, and workspace_bytes of device memory (256-byte
 * aligned) for activations, the 16-bit weight copy and scratch.
 * Returns GPT_EINVAL for an invalid config, GPT_EUNSUPPORTED for a valid one
 * these kernels do not cover (n_embd a multiple of 4 up to 2048 and head width
 * up to 128; the 16-bit modes also need n_embd % 64 == 0 and the padded vocabulary,
 * rounded up to 64, at most 53248).  Head width 64 takes the flash-attention
 * kernels; other widths a slower per-query kernel. */
int gpt_query_sizes(const gpt_config* cfg, int64_t* n_params, int64_t* workspace_bytes);

/* Bind caller-owned device buffers and create a handle.
 * params, grads, adam_m, adam_v: device fp32 [n_params] (params 16-byte
 * aligned); workspace: device memory of workspace_bytes.
 * init_params: device fp32 [n_params] in the canonical order, copied into
 * params; or NULL: params are drawn on the device from `seed` ("Let's
 * reproduce GPT-2 (124M)", chapter "Model Initialization"; "nanoGPT" Part V
 * Deep dive 1): every Linear weight and both embedding tables (pad rows
 * included) N(0, 0.02^2), attn.c_proj and mlp.c_proj weights
 * N(0, (0.02 / sqrt(2 n_layer))^2), biases 0, LayerNorm gains 1 and shifts
 * 0.  The normals come from Philox4x32-10 under the 64-bit seed through the
 * Box-Muller transform; element i's value depends only on i and the seed.
 * seed is unused when init_params is not NULL.
 * adam_m, adam_v and grads are zeroed.  In the 16-bit modes the 16-bit
 * copy of the weights and the transposed copies of the weight matrices (in
 * the workspace) are written here and, after that, by gpt_adamw_step and
 * gpt_amp_step: a caller that writes params itself must create a new handle
 * for the copies to follow.  The buffers must stay valid until gpt_destroy. */
int gpt_init(gpt_model** out, const gpt_config* cfg, float* params, float* grads,
             float* adam_m, float* adam_v, void* workspace, const float* init_params,
             uint64_t seed, void* stream);

/* Forward pass and, when targets != NULL, the loss and its gradient w.r.t.
 * the logits ("nanoGPT", Part IV Stage 4; loss of "Let's reproduce GPT-2
 * (124M)", chapter "Cross Entropy Loss").
 * idx, targets: device int32 [B*T], row-major (b, t).  A target of -1 is
 * ignored (ignore_index=-1); the loss is the mean over the others.  A target
 * outside [-1, V) is treated as ignored too and raises GPT_FLAG_BAD_TARGET.
 * loss_scale multiplies the gradient only (1/k under accumulation over k
 * micro-batches, "nanoGPT" Part IV Stage 4).
 * loss_out: device float, receives the unscaled mean loss (may be NULL).
 * logits_out: optional device buffer [B*T][Vp] (fp32 in GPT_FP32 mode, the
 * 16-bit format in GPT_BF16 and GPT_FP16 modes) receiving the logits before the loss is taken.
 * Errors: GPT_EINVAL (B < 1, B > max_batch, null idx), GPT_ESEQLEN. */
int gpt_forward_loss(gpt_model* h, const int32_t* idx, const int32_t* targets,
                     int32_t B, int32_t T, float loss_scale, float* loss_out,
                     void* logits_out, void* stream);

/* Evaluation ("nanoGPT", Part IV Stage 2, estimate_loss: the model in eval
 * mode and no gradient): the mean loss over the targets in [0, V) of one batch
 * into loss_out (device float), with no dropout and no gradient written.
 * gpt_estimate_loss averages such losses over evaluation batches.  A following
 * gpt_backward fails with GPT_ESTATE.  Errors as gpt_forward_loss; targets
 * and loss_out must not be NULL. */
int gpt_eval_loss(gpt_model* h, const int32_t* idx, const int32_t* targets, int32_t B,
                  int32_t T, float* loss_out, void* stream);

/* The pages' estimate_loss over one split ("nanoGPT", Part IV Stage 2): the
 * eval loss (as gpt_eval_loss) of each of n_batches batches, then the mean of
 * those losses (fp64 sum in a fixed order) into loss_out (device float).
 * idx, targets: device int32 [n_batches][B][T].  Errors as gpt_eval_loss;
 * GPT_EINVAL for n_batches outside [1, 1024]. */
int gpt_estimate_loss(gpt_model* h, const int32_t* idx, const int32_t* targets,
                      int32_t n_batches, int32_t B, int32_t T, float* loss_out, void* stream);

/* Backward pass of the last forward (which must have had targets).
 * zero_first != 0: grads = new gradient; else grads += new gradient
 * (accumulation until zero_grad, "nanoGPT" Deep dive 2). */
int gpt_backward(gpt_model* h, int32_t zero_first, void* stream);

/* Global-norm clipping and one AdamW update of params, adam_m, adam_v
 * ("andrej-karpathy-lets-reproduce-gpt-2", the optimization recipe: betas
 * (0.9, 0.95), eps 1e-8, clip 1.0, weight decay 0.1 on 2-D tensors only).
 *   norm = ||grads||_2 over all elements; coef = min(1, max_norm/(norm+1e-6))
 *   (max_norm <= 0: coef = 1); g = coef*grad;
 *   m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
 *   p = p (1 - lr wd [p is in a 2-D tensor]);
 *   p = p - lr (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps).
 * t: 1-based optimizer step.  norm_out: device float receiving the pre-clip
 * norm (may be NULL).  skip_nonfinite != 0: when the norm is not finite,
 * params, adam_m and adam_v are left untouched.  grads are not modified. */
int gpt_adamw_step(gpt_model* h, float lr, float beta1, float beta2, float eps,
                   float weight_decay, float max_norm, int32_t t,
                   int32_t skip_nonfinite, float* norm_out, void* stream);

/* Learning rate at optimizer iteration it ("nanoGPT", Part IV Stage 1,
 * get_lr; "Karpathy's Let's Reproduce GPT-2 in One Read", Section 3):
 * it < warmup: max_lr * (it + 1) / warmup (linear warmup);
 * warmup <= it <= decay_end: min_lr + (max_lr - min_lr) * (1 + cos(pi *
 * (it - warmup) / (decay_end - warmup))) / 2 (cosine decay);
 * it > decay_end: min_lr.  Host arithmetic in double, no device involved.
 * NaN for it < 0, warmup < 0 or decay_end <= warmup.  The pages' values:
 * max 6e-4, min 6e-5, warmup 715, decay_end 19073 (build-nanogpt) or warmup
 * 2000, decay_end 600000 (nanoGPT). */
double gpt_lr_at(int64_t it, double max_lr, double min_lr, int64_t warmup, int64_t decay_end);

/* ---------------------------------------------------------------------------
 * Dynamic loss scaling for float16 training ("nanoGPT", Part IV Stages 4-5,
 * Part V Deep dive 2 and Part VIII checks 6-7; "Let's reproduce GPT-2
 * (124M)", chapter "Float16, Gradient Scalers, BF16"): binary16 has a narrow
 * exponent range, so the loss is multiplied by a scale before the backward
 * pass, and the optimizer step unscales, clips, then steps or skips, and
 * adapts the scale.  The order of one iteration is
 *   gpt_forward_loss_scaled + gpt_backward (per micro-batch), gpt_amp_step.
 * Usable in every mode; needed in GPT_FP16.
 * ------------------------------------------------------------------------- */

/* Scaler state, in DEVICE memory, owned by the caller; the library reads and
 * updates it in stream order, so no host synchronisation is needed per step.
 * Initialise it once (e.g. {65536.f, 0, 0, 0}). */
typedef struct {
  float scale;            /* S: multiplies the loss before the backward pass */
  int32_t growth_tracker; /* clean steps since S last changed */
  int32_t steps;          /* AdamW updates applied; skipped steps are not
                             counted (the bias corrections use steps + 1) */
  int32_t found_inf;      /* 1 if the last gpt_amp_step skipped its update */
} gpt_loss_scaler;

/* gpt_forward_loss, with the gradient w.r.t. the logits further multiplied by
 * scaler->scale (read on the device when the kernel runs).  loss_out is still
 * the unscaled mean loss.  Errors: as gpt_forward_loss, GPT_EINVAL for a null
 * scaler. */
int gpt_forward_loss_scaled(gpt_model* h, const int32_t* idx, const int32_t* targets,
                            int32_t B, int32_t T, float loss_scale,
                            const gpt_loss_scaler* scaler, float* loss_out,
                            void* logits_out, void* stream);

/* The optimizer step of a loss-scaled iteration, in the pages' order, with
 * S = scaler->scale:
 *   unscale:  the update uses grads / S (grads themselves are not modified);
 *   clip:     norm = ||grads / S||_2, coef = min(1, max_norm/(norm+1e-6))
 *             (max_norm <= 0: coef = 1);
 *   step:     AdamW exactly as gpt_adamw_step at t = scaler->steps + 1 on
 *             g = coef grads / S, unless norm is not finite (an inf or NaN
 *             gradient element): then params, adam_m, adam_v stay untouched;
 *   update:   not finite: S *= backoff_factor, growth_tracker = 0,
 *             found_inf = 1; finite: steps += 1, found_inf = 0, and
 *             growth_tracker += 1, which on reaching growth_interval becomes
 *             0 with S *= growth_factor (kept only if finite).
 * Readings (the pages give no values): the library defaults 2.0, 0.5, 2000.
 * norm_out: device float receiving norm (may be NULL).  Errors: GPT_EINVAL
 * (null handle or scaler, growth_interval < 1, growth_factor < 1,
 * backoff_factor outside (0, 1]). */
int gpt_amp_step(gpt_model* h, float lr, float beta1, float beta2, float eps,
                 float weight_decay, float max_norm, gpt_loss_scaler* scaler,
                 float growth_factor, float backoff_factor, int32_t growth_interval,
                 float* norm_out, void* stream);

/* ---------------------------------------------------------------------------
 * Dropout
 * ------------------------------------------------------------------------- */

/* Dropout of a training forward ("nanoGPT", Part IV Stage 4 and Part V Deep
 * dive 1; "Build GPT from scratch", "The model in forty lines"; 0.2 for the
 * character-level model, "nanoGPT" Part VIII check 15): applied to the
 * embedding sum, to the attention probabilities (after the softmax, before
 * the product with v) and to the MLP output; a kept value is multiplied by
 * 1/(1-p).  Reading: no dropout after the attention's output projection
 * (neither page puts one there).  Masks come from Philox4x32-10 (Salmon et
 * al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) with key = seed
 * (low word first): element (row, col) of a site's matrix is kept when word
 * col % 4 of philox(counter = {col / 4, row, site * 2^24 + bh, step}) is
 * >= ceil(p * 2^32).  Sites: 0 the embedding sum (rows b*T + t, columns
 * features), 1 + 2l the attention probabilities of layer l (rows queries,
 * columns keys, bh = b * n_head + h), 2 + 2l the MLP output of layer l (as
 * the embedding); bh = 0 except for attention. */
typedef struct {
  float p;       /* probability of dropping an element, in [0, 1); 0: none */
  uint32_t step; /* counter word telling forward calls apart */
  uint64_t seed; /* Philox key */
} gpt_dropout;

/* gpt_forward_loss with optional dynamic loss scaling (scaler: as
 * gpt_forward_loss_scaled; NULL: none) and optional dropout (NULL or p = 0:
 * none).  gpt_backward uses the same masks, regenerated from the counter.
 * Errors: as gpt_forward_loss; GPT_EINVAL for p outside [0, 1);
 * GPT_EUNSUPPORTED for dropout with more than 127 layers. */
int gpt_forward_loss_ex(gpt_model* h, const int32_t* idx, const int32_t* targets,
                        int32_t B, int32_t T, float loss_scale,
                        const gpt_loss_scaler* scaler, const gpt_dropout* dropout,
                        float* loss_out, void* logits_out, void* stream);

/* ---------------------------------------------------------------------------
 * Sampling from the model ("nanoGPT", Part IV, one generation: sample.py +
 * model.py, generate), with a cache of keys and values ("Build GPT from
 * scratch", exercise "Add a KV cache") so that a step feeds one new token per
 * sequence.  Learned positions make a cache valid only while a sequence fits
 * in block_size; past it the caller runs gpt_prefill on the last block_size
 * tokens (the pages' cropping).  These calls overwrite the activations of the
 * last forward, so gpt_backward afterwards fails with GPT_ESTATE.
 * ------------------------------------------------------------------------- */

/* Bytes of a cache for B sequences of up to max_len positions:
 * kv[layer][k|v][b][head][t][head_width] in the mode's activation type
 * (bf16 in GPT_BF16 mode, binary16 in GPT_FP16 mode, fp32 in GPT_FP32 mode),
 * followed by 64 x head_width elements of slack that a decode step may read
 * (whole chunks of 64 positions) but never uses.  -1 for an invalid config
 * or size.  The caller allocates it on the device and owns it. */
int64_t gpt_kv_cache_bytes(const gpt_config* cfg, int32_t B, int32_t max_len);

/* Forward over prompts idx (device int32 [B*T0], row-major (b, t)), storing
 * every layer's keys and values of positions [0, T0) in kv (sized for exactly
 * B sequences and max_len positions, 1 <= T0 <= max_len <= block_size), and
 * the logits of each sequence's last position in logits_out (device fp32
 * [B][padded_vocab]).  Errors: GPT_EINVAL (null pointer, B outside
 * [1, max_batch]), GPT_ESEQLEN. */
int gpt_prefill(gpt_model* h, const int32_t* idx, int32_t B, int32_t T0, void* kv,
                int32_t max_len, float* logits_out, void* stream);

/* One new token per sequence, tok (device int32 [B]), all at position pos
 * (0 <= pos < max_len): its keys and values go to cache position pos,
 * attention covers positions [0, pos], and logits_out (device fp32
 * [B][padded_vocab]) receives the next-token logits.  kv, B and max_len as in
 * the gpt_prefill that filled positions [0, pos).  Errors as gpt_prefill. */
int gpt_decode_step(gpt_model* h, const int32_t* tok, int32_t B, int32_t pos, void* kv,
                    int32_t max_len, float* logits_out, void* stream);

/* One draw per row of logits (device fp32 [B][ldv], ids [0, V) used):
 * z = logits / temperature; when 0 < top_k < V, ids with z below the k-th
 * largest z are removed (ids equal to it stay); p = softmax(z); the token is
 * the first id whose cumulative p exceeds u[b] (device fp32 [B], uniforms in
 * [0, 1) that the caller draws).  tok_out: device int32 [B].  A row with no
 * distribution to draw from (a NaN or +inf logit, or u[b] negative or NaN)
 * gets -1, which a following gpt_decode_step reports as GPT_FLAG_BAD_TOKEN;
 * u[b] >= 1 takes the last kept id.
 * Errors: GPT_EINVAL (null pointer, B < 1, ldv < V, temperature <= 0),
 * GPT_EUNSUPPORTED (V above 57344). */
int gpt_sample(const float* logits, int32_t B, int32_t V, int32_t ldv, float temperature,
               int32_t top_k, const float* u, int32_t* tok_out, void* stream);

/* Options of a handle (gpt_set_option).
 * GPT_OPT_FUSED_HEAD_CE (value 0 or 1, default 1): fuse the cross-entropy into the tied
 * LM head, so that no pass over the logits follows the head's product
 * ("Let's reproduce GPT-2 (124M)", chapters "Cross Entropy Loss" and "Flash
 * Attention": do not make extra passes over a large tensor).  The head's
 * product stores p = exp(z) in place of the logits z and, in its epilogue,
 * each row's sums of p; one small pass per row takes S = sum of p, the loss
 * log S - z_y, the factor r = loss_scale / (n_valid S), r times the final
 * LayerNorm's output, and writes p_y - S at the target's column.  The logit
 * gradient is then r times a stored row: the head's weight-gradient product
 * takes the scaled LayerNorm output as its other operand, and its
 * input-gradient product multiplies its rows by r in the epilogue.
 * Applies to gpt_forward_loss with targets and without logits_out in
 * GPT_BF16 mode (other modes and calls keep the separate pass).  It carries
 * logits within about +-64 (GPT_FLAG_HEAD_RANGE otherwise).
 * GPT_OPT_TIME_WEIGHT_GRADIENTS (value 0 or 1, default 0): gpt_backward
 * records a HIP event on its stream before and after each weight-gradient
 * launch ("Let's reproduce GPT-2 (124M)", "Speed Stack": time what the step
 * spends where), for gpt_read_timing.  Only the time between the events is
 * measured; the results of the step do not change.  The library keeps the
 * events until gpt_read_timing takes them (two per launch, 98 per GPT-2
 * backward), so a caller that turns the option on reads them now and then.
 * A launch that fails leaves its opening event unmatched; the next launch's
 * pair replaces it.
 * Errors: GPT_EINVAL (null handle, unknown option or value). */
enum { GPT_OPT_FUSED_HEAD_CE = 1, GPT_OPT_TIME_WEIGHT_GRADIENTS = 2 };
int gpt_set_option(gpt_model* h, int32_t option, int32_t value);
/* The current value of an option into *value.  Errors: GPT_EINVAL. */
int gpt_get_option(gpt_model* h, int32_t option, int32_t* value);

/* With GPT_OPT_TIME_WEIGHT_GRADIENTS on: waits for the events recorded since
 * the last call, puts the summed time of the weight-gradient launches they
 * bracket in *ms (milliseconds) and their number in *launches (the final
 * split-K reduction of a backward is counted with the last launch), and
 * starts over.  Errors: GPT_EINVAL (null pointer), GPT_EHIP. */
int gpt_read_timing(gpt_model* h, double* ms, int64_t* launches);

/* Synchronise `stream`, return the device flags (GPT_FLAG_*) raised since the
 * last call in *flags, and clear them. */
int gpt_read_flags(gpt_model* h, int32_t* flags, void* stream);

void gpt_destroy(gpt_model* h);

const char* gpt_strerror(int code);

/* ---------------------------------------------------------------------------
 * Single-operation entry points.  They run one kernel of the step on caller
 * buffers so each can be checked and timed on its own.  All pointers are
 * device pointers; matrices are row-major; `act` buffers are fp32 when
 * dtype == GPT_FP32, bf16 when dtype == GPT_BF16 and binary16 when
 * dtype == GPT_FP16 (both 16-bit formats as raw uint16 storage).  Another
 * dtype value returns GPT_EINVAL.
 * ------------------------------------------------------------------------- */

/* C = A B^T over K, plus optional bias[n] ("nanoGPT" Deep dive 1: the Linear
 * layers).  A: act [M][K], B: act [N][K], bias: fp32 [N] or NULL,
 * C: act [M][N] (fp32 when out_f32 != 0).  16-bit dtypes need K % 8 == 0. */
int gpt_op_linear(int32_t dtype, const void* A, const void* B, const float* bias,
                  void* C, int32_t out_f32, int32_t M, int32_t N, int32_t K, void* stream);

/* The MLP expansion with its activation ("nanoGPT" Deep dive 1, the MLP:
 * expand, tanh-GELU; "Let's Reproduce GPT-2 in One Read", the GELU check):
 * u = A W^T + bias over K; dgelu[m][n] = gelu'(u), g[m][n] = gelu(u), with
 * gelu(u) = 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))).  A: act [M][K],
 * W: act [N][K], bias: fp32 [N] or NULL, dgelu and g: act [M][N].  The step
 * keeps gelu'(u) instead of u for its backward.  16-bit dtypes need
 * K % 8 == 0. */
int gpt_op_linear_gelu(int32_t dtype, const void* A, const void* W, const float* bias,
                       void* dgelu, void* g, int32_t M, int32_t N, int32_t K, void* stream);

/* The MLP projection's input gradient through the activation ("nanoGPT"
 * Part IV Stage 4, the backward of Deep dive 1's MLP):
 * du[m][n] = (sum_k dY[m][k] Wt[n][k]) * dgelu[m][n], and when dbias is not
 * NULL, dbias[n] (+)= sum_m du[m][n] (the expansion's bias gradient; added to
 * dbias when accumulate_bias != 0), summed from the fp32 values before du is
 * rounded.  dY: act [M][K], Wt: act [N][K] (the projection's weight
 * transposed), dgelu: act [M][N] as gpt_op_linear_gelu writes it, du: act
 * [M][N], dbias: fp32 [N].  workspace: device fp32 scratch of workspace_bytes
 * >= ceil(M/128) * N * 4 (column-sum partials), needed only with dbias;
 * GPT_EINVAL otherwise.  16-bit dtypes need K % 8 == 0. */
int gpt_op_linear_gelu_bwd(int32_t dtype, const void* dY, const void* Wt, const void* dgelu,
                           void* du, float* dbias, int32_t accumulate_bias, int32_t M, int32_t N,
                           int32_t K, float* workspace, int64_t workspace_bytes, void* stream);

/* gpt_op_linear_gelu_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the column-sum scratch taken
 * from a 4 MiB device array the library holds per device until the process
 * ends, so the call allocates nothing and needs no workspace.  The array of
 * the calling thread's current device is used, and `stream` must belong to
 * that device (GPT_EINVAL otherwise, nothing enqueued).  With dbias set,
 * ceil(M/128) * N * 4 must not exceed 4 MiB (GPT_EINVAL, nothing enqueued).  Calls that overlap on one device share the array and
 * race: serialise them (one stream, or events).  Nothing in the array needs
 * to start at zero; it keeps the last call's partials. */
int gpt_op_linear_gelu_bwd_noalloc(int32_t dtype, const void* dY, const void* Wt,
                                   const void* dgelu, void* du, float* dbias,
                                   int32_t accumulate_bias, int32_t M, int32_t N, int32_t K,
                                   void* stream);

/* dW (+)= dY^T X: dY act [M][N], X act [M][K], dW fp32 [N][K];
 * accumulate != 0 adds to dW.  The weight gradient of a Linear layer.
 * workspace: optional device fp32 scratch of workspace_bytes (NULL: none);
 * with enough of it a long reduction over M is split across workgroups and
 * the partial sums are added in a fixed order. */
int gpt_op_linear_dw(int32_t dtype, const void* dY, const void* X, float* dW,
                     int32_t accumulate, int32_t M, int32_t N, int32_t K,
                     float* workspace, int64_t workspace_bytes, void* stream);

/* count weight gradients in the order given, as the training backward
 * launches its own: product i is gpt_op_linear_dw(dtype, dY[i], X[i], dW[i],
 * accumulate[i], M[i], N[i], K[i], ...), with the same results bit for bit.
 * dY, X, dW: host arrays of device pointers; accumulate, M, N, K: host arrays
 * of count values.  A product whose reduction over M is split leaves its
 * partial sums to the next product's launch, which adds them (in the same
 * fixed order) with workgroups beside its own tiles; the last product's are
 * added after the sequence.  workspace: optional device fp32 scratch
 * (NULL: no split), used as two halves.  The dW of consecutive products must
 * not overlap unless they are the same pointer (the earlier reduction then
 * runs first).  On error the dW are unspecified. */
int gpt_op_linear_dw_seq(int32_t dtype, int32_t count, const void* const* dY,
                         const void* const* X, float* const* dW, const int32_t* accumulate,
                         const int32_t* M, const int32_t* N, const int32_t* K,
                         float* workspace, int64_t workspace_bytes, void* stream);

/* dX = dY W: dY act [M][N], W act [N][K], dX fp32 [M][K].  The input
 * gradient of a Linear layer. */
int gpt_op_linear_dx(int32_t dtype, const void* dY, const void* W, float* dX,
                     int32_t M, int32_t N, int32_t K, void* stream);

/* Causal attention forward over qkv act [B*T][3*C] (q | k | v column blocks,
 * head h at columns h*hs) -> out act [B*T][C], lse fp32 [B][H][T]
 * (natural-log row logsumexp of the scaled scores).  "nanoGPT" Deep dive 1,
 * the manual path: softmax(q k^T / sqrt(hs) with -inf above the diagonal) v. */
int gpt_op_attention_fwd(int32_t dtype, const void* qkv, void* out, float* lse,
                         int32_t B, int32_t T, int32_t H, int32_t C, void* stream);

/* Its backward: dout act [B*T][C] -> dqkv act [B*T][3*C] (every element
 * written).  D: fp32 scratch [2][B][H][T]; D[0] receives rowsum(dout * out)
 * (negated in 16-bit modes at head width 64), D[1] the row logsumexp times
 * log2(e). */
int gpt_op_attention_bwd(int32_t dtype, const void* qkv, const void* out,
                         const float* lse, const void* dout, void* dqkv, float* D,
                         int32_t B, int32_t T, int32_t H, int32_t C, void* stream);

/* y = LayerNorm(x) w + b per row (biased variance, eps 1e-5):
 * x fp32 [M][C] -> y act [M][C], mean and rstd fp32 [M]. */
int gpt_op_layernorm_fwd(int32_t dtype, const float* x, const float* w, const float* b,
                         void* y, float* mean, float* rstd, int32_t M, int32_t C,
                         void* stream);

/* y = x times the dropout multipliers of one site's matrix (see gpt_dropout):
 * x, y device fp32 [rows][cols] (cols % 4 == 0; y may equal x); site_word =
 * site * 2^24 + bh.  p = 0 copies.  The masks of every site can be checked
 * element by element through this call. */
int gpt_op_dropout(const float* x, float* y, int64_t rows, int32_t cols, float p,
                   uint64_t seed, uint32_t step, uint32_t site_word, void* stream);

/* Masked softmax cross-entropy, in place: logits act [N][ldv] -> dlogits
 * (loss_scale * (softmax - onehot) / n_valid over columns < V, zero for
 * columns in [V, ldv)); loss: device fp32 scalar = mean over the targets in
 * [0, V) (any other target is ignored: zero loss and gradient in its row).
 * row_loss: device fp32 [N] receiving each row's loss (0 if ignored);
 * n_valid: device int32 receiving the count of targets in [0, V).
 * 16-bit dtypes need ldv % 8 == 0 and ldv <= 53248. */
int gpt_op_cross_entropy(int32_t dtype, void* logits, const int32_t* targets,
                         float* loss, float* row_loss, int32_t* n_valid,
                         float loss_scale, int32_t N, int32_t V, int32_t ldv,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT_HIP_H */
