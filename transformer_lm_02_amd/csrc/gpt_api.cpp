// C ABI of libgpt_hip.so: host orchestration of one GPT-2 training step.
//
// The step is the training iteration of "nanoGPT" (stanleyjacob.dev), Part IV
// Stages 4-5: forward (embeddings, n_layer pre-norm blocks, ln_f, tied LM
// head, cross-entropy), backward (accumulating into grads until the caller
// asks for a fresh start), then global-norm clipping and AdamW.  Every call
// only enqueues kernels on the caller's stream; all device memory belongs to
// the caller (params, grads, Adam moments and one workspace).
#include <math.h>

#include <algorithm>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "gpt_hip.h"
#include "api_impl.h"
#include "kernels.h"

namespace HALF_NS {
namespace {


int fail(int code, const char* what) {
  gpt_error_text() = what;
  return code;
}
int map_rc(int rc) {
  if (rc == 0) return GPT_OK;
  if (rc == -5) return GPT_EUNSUPPORTED;
  hipError_t e = hipGetLastError();
  gpt_error_text() = hipGetErrorString(e);
  return GPT_EHIP;
}
#define CK(x)                       \
  do {                              \
    int rc_ = (x);                  \
    if (rc_) return map_rc(rc_);    \
  } while (0)
#define CKH(x)                                   \
  do {                                           \
    hipError_t e_ = (x);                         \
    if (e_ != hipSuccess) {                      \
      gpt_error_text() = hipGetErrorString(e_);             \
      return GPT_EHIP;                           \
    }                                            \
  } while (0)

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// element offsets of every tensor in the canonical flat parameter vector
struct LayerOff {
  int64_t ln1w, ln1b, attnw, attnb, aprojw, aprojb, ln2w, ln2b, fcw, fcb, mprojw, mprojb;
};
// initial value of a tensor drawn from a seed: N(0, 0.02^2), N(0, (0.02 /
// sqrt(2 L))^2) for the projections into the residual stream, or a constant
enum InitKind { INIT_STD = 0, INIT_RESID = 1, INIT_ONE = 2, INIT_ZERO = 3 };
struct ParamOff {
  int64_t wte, wpe, lnfw, lnfb, total;
  std::vector<LayerOff> layer;
  std::vector<std::pair<int64_t, int64_t>> tensors;  // (offset, count) in order
  std::vector<int> is2d;
  std::vector<int> init;  // InitKind per tensor
};

ParamOff param_offsets(const gpt_config& c) {
  ParamOff p;
  int64_t off = 0;
  const int64_t d = c.n_embd;
  auto take = [&](int64_t n, bool two_d, int init) {
    int64_t o = off;
    p.tensors.push_back({o, n});
    p.is2d.push_back(two_d);
    p.init.push_back(init);
    off += n;
    return o;
  };
  p.wte = take((int64_t)c.padded_vocab * d, true, INIT_STD);
  p.wpe = take((int64_t)c.block_size * d, true, INIT_STD);
  for (int l = 0; l < c.n_layer; ++l) {
    LayerOff L;
    L.ln1w = take(d, false, INIT_ONE);
    L.ln1b = take(d, false, INIT_ZERO);
    L.attnw = take(3 * d * d, true, INIT_STD);
    L.attnb = take(3 * d, false, INIT_ZERO);
    L.aprojw = take(d * d, true, INIT_RESID);
    L.aprojb = take(d, false, INIT_ZERO);
    L.ln2w = take(d, false, INIT_ONE);
    L.ln2b = take(d, false, INIT_ZERO);
    L.fcw = take(4 * d * d, true, INIT_STD);
    L.fcb = take(4 * d, false, INIT_ZERO);
    L.mprojw = take(4 * d * d, true, INIT_RESID);
    L.mprojb = take(d, false, INIT_ZERO);
    p.layer.push_back(L);
  }
  p.lnfw = take(d, false, INIT_ONE);
  p.lnfb = take(d, false, INIT_ZERO);
  p.total = off;
  return p;
}

// byte offsets of every buffer in the workspace
struct WsLayer {
  int64_t attnT, aprojT, fcT, mprojT;  // element offsets in the transposed copy
  size_t x_in, ln1_mean, ln1_rstd, ln1, qkv, att, lse, x_mid, ln2_mean, ln2_rstd, ln2, dgelu, g;
  size_t dmask = 0;  // the flash forward's dropout bits for its backward (16-bit, head width 64)
};
struct WsOff {
  size_t shadow = 0;
  std::vector<WsLayer> layer;
  size_t x_final, lnf_mean, lnf_rstd, lnf, logits, row_loss, nvalid, flags, scal;
  // fused head + cross-entropy (16-bit modes): row sums of exp(z) per 96
  // columns, the target logit, the gradient factors r and sc, and r * lnf
  size_t head_part = 0, head_zy = 0, head_r = 0, head_h2 = 0;
  int head_npart = 0;
  size_t dres, dres_act, dln, dbig, dO, Dbuf, ln_part, cs_part, norm_part, chunks, splitk;
  int64_t splitk_bytes;
  int64_t ln_part_elems, cs_part_elems;  // one slice of each (several slices kept)
  size_t init_tab;  // InitSeg per chunk (initialisation from a seed)
  size_t eval_losses = 0;  // per-batch losses of gpt_estimate_loss
  size_t total;
  int nchunks;
  int64_t vi;  // logits row pitch: padded_vocab rounded up to 64
  size_t wT = 0, tjobs = 0;  // transposed 16-bit weights; their job table
  int64_t wteT = 0, wT_elems = 0;
  int njobs = 0, ttiles = 0;
};

constexpr int64_t kChunk = 8192;
constexpr int kEvalBatches = 1024;  // batches one gpt_estimate_loss call averages

WsOff ws_offsets(const gpt_config& c, const ParamOff& p) {
  WsOff w;
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    size_t o = off;
    off = (size_t)round_up(off + (size_t)bytes, 256);
    return o;
  };
  const bool bf = c.mode != GPT_FP32;
  const int64_t es = bf ? 2 : 4;
  const int64_t M = (int64_t)c.max_batch * c.block_size, d = c.n_embd, H = c.n_head;
  w.vi = round_up(c.padded_vocab, 64);
  if (bf) w.shadow = take(p.total * 2);
  // transposed copies (16-bit mode): wte^T [d][vi] (columns >= Vp zero), then
  // per layer attn^T [d][3d], aproj^T [d][d], fc^T [d][4d], mproj^T [4d][d]
  int64_t te = 0;
  w.wteT = te;
  te += d * w.vi;
  std::vector<int64_t> lt;
  for (int l = 0; l < c.n_layer; ++l) {
    lt.push_back(te);
    te += 12 * d * d;
  }
  w.wT_elems = bf ? te : 0;
  if (bf) {
    w.wT = take(te * 2);
    w.njobs = 1 + 4 * c.n_layer;
    w.tjobs = take((int64_t)w.njobs * (int64_t)sizeof(TransposeJob));
  }
  for (int l = 0; l < c.n_layer; ++l) {
    WsLayer L;
    L.attnT = lt[l];
    L.aprojT = L.attnT + 3 * d * d;
    L.fcT = L.aprojT + d * d;
    L.mprojT = L.fcT + 4 * d * d;
    L.x_in = take(M * d * 4);
    L.ln1_mean = take(M * 4);
    L.ln1_rstd = take(M * 4);
    L.ln1 = take(M * d * es);
    L.qkv = take(M * 3 * d * es);
    L.att = take(M * d * es);
    L.lse = take(M * H * 4);
    L.x_mid = take(M * d * 4);
    L.ln2_mean = take(M * 4);
    L.ln2_rstd = take(M * 4);
    L.ln2 = take(M * d * es);
    L.dgelu = take(M * 4 * d * es);  // gelu'(u), kept for the backward
    L.g = take(M * 4 * d * es);
    // one bit per (query, key) of every head, as 32-bit words per 64-key
    // block and half: [b*H + h][key block][half][query]
    if (bf && d / H == 64) L.dmask = take(M * H * round_up(c.block_size, 64) / 64 * 2 * 4);
    w.layer.push_back(L);
  }
  w.x_final = take(M * d * 4);
  w.lnf_mean = take(M * 4);
  w.lnf_rstd = take(M * 4);
  w.lnf = take(M * d * es);
  w.logits = take(M * w.vi * es);
  w.row_loss = take(M * 4);
  if (bf) {
    w.head_npart = (int)cdiv(c.padded_vocab, 96);
    w.head_part = take(M * w.head_npart * 4);
    w.head_zy = take(M * 4);
    w.head_r = take(M * 4);
    w.head_h2 = take(M * d * 2);
  }
  w.nvalid = take(4);
  w.flags = take(4);
  w.scal = take(16);
  w.dres = take(M * d * 4);
  w.dres_act = take(M * d * es);
  w.dln = take(M * d * 4);
  w.dbig = take(M * 4 * d * es);
  w.dO = take(M * d * es);
  w.Dbuf = take(2 * M * H * 4);
  // Column-sum partials of the backward, one slice per producer so that all
  // of them are finished by one launch at its end: a LayerNorm slice per
  // LayerNorm (2 per layer + the final one); a column-sum slice (at most one
  // row per 128 tokens, GEMM row tiles or attention blocks, or per
  // colsum_part_rows block) for the MLP expansion bias and the q|k|v bias of
  // every layer.
  w.ln_part_elems = (int64_t)layernorm_bwd_part_rows((int)M) * 3 * d;
  w.ln_part = take((2 * c.n_layer + 1) * w.ln_part_elems * 4);
  w.cs_part_elems = std::max<int64_t>(cdiv(M, 128), colsum_part_rows((int)M)) * 4 * d;
  w.cs_part = take(2 * c.n_layer * w.cs_part_elems * 4);
  w.norm_part = take((int64_t)adamw_norm_blocks() * 8);
  // two halves, one per weight gradient in flight (SplitKChain)
  w.splitk_bytes = bf ? 2 * gemm_splitk_bytes(4 * d, d) : 0;
  w.splitk = take(w.splitk_bytes);
  int64_t nch = 0;
  for (auto& t : p.tensors) nch += (t.second + kChunk - 1) / kChunk;
  w.nchunks = (int)nch;
  w.chunks = take(nch * (int64_t)sizeof(AdamChunk));
  w.init_tab = take(nch * (int64_t)sizeof(InitSeg));
  w.eval_losses = take(kEvalBatches * 4);
  w.total = off;
  return w;
}

int validate(const gpt_config* c) {
  if (!c) return fail(GPT_EINVAL, "null config");
  if (c->vocab_size < 1 || c->padded_vocab < c->vocab_size || c->block_size < 1 ||
      c->n_layer < 1 || c->n_head < 1 || c->n_embd < 1 || c->max_batch < 1 ||
      (c->mode != GPT_FP32 && c->mode != GPT_BF16 && c->mode != GPT_FP16) || c->n_embd % c->n_head)
    return fail(GPT_EINVAL, "invalid gpt_config");
  const int hs = c->n_embd / c->n_head;
  if (c->n_embd % 4 || c->n_embd > 2048 || hs > 128)
    return fail(GPT_EUNSUPPORTED, "n_embd must be a multiple of 4, at most 2048; head width <= 128");
  if (c->mode != GPT_FP32) {
    if (c->n_embd % 64) return fail(GPT_EUNSUPPORTED, "h16 mode needs n_embd % 64 == 0");
    if (round_up(c->padded_vocab, 64) > 53248)
      return fail(GPT_EUNSUPPORTED, "h16 cross-entropy covers rows up to 53248 columns");
  }
  if ((int64_t)c->max_batch * c->block_size > (1 << 26))
    return fail(GPT_EUNSUPPORTED, "max_batch * block_size too large");
  return GPT_OK;
}

}  // namespace

struct Model {
  gpt_config cfg;
  ParamOff po;
  WsOff wo;
  float *params, *grads, *m, *v;
  char* ws;
  std::vector<AdamChunk> chunks;
  std::vector<InitSeg> init_segs;
  std::vector<TransposeJob> tjobs;
  bool have_fwd = false, have_targets = false;
  int B = 0, T = 0;
  const int32_t* idx = nullptr;
  // GPT_OPT_FUSED_HEAD_CE (on by default: measured 0.38 ms a step faster at
  // GPT-2 124M, B=16, T=1024), and whether the last forward took that path
  bool fused_ce = true, last_fused = false;
  // the fused head + cross-entropy applies: bfloat16 mode (exp(z) needs its
  // exponent range) and a padded vocabulary the pipelined GEMM covers
  bool fused_ok() const {
    return fused_ce && cfg.mode == GPT_BF16 && cfg.padded_vocab % 8 == 0 && cfg.n_embd % 8 == 0;
  }
  Drop drop;  // dropout of the last forward (site word 0); thresh 0: none
  // GPT_OPT_TIME_WEIGHT_GRADIENTS: gpt_backward records an event before and
  // after each weight-gradient launch, taking tev in order; gpt_read_timing
  // sums the intervals and starts the list over
  bool time_dw = false;
  std::vector<hipEvent_t> tev;
  size_t tev_used = 0;
  // begin: the event before a launch, which always takes an even index (a
  // begin left unmatched by a failed launch is dropped), so that the pairs
  // gpt_read_timing sums stay aligned; the count grows only once the event
  // is recorded
  int mark(hipStream_t s, bool begin) {
    if (begin && (tev_used & 1)) --tev_used;
    if (tev_used == tev.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return -4;
      tev.push_back(e);
    }
    if (hipEventRecord(tev[tev_used], s) != hipSuccess) return -4;
    ++tev_used;
    return 0;
  }
  ~Model() {
    for (hipEvent_t e : tev) (void)hipEventDestroy(e);
  }

  bool h16() const { return cfg.mode != GPT_FP32; }
  int64_t es() const { return h16() ? 2 : 4; }
  template <typename P = void>
  P* at(size_t off) const { return (P*)(ws + off); }
  float* P(int64_t off) const { return params + off; }
  float* G(int64_t off) const { return grads + off; }
  // matrix operand copy of a weight: 16-bit copy in 16-bit mode, fp32 params otherwise
  const void* W(int64_t off) const {
    return h16() ? (const void*)(at<h16_t>(wo.shadow) + off) : (const void*)(params + off);
  }
  const h16_t* WT(int64_t off) const { return at<h16_t>(wo.wT) + off; }
  // AdamW's tiles: the weight matrices with transposed copies (16-bit modes)
  TileJobs tiles() const {
    TileJobs t;
    if (!h16()) return t;
    t.dstT = at<h16_t>(wo.wT);
    t.jobs = at<TransposeJob>(wo.tjobs);
    t.njobs = wo.njobs;
    t.ntiles = wo.ttiles;
    return t;
  }
  int refresh_transposes(hipStream_t s) const {
    if (!h16()) return 0;
    return transpose_h16_launch(at<h16_t>(wo.shadow), at<h16_t>(wo.wT),
                                 at<TransposeJob>(wo.tjobs), wo.njobs, wo.ttiles, s);
  }
};


int gpt_query_sizes(const gpt_config* cfg, int64_t* n_params, int64_t* workspace_bytes) {
  int rc = validate(cfg);
  if (rc) return rc;
  ParamOff p = param_offsets(*cfg);
  WsOff w = ws_offsets(*cfg, p);
  if (n_params) *n_params = p.total;
  if (workspace_bytes) *workspace_bytes = (int64_t)w.total;
  return GPT_OK;
}

int gpt_init(Model** out, const gpt_config* cfg, float* params, float* grads, float* adam_m,
             float* adam_v, void* workspace, const float* init_params, uint64_t seed,
             void* stream) {
  if (!out) return fail(GPT_EINVAL, "null output handle");
  *out = nullptr;
  int rc = validate(cfg);
  if (rc) return rc;
  if (!params || !grads || !adam_m || !adam_v || !workspace)
    return fail(GPT_EINVAL, "null device buffer");
  if ((uintptr_t)workspace & 255) return fail(GPT_EINVAL, "workspace must be 256-byte aligned");
  if ((uintptr_t)params & 15) return fail(GPT_EINVAL, "params must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  Model* h = new Model;
  h->cfg = *cfg;
  h->po = param_offsets(*cfg);
  h->wo = ws_offsets(*cfg, h->po);
  h->params = params;
  h->grads = grads;
  h->m = adam_m;
  h->v = adam_v;
  h->ws = (char*)workspace;
  if (h->h16()) {
    const int64_t d = cfg->n_embd;
    int tiles = 0;
    auto job = [&](int64_t src, int64_t dst, int64_t rows, int64_t cols, int64_t ld) {
      h->tjobs.push_back({src, dst, (int32_t)rows, (int32_t)cols, (int32_t)ld, tiles});
      tiles += (int)(cdiv(rows, 64) * cdiv(cols, 64));
    };
    job(h->po.wte, h->wo.wteT, cfg->padded_vocab, d, h->wo.vi);
    for (int l = 0; l < cfg->n_layer; ++l) {
      const LayerOff& P = h->po.layer[l];
      const WsLayer& L = h->wo.layer[l];
      job(P.attnw, L.attnT, 3 * d, d, 3 * d);
      job(P.aprojw, L.aprojT, d, d, d);
      job(P.fcw, L.fcT, 4 * d, d, 4 * d);
      job(P.mprojw, L.mprojT, d, 4 * d, d);
    }
    h->wo.ttiles = tiles;
  }
  const float res_std = (float)(0.02 / sqrt(2.0 * cfg->n_layer));
  for (size_t i = 0; i < h->po.tensors.size(); ++i) {
    const int64_t o = h->po.tensors[i].first, n = h->po.tensors[i].second;
    const int k = h->po.init[i];
    const float sd = k == INIT_STD ? 0.02f : k == INIT_RESID ? res_std : 0.f;
    const float val = k == INIT_ONE ? 1.f : 0.f;
    // a matrix with a transposed copy is updated by AdamW tiles, not chunks
    bool tiled = false;
    for (const TransposeJob& j : h->tjobs) tiled = tiled || j.src == o;
    if (tiled && !h->po.is2d[i]) {
      delete h;
      return fail(GPT_EINVAL, "internal: a transposed weight is not 2-D");
    }
    for (int64_t c = 0; c < n; c += kChunk) {
      const int32_t cnt = (int32_t)std::min<int64_t>(kChunk, n - c);
      if (!tiled) h->chunks.push_back({o + c, cnt, h->po.is2d[i]});
      h->init_segs.push_back({o + c, cnt, 0, sd, val});
    }
  }
  const int64_t nb = h->po.total * 4;
  hipError_t e = hipSuccess;
  if (init_params && init_params != params)
    e = hipMemcpyAsync(params, init_params, nb, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemsetAsync(adam_m, 0, nb, s);
  if (e == hipSuccess) e = hipMemsetAsync(adam_v, 0, nb, s);
  if (e == hipSuccess) e = hipMemsetAsync(grads, 0, nb, s);
  if (e == hipSuccess) e = hipMemsetAsync(h->ws + h->wo.flags, 0, 4, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->ws + h->wo.chunks, h->chunks.data(), h->chunks.size() * sizeof(AdamChunk),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !init_params)
    e = hipMemcpyAsync(h->ws + h->wo.init_tab, h->init_segs.data(),
                       h->init_segs.size() * sizeof(InitSeg), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && h->h16()) {
    e = hipMemcpyAsync(h->ws + h->wo.tjobs, h->tjobs.data(), h->tjobs.size() * sizeof(TransposeJob),
                       hipMemcpyHostToDevice, s);
    // columns Vp..vi of wte^T stay zero
    if (e == hipSuccess) e = hipMemsetAsync(h->ws + h->wo.wT, 0, h->wo.wT_elems * 2, s);
    // and so do columns Vp..vi of the logits buffer, which only the
    // cross-entropy writes (the fused head's input-gradient product reads them)
    const int64_t Mx = (int64_t)cfg->max_batch * cfg->block_size;
    if (e == hipSuccess && h->wo.vi > cfg->padded_vocab)
      e = hipMemset2DAsync(h->ws + h->wo.logits + cfg->padded_vocab * 2, h->wo.vi * 2, 0,
                           (h->wo.vi - cfg->padded_vocab) * 2, Mx, s);
  }
  // the host table must outlive the copy: wait for it once, at set-up
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    gpt_error_text() = hipGetErrorString(e);
    delete h;
    return GPT_EHIP;
  }
  if (!init_params) {
    rc = init_params_launch(params, h->at<InitSeg>(h->wo.init_tab), (int)h->init_segs.size(),
                            seed, s);
    if (rc) {
      delete h;
      return map_rc(rc);
    }
  }
  if (h->h16()) {
    rc = to_h16_launch(params, h->at<h16_t>(h->wo.shadow), h->po.total, s);
    if (!rc) rc = h->refresh_transposes(s);
    if (rc) {
      delete h;
      return map_rc(rc);
    }
  }
  *out = h;
  return GPT_OK;
}

// Dropout sites of one forward: 0 the embedding sum, 1 + 2l the attention
// probabilities of layer l, 2 + 2l the MLP output of layer l (counter word 2
// = site * 2^24, plus b * n_head + h for attention).
static Drop at_site(Drop d, int site) {
  if (d.thresh) d.site = (uint32_t)site << 24;
  return d;
}
// thresh = ceil(p 2^32) (a word w keeps its element when w >= thresh, i.e.
// w / 2^32 >= p), scale = 1 / (1 - p); p = 0 gives no dropout
static int make_drop(const gpt_dropout* g, int n_layer, Drop* out) {
  *out = Drop();
  if (!g || g->p == 0.f) return GPT_OK;
  if (!(g->p > 0.f && g->p < 1.f)) return fail(GPT_EINVAL, "dropout p must be in [0, 1)");
  if (2 * n_layer + 1 > 255) return fail(GPT_EUNSUPPORTED, "dropout covers at most 127 layers");
  const double t = ceil((double)g->p * 4294967296.0);
  out->thresh = (uint32_t)(t > 4294967295.0 ? 4294967295.0 : t);
  out->scale = (float)(1.0 / (1.0 - (double)g->p));
  out->k0 = (uint32_t)g->seed;
  out->k1 = (uint32_t)(g->seed >> 32);
  out->step = g->step;
  return GPT_OK;
}

// Embedding, the L blocks and the final LayerNorm over B sequences of T
// tokens ([NG] Part IV Stage 4: GPT.forward up to ln_f), with the dropout dr
// (none for sampling).  With kv set, each block's keys and values are also
// stored in the cache kv (sized for B sequences of max_len positions) at
// positions [0, T).
static int forward_stack(Model* h, const int32_t* idx, int B, int T, void* kv, int max_len,
                         hipStream_t s, Drop dr = Drop()) {
  const gpt_config& c = h->cfg;
  const bool bf = h->h16();
  const WsOff& w = h->wo;
  const ParamOff& p = h->po;
  const int M = B * T, d = c.n_embd, H = c.n_head;
  const int64_t kv_layer = 2ll * B * H * max_len * (d / H);
  CK(embed_fwd_launch(idx, h->P(p.wte), h->P(p.wpe), h->at<float>(w.layer.empty() ? w.x_final : w.layer[0].x_in),
                      M, T, d, c.padded_vocab, h->at<int>(w.flags), s, at_site(dr, 0)));
  for (int l = 0; l < c.n_layer; ++l) {
    const WsLayer& L = w.layer[l];
    const LayerOff& P = p.layer[l];
    const size_t x_out = (l + 1 < c.n_layer) ? w.layer[l + 1].x_in : w.x_final;
    CK(layernorm_fwd_launch(bf, h->at<float>(L.x_in), h->P(P.ln1w), h->P(P.ln1b), h->at(L.ln1),
                            h->at<float>(L.ln1_mean), h->at<float>(L.ln1_rstd), M, d, s));
    GemmEpiArgs e;
    e.out = h->at(L.qkv);
    e.bias = h->P(P.attnb);
    e.ldc = 3 * d;
    CK(gemm_launch(bf, true, true, EPI_ACT, h->at(L.ln1), d, h->W(P.attnw), d, M, 3 * d, d, d, d,
                   e, s));
    if (kv)
      CK(kv_store_launch(bf, h->at(L.qkv), (char*)kv + l * kv_layer * h->es(), B, T, H, d / H,
                         max_len, 0, s));
    CK(attention_fwd_launch(bf, h->at(L.qkv), h->at(L.att), h->at<float>(L.lse), B, T, H, d, s,
                            at_site(dr, 1 + 2 * l), L.dmask ? h->at<uint32_t>(L.dmask) : nullptr));
    e = GemmEpiArgs();
    e.out = h->at(L.x_mid);
    e.aux = h->at(L.x_in);
    e.bias = h->P(P.aprojb);
    e.ldc = d;
    CK(gemm_launch(bf, true, true, EPI_RESID, h->at(L.att), d, h->W(P.aprojw), d, M, d, d, d, d, e,
                   s));
    CK(layernorm_fwd_launch(bf, h->at<float>(L.x_mid), h->P(P.ln2w), h->P(P.ln2b), h->at(L.ln2),
                            h->at<float>(L.ln2_mean), h->at<float>(L.ln2_rstd), M, d, s));
    e = GemmEpiArgs();
    e.out = h->at(L.dgelu);
    e.out2 = h->at(L.g);
    e.bias = h->P(P.fcb);
    e.ldc = 4 * d;
    CK(gemm_launch(bf, true, true, EPI_GELU, h->at(L.ln2), d, h->W(P.fcw), d, M, 4 * d, d, d, d,
                   e, s));
    e = GemmEpiArgs();
    e.out = h->at(x_out);
    e.aux = h->at(L.x_mid);
    e.bias = h->P(P.mprojb);
    e.ldc = d;
    e.drop = at_site(dr, 2 + 2 * l);
    CK(gemm_launch(bf, true, true, EPI_RESID, h->at(L.g), 4 * d, h->W(P.mprojw), 4 * d, M, d, 4 * d,
                   4 * d, 4 * d, e, s));
  }
  CK(layernorm_fwd_launch(bf, h->at<float>(w.x_final), h->P(p.lnfw), h->P(p.lnfb), h->at(w.lnf),
                          h->at<float>(w.lnf_mean), h->at<float>(w.lnf_rstd), M, d, s));
  return GPT_OK;
}

// The tied head with the cross-entropy fused (after forward_stack and the
// count of valid targets): the product's epilogue stores exp(z) and each
// row's sums, one small pass takes each row's loss, the gradient factor r,
// r * lnf and the target columns; no pass over the logits follows.
static int fused_head_loss(Model* h, const int32_t* targets, int M, float loss_scale,
                           const float* dscale, hipStream_t s) {
  const gpt_config& c = h->cfg;
  const WsOff& w = h->wo;
  const int d = c.n_embd;
  GemmEpiArgs e;
  e.out = h->at(w.logits);
  e.ldc = (int)w.vi;
  e.head.tgt = targets;
  e.head.part = h->at<float>(w.head_part);
  e.head.zy = h->at<float>(w.head_zy);
  e.head.V = c.vocab_size;
  e.head.npart = w.head_npart;
  CK(gemm_launch(true, true, true, EPI_HEAD, h->at(w.lnf), d, h->W(h->po.wte), d, M,
                 c.padded_vocab, d, d, d, e, s));
  CK(head_combine_launch(h->at<float>(w.head_part), w.head_npart, h->at<float>(w.head_zy), targets,
                         c.vocab_size, h->at<int>(w.nvalid), loss_scale, dscale,
                         h->at<h16_t>(w.lnf), d, h->at<float>(w.row_loss), h->at<float>(w.head_r),
                         h->at<h16_t>(w.head_h2), h->at<h16_t>(w.logits), (int)w.vi, M,
                         h->at<int>(w.flags), s));
  return GPT_OK;
}

int gpt_forward_loss(Model* h, const int32_t* idx, const int32_t* targets, int32_t B, int32_t T,
                     float loss_scale, const float* dscale, const gpt_dropout* dropout,
                     float* loss_out, void* logits_out, void* stream) {
  if (!h || !idx) return fail(GPT_EINVAL, "null handle or idx");
  const gpt_config& c = h->cfg;
  if (B < 1 || B > c.max_batch) return fail(GPT_EINVAL, "B outside [1, max_batch]");
  if (T < 1) return fail(GPT_EINVAL, "T < 1");
  if (T > c.block_size) return fail(GPT_ESEQLEN, "T > block_size");
  Drop dr;
  if (int rc = make_drop(dropout, c.n_layer, &dr)) return rc;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = h->h16();
  const WsOff& w = h->wo;
  const ParamOff& p = h->po;
  const int M = B * T, d = c.n_embd;
  h->have_fwd = false;

  CK(forward_stack(h, idx, B, T, nullptr, 1, s, dr));
  const bool fused = targets && !logits_out && h->fused_ok();
  if (fused) {
    CK(count_valid_launch(targets, M, c.vocab_size, h->at<int>(w.nvalid), h->at<int>(w.flags), s));
    CK(fused_head_loss(h, targets, M, loss_scale, dscale, s));
    if (loss_out) CK(loss_finalize_launch(h->at<float>(w.row_loss), M, h->at<int>(w.nvalid), loss_out, s));
  } else {
    GemmEpiArgs e;
    e.out = h->at(w.logits);
    e.ldc = (int)w.vi;
    CK(gemm_launch(bf, true, true, EPI_ACT, h->at(w.lnf), d, h->W(p.wte), d, M, c.padded_vocab, d,
                   d, d, e, s));
  }
  if (logits_out)
    CKH(hipMemcpy2DAsync(logits_out, (size_t)c.padded_vocab * h->es(), h->at(w.logits),
                         (size_t)w.vi * h->es(), (size_t)c.padded_vocab * h->es(), M,
                         hipMemcpyDeviceToDevice, s));
  if (targets && !fused) {
    CK(count_valid_launch(targets, M, c.vocab_size, h->at<int>(w.nvalid), h->at<int>(w.flags), s));
    CK(cross_entropy_launch(bf, h->at(w.logits), targets, h->at<float>(w.row_loss),
                            h->at<int>(w.nvalid), loss_scale, dscale, M, c.vocab_size, (int)w.vi,
                            s));
    if (loss_out) CK(loss_finalize_launch(h->at<float>(w.row_loss), M, h->at<int>(w.nvalid), loss_out, s));
  }
  h->have_fwd = true;
  h->have_targets = targets != nullptr;
  h->B = B;
  h->T = T;
  h->idx = idx;
  h->last_fused = fused;
  h->drop = dr;
  return GPT_OK;
}

// Evaluation ([NG] Part IV Stage 2, estimate_loss: the model in eval mode, so
// no dropout, and no gradient): the mean loss over the valid targets, the
// logits left unmodified.
int gpt_eval_loss(Model* h, const int32_t* idx, const int32_t* targets, int32_t B, int32_t T,
                  float* loss_out, void* stream) {
  if (!h || !idx || !targets || !loss_out) return fail(GPT_EINVAL, "null handle or buffer");
  const gpt_config& c = h->cfg;
  if (B < 1 || B > c.max_batch) return fail(GPT_EINVAL, "B outside [1, max_batch]");
  if (T < 1) return fail(GPT_EINVAL, "T < 1");
  if (T > c.block_size) return fail(GPT_ESEQLEN, "T > block_size");
  hipStream_t s = (hipStream_t)stream;
  const bool bf = h->h16();
  const WsOff& w = h->wo;
  const ParamOff& p = h->po;
  const int M = B * T, d = c.n_embd;
  h->have_fwd = false;
  CK(forward_stack(h, idx, B, T, nullptr, 1, s));
  CK(count_valid_launch(targets, M, c.vocab_size, h->at<int>(w.nvalid), h->at<int>(w.flags), s));
  if (h->fused_ok()) {
    // the same fused head as training, so the eval loss is the training
    // forward's loss bit for bit (the factors it leaves go unused)
    CK(fused_head_loss(h, targets, M, 1.f, nullptr, s));
  } else {
    GemmEpiArgs e;
    e.out = h->at(w.logits);
    e.ldc = (int)w.vi;
    CK(gemm_launch(bf, true, true, EPI_ACT, h->at(w.lnf), d, h->W(p.wte), d, M, c.padded_vocab, d,
                   d, d, e, s));
    CK(cross_entropy_launch(bf, h->at(w.logits), targets, h->at<float>(w.row_loss),
                            h->at<int>(w.nvalid), 1.f, nullptr, M, c.vocab_size, (int)w.vi, s, 0));
  }
  CK(loss_finalize_launch(h->at<float>(w.row_loss), M, h->at<int>(w.nvalid), loss_out, s));
  return GPT_OK;
}

// The pages' estimate_loss over one split ([NG] Part IV Stage 2): the eval
// loss of each of n_batches batches (idx, targets: [n_batches][B][T]), then
// their mean in a fixed order (fp64) into loss_out, all on the device.
int gpt_estimate_loss(Model* h, const int32_t* idx, const int32_t* targets, int32_t n_batches,
                      int32_t B, int32_t T, float* loss_out, void* stream) {
  if (!h || !idx || !targets || !loss_out) return fail(GPT_EINVAL, "null handle or buffer");
  if (n_batches < 1 || n_batches > kEvalBatches)
    return fail(GPT_EINVAL, "n_batches outside [1, 1024]");
  float* losses = h->at<float>(h->wo.eval_losses);
  const int64_t n = (int64_t)B * T;
  for (int k = 0; k < n_batches; ++k)
    if (int rc = gpt_eval_loss(h, idx + k * n, targets + k * n, B, T, losses + k, stream)) return rc;
  CK(mean_launch(losses, n_batches, loss_out, (hipStream_t)stream));
  return GPT_OK;
}

// ---------------------------------------------------------------- sampling
int64_t gpt_kv_cache_bytes(const gpt_config* c, int32_t B, int32_t max_len) {
  if (validate(c) != GPT_OK || B < 1 || max_len < 1) return -1;
  const int64_t es = c->mode != GPT_FP32 ? 2 : 4;
  // + 64 rows of one head: the decode attention reads whole chunks of 64
  // value rows, past the last sequence's len up to 63 rows beyond the end
  return ((int64_t)c->n_layer * 2 * B * c->n_embd * max_len + 64ll * (c->n_embd / c->n_head)) * es;
}

static int check_decode_args(Model* h, int B, int max_len, const void* kv, const float* logits_out) {
  const gpt_config& c = h->cfg;
  if (!kv || !logits_out) return fail(GPT_EINVAL, "null cache or logits buffer");
  if (B < 1 || B > c.max_batch) return fail(GPT_EINVAL, "B outside [1, max_batch]");
  if (max_len < 1 || max_len > c.block_size) return fail(GPT_ESEQLEN, "max_len outside [1, block_size]");
  return GPT_OK;
}

// head over one row per sequence: logits [B][padded_vocab] fp32 = rows of
// lnf (row pitch lda elements) times wte^T
static int head_rows(Model* h, const void* rows, int lda, int B, float* logits_out, hipStream_t s) {
  const gpt_config& c = h->cfg;
  GemmEpiArgs e;
  e.out = logits_out;
  e.ldc = c.padded_vocab;
  CK(gemm_launch(h->h16(), true, true, EPI_F32, rows, lda, h->W(h->po.wte), c.n_embd, B,
                 c.padded_vocab, c.n_embd, c.n_embd, c.n_embd, e, s));
  return GPT_OK;
}

int gpt_prefill(Model* h, const int32_t* idx, int32_t B, int32_t T0, void* kv, int32_t max_len,
                float* logits_out, void* stream) {
  if (!h || !idx) return fail(GPT_EINVAL, "null handle or idx");
  CK(check_decode_args(h, B, max_len, kv, logits_out));
  if (T0 < 1 || T0 > max_len) return fail(GPT_ESEQLEN, "prompt length outside [1, max_len]");
  hipStream_t s = (hipStream_t)stream;
  h->have_fwd = false;
  const int d = h->cfg.n_embd;
  CK(forward_stack(h, idx, B, T0, kv, max_len, s));
  // the last position of every sequence: row b*T0 + T0-1 of lnf
  CK(head_rows(h, (const char*)h->at(h->wo.lnf) + (size_t)(T0 - 1) * d * h->es(), T0 * d, B,
               logits_out, s));
  return GPT_OK;
}

int gpt_decode_step(Model* h, const int32_t* tok, int32_t B, int32_t pos, void* kv,
                    int32_t max_len, float* logits_out, void* stream) {
  if (!h || !tok) return fail(GPT_EINVAL, "null handle or tokens");
  CK(check_decode_args(h, B, max_len, kv, logits_out));
  if (pos < 0 || pos >= max_len) return fail(GPT_ESEQLEN, "position outside [0, max_len)");
  hipStream_t s = (hipStream_t)stream;
  h->have_fwd = false;
  const gpt_config& c = h->cfg;
  const bool bf = h->h16();
  const WsOff& w = h->wo;
  const ParamOff& p = h->po;
  const int d = c.n_embd, H = c.n_head, hs = d / H;
  const int64_t kv_layer = 2ll * B * H * max_len * hs;
  // B rows, one per sequence, through the layer-0 activation buffers: x
  // alternates between x_in and x_mid
  const WsLayer& L = w.layer[0];
  float* xa = h->at<float>(L.x_in);
  float* xb = h->at<float>(L.x_mid);
  CK(embed_fwd_launch(tok, h->P(p.wte), h->P(p.wpe) + (size_t)pos * d, xa, B, 1, d, c.padded_vocab,
                      h->at<int>(w.flags), s));
  // few-row products (gemv_launch) where the rows fit; the tiled GEMM
  // path otherwise (it returns -5 when a shape or alignment does not suit)
  auto gemv = [&](int epi, const void* A, const float* lnw, const float* lnb, const void* W,
                  const float* bias, const float* aux, void* out, int N, int K, int ldo, void* kvc)
      -> int {
    return gemv_launch(bf, epi, A, lnw, lnb, W, bias, aux, out, B, N, K, ldo, kvc, H, hs, max_len,
                       pos, s);
  };
  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& P = p.layer[l];
    void* kvl = (char*)kv + l * kv_layer * h->es();
    // LayerNorm 1 + q|k|v projection + cache store
    int rc = gemv(0, xa, h->P(P.ln1w), h->P(P.ln1b), h->W(P.attnw), h->P(P.attnb), nullptr,
                  h->at(L.qkv), 3 * d, d, 3 * d, kvl);
    if (rc == -5) {
      CK(layernorm_fwd_launch(bf, xa, h->P(P.ln1w), h->P(P.ln1b), h->at(L.ln1),
                              h->at<float>(L.ln1_mean), h->at<float>(L.ln1_rstd), B, d, s));
      GemmEpiArgs e;
      e.out = h->at(L.qkv);
      e.bias = h->P(P.attnb);
      e.ldc = 3 * d;
      CK(gemm_launch(bf, true, true, EPI_ACT, h->at(L.ln1), d, h->W(P.attnw), d, B, 3 * d, d, d, d,
                     e, s));
      CK(kv_store_launch(bf, h->at(L.qkv), kvl, B, 1, H, hs, max_len, pos, s));
    } else {
      CK(rc);
    }
    CK(decode_attn_launch(bf, h->at(L.qkv), kvl, h->at(L.att), B, H, hs, max_len, pos + 1, s));
    // attention projection + residual
    rc = gemv(2, h->at(L.att), nullptr, nullptr, h->W(P.aprojw), h->P(P.aprojb), xa, xb, d, d, d,
              nullptr);
    if (rc == -5) {
      GemmEpiArgs e;
      e.out = xb;
      e.aux = xa;
      e.bias = h->P(P.aprojb);
      e.ldc = d;
      CK(gemm_launch(bf, true, true, EPI_RESID, h->at(L.att), d, h->W(P.aprojw), d, B, d, d, d, d,
                     e, s));
    } else {
      CK(rc);
    }
    // LayerNorm 2 + MLP expansion + GELU
    rc = gemv(3, xb, h->P(P.ln2w), h->P(P.ln2b), h->W(P.fcw), h->P(P.fcb), nullptr, h->at(L.g),
              4 * d, d, 4 * d, nullptr);
    if (rc == -5) {
      CK(layernorm_fwd_launch(bf, xb, h->P(P.ln2w), h->P(P.ln2b), h->at(L.ln2),
                              h->at<float>(L.ln2_mean), h->at<float>(L.ln2_rstd), B, d, s));
      GemmEpiArgs e;
      e.out = h->at(L.dgelu);
      e.out2 = h->at(L.g);
      e.bias = h->P(P.fcb);
      e.ldc = 4 * d;
      CK(gemm_launch(bf, true, true, EPI_GELU, h->at(L.ln2), d, h->W(P.fcw), d, B, 4 * d, d, d, d,
                     e, s));
    } else {
      CK(rc);
    }
    // MLP projection + residual
    rc = gemv(2, h->at(L.g), nullptr, nullptr, h->W(P.mprojw), h->P(P.mprojb), xb, xa, d, 4 * d, d,
              nullptr);
    if (rc == -5) {
      GemmEpiArgs e;
      e.out = xa;
      e.aux = xb;
      e.bias = h->P(P.mprojb);
      e.ldc = d;
      CK(gemm_launch(bf, true, true, EPI_RESID, h->at(L.g), 4 * d, h->W(P.mprojw), 4 * d, B, d,
                     4 * d, 4 * d, 4 * d, e, s));
    } else {
      CK(rc);
    }
  }
  // final LayerNorm + head over every padded column
  int rc = gemv(1, xa, h->P(p.lnfw), h->P(p.lnfb), h->W(p.wte), nullptr, nullptr, logits_out,
                c.padded_vocab, d, c.padded_vocab, nullptr);
  if (rc == -5) {
    CK(layernorm_fwd_launch(bf, xa, h->P(p.lnfw), h->P(p.lnfb), h->at(w.lnf),
                            h->at<float>(w.lnf_mean), h->at<float>(w.lnf_rstd), B, d, s));
    CK(head_rows(h, h->at(w.lnf), d, B, logits_out, s));
  } else {
    CK(rc);
  }
  return GPT_OK;
}

int gpt_sample(const float* logits, int32_t B, int32_t V, int32_t ldv, float temperature,
               int32_t top_k, const float* u, int32_t* tok_out, void* stream) {
  if (!logits || !u || !tok_out) return fail(GPT_EINVAL, "null sampling buffer");
  if (B < 1 || V < 1 || ldv < V) return fail(GPT_EINVAL, "bad sampling shape");
  if (!(temperature > 0.f)) return fail(GPT_EINVAL, "temperature must be > 0");
  CK(sample_launch(logits, B, V, ldv, temperature, top_k, u, tok_out, (hipStream_t)stream));
  return GPT_OK;
}

int gpt_backward(Model* h, int32_t zero_first, void* stream) {
  if (!h) return fail(GPT_EINVAL, "null handle");
  if (!h->have_fwd || !h->have_targets)
    return fail(GPT_ESTATE, "backward needs a preceding forward with targets");
  hipStream_t s = (hipStream_t)stream;
  const gpt_config& c = h->cfg;
  const bool bf = h->h16();
  const WsOff& w = h->wo;
  const ParamOff& p = h->po;
  const int B = h->B, T = h->T, M = B * T, d = c.n_embd, H = c.n_head;
  const int beta = zero_first ? 0 : 1;
  const int vi = (int)w.vi;
  float* dres = h->at<float>(w.dres);
  void* dres_act = h->at(w.dres_act);
  void* dln = h->at(w.dln);  // input gradients of the LayerNorms, in the activation type
  void* dbig = h->at(w.dbig);
  // the column-sum partials each producer leaves (bias and LayerNorm weight
  // gradients), finished together at the end
  std::vector<ColsumJob> jobs;
  jobs.reserve(4 * c.n_layer + 1);
  int n_ln = 0, n_cs = 0;
  auto ln_slice = [&]() { return h->at<float>(w.ln_part) + (n_ln++) * w.ln_part_elems; };
  auto cs_slice = [&]() { return h->at<float>(w.cs_part) + (n_cs++) * w.cs_part_elems; };
  auto keep = [&](const ColsumJob& j) {
    if (j.part) jobs.push_back(j);
  };
  ColsumJob job;
  float* sk = w.splitk_bytes ? h->at<float>(w.splitk) : nullptr;
  const int64_t skb = w.splitk_bytes;
  // the weight gradients pass their split-K reductions along (each runs
  // inside the next weight-gradient launch), over the two halves of the
  // split-K scratch
  SplitKChain chain;
  if (sk) {
    chain.ws_bytes = (skb / 2) & ~(int64_t)255;
    chain.ws[0] = sk;
    chain.ws[1] = (float*)((char*)sk + chain.ws_bytes);
  }

  // LM head: dwte (+)= dlogits^T lnf ; dlnf = dlogits wte.  The input
  // gradients of the LayerNorms (dlnf, dln2, dln1) are stored in the
  // activation type, as the matrix products' outputs are under 16-bit mixed
  // precision; the LayerNorm backward reads them into fp32.
  if (h->last_fused) {
    // fused head: the buffer holds exp(z) with exp(z_y) - S at each row's
    // target, so dz = r times a row of it and is never stored: dwte (+)=
    // buffer^T (r lnf); dlnf = r (buffer wte) in the product's epilogue
    GemmEpiArgs e;
    e.out = h->G(p.wte);
    e.ldc = d;
    e.beta = beta;
    e.chain = &chain;
    if (h->time_dw) CK(h->mark(s, true));
    CK(gemm_launch(bf, false, false, EPI_ACCUM, h->at(w.logits), vi, h->at(w.head_h2), d,
                   c.padded_vocab, d, M, M, M, e, s, sk, skb));
    if (h->time_dw) CK(h->mark(s, false));
    e = GemmEpiArgs();
    e.out = dln;
    e.ldc = d;
    e.head.r = h->at<float>(w.head_r);
    CK(gemm_launch(bf, true, true, EPI_HEAD_DX, h->at(w.logits), vi, h->WT(w.wteT), vi, M, d, vi, vi,
                   vi, e, s));
  } else {
    GemmEpiArgs e;
    e.out = h->G(p.wte);
    e.ldc = d;
    e.beta = beta;
    e.chain = &chain;
    if (h->time_dw) CK(h->mark(s, true));
    CK(gemm_launch(bf, false, false, EPI_ACCUM, h->at(w.logits), vi, h->at(w.lnf), d,
                   c.padded_vocab, d, M, M, M, e, s, sk, skb));
    if (h->time_dw) CK(h->mark(s, false));
    e = GemmEpiArgs();
    e.out = dln;
    e.ldc = d;
    if (bf)
      CK(gemm_launch(bf, true, true, EPI_ACT, h->at(w.logits), vi, h->WT(w.wteT), vi, M, d, vi, vi,
                     vi, e, s));
    else
      CK(gemm_launch(bf, true, false, EPI_ACT, h->at(w.logits), vi, h->W(p.wte), d, M, d, vi, vi,
                     c.padded_vocab, e, s));
  }
  // with dropout, the LayerNorm backward that yields the gradient at a block's
  // output also forms the masked copy that the MLP projection's backward reads
  // (dres itself, the residual's gradient, stays unmasked)
  const Drop dr = h->drop;
  CK(layernorm_bwd_launch(bf, dln, h->at<float>(w.x_final), h->at<float>(w.lnf_mean),
                          h->at<float>(w.lnf_rstd), h->P(p.lnfw), dres, dres_act, 0, ln_slice(),
                          h->G(p.lnfw), h->G(p.lnfb), h->G(p.layer[c.n_layer - 1].mprojb), beta, M,
                          d, s, &(job = ColsumJob()), at_site(dr, 2 + 2 * (c.n_layer - 1))));
  keep(job);
  for (int l = c.n_layer - 1; l >= 0; --l) {
    const WsLayer& L = w.layer[l];
    const LayerOff& P = p.layer[l];
    // MLP projection: dW (+)= dres^T g ; du = (dres Wm) * gelu'(u)
    GemmEpiArgs e;
    e.out = h->G(P.mprojw);
    e.ldc = 4 * d;
    e.beta = beta;
    e.chain = &chain;
    if (h->time_dw) CK(h->mark(s, true));
    CK(gemm_launch(bf, false, false, EPI_ACCUM, dres_act, d, h->at(L.g), 4 * d, d, 4 * d, M, M, M, e, s, sk, skb));
    if (h->time_dw) CK(h->mark(s, false));
    e = GemmEpiArgs();
    e.out = dbig;
    e.aux = h->at(L.dgelu);
    e.ldc = 4 * d;
    e.cs_part = cs_slice();  // MLP expansion bias: db = colsum(du), formed alongside
    e.cs_out = h->G(P.fcb);
    e.cs_beta = beta;
    e.cs_defer = &(job = ColsumJob());
    if (bf)
      CK(gemm_launch(bf, true, true, EPI_GELU_BWD, dres_act, d, h->WT(L.mprojT), d, M, 4 * d, d, d,
                     d, e, s));
    else
      CK(gemm_launch(bf, true, false, EPI_GELU_BWD, dres_act, d, h->W(P.mprojw), 4 * d, M, 4 * d, d,
                     d, d, e, s));
    keep(job);
    // MLP expansion: dW (+)= du^T ln2 ; dln2 = du Wfc
    e = GemmEpiArgs();
    e.out = h->G(P.fcw);
    e.ldc = d;
    e.beta = beta;
    e.chain = &chain;
    if (h->time_dw) CK(h->mark(s, true));
    CK(gemm_launch(bf, false, false, EPI_ACCUM, dbig, 4 * d, h->at(L.ln2), d, 4 * d, d, M, M, M, e, s, sk, skb));
    if (h->time_dw) CK(h->mark(s, false));
    e = GemmEpiArgs();
    e.out = dln;
    e.ldc = d;
    if (bf)
      CK(gemm_launch(bf, true, true, EPI_ACT, dbig, 4 * d, h->WT(L.fcT), 4 * d, M, d, 4 * d, 4 * d,
                     4 * d, e, s));
    else
      CK(gemm_launch(bf, true, false, EPI_ACT, dbig, 4 * d, h->W(P.fcw), d, M, d, 4 * d, 4 * d,
                     4 * d, e, s));
    CK(layernorm_bwd_launch(bf, dln, h->at<float>(L.x_mid), h->at<float>(L.ln2_mean),
                            h->at<float>(L.ln2_rstd), h->P(P.ln2w), dres, dres_act, 1, ln_slice(),
                            h->G(P.ln2w), h->G(P.ln2b), h->G(P.aprojb), beta, M, d, s,
                            &(job = ColsumJob())));
    keep(job);
    // attention projection: dW (+)= dres^T att ; datt = dres Wa
    e = GemmEpiArgs();
    e.out = h->G(P.aprojw);
    e.ldc = d;
    e.beta = beta;
    e.chain = &chain;
    if (h->time_dw) CK(h->mark(s, true));
    CK(gemm_launch(bf, false, false, EPI_ACCUM, dres_act, d, h->at(L.att), d, d, d, M, M, M, e, s, sk, skb));
    if (h->time_dw) CK(h->mark(s, false));
    e = GemmEpiArgs();
    e.out = h->at(w.dO);
    e.ldc = d;
    if (bf)
      CK(gemm_launch(bf, true, true, EPI_ACT, dres_act, d, h->WT(L.aprojT), d, M, d, d, d, d, e, s));
    else
      CK(gemm_launch(bf, true, false, EPI_ACT, dres_act, d, h->W(P.aprojw), d, M, d, d, d, d, e, s));
    // attention; the fused projection's bias gradient db = colsum(dqkv) is
    // formed by the attention backward
    CK(attention_bwd_launch(bf, h->at(L.qkv), h->at(L.att), h->at<float>(L.lse), h->at(w.dO), dbig,
                            h->at<float>(w.Dbuf), B, T, H, d, cs_slice(), h->G(P.attnb), beta, s,
                            &(job = ColsumJob()), at_site(dr, 1 + 2 * l),
                            L.dmask ? h->at<uint32_t>(L.dmask) : nullptr));
    keep(job);
    // fused q|k|v projection: dW (+)= dqkv^T ln1 ; dln1 = dqkv Wqkv
    e = GemmEpiArgs();
    e.out = h->G(P.attnw);
    e.ldc = d;
    e.beta = beta;
    e.chain = &chain;
    if (h->time_dw) CK(h->mark(s, true));
    CK(gemm_launch(bf, false, false, EPI_ACCUM, dbig, 3 * d, h->at(L.ln1), d, 3 * d, d, M, M, M, e, s, sk, skb));
    if (l == 0) CK(splitk_chain_flush(&chain, s));  // the last weight gradient's reduction
    if (h->time_dw) CK(h->mark(s, false));
    e = GemmEpiArgs();
    e.out = dln;
    e.ldc = d;
    if (bf)
      CK(gemm_launch(bf, true, true, EPI_ACT, dbig, 3 * d, h->WT(L.attnT), 3 * d, M, d, 3 * d, 3 * d,
                     3 * d, e, s));
    else
      CK(gemm_launch(bf, true, false, EPI_ACT, dbig, 3 * d, h->W(P.attnw), d, M, d, 3 * d, 3 * d,
                     3 * d, e, s));
    CK(layernorm_bwd_launch(bf, dln, h->at<float>(L.x_in), h->at<float>(L.ln1_mean),
                            h->at<float>(L.ln1_rstd), h->P(P.ln1w), dres, dres_act, 1, ln_slice(),
                            h->G(P.ln1w), h->G(P.ln1b), l > 0 ? h->G(p.layer[l - 1].mprojb) : nullptr,
                            beta, M, d, s, &(job = ColsumJob()),
                            l > 0 ? at_site(dr, 2 + 2 * (l - 1)) : Drop()));
    keep(job);
  }
  CK(splitk_chain_flush(&chain, s));  // nothing pending unless the layer loop was empty
  CK(colsum_finalize_group_launch(jobs.data(), (int)jobs.size(), beta, s));
  // the embedding sum's dropout: the gradient that reaches wte and wpe
  CK(dropout_rows_launch(dres, dres, M, d, at_site(dr, 0), s));
  // embeddings: dwte[idx] += dx ; dwpe[t] (+)= sum_b dx
  CK(embed_bwd_launch(h->idx, dres, h->G(p.wte), h->G(p.wpe), B, T, c.block_size, d,
                      c.padded_vocab, beta, s));
  return GPT_OK;
}

int gpt_adamw_step(Model* h, float lr, float beta1, float beta2, float eps, float weight_decay,
                   float max_norm, int32_t t, int32_t skip_nonfinite, float* norm_out,
                   void* stream) {
  if (!h) return fail(GPT_EINVAL, "null handle");
  if (t < 1) return fail(GPT_EINVAL, "t must be >= 1");
  hipStream_t s = (hipStream_t)stream;
  const WsOff& w = h->wo;
  CK(adamw_launch(h->params, h->grads, h->m, h->v,
                  h->h16() ? h->at<h16_t>(w.shadow) : nullptr, h->po.total,
                  h->at<AdamChunk>(w.chunks), (int)h->chunks.size(), h->tiles(),
                  h->at<double>(w.norm_part), h->at<float>(w.scal), norm_out, lr, beta1, beta2, eps,
                  weight_decay, max_norm, t, skip_nonfinite, s));
  return GPT_OK;
}

// Dynamic loss scaling: unscale (multiply by 1/scale), clip against the norm of
// the unscaled gradients, AdamW at step steps+1 unless the norm is not finite,
// then the scale update, all on the device.
int gpt_amp_step(Model* h, float lr, float beta1, float beta2, float eps, float weight_decay,
                 float max_norm, gpt_loss_scaler* scaler, float growth_factor, float backoff_factor,
                 int32_t growth_interval, float* norm_out, void* stream) {
  if (!h || !scaler) return fail(GPT_EINVAL, "null handle or scaler");
  if (growth_interval < 1 || !(growth_factor >= 1.f) || !(backoff_factor > 0.f) ||
      !(backoff_factor <= 1.f))
    return fail(GPT_EINVAL, "bad loss-scaler constants");
  hipStream_t s = (hipStream_t)stream;
  const WsOff& w = h->wo;
  CK(adamw_amp_launch(h->params, h->grads, h->m, h->v, h->h16() ? h->at<h16_t>(w.shadow) : nullptr,
                      h->po.total, h->at<AdamChunk>(w.chunks), (int)h->chunks.size(), h->tiles(),
                      h->at<double>(w.norm_part), h->at<float>(w.scal), norm_out, lr, beta1, beta2,
                      eps, weight_decay, max_norm, (float*)scaler, growth_factor, backoff_factor,
                      growth_interval, s));
  return GPT_OK;
}

int gpt_set_option(Model* h, int32_t option, int32_t value) {
  if (!h) return fail(GPT_EINVAL, "null handle");
  if (option != GPT_OPT_FUSED_HEAD_CE && option != GPT_OPT_TIME_WEIGHT_GRADIENTS)
    return fail(GPT_EINVAL, "unknown option");
  if (value != 0 && value != 1) return fail(GPT_EINVAL, "option value must be 0 or 1");
  if (option == GPT_OPT_FUSED_HEAD_CE) h->fused_ce = value != 0;
  else h->time_dw = value != 0;
  return GPT_OK;
}

int gpt_get_option(Model* h, int32_t option, int32_t* value) {
  if (!h || !value) return fail(GPT_EINVAL, "null handle or value");
  if (option == GPT_OPT_FUSED_HEAD_CE) {
    *value = h->fused_ce ? 1 : 0;
    return GPT_OK;
  }
  if (option == GPT_OPT_TIME_WEIGHT_GRADIENTS) {
    *value = h->time_dw ? 1 : 0;
    return GPT_OK;
  }
  return fail(GPT_EINVAL, "unknown option");
}

int gpt_read_timing(Model* h, double* ms, int64_t* launches) {
  if (!h || !ms || !launches) return fail(GPT_EINVAL, "null handle or output");
  double total = 0.0;
  for (size_t i = 0; i + 1 < h->tev_used; i += 2) {
    CKH(hipEventSynchronize(h->tev[i + 1]));
    float t = 0.f;
    CKH(hipEventElapsedTime(&t, h->tev[i], h->tev[i + 1]));
    total += t;
  }
  *ms = total;
  *launches = (int64_t)(h->tev_used / 2);
  h->tev_used = 0;
  return GPT_OK;
}

int gpt_read_flags(Model* h, int32_t* flags, void* stream) {
  if (!h || !flags) return fail(GPT_EINVAL, "null argument");
  hipStream_t s = (hipStream_t)stream;
  int32_t v = 0;
  CKH(hipMemcpyAsync(&v, h->ws + h->wo.flags, 4, hipMemcpyDeviceToHost, s));
  CKH(hipStreamSynchronize(s));
  CKH(hipMemsetAsync(h->ws + h->wo.flags, 0, 4, s));
  *flags = v;
  return GPT_OK;
}

void gpt_destroy(Model* h) { delete h; }


// ----------------------------------------------------------------- single ops
int gpt_op_linear(int32_t h16, const void* A, const void* B, const float* bias, void* C,
                  int32_t out_f32, int32_t M, int32_t N, int32_t K, void* stream) {
  if (!A || !B || !C || M < 0 || N < 0 || K < 1) return fail(GPT_EINVAL, "bad linear arguments");
  GemmEpiArgs e;
  e.out = C;
  e.bias = bias;
  e.ldc = N;
  CK(gemm_launch(h16 != 0, true, true, out_f32 ? EPI_F32 : EPI_ACT, A, K, B, K, M, N, K, K, K, e,
                 (hipStream_t)stream));
  return GPT_OK;
}

// MLP expansion forward (fc + bias + tanh-GELU): u = A W^T + bias;
// dgelu = gelu'(u), g = gelu(u), both in the activation type
int gpt_op_linear_gelu(int32_t h16, const void* A, const void* W, const float* bias, void* dgelu,
                       void* g, int32_t M, int32_t N, int32_t K, void* stream) {
  if (!A || !W || !dgelu || !g || M < 0 || N < 0 || K < 1)
    return fail(GPT_EINVAL, "bad linear_gelu arguments");
  GemmEpiArgs e;
  e.out = dgelu;
  e.out2 = g;
  e.bias = bias;
  e.ldc = N;
  CK(gemm_launch(h16 != 0, true, true, EPI_GELU, A, K, W, K, M, N, K, K, K, e,
                 (hipStream_t)stream));
  return GPT_OK;
}

// Column-sum scratch of the GELU-derivative product: one fp32 row per 128 rows
int64_t op_gelu_bwd_scratch_bytes(int64_t M, int64_t N) { return cdiv(M, 128) * N * 4; }

// MLP projection backward into the expansion: du = (dY Wt^T) * dgelu and,
// when dbias is set, dbias (+)= colsum(du) through the fp32 scratch
int gpt_op_linear_gelu_bwd(int32_t h16, const void* dY, const void* Wt, const void* dgelu,
                           void* du, float* dbias, int32_t accumulate_bias, int32_t M, int32_t N,
                           int32_t K, float* workspace, int64_t workspace_bytes, void* stream) {
  if (!dY || !Wt || !dgelu || !du || M < 0 || N < 1 || K < 1)
    return fail(GPT_EINVAL, "bad linear_gelu_bwd arguments");
  if (dbias && (!workspace || workspace_bytes < op_gelu_bwd_scratch_bytes(M, N)))
    return fail(GPT_EINVAL, "linear_gelu_bwd: workspace below ceil(M/128)*N*4 bytes");
  GemmEpiArgs e;
  e.out = du;
  e.aux = dgelu;
  e.ldc = N;
  if (dbias) {
    e.cs_part = workspace;
    e.cs_out = dbias;
    e.cs_beta = accumulate_bias ? 1 : 0;
  }
  CK(gemm_launch(h16 != 0, true, true, EPI_GELU_BWD, dY, K, Wt, K, M, N, K, K, K, e,
                 (hipStream_t)stream));
  return GPT_OK;
}

int gpt_op_linear_dw(int32_t h16, const void* dY, const void* X, float* dW, int32_t accumulate,
                     int32_t M, int32_t N, int32_t K, float* workspace, int64_t workspace_bytes,
                     void* stream) {
  if (!dY || !X || !dW || M < 1 || N < 0 || K < 0) return fail(GPT_EINVAL, "bad linear_dw arguments");
  GemmEpiArgs e;
  e.out = dW;
  e.ldc = K;
  e.beta = accumulate ? 1 : 0;
  CK(gemm_launch(h16 != 0, false, false, EPI_ACCUM, dY, N, X, K, N, K, M, M, M, e,
                 (hipStream_t)stream, workspace, workspace ? workspace_bytes : 0));
  return GPT_OK;
}

int gpt_op_linear_dw_seq(int32_t h16, int32_t count, const void* const* dY, const void* const* X,
                         float* const* dW, const int32_t* accumulate, const int32_t* M,
                         const int32_t* N, const int32_t* K, float* workspace,
                         int64_t workspace_bytes, void* stream) {
  if (count < 0 || (count > 0 && (!dY || !X || !dW || !accumulate || !M || !N || !K)))
    return fail(GPT_EINVAL, "bad linear_dw_seq arguments");
  for (int i = 0; i < count; ++i)
    if (!dY[i] || !X[i] || !dW[i] || M[i] < 1 || N[i] < 0 || K[i] < 0)
      return fail(GPT_EINVAL, "bad linear_dw_seq arguments");
  hipStream_t s = (hipStream_t)stream;
  SplitKChain chain;
  if (workspace && workspace_bytes > 0) {
    chain.ws_bytes = (workspace_bytes / 2) & ~(int64_t)255;
    chain.ws[0] = workspace;
    chain.ws[1] = (float*)((char*)workspace + chain.ws_bytes);
  }
  for (int i = 0; i < count; ++i) {
    // a product that adds into the previous product's gradient waits for
    // that product's reduction
    if (i > 0 && dW[i] == dW[i - 1]) CK(splitk_chain_flush(&chain, s));
    GemmEpiArgs e;
    e.out = dW[i];
    e.ldc = K[i];
    e.beta = accumulate[i] ? 1 : 0;
    e.chain = &chain;
    CK(gemm_launch(h16 != 0, false, false, EPI_ACCUM, dY[i], N[i], X[i], K[i], N[i], K[i], M[i],
                   M[i], M[i], e, s, workspace, workspace ? workspace_bytes : 0));
  }
  CK(splitk_chain_flush(&chain, s));
  return GPT_OK;
}

int gpt_op_linear_dx(int32_t h16, const void* dY, const void* W, float* dX, int32_t M, int32_t N,
                     int32_t K, void* stream) {
  if (!dY || !W || !dX || M < 0 || N < 1 || K < 0) return fail(GPT_EINVAL, "bad linear_dx arguments");
  GemmEpiArgs e;
  e.out = dX;
  e.ldc = K;
  CK(gemm_launch(h16 != 0, true, false, EPI_F32, dY, N, W, K, M, K, N, N, N, e,
                 (hipStream_t)stream));
  return GPT_OK;
}

int gpt_op_attention_fwd(int32_t h16, const void* qkv, void* out, float* lse, int32_t B, int32_t T,
                         int32_t H, int32_t C, void* stream) {
  if (!qkv || !out || !lse || B < 1 || T < 1 || H < 1 || C % H) return fail(GPT_EINVAL, "bad attention arguments");
  CK(attention_fwd_launch(h16 != 0, qkv, out, lse, B, T, H, C, (hipStream_t)stream));
  return GPT_OK;
}

int gpt_op_attention_bwd(int32_t h16, const void* qkv, const void* out, const float* lse,
                         const void* dout, void* dqkv, float* D, int32_t B, int32_t T, int32_t H,
                         int32_t C, void* stream) {
  if (!qkv || !out || !lse || !dout || !dqkv || !D || B < 1 || T < 1 || H < 1 || C % H)
    return fail(GPT_EINVAL, "bad attention arguments");
  CK(attention_bwd_launch(h16 != 0, qkv, out, lse, dout, dqkv, D, B, T, H, C, nullptr, nullptr, 0,
                          (hipStream_t)stream));
  return GPT_OK;
}

int gpt_op_layernorm_fwd(int32_t h16, const float* x, const float* w, const float* b, void* y,
                         float* mean, float* rstd, int32_t M, int32_t C, void* stream) {
  if (!x || !w || !b || !y || !mean || !rstd || M < 0 || C < 1) return fail(GPT_EINVAL, "bad layernorm arguments");
  CK(layernorm_fwd_launch(h16 != 0, x, w, b, y, mean, rstd, M, C, (hipStream_t)stream));
  return GPT_OK;
}

int gpt_op_dropout(const float* x, float* y, int64_t rows, int32_t cols, float p, uint64_t seed,
                   uint32_t step, uint32_t site_word, void* stream) {
  if (!x || !y || rows < 0 || cols < 1 || cols % 4) return fail(GPT_EINVAL, "bad dropout arguments");
  gpt_dropout g{p, step, seed};
  Drop dr;
  if (int rc = make_drop(&g, 0, &dr)) return rc;
  dr.site = site_word;
  CK(dropout_rows_launch(x, y, rows, cols, dr, (hipStream_t)stream));
  return GPT_OK;
}

int gpt_op_cross_entropy(int32_t h16, void* logits, const int32_t* targets, float* loss,
                         float* row_loss, int32_t* n_valid, float loss_scale, int32_t N, int32_t V,
                         int32_t ldv, void* stream) {
  if (!logits || !targets || !loss || !row_loss || !n_valid || N < 1 || V < 1 || ldv < V)
    return fail(GPT_EINVAL, "bad cross-entropy arguments");
  hipStream_t s = (hipStream_t)stream;
  CK(count_valid_launch(targets, N, V, n_valid, nullptr, s));
  CK(cross_entropy_launch(h16 != 0, logits, targets, row_loss, n_valid, loss_scale, nullptr, N, V,
                          ldv, s));
  CK(loss_finalize_launch(row_loss, N, n_valid, loss, s));
  return GPT_OK;
}

}  // namespace HALF_NS
