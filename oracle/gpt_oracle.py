"""Plain CPU oracle for one GPT-2 training step, and for sampling from the model.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the build entry
point, and the CPU-baseline leg of the benchmark use it.  It shares no code
with the HIP library and imports nothing from the product package.

What it computes is the plain definition of the model and of the step, in
float64 by default (every function takes the array dtype it is given), with
numpy's matmul as the only library primitive.  No blocking, no fusion, no
online softmax: attention materialises the full T x T score matrix, the
cross-entropy materialises the probabilities, AdamW is written per element.

Sources (page title, section):
  [NG]  "nanoGPT" (stanleyjacob.dev), Part IV "The full life of one training
        iteration" (Stages 1-6) and Part V "Internals deep dives" (Deep dive 1:
        model.py, Deep dive 2: train.py).
  [RC]  "Let's reproduce GPT-2 (124M)" (library.recl.app chapter notes), chapters
        "Cross Entropy Loss", "Model Initialization", "Float16, Gradient
        Scalers, BF16", "Nice/Ugly Numbers", "Gradient Accumulation".
  [YT]  "andrej-karpathy-lets-reproduce-gpt-2" (youtube.nixfred.com), "The
        optimization recipe, borrowed from the GPT-3 paper".
  [SO]  "Karpathy's Let's Reproduce GPT-2 in One Read" (sotaaz.com), "One check
        we ran: the GELU in nanoGPT is not GPT-2's" and "Section 3".
  [BK]  "Build GPT from scratch (nanoGPT walkthrough)" (learn.byteknotlabs.com),
        "The model in forty lines" and "Common pitfalls".

Readings taken where the pages are silent (each repeated where it is used):
  * LayerNorm: biased variance, epsilon 1e-5 (the defaults of the PyTorch
    LayerNorm the pages call; no value is printed).
  * GELU: the tanh approximation ([SO] says GPT-2 uses it), with the constants
    sqrt(2/pi) and 0.044715 of Hendrycks & Gimpel; its derivative is that of
    the tanh form.
  * Padded vocabulary columns v >= V are excluded from the softmax and get a
    zero gradient (the pages let the network learn to push them down; the
    workload definition masks them).
  * AdamW order: decoupled decay p <- p (1 - lr wd) first, then the Adam step
    with eps added outside the square root; bias correction uses the 1-based
    optimizer step t.
  * Clipping: coef = min(1, max_norm / (norm + 1e-6)), applied always.
  * Sampling: the top-k cutoff keeps values equal to the k-th largest;
    top_k <= 0 keeps all; the multinomial draw is by inverse CDF in token-id
    order with a uniform supplied by the caller.
  * Dropout: at the embedding sum, on the attention probabilities and on the
    MLP output (not after the attention's output projection, which neither
    page names); masks from Philox4x32-10 keyed by a seed, with the counter
    layout of dropout_mult; a kept value is multiplied by 1/(1-p).
    The generator is pinned to the known-answer vectors published with its
    definition (multipliers, key schedule and rounds at 32 bits), its round
    structure also through numpy's 64-bit Philox, and the key increments
    through their definitions.
  * Dynamic loss scaling (float16): initial scale 2^16, growth factor 2
    after 2000 consecutive clean steps, backoff factor 0.5 on a step with an
    inf or NaN gradient (the defaults of the GradScaler the pages construct;
    no value is printed); a grown scale is kept only if it is finite; a
    skipped step leaves params, m, v and the optimizer step count unchanged.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

LN_EPS = 1e-5
GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


# --------------------------------------------------------------------------
# configuration and parameter layout
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    """GPTConfig of [NG] Deep dive 1: block size, vocab, layers, heads, width.

    `vocab_size` is the real vocabulary V; `padded_vocab` (>= V) is the row
    count of the tied embedding ([RC] "Nice/Ugly Numbers": 50257 -> 50304).
    """
    vocab_size: int
    padded_vocab: int
    block_size: int
    n_layer: int
    n_head: int
    n_embd: int

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head


def param_shapes(cfg: Config, bias: bool = True, tied: bool = True):
    """Canonical flat parameter order, as (name, shape) pairs.

    Token table, position table, then per block ln_1, the fused q|k|v linear,
    the attention output projection, ln_2, the MLP expansion to 4*d and its
    projection back, then ln_f ([NG] Deep dive 1; [NG] Part IV Stage 4 for the
    block wiring).  Linear weights are stored [out, in].  With `tied` the LM
    head is the token table itself ([NG] Deep dive 1, weight tying), so no
    extra tensor appears; `tied=False` and `bias=False` exist only for the
    parameter-count checks of other models the pages describe.
    """
    d, L = cfg.n_embd, cfg.n_layer
    out = [("wte", (cfg.padded_vocab, d)), ("wpe", (cfg.block_size, d))]
    for l in range(L):
        p = f"h{l}."
        out.append((p + "ln1.w", (d,)))
        if bias:
            out.append((p + "ln1.b", (d,)))
        out.append((p + "attn.w", (3 * d, d)))
        if bias:
            out.append((p + "attn.b", (3 * d,)))
        out.append((p + "aproj.w", (d, d)))
        if bias:
            out.append((p + "aproj.b", (d,)))
        out.append((p + "ln2.w", (d,)))
        if bias:
            out.append((p + "ln2.b", (d,)))
        out.append((p + "fc.w", (4 * d, d)))
        if bias:
            out.append((p + "fc.b", (4 * d,)))
        out.append((p + "mproj.w", (d, 4 * d)))
        if bias:
            out.append((p + "mproj.b", (d,)))
    out.append(("lnf.w", (d,)))
    if bias:
        out.append(("lnf.b", (d,)))
    if not tied:
        out.append(("lm_head", (cfg.padded_vocab, d)))
    return out


def num_params(cfg: Config, bias: bool = True, tied: bool = True,
               non_embedding: bool = False) -> int:
    """Parameter count; the tied matrix is counted once.

    With `non_embedding` only the position table is subtracted, which is the
    get_num_params convention of [NG] Deep dive 1 ("123.65M").
    """
    n = sum(int(np.prod(s)) for _, s in param_shapes(cfg, bias, tied))
    if non_embedding:
        n -= cfg.block_size * cfg.n_embd
    return n


def unpack(flat: np.ndarray, cfg: Config) -> dict:
    """Views into a flat parameter (or gradient) vector, by name."""
    views, off = {}, 0
    for name, shape in param_shapes(cfg):
        n = int(np.prod(shape))
        views[name] = flat[off:off + n].reshape(shape)
        off += n
    assert off == flat.size, (off, flat.size)
    return views


def decay_mask(cfg: Config, dtype=np.float64) -> np.ndarray:
    """1 for tensors with two or more dimensions, else 0 ([NG] Deep dive 1,
    configure_optimizers; [YT] "weight decay of 0.1, applied only to the two
    dimensional parameters")."""
    parts = []
    for _, shape in param_shapes(cfg):
        parts.append(np.full(int(np.prod(shape)), 1.0 if len(shape) >= 2 else 0.0, dtype))
    return np.concatenate(parts)


# --------------------------------------------------------------------------
# the operations of the forward pass and their derivatives
# --------------------------------------------------------------------------
def layernorm_fwd(x, w, b, eps=LN_EPS):
    """Per-row normalisation over the last axis, then the affine map.

    mean and biased variance over the features; y = (x - mean)/sqrt(var+eps)*w+b.
    Returns y and the cache (xhat, rstd) for the backward.
    """
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    return xhat * w + b, (xhat, rstd)


def layernorm_bwd(dy, w, cache):
    """Derivative of layernorm_fwd: returns dx, dw, db.

    With g = dy*w: dx = rstd * (g - mean(g) - xhat * mean(g*xhat)) per row.
    """
    xhat, rstd = cache
    g = dy * w
    dx = rstd * (g - g.mean(axis=-1, keepdims=True)
                 - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    red = tuple(range(dy.ndim - 1))
    return dx, (dy * xhat).sum(axis=red), dy.sum(axis=red)


def gelu_fwd(u):
    """tanh-approximate GELU ([SO] "the GELU in nanoGPT is not GPT-2's")."""
    return 0.5 * u * (1.0 + np.tanh(GELU_C * (u + GELU_A * u ** 3)))


def gelu_bwd(u):
    """d gelu_fwd / du, the derivative of the tanh form itself."""
    t = np.tanh(GELU_C * (u + GELU_A * u ** 3))
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * GELU_C * (1.0 + 3.0 * GELU_A * u * u)


def causal_attention_fwd(q, k, v, z=None):
    """The manual attention path of [NG] Deep dive 1 (the semantics of the
    fused flash kernel): scores q k^T / sqrt(hs), entries above the diagonal
    set to -inf before the softmax ([BK] "Common pitfalls"), row softmax,
    dropout on the probabilities, then the weighted sum of v.  q, k, v:
    (..., T, hs); z (optional, (..., T, T)): the dropout multipliers (0 or
    1/(1-p)) applied to the probabilities.  Returns out and P (before
    dropout).
    """
    T, hs = q.shape[-2], q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(hs)
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(future, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=-1, keepdims=True)
    return (p if z is None else p * z) @ v, p


def causal_attention_bwd(dout, q, k, v, p, z=None):
    """Derivative of causal_attention_fwd: returns dq, dk, dv.

    With Pd = P * z (P when there is no dropout): dV = Pd^T dO;
    dP = (dO V^T) * z; dS = P * (dP - rowsum(P * dP)); the masked entries
    have P = 0 and so get no gradient; dQ = dS K / sqrt(hs),
    dK = dS^T Q / sqrt(hs).
    """
    hs = q.shape[-1]
    pd = p if z is None else p * z
    dv = np.swapaxes(pd, -1, -2) @ dout
    dp = dout @ np.swapaxes(v, -1, -2)
    if z is not None:
        dp = dp * z
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    dq = ds @ k / math.sqrt(hs)
    dk = np.swapaxes(ds, -1, -2) @ q / math.sqrt(hs)
    return dq, dk, dv


def cross_entropy(logits, targets, vocab_size, loss_scale=1.0):
    """Mean next-token negative log-likelihood and its gradient ([RC] "Cross
    Entropy Loss"; [NG] Part IV Stage 4: F.cross_entropy with ignore_index=-1).

    logits: (N, Vp); targets: (N,) with -1 meaning "no target".  Only the
    first `vocab_size` columns take part; padded columns get zero gradient.
    Returns (loss, dlogits) where loss is the unscaled mean over the
    non-ignored rows and dlogits = loss_scale * (softmax - onehot) / n_valid.
    """
    n, vp = logits.shape
    z = logits[:, :vocab_size]
    valid = targets >= 0
    n_valid = int(valid.sum())
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    sumexp = e.sum(axis=1, keepdims=True)
    lse = (zmax + np.log(sumexp))[:, 0]
    rows = np.nonzero(valid)[0]
    nll = lse[rows] - z[rows, targets[rows]]
    loss = float(nll.sum() / n_valid) if n_valid else 0.0
    dlogits = np.zeros_like(logits)
    if n_valid:
        prob = e / sumexp
        prob[rows, targets[rows]] -= 1.0
        prob[~valid] = 0.0
        dlogits[:, :vocab_size] = prob * (loss_scale / n_valid)
    return loss, dlogits


# --------------------------------------------------------------------------
# dropout from a counter-based generator
# --------------------------------------------------------------------------
# Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
# Easy as 1, 2, 3", SC'11): multipliers of the two 32-bit products, and the
# key increments (the fractional parts of the golden ratio and of sqrt(3),
# in 32-bit fixed point).
PHILOX_M32 = (0xD2511F53, 0xCD9E8D57)
PHILOX_W32 = (0x9E3779B9, 0xBB67AE85)


def philox(counter, key, width=32, mults=PHILOX_M32, weyl=PHILOX_W32, rounds=10):
    """The Philox bijection of four words: each round multiplies words 0 and
    2 by the two constants, and the new words are (hi(M1 c2) ^ c1 ^ k0,
    lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key is increased by
    the Weyl constants between rounds.  counter: four broadcastable integer
    arrays, key: two integers.  width 32 works on uint64 arrays (a 32 x 32
    product fits); width 64 on Python integers (the 64-bit variant, used only
    to check the round structure).  Returns the four output words."""
    mask = (1 << width) - 1
    if width == 32:
        c = [np.asarray(x, dtype=np.uint64) & np.uint64(mask) for x in counter]
        k0, k1 = np.uint64(key[0] & mask), np.uint64(key[1] & mask)
        M0, M1 = np.uint64(mults[0]), np.uint64(mults[1])
        W0, W1, msk, sh = np.uint64(weyl[0]), np.uint64(weyl[1]), np.uint64(mask), np.uint64(32)
    else:
        c = [np.asarray(x, dtype=object) for x in counter]
        k0, k1 = key[0] & mask, key[1] & mask
        (M0, M1), (W0, W1), msk, sh = mults, weyl, mask, width
    for r in range(rounds):
        if r:
            k0, k1 = (k0 + W0) & msk, (k1 + W1) & msk
        p0, p1 = M0 * c[0], M1 * c[2]
        c = [(p1 >> sh) ^ c[1] ^ k0, p1 & msk, (p0 >> sh) ^ c[3] ^ k1, p0 & msk]
    return c


@dataclass(frozen=True)
class Dropout:
    """Dropout of probability p ([NG] Part IV Stage 4 and Deep dive 1; [BK]
    "The model in forty lines"; [NG] Part VIII check 15 gives 0.2 for the
    character-level model) with masks drawn from Philox4x32-10 keyed by a
    64-bit seed; step tells calls apart (one per forward)."""
    p: float
    seed: int
    step: int = 0


def dropout_threshold(p: float) -> int:
    """A 32-bit word w keeps its element when w >= this (so w / 2^32 >= p)."""
    return min((1 << 32) - 1, math.ceil(p * 4294967296.0))


def dropout_mult(dr: Dropout, site: int, bh, rows: int, cols: int, dtype=np.float64):
    """The multipliers (0 or 1/(1-p)) of one site's matrix, shape
    (len(bh), rows, cols).  Element (r, c) of head bh is kept when word c % 4
    of Philox4x32-10 with key (seed low 32 bits, seed high 32 bits) and
    counter (c // 4, r, site * 2^24 + bh, step) is >= dropout_threshold(p).
    Sites: 0 the embedding sum, 1 + 2l the attention probabilities of layer
    l (rows queries, columns keys, bh = b * n_head + h), 2 + 2l the MLP
    output of layer l (rows b * T + t, columns features, bh = 0)."""
    bh = np.atleast_1d(np.asarray(bh, dtype=np.int64))
    g = np.arange((cols + 3) // 4, dtype=np.int64)[None, None, :]
    r = np.arange(rows, dtype=np.int64)[None, :, None]
    c2 = ((site << 24) + bh)[:, None, None]
    words = philox((g, r, c2, dr.step), (dr.seed & 0xFFFFFFFF, dr.seed >> 32))
    w = np.stack(np.broadcast_arrays(*words), axis=-1).reshape(len(bh), rows, -1)[:, :, :cols]
    keep = w >= np.uint64(dropout_threshold(dr.p))
    return keep.astype(dtype) * (1.0 / (1.0 - dr.p))


# --------------------------------------------------------------------------
# the model: forward and backward
# --------------------------------------------------------------------------
def forward(flat_params, idx, targets, cfg: Config, loss_scale=1.0,
            dtype=np.float64, dropout: Dropout | None = None):
    """GPT.forward of [NG] Part IV Stage 4 and Deep dive 1.

    token rows of wte plus position rows of wpe; per block
    x = x + attn(ln_1(x)); x = x + mlp(ln_2(x)); ln_f; logits = h wte^T over
    all padded_vocab columns; cross-entropy against the targets.
    idx, targets: int arrays (B, T), T <= block_size ([RC] "Implementing the
    forward pass to get logits").  Returns (logits (B,T,Vp), loss, cache);
    loss is None when targets is None.
    dropout (p > 0): the three places the pages name - the embedding sum
    ([NG] Part IV Stage 4), the attention probabilities and the MLP output
    ([NG] Deep dive 1; [BK] "The model in forty lines").  Reading: the
    attention's output projection is not followed by dropout (neither page
    puts one there).  Masks from dropout_mult.
    """
    P = unpack(np.asarray(flat_params, dtype=dtype), cfg)
    B, T = idx.shape
    if T > cfg.block_size:
        raise ValueError("sequence longer than block_size")
    d, H, hs = cfg.n_embd, cfg.n_head, cfg.head_dim
    drop = dropout is not None and dropout.p > 0
    x = P["wte"][idx] + P["wpe"][:T]
    z_emb = None
    if drop:
        z_emb = dropout_mult(dropout, 0, 0, B * T, d, dtype)[0].reshape(B, T, d)
        x = x * z_emb
    layers = []
    for l in range(cfg.n_layer):
        p = f"h{l}."
        c = {"x_in": x}
        h1, c["ln1"] = layernorm_fwd(x, P[p + "ln1.w"], P[p + "ln1.b"])
        qkv = h1 @ P[p + "attn.w"].T + P[p + "attn.b"]
        # split the 3d columns into q | k | v, then d columns into heads
        q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(B, T, H, hs).transpose(0, 2, 1, 3)
                   for i in range(3))
        z_att = None
        if drop:
            z_att = dropout_mult(dropout, 1 + 2 * l, np.arange(B * H), T, T, dtype).reshape(B, H, T, T)
        o, att_p = causal_attention_fwd(q, k, v, z_att)
        o = o.transpose(0, 2, 1, 3).reshape(B, T, d)
        x = x + (o @ P[p + "aproj.w"].T + P[p + "aproj.b"])
        c.update(h1=h1, q=q, k=k, v=v, att_p=att_p, z_att=z_att, o=o, x_mid=x)
        h2, c["ln2"] = layernorm_fwd(x, P[p + "ln2.w"], P[p + "ln2.b"])
        u = h2 @ P[p + "fc.w"].T + P[p + "fc.b"]
        g = gelu_fwd(u)
        y = g @ P[p + "mproj.w"].T + P[p + "mproj.b"]
        z_mlp = None
        if drop:
            z_mlp = dropout_mult(dropout, 2 + 2 * l, 0, B * T, d, dtype)[0].reshape(B, T, d)
            y = y * z_mlp
        x = x + y
        c.update(h2=h2, u=u, g=g, z_mlp=z_mlp)
        layers.append(c)
    hf, lnf_cache = layernorm_fwd(x, P["lnf.w"], P["lnf.b"])
    logits = hf @ P["wte"].T
    loss, dlogits = None, None
    if targets is not None:
        loss, dlogits = cross_entropy(logits.reshape(B * T, -1), targets.reshape(-1),
                                      cfg.vocab_size, loss_scale)
        dlogits = dlogits.reshape(logits.shape)
    cache = dict(P=P, idx=idx, layers=layers, hf=hf, lnf=lnf_cache, dlogits=dlogits, z_emb=z_emb)
    return logits, loss, cache


def backward(cache, cfg: Config, dtype=np.float64):
    """Analytic derivative of forward(...) w.r.t. every parameter.

    Returns a flat gradient vector in the canonical order.  The tied matrix
    receives the sum of its head and embedding gradients ([NG] Deep dive 1).
    """
    P, idx = cache["P"], cache["idx"]
    B, T = idx.shape
    d, H, hs = cfg.n_embd, cfg.n_head, cfg.head_dim
    grads = np.zeros(num_params(cfg), dtype=dtype)
    G = unpack(grads, cfg)
    dlogits = cache["dlogits"]
    # head: logits = hf wte^T
    G["wte"][...] += dlogits.reshape(B * T, -1).T @ cache["hf"].reshape(B * T, d)
    dhf = dlogits @ P["wte"]
    dx, G["lnf.w"][...], G["lnf.b"][...] = layernorm_bwd(dhf, P["lnf.w"], cache["lnf"])
    for l in reversed(range(cfg.n_layer)):
        p, c = f"h{l}.", cache["layers"][l]
        # MLP branch: x = x_mid + z * (g Wm^T + bm), g = gelu(u), u = h2 Wfc^T + bfc
        dy = dx if c["z_mlp"] is None else dx * c["z_mlp"]
        G[p + "mproj.w"][...] = dy.reshape(-1, d).T @ c["g"].reshape(-1, 4 * d)
        G[p + "mproj.b"][...] = dy.reshape(-1, d).sum(axis=0)
        dg = dy @ P[p + "mproj.w"]
        du = dg * gelu_bwd(c["u"])
        G[p + "fc.w"][...] = du.reshape(-1, 4 * d).T @ c["h2"].reshape(-1, d)
        G[p + "fc.b"][...] = du.reshape(-1, 4 * d).sum(axis=0)
        dh2 = du @ P[p + "fc.w"]
        dln, G[p + "ln2.w"][...], G[p + "ln2.b"][...] = layernorm_bwd(dh2, P[p + "ln2.w"], c["ln2"])
        dx = dx + dln
        # attention branch: x_mid = x_in + o Wa^T + ba
        G[p + "aproj.w"][...] = dx.reshape(-1, d).T @ c["o"].reshape(-1, d)
        G[p + "aproj.b"][...] = dx.reshape(-1, d).sum(axis=0)
        do = (dx @ P[p + "aproj.w"]).reshape(B, T, H, hs).transpose(0, 2, 1, 3)
        dq, dk, dv = causal_attention_bwd(do, c["q"], c["k"], c["v"], c["att_p"], c["z_att"])
        dqkv = np.concatenate([t.transpose(0, 2, 1, 3).reshape(B, T, d) for t in (dq, dk, dv)],
                              axis=-1)
        G[p + "attn.w"][...] = dqkv.reshape(-1, 3 * d).T @ c["h1"].reshape(-1, d)
        G[p + "attn.b"][...] = dqkv.reshape(-1, 3 * d).sum(axis=0)
        dh1 = dqkv @ P[p + "attn.w"]
        dln, G[p + "ln1.w"][...], G[p + "ln1.b"][...] = layernorm_bwd(dh1, P[p + "ln1.w"], c["ln1"])
        dx = dx + dln
    # embeddings: x = z * (wte[idx] + wpe[:T])
    if cache["z_emb"] is not None:
        dx = dx * cache["z_emb"]
    np.add.at(G["wte"], idx.reshape(-1), dx.reshape(-1, d))
    G["wpe"][:T] += dx.sum(axis=0)
    return grads


def loss_and_grads(flat_params, idx, targets, cfg: Config, loss_scale=1.0,
                   dtype=np.float64, dropout: Dropout | None = None):
    """One forward plus backward: (loss, flat grads, logits)."""
    logits, loss, cache = forward(flat_params, idx, targets, cfg, loss_scale, dtype, dropout)
    return loss, backward(cache, cfg, dtype), logits


def estimate_loss(flat_params, batches, cfg: Config, dtype=np.float64) -> float:
    """The eval gate's loss estimate ([NG] Part IV Stage 2): the model in eval
    mode (no dropout, no gradient), the mean of the per-batch mean losses over
    the given batches of one split."""
    return float(np.mean([forward(flat_params, idx, tgt, cfg, dtype=dtype)[1]
                          for idx, tgt in batches]))


# --------------------------------------------------------------------------
# the optimizer step
# --------------------------------------------------------------------------
def grad_norm(grads) -> float:
    """Global L2 norm over every gradient element, summed in float64."""
    g = np.asarray(grads, dtype=np.float64)
    return float(math.sqrt(float(np.dot(g, g))))


def clip_coef(norm: float, max_norm: float) -> float:
    """Global-norm clipping coefficient ([NG] Part IV Stage 5: the gradient is
    rescaled if its global norm exceeds 1.0).  Reading: min(1, max/(n+1e-6));
    max_norm <= 0 disables clipping."""
    if max_norm <= 0:
        return 1.0
    return min(1.0, max_norm / (norm + 1e-6))


def adamw(params, grads, m, v, mask, t, lr, beta1=0.9, beta2=0.95, eps=1e-8,
          weight_decay=0.1, coef=1.0):
    """One AdamW update ([YT] recipe: betas (0.9, 0.95), eps 1e-8, decay 0.1
    on 2-D tensors only; decoupled decay as named in [RC] glossary).

    Per element: g = coef*grad; m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
    p = p (1 - lr wd mask); p = p - lr * (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps).
    Returns new (params, m, v); the inputs are not modified.
    """
    g = grads * coef
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    p = params * (1.0 - lr * weight_decay * mask)
    p = p - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v


def get_lr(it: int, max_lr=6e-4, min_lr=None, warmup=715, decay_end=19073) -> float:
    """Learning rate at optimizer iteration `it` ([NG] Part IV Stage 1 and
    Deep dive 2; [SO] Section 3): linear warmup max*(it+1)/warmup, cosine
    decay from max to min between warmup and decay_end, min afterwards;
    min defaults to a tenth of the peak."""
    if min_lr is None:
        min_lr = 0.1 * max_lr
    if it < warmup:
        return max_lr * (it + 1) / warmup
    if it > decay_end:
        return min_lr
    ratio = (it - warmup) / (decay_end - warmup)
    return min_lr + 0.5 * (1.0 + math.cos(math.pi * ratio)) * (max_lr - min_lr)


def train_step(params, m, v, t, micro_batches, cfg: Config, lr, beta1=0.9,
               beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
               skip_nonfinite=False, dtype=np.float64):
    """One optimizer iteration ([NG] Part IV Stages 4-5).

    micro_batches: list of (idx, targets).  Each micro-loss is scaled by
    1/len(micro_batches) so the summed gradients are the mean ([YT] "Batch
    size by gradient accumulation"); then the global norm, clipping, AdamW.
    Returns dict(params, m, v, loss (mean of micro-losses), norm (pre-clip),
    grads (the accumulated, unclipped gradient)).
    """
    k = len(micro_batches)
    grads = np.zeros(num_params(cfg), dtype=dtype)
    losses = []
    for idx, tgt in micro_batches:
        loss, g, _ = loss_and_grads(params, idx, tgt, cfg, 1.0 / k, dtype)
        grads += g
        losses.append(loss)
    norm = grad_norm(grads)
    if skip_nonfinite and not math.isfinite(norm):
        return dict(params=params.copy(), m=m.copy(), v=v.copy(),
                    loss=float(np.mean(losses)), norm=norm, grads=grads)
    coef = clip_coef(norm, max_norm)
    p, m2, v2 = adamw(np.asarray(params, dtype), grads, np.asarray(m, dtype),
                      np.asarray(v, dtype), decay_mask(cfg, dtype), t, lr, beta1,
                      beta2, eps, weight_decay, coef)
    return dict(params=p, m=m2, v=v2, loss=float(np.mean(losses)), norm=norm,
                grads=grads)


# --------------------------------------------------------------------------
# float16 training: dynamic loss scaling
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class LossScaler:
    """State of the dynamic loss scale of float16 training ([NG] Part IV
    Stage 4 and Stage 5; Part V Deep dive 2; [RC] "Float16, Gradient Scalers,
    BF16").  scale multiplies the loss before the backward pass; growth_tracker
    counts clean steps since the scale last changed; steps counts the AdamW
    updates actually applied (a skipped step does not advance the bias
    correction, since the optimizer is not called)."""
    scale: float = 65536.0
    growth_tracker: int = 0
    steps: int = 0


def scaler_update(state: LossScaler, found_inf: bool, growth_factor=2.0,
                  backoff_factor=0.5, growth_interval=2000) -> LossScaler:
    """The scale after one step ([NG] Part IV Stage 5: an overflow shrinks the
    scale; the scale is adjusted for the next iteration).  Readings: the
    library defaults the pages' GradScaler is built with (growth 2, backoff
    0.5, growth every 2000 clean steps); a step with an overflow multiplies
    the scale by the backoff factor and restarts the count; the count reaching
    the interval multiplies it by the growth factor (kept only if finite) and
    restarts the count."""
    if found_inf:
        return LossScaler(state.scale * backoff_factor, 0, state.steps)
    clean = state.growth_tracker + 1
    if clean == growth_interval:
        grown = state.scale * growth_factor
        return LossScaler(grown if math.isfinite(grown) else state.scale, 0, state.steps + 1)
    return LossScaler(state.scale, clean, state.steps + 1)


def amp_step(params, scaled_grads, m, v, mask, state: LossScaler, lr, beta1=0.9,
             beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0, growth_factor=2.0,
             backoff_factor=0.5, growth_interval=2000):
    """The float16 optimizer step in the pages' order ([NG] Part IV Stage 5;
    Part VIII checks 6 and 7): unscale the gradients (multiply by 1/scale),
    clip against the norm of the unscaled gradients, apply AdamW unless an
    element is inf or NaN (then leave params, m and v as they are), update
    the scale.  Returns dict(params, m, v, norm (of the unscaled gradients),
    found_inf, state (the updated LossScaler))."""
    grads = np.asarray(scaled_grads) * (1.0 / state.scale)
    found_inf = not bool(np.all(np.isfinite(grads)))
    norm = grad_norm(grads)
    if found_inf:
        p, m2, v2 = params.copy(), m.copy(), v.copy()
    else:
        p, m2, v2 = adamw(params, grads, m, v, mask, state.steps + 1, lr, beta1, beta2, eps,
                          weight_decay, clip_coef(norm, max_norm))
    new = scaler_update(state, found_inf, growth_factor, backoff_factor, growth_interval)
    return dict(params=p, m=m2, v=v2, norm=norm, found_inf=found_inf, state=new)


def train_step_amp(params, m, v, state: LossScaler, micro_batches, cfg: Config, lr,
                   beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
                   growth_factor=2.0, backoff_factor=0.5, growth_interval=2000,
                   dtype=np.float64):
    """One float16-style iteration ([NG] Part IV Stages 4-5): every micro-loss
    is multiplied by scale / k before its backward pass (the scaled backward),
    the gradients accumulate, then amp_step.  Returns amp_step's dict plus
    loss (the mean of the unscaled micro-losses) and grads (the accumulated,
    still scaled gradient)."""
    k = len(micro_batches)
    grads = np.zeros(num_params(cfg), dtype=dtype)
    losses = []
    for idx, tgt in micro_batches:
        loss, g, _ = loss_and_grads(params, idx, tgt, cfg, state.scale / k, dtype)
        grads += g
        losses.append(loss)
    out = amp_step(np.asarray(params, dtype), grads, np.asarray(m, dtype), np.asarray(v, dtype),
                   decay_mask(cfg, dtype), state, lr, beta1, beta2, eps, weight_decay, max_norm,
                   growth_factor, backoff_factor, growth_interval)
    out.update(loss=float(np.mean(losses)), grads=grads)
    return out


def flops_per_token(cfg: Config, T: int) -> int:
    """Model FLOPs per token of [NG] Part IV Stage 6 (estimate_mfu):
    6N + 12*L*H*Q*T, N the non-embedding parameter count, Q the head width."""
    N = num_params(cfg, non_embedding=True)
    return 6 * N + 12 * cfg.n_layer * cfg.n_head * cfg.head_dim * T


# --------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------
def topk_sample(logits_row, vocab_size, temperature, top_k, u, dtype=np.float64):
    """One draw of GPT.generate ([NG] Part IV, "one generation (sample.py +
    model.py, generate)"): the last position's logits over the real
    vocabulary divided by the temperature; every logit below the top-k
    cutoff (the k-th largest value) removed, values equal to it kept;
    softmax; one multinomial draw.

    Readings: top_k <= 0 keeps every id (the pages' cutoff is optional);
    the draw is by inverse CDF in token-id order with the uniform u in
    [0, 1) supplied by the caller, i.e. the first id whose cumulative
    probability exceeds u (the pages name torch.multinomial, whose internal
    algorithm they do not give; every exact sampler has this distribution).
    Returns (token, probs over the first vocab_size ids).
    """
    z = np.asarray(logits_row, dtype=dtype)[:vocab_size] / dtype(temperature)
    if 0 < top_k < vocab_size:
        cutoff = np.sort(z)[vocab_size - top_k]  # the k-th largest
        z = np.where(z < cutoff, -np.inf, z)
    p = np.exp(z - z.max())
    p = p / p.sum()
    c = np.cumsum(p)
    tok = int(np.searchsorted(c, u, side="right"))
    return min(tok, vocab_size - 1), p


def generate(flat_params, idx, cfg: Config, n_new, temperature, top_k, us,
             dtype=np.float64):
    """GPT.generate of [NG] Part IV ("one generation"): per new token, crop
    the context to its last block_size tokens, run the whole forward (no
    cache), take the last position's logits and draw with topk_sample;
    append and repeat.  us: uniforms (B, n_new).  Returns (tokens (B,
    T0 + n_new), last-position logits (n_new, B, Vp))."""
    idx = np.asarray(idx)
    steps = []
    for i in range(n_new):
        ctx = idx[:, -cfg.block_size:]
        logits, _, _ = forward(flat_params, ctx, None, cfg, dtype=dtype)
        last = logits[:, -1, :]
        steps.append(last)
        nxt = [topk_sample(last[b], cfg.vocab_size, temperature, top_k, us[b, i], dtype)[0]
               for b in range(idx.shape[0])]
        idx = np.concatenate([idx, np.asarray(nxt, dtype=idx.dtype)[:, None]], axis=1)
    return idx, np.stack(steps)
