"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random numbers and lays them out; it holds none of the
model's arithmetic.  Both the HIP path and the CPU oracle receive what it
produces, so neither side's result can leak into the other's inputs.

Workloads (sizes as the pages give them):
  * "tiny"   vocab 65, T 64, 2 layers, 4 heads, width 64, batch 4 - uniform ids.
  * "char"   vocab 65, T 256, 6 layers, 6 heads, width 384, batch 64 - the
             Shakespeare-char model of "nanoGPT" (stanleyjacob.dev) Part II,
             uniform ids standing in for the 65-character corpus.
  * "gpt2"   GPT-2 124M: vocab 50257 padded to 50304, T 1024, 12 layers,
             12 heads, width 768, micro-batch 16 ("Let's reproduce GPT-2
             (124M)", Speed Stack chapters) - Zipf(1.1) ids standing in for
             FineWeb-Edu BPE tokens.
  * "gpt2_1p5b"  the 1.5B shape: width 1600, 48 layers, 25 heads, batch 8.
Targets are the inputs shifted by one token ("nanoGPT", Part IV Stage 3).
"""
from __future__ import annotations

import math

import numpy as np

WORKLOADS = {
    "tiny": dict(vocab_size=65, padded_vocab=65, block_size=64, n_layer=2,
                 n_head=4, n_embd=64, batch=4, tokens="uniform"),
    "char": dict(vocab_size=65, padded_vocab=65, block_size=256, n_layer=6,
                 n_head=6, n_embd=384, batch=64, tokens="uniform"),
    "gpt2": dict(vocab_size=50257, padded_vocab=50304, block_size=1024,
                 n_layer=12, n_head=12, n_embd=768, batch=16, tokens="zipf"),
    "gpt2_1p5b": dict(vocab_size=50257, padded_vocab=50304, block_size=1024,
                      n_layer=48, n_head=25, n_embd=1600, batch=8, tokens="zipf"),
}

MODEL_KEYS = ("vocab_size", "padded_vocab", "block_size", "n_layer", "n_head", "n_embd")


def model_dims(workload: dict) -> dict:
    return {k: workload[k] for k in MODEL_KEYS}


def uniform_tokens(batch: int, T: int, vocab: int, seed: int):
    """(idx, targets) int32 [batch, T]: ids uniform in [0, vocab)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(0, vocab, size=(batch, T + 1))
    return a[:, :T].astype(np.int32), a[:, 1:].astype(np.int32)


def zipf_tokens(batch: int, T: int, vocab: int, seed: int, s: float = 1.1):
    """(idx, targets) int32 [batch, T]: ids with P(id = i) proportional to
    (i + 1)^-s over [0, vocab), drawn by inverse CDF."""
    rng = np.random.default_rng(seed)
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(size=(batch, T + 1))
    a = np.minimum(np.searchsorted(cdf, u, side="right"), vocab - 1)
    return a[:, :T].astype(np.int32), a[:, 1:].astype(np.int32)


def tokens(workload: dict, seed: int, batch: int | None = None, T: int | None = None):
    batch = workload["batch"] if batch is None else batch
    T = workload["block_size"] if T is None else T
    if workload["tokens"] == "zipf":
        return zipf_tokens(batch, T, workload["vocab_size"], seed)
    return uniform_tokens(batch, T, workload["vocab_size"], seed)


def _tensor_list(dims: dict):
    """Canonical parameter order with each tensor's kind:
    'emb' (embedding table), 'w' (linear weight), 'wres' (linear weight that
    writes into the residual stream), 'b' (bias), 'g' (LayerNorm gain),
    'beta' (LayerNorm shift)."""
    d, L = dims["n_embd"], dims["n_layer"]
    out = [("wte", (dims["padded_vocab"], d), "emb"), ("wpe", (dims["block_size"], d), "emb")]
    for l in range(L):
        out += [
            (f"h{l}.ln1.w", (d,), "g"), (f"h{l}.ln1.b", (d,), "beta"),
            (f"h{l}.attn.w", (3 * d, d), "w"), (f"h{l}.attn.b", (3 * d,), "b"),
            (f"h{l}.aproj.w", (d, d), "wres"), (f"h{l}.aproj.b", (d,), "b"),
            (f"h{l}.ln2.w", (d,), "g"), (f"h{l}.ln2.b", (d,), "beta"),
            (f"h{l}.fc.w", (4 * d, d), "w"), (f"h{l}.fc.b", (4 * d,), "b"),
            (f"h{l}.mproj.w", (d, 4 * d), "wres"), (f"h{l}.mproj.b", (d,), "b"),
        ]
    out += [("lnf.w", (d,), "g"), ("lnf.b", (d,), "beta")]
    return out


def n_params(dims: dict) -> int:
    return sum(int(np.prod(s)) for _, s, _ in _tensor_list(dims))


def init_params(dims: dict, seed: int, dtype=np.float32, std: float = 0.02) -> np.ndarray:
    """Flat initial parameters: N(0, std) for embeddings and linear weights,
    N(0, std / sqrt(2 * n_layer)) for the two projections per block that write
    into the residual stream, zero biases, LayerNorm gain 1 and shift 0
    ("Let's reproduce GPT-2 (124M)", chapter "Model Initialization")."""
    rng = np.random.default_rng(seed)
    parts = []
    res_std = std / math.sqrt(2 * dims["n_layer"])
    for _, shape, kind in _tensor_list(dims):
        n = int(np.prod(shape))
        if kind in ("emb", "w"):
            parts.append(rng.standard_normal(n, dtype=np.float32) * np.float32(std))
        elif kind == "wres":
            parts.append(rng.standard_normal(n, dtype=np.float32) * np.float32(res_std))
        elif kind == "g":
            parts.append(np.ones(n, np.float32))
        else:
            parts.append(np.zeros(n, np.float32))
    return np.concatenate(parts).astype(dtype)


def perturbed_params(dims: dict, seed: int, scale: float = 0.02) -> np.ndarray:
    """Like init_params but with every tensor (biases and LayerNorm affine
    included) perturbed, so that gradient checks exercise all terms."""
    rng = np.random.default_rng(seed + 7919)
    p = init_params(dims, seed)
    return (p + rng.standard_normal(p.size).astype(np.float32) * np.float32(scale)).astype(np.float32)


def synthetic_grads(n: int, seed: int, scale: float = 1e-3) -> np.ndarray:
    """Gradient-like float32 vector (heavy-tailed) for optimizer-only checks."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(n).astype(np.float32) * np.float32(scale)
    g *= np.exp(rng.standard_normal(n) * 1.5).astype(np.float32)
    return g.astype(np.float32)


def tensor_offsets(dims: dict) -> dict:
    """name -> (offset, shape) in the flat parameter vector."""
    out, off = {}, 0
    for name, shape, _ in _tensor_list(dims):
        out[name] = (off, shape)
        off += int(np.prod(shape))
    return out
