"""Step-level parity on the GPU through the C-ABI: gpt_forward_loss,
gpt_backward and gpt_adamw_step against the float64 CPU oracle on the same
seeded parameters and tokens.

Tolerances:
  * fp32 mode: logits within 1e-4 relative; gradients within 1e-4 relative
    per tensor; AdamW-updated weights within 1e-3 relative.
  * bf16 mode: loss within 2e-2 absolute; per-tensor gradient cosine >= 0.995.
  * AdamW itself: 1e-3 relative on identical synthetic inputs.
The key-bias slice of every attn.b (its gradient is zero in exact arithmetic,
since the softmax ignores a per-row constant) is left out of gradient
cosines and updated-weight comparisons: its sign is rounding noise on both
sides, and Adam's first step turns that noise into a full lr-sized move.
"""
import math

import numpy as np
import pytest

from oracle import gpt_oracle as O
from tests.helpers import case, cosine, max_rel, rel_err, to_np
from transformer_lm_02_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global bd
    from transformer_lm_02_amd import binding as bd_mod
    bd = bd_mod
    yield


def ocfg(dims):
    return O.Config(**{k: dims[k] for k in synth.MODEL_KEYS})


def kbias_mask(dims):
    """True for every element except the key-bias slices."""
    keep = np.ones(synth.n_params(dims), bool)
    offs = synth.tensor_offsets(dims)
    d = dims["n_embd"]
    for l in range(dims["n_layer"]):
        off, _ = offs[f"h{l}.attn.b"]
        keep[off + d:off + 2 * d] = False
    return keep


def per_tensor(dims, flat):
    offs = synth.tensor_offsets(dims)
    return {n: flat[o:o + int(np.prod(s))] for n, (o, s) in offs.items()}


def dev_tokens(idx, tgt):
    return torch.as_tensor(idx).cuda(), torch.as_tensor(tgt).cuda()


def check_grads(dims, got, ref, min_cos=None, max_rel_err=None):
    keep = kbias_mask(dims)
    G, R, K = per_tensor(dims, got), per_tensor(dims, ref), per_tensor(dims, keep)
    worst = []
    for n in G:
        g, r = G[n][K[n]], R[n][K[n]]
        if np.linalg.norm(r) == 0:
            assert np.abs(g).max() <= 1e-6, n
            continue
        if min_cos is not None:
            c = cosine(g, r)
            worst.append((c, n))
            assert c >= min_cos, (n, c)
        if max_rel_err is not None:
            e = rel_err(g, r)
            worst.append((-e, n))
            assert e <= max_rel_err, (n, e)
    return sorted(worst)[:3]


# ---------------------------------------------------------------- fp32 mode, tiny model
def test_tiny_fp32_full_step_parity():
    dims = synth.WORKLOADS["tiny"]
    case("tiny fp32 step B=4 T=64")
    params = synth.init_params(dims, seed=1337)
    idx, tgt = synth.tokens(dims, seed=1338)
    cfg = ocfg(dims)
    ref = O.train_step(params.astype(np.float64), np.zeros(params.size), np.zeros(params.size), 1,
                       [(idx, tgt)], cfg, lr=1e-3)
    ref_logits, ref_loss, _ = O.forward(params, idx, tgt, cfg)

    m = bd.GPT(dims, bd.GPT_FP32, max_batch=4, init_params=params)
    di, dt = dev_tokens(idx, tgt)
    loss, logits = m.forward(di, dt, logits=True)
    m.backward(zero_first=True)
    norm = m.adamw_step(lr=1e-3, t=1)
    torch.cuda.synchronize()
    got_logits = to_np(logits)
    V = dims["vocab_size"]
    assert rel_err(got_logits[..., :V], ref_logits[..., :V]) <= 1e-4
    assert max_rel(got_logits[..., :V], ref_logits[..., :V]) <= 1e-4
    assert abs(float(loss.item()) - ref_loss) <= 1e-5
    check_grads(dims, to_np(m.grads), ref["grads"], max_rel_err=1e-4)
    assert abs(float(norm.item()) - ref["norm"]) <= 1e-5 * ref["norm"]
    keep = kbias_mask(dims)
    got_p = to_np(m.params)
    assert rel_err(got_p[keep], ref["params"][keep]) <= 1e-3
    for n, g in per_tensor(dims, got_p).items():
        r = per_tensor(dims, ref["params"])[n]
        k = per_tensor(dims, keep)[n]
        assert rel_err(g[k], r[k]) <= 1e-3, n
    m.close()


@pytest.mark.parametrize("pattern", ["one_id", "two_ids", "cycle"])
def test_tiny_fp32_embedding_gradient_repeated_ids(pattern):
    """The embedding backward adds the rows of each id inside a workgroup of
    256 rows (runs of at most 16 rows per wave) before its atomic adds:
    three workgroups of one repeated id, of two alternating ids, and of ids
    cycling through the vocabulary, against the oracle's gradients at 1e-4."""
    dims = synth.WORKLOADS["tiny"]
    B, T, V = 12, dims["block_size"], dims["vocab_size"]
    case(f"tiny fp32 embedding gradient tokens={pattern} B={B} T={T}")
    params = synth.perturbed_params(dims, seed=51)
    n = np.arange(B * T).reshape(B, T)
    idx = {"one_id": np.full((B, T), 7), "two_ids": 3 + 50 * (n % 2), "cycle": n % V}[pattern]
    idx = idx.astype(np.int32)
    tgt = np.random.default_rng(52).integers(0, V, size=(B, T)).astype(np.int32)
    _, ref_g, _ = O.loss_and_grads(params, idx, tgt, ocfg(dims))
    m = bd.GPT(dims, bd.GPT_FP32, max_batch=B, init_params=params)
    m.forward(*dev_tokens(idx, tgt))
    m.backward(zero_first=True)
    torch.cuda.synchronize()
    check_grads(dims, to_np(m.grads), ref_g, max_rel_err=1e-4)
    m.close()


def test_tiny_fp32_gradient_accumulation():
    dims = synth.WORKLOADS["tiny"]
    case("tiny fp32 accumulation 4 x B=1")
    params = synth.perturbed_params(dims, seed=5)
    idx, tgt = synth.tokens(dims, seed=6)
    _, ref_g, _ = O.loss_and_grads(params, idx, tgt, ocfg(dims))
    m = bd.GPT(dims, bd.GPT_FP32, max_batch=4, init_params=params)
    for i in range(4):
        di, dt = dev_tokens(idx[i:i + 1], tgt[i:i + 1])
        m.forward(di, dt, loss_scale=0.25)
        m.backward(zero_first=(i == 0))
    torch.cuda.synchronize()
    check_grads(dims, to_np(m.grads), ref_g, max_rel_err=1e-4)
    m.close()


def test_tiny_fp32_ignored_targets_and_short_sequence():
    dims = synth.WORKLOADS["tiny"]
    case("tiny fp32 B=3 T=37 with ignored targets")
    params = synth.perturbed_params(dims, seed=7)
    idx, tgt = synth.tokens(dims, seed=8, batch=3, T=37)
    tgt[0, :5] = -1
    tgt[2, 30] = -1
    ref_loss, ref_g, ref_logits = O.loss_and_grads(params, idx, tgt, ocfg(dims))
    m = bd.GPT(dims, bd.GPT_FP32, max_batch=4, init_params=params)
    loss, logits = m.forward(*dev_tokens(idx, tgt), logits=True)
    m.backward()
    torch.cuda.synchronize()
    assert abs(float(loss.item()) - ref_loss) <= 1e-5
    assert rel_err(to_np(logits), ref_logits) <= 1e-4
    check_grads(dims, to_np(m.grads), ref_g, max_rel_err=1e-4)
    m.close()


# ---------------------------------------------------------------- bf16 mode
def bf16_step_parity(name, batch, T=None, seed=0, **override):
    dims = dict(synth.WORKLOADS[name], **override)
    T = T or dims["block_size"]
    case(f"{name} bf16 step B={batch} T={T}")
    params = synth.init_params(dims, seed=1337 + seed)
    idx, tgt = synth.tokens(dims, seed=1338 + seed, batch=batch, T=T)
    ref_loss, ref_g, _ = O.loss_and_grads(params, idx, tgt, ocfg(dims))
    m = bd.GPT(dims, bd.GPT_BF16, max_batch=batch, init_params=params)
    loss, _ = m.forward(*dev_tokens(idx, tgt))
    m.backward()
    torch.cuda.synchronize()
    got_loss = float(loss.item())
    assert abs(got_loss - ref_loss) <= 2e-2, (got_loss, ref_loss)
    worst = check_grads(dims, to_np(m.grads), ref_g, min_cos=0.995)
    print(f"loss gpu {got_loss:.5f} oracle {ref_loss:.5f}; lowest cosines {worst}", flush=True)
    m.close()


def test_char_bf16_step_parity_full_batch():
    bf16_step_parity("char", batch=64)


def test_gpt2_bf16_step_parity_two_sequences():
    bf16_step_parity("gpt2", batch=2)


def test_gpt2_bf16_ragged_short_batch():
    bf16_step_parity("gpt2", batch=3, T=200, seed=4)


def test_gpt2_1p5b_width_two_layers_bf16_parity():
    """The 1.5B shape's layer width (d 1600, 25 heads of 64, MLP 6400, padded
    vocabulary) with two layers: every per-layer kernel at that shape; depth
    only repeats them."""
    bf16_step_parity("gpt2_1p5b", batch=1, T=256, seed=6, n_layer=2)


def test_gpt2_bf16_gradient_accumulation():
    """Two micro-batches with loss scale 1/2, the second accumulating into
    the first's gradients, against the oracle on the two sequences as one
    batch ("Let's reproduce GPT-2 (124M)", chapter "Gradient Accumulation")."""
    dims = synth.WORKLOADS["gpt2"]
    case("gpt2 bf16 accumulation 2 x B=1 T=128")
    params = synth.init_params(dims, seed=1341)
    idx, tgt = synth.tokens(dims, seed=1342, batch=2, T=128)
    ref_loss, ref_g, _ = O.loss_and_grads(params, idx, tgt, ocfg(dims))
    m = bd.GPT(dims, bd.GPT_BF16, max_batch=1, init_params=params)
    losses = []
    for i in range(2):
        loss, _ = m.forward(*dev_tokens(idx[i:i + 1], tgt[i:i + 1]), loss_scale=0.5)
        losses.append(float(loss.item()))
        m.backward(zero_first=(i == 0))
    torch.cuda.synchronize()
    assert abs(0.5 * sum(losses) - ref_loss) <= 2e-2, (losses, ref_loss)
    worst = check_grads(dims, to_np(m.grads), ref_g, min_cos=0.995)
    print(f"lowest cosines {worst}", flush=True)
    m.close()


def test_gpt2_full_batch_sampled_logits_and_properties():
    """The benchmark's launch configuration (B=16, T=1024): logits of sampled
    sequences against the oracle run on those sequences alone (the forward
    treats sequences independently), loss in the initial-loss band, and a
    bit-identical second forward."""
    dims = synth.WORKLOADS["gpt2"]
    case("gpt2 bf16 B=16 T=1024 sampled sequences")
    params = synth.init_params(dims, seed=1337)
    idx, tgt = synth.tokens(dims, seed=1338)
    m = bd.GPT(dims, bd.GPT_BF16, max_batch=16, init_params=params)
    di, dt = dev_tokens(idx, tgt)
    loss, logits = m.forward(di, dt, logits=True)
    torch.cuda.synchronize()
    lg = logits.clone()
    V = dims["vocab_size"]
    lnv = math.log(V)
    assert lnv - 0.1 <= float(loss.item()) <= lnv + 2e-4 * 768 + 0.1
    for b in (0, 11):
        ref, _, _ = O.forward(params, idx[b:b + 1], tgt[b:b + 1], ocfg(dims))
        got = to_np(lg[b, :, :V])
        assert cosine(got, ref[0, :, :V]) >= 0.999
        assert rel_err(got, ref[0, :, :V]) <= 3e-2
    _, logits2 = m.forward(di, dt, logits=True)
    torch.cuda.synchronize()
    assert torch.equal(lg, logits2)
    m.backward()
    norm = m.adamw_step(lr=6e-4, t=1)
    torch.cuda.synchronize()
    assert math.isfinite(float(norm.item()))
    m.close()


def test_bf16_causal_invariance_bit_identical():
    dims = synth.WORKLOADS["char"]
    case("char bf16 causal bit-identity B=4 T=256")
    params = synth.perturbed_params(dims, seed=3)
    idx, tgt = synth.tokens(dims, seed=4, batch=4)
    m = bd.GPT(dims, bd.GPT_BF16, max_batch=4, init_params=params)
    _, l0 = m.forward(*dev_tokens(idx, tgt), logits=True)
    l0 = l0.clone()
    rng = np.random.default_rng(5)
    for t in (0, 100, 200):
        idx2, tgt2 = idx.copy(), tgt.copy()
        idx2[:, t + 1:] = rng.integers(0, 65, idx2[:, t + 1:].shape)
        _, l1 = m.forward(*dev_tokens(idx2, tgt2), logits=True)
        torch.cuda.synchronize()
        assert torch.equal(l0[:, :t + 1], l1[:, :t + 1])
        assert not torch.equal(l0[:, t + 1:], l1[:, t + 1:])
    m.close()


# ---------------------------------------------------------------- AdamW on identical inputs
@pytest.mark.parametrize("max_norm,scale", [(1.0, 1e-3), (1.0, 1.0), (0.0, 1e-2)])
def test_adamw_kernel_matches_oracle(max_norm, scale):
    dims = synth.WORKLOADS["char"]
    case(f"adamw char params max_norm={max_norm} grad scale={scale}")
    n = synth.n_params(dims)
    params = synth.perturbed_params(dims, seed=11)
    rng = np.random.default_rng(12)
    m0 = rng.standard_normal(n).astype(np.float32) * np.float32(1e-3)
    v0 = (rng.standard_normal(n).astype(np.float32) * np.float32(1e-3)) ** 2
    g = synth.synthetic_grads(n, seed=13, scale=scale)
    t, lr = 3, 6e-4
    norm = O.grad_norm(g.astype(np.float64))
    coef = O.clip_coef(norm, max_norm)
    mask = O.decay_mask(ocfg(dims))
    ref_p, ref_m, ref_v = O.adamw(params.astype(np.float64), g.astype(np.float64),
                                  m0.astype(np.float64), v0.astype(np.float64), mask, t, lr,
                                  coef=coef)
    mdl = bd.GPT(dims, bd.GPT_BF16, max_batch=1, init_params=params)
    mdl.grads.copy_(torch.as_tensor(g))
    mdl.adam_m.copy_(torch.as_tensor(m0))
    mdl.adam_v.copy_(torch.as_tensor(v0))
    got_norm = mdl.adamw_step(lr=lr, t=t, max_norm=max_norm)
    torch.cuda.synchronize()
    assert abs(float(got_norm.item()) - norm) <= 1e-5 * norm
    assert rel_err(to_np(mdl.params), ref_p) <= 1e-3
    assert max_rel(to_np(mdl.params) - params, ref_p - params) <= 1e-3
    assert rel_err(to_np(mdl.adam_m), ref_m) <= 1e-5
    assert rel_err(to_np(mdl.adam_v), ref_v) <= 1e-5
    assert np.array_equal(to_np(mdl.grads), g.astype(np.float64))  # grads untouched
    mdl.close()


def test_adamw_skips_nonfinite_gradients():
    dims = synth.WORKLOADS["tiny"]
    case("adamw skip on non-finite norm")
    params = synth.perturbed_params(dims, seed=14)
    mdl = bd.GPT(dims, bd.GPT_FP32, max_batch=1, init_params=params)
    g = synth.synthetic_grads(params.size, seed=15)
    g[123] = np.inf
    mdl.grads.copy_(torch.as_tensor(g))
    norm = mdl.adamw_step(lr=1e-3, t=1, skip_nonfinite=True)
    torch.cuda.synchronize()
    assert not math.isfinite(float(norm.item()))
    assert np.array_equal(to_np(mdl.params), params.astype(np.float64))
    assert float(mdl.adam_m.abs().max().item()) == 0.0
    mdl.close()


# ---------------------------------------------------------------- error paths
def test_error_paths_and_bad_token_flag():
    dims = synth.WORKLOADS["tiny"]
    case("error paths tiny fp32")
    params = synth.init_params(dims, seed=1)
    m = bd.GPT(dims, bd.GPT_FP32, max_batch=2, init_params=params)
    with pytest.raises(bd.GptError) as e:
        m.backward()
    assert e.value.code == bd.GPT_ESTATE
    idx, tgt = synth.tokens(dims, seed=2, batch=2)
    long_idx = torch.zeros((2, 65), dtype=torch.int32, device="cuda")
    with pytest.raises(bd.GptError) as e:
        m.forward(long_idx, long_idx)
    assert e.value.code == bd.GPT_ESEQLEN
    with pytest.raises(bd.GptError) as e:
        m.forward(torch.zeros((3, 8), dtype=torch.int32, device="cuda"))
    assert e.value.code == bd.GPT_EINVAL
    idx[1, 7] = 9999  # outside [0, 65)
    loss, _ = m.forward(*dev_tokens(idx, tgt))
    assert m.read_flags() == bd.GPT_FLAG_BAD_TOKEN
    assert math.isfinite(float(loss.item()))
    assert m.read_flags() == 0
    m.close()
