"""Float16 training with dynamic loss scaling on the GPU through the C-ABI
(GPT_FP16 mode, gpt_forward_loss_scaled, gpt_amp_step) against the float64
CPU oracle.

Tolerances:
  * single ops in binary16: as their bf16 counterparts, or tighter where the
    format's 11-bit significand allows (stated per test);
  * a loss-scaled step: loss within 1e-2 absolute; per-tensor cosine of the
    unscaled gradients (grads / scale) >= 0.998;
  * gpt_amp_step on identical inputs: the scale, the growth count, the
    update count and the skip flag exactly; the norm within 1e-5 relative;
    parameters within 1e-3 relative (AdamW's fp32 rounding, as for
    gpt_adamw_step); a skipped step leaves params, m and v bit-identical;
  * fp32 mode under a power-of-two scale: the oracle's float16-style
    iteration (train_step_amp) within the fp32 step tolerances.
"""
import math

import numpy as np
import pytest

from oracle import gpt_oracle as O
from tests.helpers import case, cosine, max_rel, rel_err, to_dev, to_np
from tests.test_gpu_step import check_grads, dev_tokens, kbias_mask, ocfg, per_tensor
from transformer_lm_02_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global bd
    from transformer_lm_02_amd import binding as bd_mod
    bd = bd_mod
    yield


def f16_round(a):
    """Round to IEEE binary16 (nearest-even) and return float64."""
    return np.asarray(a, np.float32).astype(np.float16).astype(np.float64)


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(scale)


# ---------------------------------------------------------------- single ops in binary16
@pytest.mark.parametrize("M,N,K", [(256, 2304, 768), (300, 200, 136), (129, 50304, 768),
                                   (1000, 768, 3072)])
def test_linear_family_fp16(M, N, K):
    case(f"linear family fp16 M={M} N={N} K={K}")
    A, B = f16_round(rnd((M, K), 1)), f16_round(rnd((N, K), 2, 0.05))
    bias = rnd(N, 3)
    ref = A @ B.T + bias
    Ad, Bd = to_dev(A, torch.float16), to_dev(B, torch.float16)
    got = to_np(bd.op_linear(Ad, Bd, torch.as_tensor(bias).cuda(), out_f32=True))
    assert rel_err(got, ref) < 1e-5 and max_rel(got, ref) < 1e-4
    got16 = to_np(bd.op_linear(Ad, Bd, torch.as_tensor(bias).cuda(), out_f32=False))
    assert max_rel(got16, ref) < 1e-3  # one binary16 rounding of the output
    dY = f16_round(rnd((M, N), 4, 0.01))
    dYd = to_dev(dY, torch.float16)
    got = to_np(bd.op_linear_dw(dYd, Ad))
    assert rel_err(got, dY.T @ A) < 1e-5
    got = to_np(bd.op_linear_dx(dYd, Bd))
    assert rel_err(got, dY @ B) < 1e-5


def split_heads(qkv, B, T, H):
    C = qkv.shape[1] // 3
    hs = C // H
    return [qkv[:, i * C:(i + 1) * C].reshape(B, T, H, hs).transpose(0, 2, 1, 3) for i in range(3)]


def merge_heads(x):
    B, H, T, hs = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B * T, H * hs)


@pytest.mark.parametrize("B,T,H,hs", [(2, 256, 3, 64), (1, 200, 2, 64), (3, 65, 1, 64),
                                      (2, 96, 2, 32)])
def test_attention_fwd_bwd_fp16(B, T, H, hs):
    """binary16 probabilities carry 3 more significand bits than bfloat16:
    the output within 5e-3 of the largest (bf16: 2e-2)."""
    case(f"attention fp16 B={B} T={T} H={H} hs={hs}")
    C = H * hs
    qkv = f16_round(rnd((B * T, 3 * C), 12))
    q, k, v = split_heads(qkv, B, T, H)
    ref_o, ref_p = O.causal_attention_fwd(q, k, v)
    qd = to_dev(qkv, torch.float16)
    out, lse = bd.op_attention_fwd(qd, B, T, H)
    assert max_rel(to_np(out), merge_heads(ref_o)) < 5e-3
    dout = f16_round(rnd((B * T, C), 13))
    do = dout.reshape(B, T, H, hs).transpose(0, 2, 1, 3)
    ref_d = np.concatenate([merge_heads(t) for t in O.causal_attention_bwd(do, q, k, v, ref_p)], 1)
    got_d = to_np(bd.op_attention_bwd(qd, out, lse, to_dev(dout, torch.float16), B, T, H))
    for i, name in enumerate("qkv"):
        g, r = got_d[:, i * C:(i + 1) * C], ref_d[:, i * C:(i + 1) * C]
        assert cosine(g, r) > 0.9999, name
        assert rel_err(g, r) < 8e-3, name


def test_layernorm_and_cross_entropy_fp16():
    case("layernorm fp16 M=1000 C=768; cross-entropy fp16 N=512 V=50257")
    x = rnd((1000, 768), 16, 3.0) + 1.0
    w, b = rnd(768, 17) + 1.0, rnd(768, 18)
    ref, _ = O.layernorm_fwd(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    y, _, _ = bd.op_layernorm_fwd(torch.as_tensor(x).cuda(), torch.as_tensor(w).cuda(),
                                  torch.as_tensor(b).cuda(), fp16=True)
    assert y.dtype == torch.float16 and max_rel(to_np(y), ref) < 1e-3
    N, V, ldv = 512, 50257, 50304
    z = f16_round(rnd((N, ldv), 19, 2.0))
    tgt = np.random.default_rng(20).integers(0, V, N).astype(np.int32)
    tgt[::17] = -1
    # a loss scale that keeps the gradients in binary16's normal range
    loss_ref, dz_ref = O.cross_entropy(z, tgt, V, loss_scale=4096.0)
    zd = to_dev(z, torch.float16)
    loss, _, nv = bd.op_cross_entropy(zd, torch.as_tensor(tgt).cuda(), V, loss_scale=4096.0)
    assert int(nv.item()) == int((tgt >= 0).sum())
    assert abs(float(loss.item()) - loss_ref) < 1e-4 * loss_ref
    got = to_np(zd)
    assert np.all(got[:, V:] == 0)
    assert max_rel(got, dz_ref) < 2e-3


# ---------------------------------------------------------------- loss-scaled steps
def scaled_step(m, idx, tgt, scale, loss_scale=1.0):
    m.init_scaler(scale)
    loss, _ = m.forward(*dev_tokens(idx, tgt), loss_scale=loss_scale, scaled=True)
    m.backward()
    torch.cuda.synchronize()
    return float(loss.item()), to_np(m.grads) / scale


@pytest.mark.parametrize("name,batch,T", [("char", 64, None), ("gpt2", 2, None),
                                          ("gpt2", 3, 200)])
def test_fp16_scaled_step_parity(name, batch, T):
    dims = synth.WORKLOADS[name]
    T = T or dims["block_size"]
    case(f"{name} fp16 loss-scaled step B={batch} T={T} scale 2^16")
    params = synth.init_params(dims, seed=1337)
    idx, tgt = synth.tokens(dims, seed=1338, batch=batch, T=T)
    ref_loss, ref_g, _ = O.loss_and_grads(params, idx, tgt, ocfg(dims))
    m = bd.GPT(dims, bd.GPT_FP16, max_batch=batch, init_params=params)
    loss, g = scaled_step(m, idx, tgt, 65536.0)
    assert abs(loss - ref_loss) <= 1e-2, (loss, ref_loss)
    worst = check_grads(dims, g, ref_g, min_cos=0.998)
    print(f"loss gpu {loss:.5f} oracle {ref_loss:.5f}; lowest cosines {worst}", flush=True)
    m.close()


def test_fp16_small_gradients_need_the_scale():
    """A loss multiplied by 2^-14 (as under a long accumulation) over 2048
    tokens: every logit gradient is at most 2^-25, half of binary16's
    smallest subnormal, so without a loss scale they all round to zero and
    every gradient vanishes; a scale of 2^16 brings them back into range and
    the unscaled result matches the oracle ("nanoGPT", Part V Deep dive 2:
    small float16 gradients underflow to zero)."""
    dims = synth.WORKLOADS["char"]
    case("char fp16 loss 2^-14 with and without scale B=8")
    params = synth.init_params(dims, seed=3)
    idx, tgt = synth.tokens(dims, seed=4, batch=8)
    ls = 2.0 ** -14
    _, ref_g, _ = O.loss_and_grads(params, idx, tgt, ocfg(dims), loss_scale=ls)
    m = bd.GPT(dims, bd.GPT_FP16, max_batch=8, init_params=params)
    _, g1 = scaled_step(m, idx, tgt, 1.0, loss_scale=ls)
    _, g2 = scaled_step(m, idx, tgt, 65536.0, loss_scale=ls)
    keep = kbias_mask(dims)
    lost = np.linalg.norm(g1[keep]) / np.linalg.norm(ref_g[keep])
    assert lost == 0.0, lost
    assert cosine(g2[keep], ref_g[keep]) >= 0.998
    assert abs(np.linalg.norm(g2[keep]) / np.linalg.norm(ref_g[keep]) - 1) < 1e-2
    print(f"norm ratio without scale {lost:.3e}", flush=True)
    m.close()


def test_fp16_overflow_skips_the_step_and_backs_off():
    """A scale of 2^40 overflows binary16 in the backward pass: the step is
    skipped (params, m and v bit-identical), the scale halves, no update is
    counted; the following step at 2^16 is clean and counted."""
    dims = synth.WORKLOADS["char"]
    case("char fp16 overflow at scale 2^40 B=4")
    params = synth.init_params(dims, seed=5)
    idx, tgt = synth.tokens(dims, seed=6, batch=4)
    m = bd.GPT(dims, bd.GPT_FP16, max_batch=4, init_params=params)
    m.init_scaler(2.0 ** 40)
    m.forward(*dev_tokens(idx, tgt), scaled=True)
    m.backward()
    p0 = to_np(m.params)
    norm = m.amp_step(lr=1e-3)
    torch.cuda.synchronize()
    assert not math.isfinite(float(norm.item()))
    assert m.scaler_state() == (2.0 ** 39, 0, 0, 1)
    assert np.array_equal(to_np(m.params), p0)
    assert float(m.adam_m.abs().max().item()) == 0.0 and float(m.adam_v.abs().max().item()) == 0.0
    m.init_scaler(65536.0, 0, 0)
    m.forward(*dev_tokens(idx, tgt), scaled=True)
    m.backward()
    norm = m.amp_step(lr=1e-3)
    torch.cuda.synchronize()
    assert math.isfinite(float(norm.item()))
    assert m.scaler_state() == (65536.0, 1, 1, 0)
    assert not np.array_equal(to_np(m.params), p0)
    m.close()


def test_amp_step_kernel_matches_oracle_over_a_sequence():
    """Identical scaled gradients on both sides for six steps with growth
    every 2 clean steps, an inf planted at step 3 and a NaN at step 6,
    gradient sizes below and above the clip threshold."""
    dims = synth.WORKLOADS["char"]
    case("amp_step char params six steps")
    n = synth.n_params(dims)
    p = synth.perturbed_params(dims, seed=21).astype(np.float64)
    mask = O.decay_mask(ocfg(dims))
    m_ref, v_ref = np.zeros(n), np.zeros(n)
    st = O.LossScaler()
    mdl = bd.GPT(dims, bd.GPT_BF16, max_batch=1, init_params=p.astype(np.float32))
    # the global norm is about 3.1e4 times the size: steps 1 and 4 stay below
    # the clip threshold of 1, the others are clipped
    sizes = [1e-5, 1e-4, 1e-5, 2e-5, 1e-3, 1e-5]
    for i, sz in enumerate(sizes):
        g = synth.synthetic_grads(n, seed=30 + i, scale=sz).astype(np.float64)
        gs = (g * st.scale).astype(np.float32)
        if i == 2:
            gs[1234] = np.inf
        if i == 5:
            gs[n - 7] = np.nan
        ref = O.amp_step(p, gs.astype(np.float64), m_ref, v_ref, mask, st, 6e-4, growth_interval=2)
        mdl.grads.copy_(torch.as_tensor(gs))
        norm = float(mdl.amp_step(lr=6e-4, growth_interval=2).item())
        torch.cuda.synchronize()
        st = ref["state"]
        assert mdl.scaler_state() == (st.scale, st.growth_tracker, st.steps, int(ref["found_inf"])), i
        if ref["found_inf"]:
            assert not math.isfinite(norm)
        else:
            assert abs(norm - ref["norm"]) <= 1e-5 * ref["norm"], i
        p, m_ref, v_ref = ref["params"], ref["m"], ref["v"]
        assert rel_err(to_np(mdl.params), p) <= 1e-3, i
        assert rel_err(to_np(mdl.adam_m), m_ref) <= 1e-5, i
        assert rel_err(to_np(mdl.adam_v), v_ref) <= 1e-5, i
    assert st.steps == 4 and st.scale == 65536.0
    mdl.close()


def test_fp32_mode_three_loss_scaled_iterations_match_oracle():
    """The whole float16-style iteration through the library (scaled
    forward, backward, gpt_amp_step) in fp32 mode, where a power-of-two
    scale is exact: three iterations with growth every 2 clean steps
    against the oracle's train_step_amp; the scale doubles after the second."""
    dims = synth.WORKLOADS["tiny"]
    case("tiny fp32 three loss-scaled iterations")
    params = synth.init_params(dims, seed=1337)
    p = params.astype(np.float64)
    m_ref, v_ref = np.zeros(p.size), np.zeros(p.size)
    st = O.LossScaler()
    mdl = bd.GPT(dims, bd.GPT_FP32, max_batch=4, init_params=params)
    for it in range(3):
        idx, tgt = synth.tokens(dims, seed=1338 + it)
        ref = O.train_step_amp(p, m_ref, v_ref, st, [(idx, tgt)], ocfg(dims), lr=1e-3,
                               growth_interval=2)
        loss, _ = mdl.forward(*dev_tokens(idx, tgt), scaled=True)
        mdl.backward()
        norm = float(mdl.amp_step(lr=1e-3, growth_interval=2).item())
        torch.cuda.synchronize()
        assert abs(float(loss.item()) - ref["loss"]) <= 1e-5
        assert abs(norm - ref["norm"]) <= 1e-5 * ref["norm"]
        st = ref["state"]
        assert mdl.scaler_state() == (st.scale, st.growth_tracker, st.steps, 0)
        p, m_ref, v_ref = ref["params"], ref["m"], ref["v"]
        keep = kbias_mask(dims)
        assert rel_err(to_np(mdl.params)[keep], p[keep]) <= 1e-3, it
    assert st.scale == 131072.0 and st.steps == 3
    mdl.close()


# ---------------------------------------------------------------- sampling in fp16 mode
def test_fp16_prefill_and_decode_logits_match_oracle():
    dims = dict(vocab_size=300, padded_vocab=320, block_size=48, n_layer=2, n_head=2, n_embd=128)
    case("fp16 decode parity B=2 T0=5 +4")
    params = synth.perturbed_params(dims, seed=11)
    B, T0, n = 2, 5, 4
    seq = np.random.default_rng(12).integers(0, 300, size=(B, T0 + n)).astype(np.int32)
    m = bd.GPT(dims, bd.GPT_FP16, max_batch=B, init_params=params)
    kv, L = m.kv_cache(B, dims["block_size"])
    got = [to_np(m.prefill(torch.as_tensor(seq[:, :T0]).cuda(), kv, L))]
    for i in range(n):
        got.append(to_np(m.decode_step(torch.as_tensor(seq[:, T0 + i]).cuda(), T0 + i, kv, L)))
    torch.cuda.synchronize()
    cfg = O.Config(**{k: dims[k] for k in synth.MODEL_KEYS})
    for i, g in enumerate(got):
        ref, _, _ = O.forward(params, seq[:, :T0 + i], None, cfg)
        assert rel_err(g[:, :300], ref[:, -1, :300]) <= 1e-2, i
    m.close()
