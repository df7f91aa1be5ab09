"""Initialisation on the device from a seed (gpt_init with no initial
parameters), against what "Let's reproduce GPT-2 (124M)", chapter "Model
Initialization", fixes: every Linear weight and both embedding tables
N(0, 0.02^2), the two projections per block into the residual stream
N(0, (0.02 / sqrt(2 n_layer))^2), biases 0, LayerNorm gains 1 and shifts 0,
and an initial loss of about ln V.

The values are draws, so they are checked by their distribution: each
tensor's mean and standard deviation within a few standard errors, a
Kolmogorov-Smirnov distance to the normal law, no correlation between
neighbours, exact constants, the same values for the same seed in every mode
and different ones for another seed.
"""
import math

import numpy as np
import pytest

from oracle import gpt_oracle as O
from tests.helpers import case, to_np
from tests.test_gpu_step import dev_tokens, ocfg, per_tensor
from transformer_lm_02_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global bd
    from transformer_lm_02_amd import binding as bd_mod
    bd = bd_mod
    yield


def expected(name, L):
    """('normal', std) or ('const', value) for a tensor name."""
    if name.endswith("ln1.w") or name.endswith("ln2.w") or name == "lnf.w":
        return "const", 1.0
    if name.endswith(".b"):
        return "const", 0.0
    if name.endswith("aproj.w") or name.endswith("mproj.w"):
        return "normal", 0.02 / math.sqrt(2 * L)
    return "normal", 0.02


def ks_normal(x, std):
    """Kolmogorov-Smirnov distance of a sample to N(0, std^2)."""
    from scipy.stats import norm
    x = np.sort(np.asarray(x, np.float64) / std)
    n = x.size
    cdf = norm.cdf(x)
    return float(max((np.arange(1, n + 1) / n - cdf).max(), (cdf - np.arange(n) / n).max()))


def test_seeded_init_matches_the_pages_distribution_gpt2():
    dims = synth.WORKLOADS["gpt2"]
    L = dims["n_layer"]
    case("gpt2 bf16 init from seed 1234")
    m = bd.GPT(dims, bd.GPT_BF16, max_batch=4, seed=1234)
    p = to_np(m.params)
    for name, t in per_tensor(dims, p).items():
        kind, val = expected(name, L)
        if kind == "const":
            assert np.all(t == val), name
            continue
        n = t.size
        mean, sd = float(t.mean()), float(t.std())
        assert abs(mean) <= 5 * val / math.sqrt(n), (name, mean)
        assert abs(sd / val - 1) <= 5 / math.sqrt(2 * n) + 1e-3, (name, sd, val)
        r = float(np.corrcoef(t[:-1], t[1:])[0, 1])
        assert abs(r) <= 5 / math.sqrt(n), (name, r)
    wte = per_tensor(dims, p)["wte"]
    sample = wte[::97][:200000]
    # critical distance at the 0.1 % level is 1.95 / sqrt(n) = 0.0044
    assert ks_normal(sample, 0.02) < 0.0044
    mproj = per_tensor(dims, p)["h0.mproj.w"]
    assert ks_normal(mproj[:200000], 0.02 / math.sqrt(2 * L)) < 0.0044
    # the initial loss: about ln V ("Let's reproduce GPT-2 (124M)", the loss
    # at initialisation), within the band of the oracle's init-loss pin
    idx, tgt = synth.tokens(dims, seed=1338, batch=4)
    loss, _ = m.forward(*dev_tokens(idx, tgt))
    lnv = math.log(dims["vocab_size"])
    got = float(loss.item())
    assert lnv - 0.1 <= got <= lnv + 2e-4 * dims["n_embd"] + 0.1, got
    # the oracle on the device's parameters agrees on one sequence
    ref_logits, ref_loss, _ = O.forward(p, idx[:1], tgt[:1], ocfg(dims))
    loss1, _ = m.forward(*dev_tokens(idx[:1], tgt[:1]))
    assert abs(float(loss1.item()) - ref_loss) <= 2e-2
    m.close()


def test_seeded_init_is_a_function_of_the_seed():
    dims = synth.WORKLOADS["tiny"]
    case("tiny init: same seed in fp32, bf16 and fp16 modes; another seed")
    got = []
    for mode in (bd.GPT_FP32, bd.GPT_BF16, bd.GPT_FP16):
        m = bd.GPT(dims, mode, max_batch=1, seed=77)
        got.append(to_np(m.params))
        assert float(m.adam_m.abs().max().item()) == 0.0
        assert float(m.grads.abs().max().item()) == 0.0
        m.close()
    assert np.array_equal(got[0], got[1]) and np.array_equal(got[0], got[2])
    m = bd.GPT(dims, bd.GPT_FP32, max_batch=1, seed=78)
    other = to_np(m.params)
    m.close()
    w0, w1 = per_tensor(dims, got[0])["wte"], per_tensor(dims, other)["wte"]
    assert not np.array_equal(w0, w1)
    assert abs(float(np.corrcoef(w0, w1)[0, 1])) < 5 / math.sqrt(w0.size)
    # the seed's upper 32 bits take part too
    m = bd.GPT(dims, bd.GPT_FP32, max_batch=1, seed=77 + (1 << 32))
    high = to_np(m.params)
    m.close()
    assert not np.array_equal(per_tensor(dims, high)["wte"], w0)
