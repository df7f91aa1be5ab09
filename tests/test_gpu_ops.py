"""Kernel-level parity on the GPU: each single-op entry point of the C-ABI
against the plain definition (the oracle's functions, or numpy float64 for a
bare matrix product) on the same seeded inputs.  Shapes span several tiles
and ragged tails; bf16 inputs are rounded to bf16 before the reference sees
them, so the tolerances measure only the kernel's own arithmetic."""
import math

import numpy as np
import pytest

from oracle import gpt_oracle as O
from tests.helpers import bf16_round, case, cosine, max_rel, rel_err, to_dev, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global bd
    from transformer_lm_02_amd import binding as bd_mod
    bd = bd_mod
    yield


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(scale)


# ---------------------------------------------------------------- matrix products
LINEAR_SHAPES = [(256, 2304, 768), (300, 200, 136), (1000, 768, 3072), (64, 128, 64),
                 (129, 50304, 768), (4100, 4800, 1600), (4100, 6400, 768), (256, 65, 64)]


@pytest.mark.parametrize("M,N,K", LINEAR_SHAPES)
def test_linear_bf16(M, N, K):
    case(f"linear bf16 M={M} N={N} K={K}")
    A, B = bf16_round(rnd((M, K), 1)), bf16_round(rnd((N, K), 2, 0.05))
    bias = rnd(N, 3)
    ref = A @ B.T + bias
    C = bd.op_linear(to_dev(A, torch.bfloat16), to_dev(B, torch.bfloat16),
                     torch.as_tensor(bias).cuda(), out_f32=True)
    got = to_np(C)
    assert rel_err(got, ref) < 1e-5 and max_rel(got, ref) < 1e-4
    Cb = bd.op_linear(to_dev(A, torch.bfloat16), to_dev(B, torch.bfloat16),
                      torch.as_tensor(bias).cuda(), out_f32=False)
    assert max_rel(to_np(Cb), ref) < 8e-3


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("M,N,K", [(16384, 768, 768), (1000, 384, 1536), (77, 64, 64),
                                   (2048, 50304, 768), (8192, 1600, 4800), (16384, 2304, 768),
                                   (3001, 768, 3072)])
def test_linear_dw_bf16(M, N, K, split):
    case(f"linear_dw bf16 M={M} N={N} K={K} split-K workspace={split}")
    dY, X = bf16_round(rnd((M, N), 4, 0.01)), bf16_round(rnd((M, K), 5))
    ref = dY.T @ X
    ws = torch.empty(16 * N * K, dtype=torch.float32, device="cuda") if split else None
    got = to_np(bd.op_linear_dw(to_dev(dY, torch.bfloat16), to_dev(X, torch.bfloat16), workspace=ws))
    assert rel_err(got, ref) < 1e-5 and max_rel(got, ref) < 1e-4
    # accumulate
    dW = torch.as_tensor(np.ones((N, K), np.float32)).cuda()
    got2 = to_np(bd.op_linear_dw(to_dev(dY, torch.bfloat16), to_dev(X, torch.bfloat16), dW,
                                 workspace=ws))
    assert rel_err(got2, ref + 1.0) < 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_linear_dw_seq_equals_one_at_a_time(dtype):
    """gpt_op_linear_dw_seq, where each product's split-K reduction runs
    inside the next product's launch, against gpt_op_linear_dw called once
    per product in the same order: equal bit for bit.  The sequence holds
    split products (4096 tokens, 16 splits), one with enough tiles not to
    split, one with the 1024 tiles or more that take the wide tiles (after a
    pending reduction, which it hosts), two in a row adding into one
    gradient, one on the plain kernel (300 tokens) after a pending
    reduction, and accumulation."""
    case(f"linear_dw_seq vs linear_dw, 8 products, {dtype}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float16
    seq = [  # (M tokens, N, K, accumulate, gradient index)
        (4096, 768, 256, 0, 0),
        (1024, 4096, 4096, 0, 5),
        (4096, 256, 768, 1, 1),
        (1024, 3072, 2304, 0, 2),
        (4096, 384, 384, 0, 3),
        (4096, 384, 384, 1, 3),
        (300, 104, 136, 1, 4),
        (4096, 768, 256, 1, 0),
    ]
    shapes = {0: (768, 256), 1: (256, 768), 2: (3072, 2304), 3: (384, 384), 4: (104, 136),
              5: (4096, 4096)}
    inputs = [(to_dev(bf16_round(rnd((M, N), 40 + i, 0.01)), dt),
               to_dev(bf16_round(rnd((M, K), 50 + i)), dt))
              for i, (M, N, K, _, _) in enumerate(seq)]
    init = {g: rnd(s, 60 + g) for g, s in shapes.items()}
    ws = torch.empty(3 * 16 * 768 * 256, dtype=torch.float32, device="cuda")
    one = {g: torch.as_tensor(v).cuda() for g, v in init.items()}
    for (M, N, K, acc, g), (dY, X) in zip(seq, inputs):
        if acc:
            bd.op_linear_dw(dY, X, one[g], workspace=ws)
        else:
            one[g].copy_(bd.op_linear_dw(dY, X, workspace=ws))
    chained = {g: torch.as_tensor(v).cuda() for g, v in init.items()}
    bd.op_linear_dw_seq([(dY, X, chained[g], acc)
                         for (M, N, K, acc, g), (dY, X) in zip(seq, inputs)], ws)
    torch.cuda.synchronize()
    for g in shapes:
        a, b = to_np(one[g]), to_np(chained[g])
        assert np.array_equal(a, b), (g, float(np.abs(a - b).max()))
    # and the values themselves: gradient 3 is the sum of its two products
    ref = sum(to_np(dY).astype(np.float64).T @ to_np(X).astype(np.float64)
              for dY, X in inputs[4:6])
    assert rel_err(to_np(chained[3]), ref) < 1e-5
    dY, X = inputs[1]
    ref = to_np(dY).astype(np.float64).T @ to_np(X).astype(np.float64)
    assert rel_err(to_np(chained[5]), ref) < 1e-5


@pytest.mark.parametrize("M,N,K", [(16384, 768, 768), (300, 200, 136), (512, 50304, 768),
                                   (1000, 3072, 768), (257, 4800, 1600), (4100, 768, 6400)])
def test_linear_dx_bf16(M, N, K):
    case(f"linear_dx bf16 M={M} N={N} K={K}")
    dY, W = bf16_round(rnd((M, N), 6, 0.01)), bf16_round(rnd((N, K), 7, 0.02))
    ref = dY @ W
    got = to_np(bd.op_linear_dx(to_dev(dY, torch.bfloat16), to_dev(W, torch.bfloat16)))
    assert rel_err(got, ref) < 1e-5 and max_rel(got, ref) < 1e-4


# The MLP expansion's two epilogues at the step's own shapes: 16384 x 3072 x
# 768 (GPT-2 124M, B=16 T=1024) and 8192 x 6400 x 1600 (the 1.5B shape, B=8)
# take the widest tiles; 2048 x 3072 x 768 and a ragged shape take the others.
GELU_SHAPES = [(16384, 3072, 768), (8192, 6400, 1600), (2048, 3072, 768), (300, 200, 136)]


@pytest.mark.parametrize("M,N,K", GELU_SHAPES)
def test_linear_gelu_forward_bf16(M, N, K):
    """u = A W^T + b; the kernel stores gelu'(u) and gelu(u) in bf16: every
    element against the tanh form's definition in float64."""
    case(f"linear+gelu bf16 M={M} N={N} K={K}")
    A, W = bf16_round(rnd((M, K), 40)), bf16_round(rnd((N, K), 41, 1.5 / math.sqrt(K)))
    bias = rnd(N, 42, 0.5)
    u = A @ W.T + bias
    dg, g = bd.op_linear_gelu(to_dev(A, torch.bfloat16), to_dev(W, torch.bfloat16),
                              torch.as_tensor(bias).cuda())
    torch.cuda.synchronize()
    for got, ref in ((to_np(g), O.gelu_fwd(u)), (to_np(dg), O.gelu_bwd(u))):
        # bf16 output: half an ulp of the value, plus the fp32 accumulation
        err = np.abs(got - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-4 * np.abs(ref).max()), float(err.max())
        assert rel_err(got, ref) < 4e-3


@pytest.mark.parametrize("M,N,K", GELU_SHAPES)
def test_linear_gelu_backward_bf16(M, N, K):
    """du = (dY Wt^T) * gelu'(u) in bf16 and the bias gradient colsum(du) in
    fp32, accumulated onto an existing value: every element against float64."""
    case(f"linear gelu-backward bf16 M={M} N={N} K={K}")
    dY = bf16_round(rnd((M, K), 43, 0.01))
    Wt = bf16_round(rnd((N, K), 44, 0.02))
    dgelu = bf16_round(np.random.default_rng(45).uniform(-0.15, 1.15, (M, N)))
    du_ref = (dY @ Wt.T) * dgelu
    db0 = rnd(N, 46)
    db_ref = db0 + du_ref.sum(axis=0)
    db = torch.as_tensor(db0).cuda()
    du = bd.op_linear_gelu_bwd(to_dev(dY, torch.bfloat16), to_dev(Wt, torch.bfloat16),
                               to_dev(dgelu, torch.bfloat16), dbias=db, accumulate_bias=True)
    torch.cuda.synchronize()
    got = to_np(du)
    err = np.abs(got - du_ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(du_ref) + 2e-4 * np.abs(du_ref).max()), float(err.max())
    assert rel_err(got, du_ref) < 4e-3
    assert max_rel(to_np(db) - db0, db_ref - db0) < 1e-4
    # without the bias gradient no scratch is needed
    du2 = bd.op_linear_gelu_bwd(to_dev(dY, torch.bfloat16), to_dev(Wt, torch.bfloat16),
                                to_dev(dgelu, torch.bfloat16))
    assert torch.equal(du, du2)


@pytest.mark.parametrize("M,N,K", [(256, 192, 64), (70, 33, 17)])
def test_linear_family_fp32(M, N, K):
    case(f"linear family fp32 M={M} N={N} K={K}")
    A, B, bias = rnd((M, K), 8), rnd((N, K), 9), rnd(N, 10)
    got = to_np(bd.op_linear(to_dev(A, torch.float32), to_dev(B, torch.float32),
                             torch.as_tensor(bias).cuda(), out_f32=True))
    assert rel_err(got, A.astype(np.float64) @ B.T + bias) < 1e-6
    dY = rnd((M, N), 11)
    got = to_np(bd.op_linear_dw(to_dev(dY, torch.float32), to_dev(A, torch.float32)))
    assert rel_err(got, dY.astype(np.float64).T @ A) < 1e-6
    got = to_np(bd.op_linear_dx(to_dev(dY, torch.float32), to_dev(B, torch.float32)))
    assert rel_err(got, dY.astype(np.float64) @ B) < 1e-6


# ---------------------------------------------------------------- attention
def split_heads(qkv, B, T, H):
    C = qkv.shape[1] // 3
    hs = C // H
    return [qkv[:, i * C:(i + 1) * C].reshape(B, T, H, hs).transpose(0, 2, 1, 3) for i in range(3)]


def merge_heads(x):
    B, H, T, hs = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B * T, H * hs)


ATTN_CASES = [  # (bf16, B, T, H, hs)
    (True, 2, 256, 3, 64), (True, 1, 200, 2, 64), (True, 1, 1024, 2, 64), (True, 3, 65, 1, 64),
    (True, 1, 1, 2, 64), (True, 2, 96, 2, 32), (False, 4, 64, 4, 16), (False, 1, 37, 2, 24)]


@pytest.mark.parametrize("bf,B,T,H,hs", ATTN_CASES)
def test_attention_fwd_bwd(bf, B, T, H, hs):
    case(f"attention bf16={bf} B={B} T={T} H={H} hs={hs}")
    C = H * hs
    dt = torch.bfloat16 if bf else torch.float32
    rd = bf16_round if bf else (lambda a: np.asarray(a, np.float64))
    qkv = rd(rnd((B * T, 3 * C), 12))
    q, k, v = split_heads(qkv, B, T, H)
    ref_o, ref_p = O.causal_attention_fwd(q, k, v)
    s = (q @ k.transpose(0, 1, 3, 2)) / math.sqrt(hs)
    s = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, s)
    ref_lse = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    dqkv_dev = to_dev(qkv, dt)
    out, lse = bd.op_attention_fwd(dqkv_dev, B, T, H)
    got_o = to_np(out)
    tol = 2e-2 if bf else 1e-5
    assert max_rel(got_o, merge_heads(ref_o)) < tol
    assert np.abs(to_np(lse) - ref_lse).max() < (2e-3 if bf else 1e-5)

    dout = rd(rnd((B * T, C), 13))
    do = dout.reshape(B, T, H, hs).transpose(0, 2, 1, 3)
    dq, dk, dv = O.causal_attention_bwd(do, q, k, v, ref_p)
    ref_d = np.concatenate([merge_heads(t) for t in (dq, dk, dv)], axis=1)
    got_d = to_np(bd.op_attention_bwd(dqkv_dev, out, lse, to_dev(dout, dt), B, T, H))
    scale = np.linalg.norm(ref_d)
    for i, name in enumerate("qkv"):
        g, r = got_d[:, i * C:(i + 1) * C], ref_d[:, i * C:(i + 1) * C]
        if np.linalg.norm(r) < 1e-9 * scale:
            # a single key (T = 1): the softmax is constant, so the query
            # gradient is zero up to rounding; its direction is noise
            assert np.linalg.norm(g) < (1e-4 if bf else 1e-9) * scale, name
        elif bf:
            assert cosine(g, r) > 0.999, name
            assert rel_err(g, r) < 3e-2, name
        else:
            assert rel_err(g, r) < 1e-5, name


def test_attention_forward_is_deterministic_and_causal():
    case("attention causal bit-identity bf16 B=2 T=512 H=2")
    B, T, H, hs = 2, 512, 2, 64
    C = H * hs
    qkv = bf16_round(rnd((B * T, 3 * C), 14))
    out0, _ = bd.op_attention_fwd(to_dev(qkv, torch.bfloat16), B, T, H)
    out1, _ = bd.op_attention_fwd(to_dev(qkv, torch.bfloat16), B, T, H)
    assert torch.equal(out0, out1)
    t = 300
    qkv2 = qkv.reshape(B, T, 3 * C).copy()
    qkv2[:, t + 1:] = bf16_round(rnd(qkv2[:, t + 1:].shape, 15))
    out2, _ = bd.op_attention_fwd(to_dev(qkv2.reshape(B * T, 3 * C), torch.bfloat16), B, T, H)
    a = out0.view(B, T, C)[:, :t + 1]
    b = out2.view(B, T, C)[:, :t + 1]
    assert torch.equal(a, b)


# ---------------------------------------------------------------- layernorm
@pytest.mark.parametrize("bf,M,C", [(True, 1000, 768), (True, 333, 1600), (False, 256, 64),
                                    (True, 16384, 768), (False, 7, 384)])
def test_layernorm_fwd(bf, M, C):
    case(f"layernorm bf16={bf} M={M} C={C}")
    x = rnd((M, C), 16, 3.0) + 1.0
    w, b = rnd(C, 17) + 1.0, rnd(C, 18)
    ref, (xhat, rstd) = O.layernorm_fwd(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    y, mean, rs = bd.op_layernorm_fwd(torch.as_tensor(x).cuda(), torch.as_tensor(w).cuda(),
                                      torch.as_tensor(b).cuda(), bf16=bf)
    assert max_rel(to_np(y), ref) < (8e-3 if bf else 2e-6)
    assert np.abs(to_np(mean) - x.astype(np.float64).mean(1)).max() < 1e-5
    assert max_rel(to_np(rs), rstd[:, 0]) < 1e-5


# ---------------------------------------------------------------- cross-entropy
@pytest.mark.parametrize("bf,N,V,ldv", [(True, 512, 50257, 50304), (True, 300, 65, 128),
                                        (False, 256, 65, 65), (False, 100, 37, 64),
                                        (True, 2048, 50257, 50304)])
def test_cross_entropy(bf, N, V, ldv):
    case(f"cross-entropy bf16={bf} N={N} V={V} ldv={ldv}")
    rd = bf16_round if bf else (lambda a: np.asarray(a, np.float64))
    z = rd(rnd((N, ldv), 19, 2.0))
    tgt = np.random.default_rng(20).integers(0, V, N).astype(np.int32)
    tgt[::17] = -1
    loss_ref, dz_ref = O.cross_entropy(z, tgt, V, loss_scale=0.5)
    zd = to_dev(z, torch.bfloat16 if bf else torch.float32)
    loss, row, nv = bd.op_cross_entropy(zd, torch.as_tensor(tgt).cuda(), V, loss_scale=0.5)
    assert int(nv.item()) == int((tgt >= 0).sum())
    assert abs(float(loss.item()) - loss_ref) < (1e-4 if bf else 1e-5) * max(1.0, loss_ref)
    got = to_np(zd)
    assert np.all(got[:, V:] == 0)
    assert max_rel(got, dz_ref) < (1e-2 if bf else 1e-5)
