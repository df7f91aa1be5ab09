"""gpt_op_linear_gelu_bwd_noalloc, the entry point that allocates nothing,
through the C-ABI: the same du and bias gradient as gpt_op_linear_gelu_bwd
(which takes its column-sum scratch from the caller) on two calls in a row,
the second smaller than the first, and both against float64 numpy at the
bar of the single-op parity tests.  (Its refusal of sizes beyond the scratch
is host code, checked without a GPU in test_abi.py.)"""
import numpy as np
import pytest

from tests.helpers import bf16_round, case, max_rel, rel_err, to_dev, to_np

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


def one_call(M, N, K, seed):
    case(f"gelu-backward no-alloc vs workspace M={M} N={N} K={K}")
    dY = bf16_round(rnd((M, K), seed, 0.01))
    Wt = bf16_round(rnd((N, K), seed + 1, 0.02))
    dgelu = bf16_round(np.random.default_rng(seed + 2).uniform(-0.15, 1.15, (M, N)))
    db0 = rnd(N, seed + 3)
    a, w, g = (to_dev(x, torch.bfloat16) for x in (dY, Wt, dgelu))
    db_ws = torch.as_tensor(db0).cuda()
    db_na = torch.as_tensor(db0).cuda()
    du_ws = bd.op_linear_gelu_bwd(a, w, g, dbias=db_ws, accumulate_bias=True)
    du_na = bd.op_linear_gelu_bwd_noalloc(a, w, g, dbias=db_na, accumulate_bias=True)
    torch.cuda.synchronize()
    assert torch.equal(du_na, du_ws)
    assert torch.equal(db_na, db_ws)
    du_ref = (dY @ Wt.T) * dgelu
    got = to_np(du_na)
    err = np.abs(got - du_ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(du_ref) + 2e-4 * np.abs(du_ref).max())
    assert rel_err(got, du_ref) < 4e-3
    assert max_rel(to_np(db_na) - db0, du_ref.sum(axis=0)) < 1e-4


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    one_call(16384, 3072, 768, 60)
    one_call(300, 200, 136, 70)  # smaller: the array keeps the first call's partials


def test_noalloc_without_bias_gradient():
    case("gelu-backward no-alloc without a bias gradient")
    M, N, K = 256, 192, 64
    a = to_dev(bf16_round(rnd((M, K), 80, 0.01)), torch.bfloat16)
    w = to_dev(bf16_round(rnd((N, K), 81, 0.02)), torch.bfloat16)
    g = to_dev(bf16_round(rnd((M, N), 82)), torch.bfloat16)
    assert torch.equal(bd.op_linear_gelu_bwd_noalloc(a, w, g), bd.op_linear_gelu_bwd(a, w, g))
