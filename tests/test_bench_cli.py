"""bench.py without a GPU: its refusal of more than one GPU, its FLOP count
per token against the per-token figures derived from the pages' MFU
estimator ("nanoGPT" Part IV Stage 6: 6 N + 12 L H Q T, N without the
position table), the weight-gradient group it times, and the committed counter
record its traffic figure comes from."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from transformer_lm_02_amd import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,per_token", [
    # 6 x 123,689,472 + 12 x 12 x 12 x 64 x 1024
    ("gpt2", 855_383_040),
    # 6 x 10,672,512 + 12 x 6 x 6 x 64 x 256
    ("char", 71_112_960),
    # 6 x 1,556,048,000 + 12 x 48 x 25 x 64 x 1024
    ("gpt2_1p5b", 10_280_006_400),
])
def test_flops_per_token(name, per_token):
    dims = synth.WORKLOADS[name]
    assert bench.flops_per_token(dims, dims["block_size"]) == per_token


def test_weight_gradient_group():
    """49 launches per step (four per block and the head's), each 2 M N K over
    the 16384 tokens: 4.05 TFLOP in all, in the backward's order."""
    dims = synth.WORKLOADS["gpt2"]
    kern, entry, shapes = bench.gemm_groups(16, 1024, dims)["weight_gradients"]
    assert entry == "linear_dw_seq"
    assert sum(n for (_, _, _, n) in shapes) == 49
    flops = sum(2.0 * M * N * K * n for (M, N, K, n) in shapes)
    d, vi = 768, 50304
    assert flops == 2.0 * 16384 * (12 * (4 * d * d * 2 + d * d + 3 * d * d) + vi * d)
    ops = [(i, i, i, None, M, N, K, n) for i, (M, N, K, n) in enumerate(shapes)]
    once = [o for o in ops if o[-1] == 1]
    assert len(once) == 1 and once[0][5] == vi


def test_committed_traffic_counters_match_the_kernel_sources():
    """The HBM bytes bench.py reports as roofline.traffic come from the
    committed counter record of the weight-gradient group, which holds the
    hash of the matrix-product sources it was taken on.  A change to those
    sources without new counter runs would report traffic as null; this
    fails first.  The record's per-launch figure is the sum of its read and
    write parts and lies above the algorithmic bytes."""
    import json
    with open(os.path.join(ROOT, "profiles", "traffic_weight_gradients.json")) as fh:
        rec = json.load(fh)
    assert rec["sources_hash"] == bench.sources_hash()
    assert bench.measured_traffic("weight_gradients") == rec["bytes_per_launch"]
    # each of the three is rounded to a byte on its own
    assert abs(rec["bytes_per_launch"] - rec["read_bytes_per_launch"]
               - rec["write_bytes_per_launch"]) <= 1
    assert rec["algorithmic_bytes_per_launch"] < rec["bytes_per_launch"]
    assert rec["launches_per_step"] == 49
