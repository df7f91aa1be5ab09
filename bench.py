"""Throughput of one GPT-2 124M bf16 training step on one MI355X.

A step is forward + loss, backward and one AdamW update (with global-norm
clipping) on a micro-batch of B=16 sequences of T=1024 tokens: the workload of
"Let's reproduce GPT-2 (124M)" (Speed Stack chapters; 90 ms per step on one
A100 after every lever).  Inputs are synthetic: Zipf(1.1) token ids over the
GPT-2 vocabulary, N(0, 0.02) weights with 0.02/sqrt(24) residual
projections, all resident in HBM before the timed region.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--fp16]
                    [--dropout P] [--accum K] [--workload gpt2|char|gpt2_1p5b]

Prints one JSON line.  --fp16 times the same step in IEEE half precision
with dynamic loss scaling (scaled forward, backward, then unscale, clip,
AdamW or skip and scale update on the device).  --dropout P times it with
dropout P at the embedding sum, the attention probabilities and the MLP output
(a fresh Philox counter word per step).  --accum K makes a step one optimizer
iteration over K accumulated micro-batches (loss scaled by 1/K, the first
backward replacing the gradients, the others adding; K = 32 is the pages'
524,288-token batch), then clipping and AdamW.  --workload times another model
of the pages at its own batch: the character-level model (vocab 65, T 256, 6
layers of width 384, B 64; the pages train it with dropout 0.2) or the 1.5B
shape (width 1600, 48 layers, B 8).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "gpt2"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
A100_TOKENS_PER_S = 182000.0  # the pages' number for this workload (A100 SXM, 90 ms)


def flops_per_token(dims, T):
    """6N + 12 L H Q T with N the non-embedding parameters (position table
    excluded), as the MFU estimator of "nanoGPT" Part IV Stage 6."""
    from transformer_lm_02_amd import synth
    N = synth.n_params(dims) - dims["block_size"] * dims["n_embd"]
    hs = dims["n_embd"] // dims["n_head"]
    return 6 * N + 12 * dims["n_layer"] * dims["n_head"] * hs * T


# The step's matrix products, grouped by the kernel instantiation the library
# runs them with at this workload (the template names rocprofv3 reports).
# Each group is replayed through the single-op entry point that runs the same
# kernel at the same shapes, one step's launches at a time, with events on
# the stream the launches go to; the weight-gradient group is also timed
# inside training steps (events the library records around its launches),
# which replaces its replay.  The group with the largest time per step is the
# dominant kernel that `roofline` reports.  Not timed here (no single-op
# entry point): the attention- and MLP-projection forwards (residual
# epilogue, 8 % of the step) and the two products of the fused head with the
# cross-entropy (one launch each, 14 % of the step).
TRAFFIC_SOURCES = ["transformer_lm_02_amd/csrc/gemm2.hip", "transformer_lm_02_amd/csrc/gemm.h",
                   "transformer_lm_02_amd/csrc/common.h"]


def gemm_groups(B, T, dims):
    """name -> (kernel template, entry point, [(M, N, K, launches per step)]).
    Shapes are the entry point's: linear C[M][N] = A[M][K] B[N][K]^T;
    linear_dw_seq dW[N][K] = dY[M][N]^T X[M][K], launched in the backward's
    order (the head, then per layer the first four shapes in turn);
    gelu / gelu_bwd as linear."""
    M, d, L = B * T, dims["n_embd"], dims["n_layer"]
    vi = -(-dims["padded_vocab"] // 64) * 64
    return {
        "weight_gradients": (
            "gemm2_kernel<128, 128, false, false, 5, 2, 64, 2> (layers; split-K reductions "
            "inside the next launch) + gemm2_kernel<128, 256, false, false, 5, 2, 48, 2> (head) "
            "+ splitk_reduce_kernel",
            "linear_dw_seq",
            [(M, vi, d, 1), (M, d, 4 * d, L), (M, 4 * d, d, L), (M, d, d, L), (M, 3 * d, d, L)]),
        "input_gradients_and_qkv": (
            "gemm2_kernel<128, 192, true, true, 0, 2, 64, 2>", "linear",
            [(M, d, 4 * d, L), (M, d, 3 * d, L), (M, d, d, L), (M, 3 * d, d, L)]),
        "mlp_expansion_gelu": ("gemm2_kernel<256, 192, true, true, 3, 2, 32, 2>", "gelu",
                               [(M, 4 * d, d, L)]),
        "mlp_projection_dx_gelu_bwd": ("gemm2_kernel<256, 192, true, true, 4, 2, 32, 2>",
                                       "gelu_bwd", [(M, 4 * d, d, L)]),
    }


def sources_hash():
    """Hash of the product kernels' sources with comments and blank space
    removed, so that an edit of a comment does not void measured counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()[:16]


def measured_traffic(group):
    """HBM bytes per launch of a group from the committed FETCH_SIZE /
    WRITE_SIZE counter runs, or None when there are none or the kernel
    sources changed since they were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", f"traffic_{group}.json")) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("sources_hash") != sources_hash():
        return None
    return rec.get("bytes_per_launch")


def group_operands(torch, shapes, entry, dt):
    g = torch.Generator(device="cuda").manual_seed(7)
    ops = []
    for (M, N, K, n) in shapes:
        if entry == "linear_dw_seq":
            a = (torch.randn((M, N), device="cuda", generator=g) * 1e-3).to(dt)
            b = (torch.randn((M, K), device="cuda", generator=g)).to(dt)
            c = torch.empty((N, K), dtype=torch.float32, device="cuda")
            aux = None
        else:
            a = (torch.randn((M, K), device="cuda", generator=g) * 1e-3).to(dt)
            b = (torch.randn((N, K), device="cuda", generator=g) * 0.02).to(dt)
            c = torch.empty((M, N), dtype=dt, device="cuda")
            aux = torch.empty((M, N), dtype=dt, device="cuda") if entry in ("gelu", "gelu_bwd") else None
        ops.append((a, b, c, aux, M, N, K, n))
    return ops


def launch_group(bd, entry, ops, ws, stream_ptr, reps=1):
    import ctypes
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    if entry == "linear_dw_seq":
        # the backward's order: shapes with one launch first (the head), then
        # one launch of every other shape per layer
        once = [o for o in ops if o[-1] == 1]
        per = [o for o in ops if o[-1] > 1]
        seq = once + [o for _ in range(max([o[-1] for o in per] or [0])) for o in per]
        items = [(o[0], o[1], o[2], False) for o in seq]
        for _ in range(reps):
            bd.op_linear_dw_seq(items, ws)
        return
    for _ in range(reps):
        for (a, b, c, aux, M, N, K, n) in ops:
            dt = bd._bf(a)
            for _ in range(n):
                if entry == "linear":
                    rc = bd.lib.gpt_op_linear(dt, vp(a), vp(b), None, vp(c), 0, M, N, K, stream_ptr)
                elif entry == "gelu":
                    rc = bd.lib.gpt_op_linear_gelu(dt, vp(a), vp(b), None, vp(c), vp(aux), M, N, K,
                                                   stream_ptr)
                else:  # gelu_bwd with the bias gradient's column sums, as in the step
                    rc = bd.lib.gpt_op_linear_gelu_bwd(dt, vp(a), vp(b), vp(aux), vp(c), vp(ws[:N]),
                                                       0, M, N, K, vp(ws[N:]), wsb - 4 * N,
                                                       stream_ptr)
                bd.check(rc, entry)


def time_gemm_groups(torch, bd, B, T, dims, reps=3, fp16=False):
    """Per group: one step's launches, timed with events on the current
    stream over `reps` repetitions after one untimed pass."""
    import ctypes
    dt = torch.float16 if fp16 else torch.bfloat16
    s = torch.cuda.current_stream()
    sp = ctypes.c_void_p(s.cuda_stream)
    d = dims["n_embd"]
    # the step's split-K scratch: 16 partial slices of the widest layer matrix
    ws = torch.empty(16 * 4 * d * d, dtype=torch.float32, device="cuda")
    out = {}
    for name, (kern, entry, shapes) in gemm_groups(B, T, dims).items():
        ops = group_operands(torch, shapes, entry, dt)
        launch_group(bd, entry, ops, ws, sp, 1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        launch_group(bd, entry, ops, ws, sp, reps)
        e1.record(s)
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / reps
        n_launch = sum(o[-1] for o in ops)
        flops = sum(2.0 * M * N * K * n for (M, N, K, n) in shapes)
        out[name] = {"kernel": ("f16::" if fp16 else "b16::") + kern, "entry": entry,
                     "ms_per_step": ms_step, "launches_per_step": n_launch,
                     "flops_per_step": flops}
        del ops
    return out


def roofline_from_groups(groups, fp16=False, instep=None):
    """The group with the largest time per step.  instep: the weight-gradient
    group timed inside training steps (events around its launches), which
    then replaces that group's replay through the single-op entry point."""
    replay = {k: round(v["ms_per_step"], 4) for k, v in groups.items()}
    if (instep and "weight_gradients" in groups
            and round(instep["launches_per_step"]) == groups["weight_gradients"]["launches_per_step"]):
        g = dict(groups["weight_gradients"])
        g["ms_per_step"] = instep["ms_per_step"]
        g["timing"] = f"in-step HIP events over {instep['steps']} steps"
        groups = dict(groups, weight_gradients=g)
    name = max(groups, key=lambda k: groups[k]["ms_per_step"])
    g = groups[name]
    n = g["launches_per_step"]
    ms_launch = g["ms_per_step"] / n
    achieved = g["flops_per_step"] / (g["ms_per_step"] * 1e-3) / 1e12
    return {"kernel": g["kernel"], "group": name, "bound": "mfma",
            "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None if fp16 else measured_traffic(name),
            "launches_per_step": n, "ms_per_launch": round(ms_launch, 4),
            "flops_per_launch": g["flops_per_step"] / n,
            "timing": g.get("timing", "replay of the step's launches through the single-op entry "
                                      "point"),
            "groups_ms_per_step_replayed": replay}


def probe(torch, bd, B, T, dims, group):
    """For counter runs: one step's launches of one group, then a plain 1 GiB
    device copy (the calibration of FETCH_SIZE / WRITE_SIZE)."""
    import ctypes
    kern, entry, shapes = gemm_groups(B, T, dims)[group]
    ops = group_operands(torch, shapes, entry, torch.bfloat16)
    ws = torch.empty(16 * 4 * dims["n_embd"] ** 2, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    launch_group(bd, entry, ops, ws, ctypes.c_void_p(s.cuda_stream), 1)
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": group, "kernel": kern, "launches": shapes,
                      "copy_bytes": src.numel() * 4, "sources_hash": sources_hash()}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(dims, seed=1338):
    """The oracle (as it stands, in its float32 mode) on a bounded sample of
    the workload: one full step (forward, backward, clip, AdamW) on one
    sequence of 1024 tokens with the full model, once with every BLAS thread
    of the host and once with one; tokens/s scales linearly in the batch."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import gpt_oracle as O
    from transformer_lm_02_amd import synth
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    cfg = O.Config(**{k: dims[k] for k in synth.MODEL_KEYS})
    params = synth.init_params(dims, seed=1337)
    idx, tgt = synth.tokens(dims, seed=seed, batch=1)
    zeros = np.zeros_like(params)

    def run():
        t0 = time.perf_counter()
        O.train_step(params, zeros, zeros, 1, [(idx, tgt)], cfg, lr=6e-4, dtype=np.float32)
        return time.perf_counter() - t0

    dt = run()
    with threadpool_limits(1):
        dt1 = run()
    return {"value": round(idx.size / dt, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_thread": {"value": round(idx.size / dt1, 2), "unit": "tokens/s", "cores": 1,
                              "s_per_step": round(dt1, 2)},
            "s_per_step": round(dt, 2),
            "sample": f"1 x 1024 tokens, full 124M model, float32 numpy oracle step "
                      f"(fwd+bwd+clip+AdamW): {dt:.1f} s on {cores} threads, {dt1:.1f} s on 1"}


def decode_bench(torch, bd, synth, dims, B, prompt, n_new, temperature=0.8, top_k=200):
    """Sampling with the key/value cache ("nanoGPT" Part IV, one generation;
    "Build GPT from scratch", exercise "Add a KV cache"): one prefill of the
    prompt, then n_new draws, each a decode step and a sample, timed with one
    event per token.  Prints one JSON line."""
    params = synth.init_params(dims, seed=1337)
    model = bd.GPT(dims, bd.GPT_BF16, max_batch=B, init_params=params)
    idx = torch.as_tensor(synth.tokens(synth.WORKLOADS[WORKLOAD], seed=1338, batch=B, T=prompt)[0]).cuda()
    g = torch.Generator(device="cuda").manual_seed(1339)
    u = torch.rand((n_new, B), generator=g, dtype=torch.float32, device="cuda")
    kv, L = model.kv_cache(B, dims["block_size"])
    V = dims["vocab_size"]
    s = torch.cuda.current_stream()

    def run(timed):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_new + 2)]
        ev[0].record(s)
        logits = model.prefill(idx, kv, L)
        ev[1].record(s)
        for i in range(n_new):
            tok = bd.sample(logits, V, temperature, top_k, u[i])
            if i + 1 < n_new:
                model.decode_step(tok, prompt + i, kv, L, logits)
            ev[i + 2].record(s)
        torch.cuda.synchronize()
        return ev

    run(False)  # warm-up: the same work once
    ev = run(True)
    prefill_ms = ev[0].elapsed_time(ev[1])
    per_tok = [ev[i + 1].elapsed_time(ev[i + 2]) for i in range(1, n_new)]
    total_ms = ev[1].elapsed_time(ev[-1])
    srt = sorted(per_tok)
    pct = lambda q: srt[min(len(srt) - 1, int(round(q * (len(srt) - 1))))]
    early = sum(per_tok[:64]) / 64
    late = sum(per_tok[-64:]) / 64
    # bytes one decode step must read: every bf16 matrix (the tied embedding
    # once) and the cache of the positions it attends to (mean position)
    d, Lyr, Vp = dims["n_embd"], dims["n_layer"], dims["padded_vocab"]
    w_bytes = 2 * (Lyr * 12 * d * d + Vp * d)
    kv_bytes = 2 * Lyr * 2 * B * d * (prompt + n_new / 2)
    step_ms = total_ms / n_new
    achieved = (w_bytes + kv_bytes) / (step_ms * 1e-3) / 1e9
    out = {
        "metric": f"decode tokens/s with a KV cache (temperature {temperature}, top-k {top_k}), "
                  f"GPT-2 124M bf16, B={B}, 1 MI355X",
        "value": round(B * n_new / (total_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": n_new, "warmup": 1, "ms_per_token": round(step_ms, 4),
        "ms_per_token_p10_p50_p90": [round(pct(0.1), 4), round(pct(0.5), 4), round(pct(0.9), 4)],
        "ms_per_token_first64_last64": [round(early, 4), round(late, 4)],
        "prefill_ms": round(prefill_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (Zipf(1.1) prompt; random-init weights)",
        "config": {"workload": f"GPT-2 124M sampling, prompt {prompt}, {n_new} new tokens, "
                               f"positions {prompt}..{prompt + n_new - 1}", "batch": B},
        "roofline": {"kernel": "whole decode step (weights + cache read once per token)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_step": int(w_bytes + kv_bytes)},
        "cpu_baseline": None,
    }
    model.close()
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--decode", type=int, default=0, metavar="B",
                    help="instead of training, time sampling with the KV cache for B sequences")
    ap.add_argument("--workload", default=WORKLOAD, choices=["gpt2", "char", "gpt2_1p5b"],
                    help="model and batch (default: GPT-2 124M, B=16, T=1024)")
    ap.add_argument("--accum", type=int, default=1, metavar="K",
                    help="micro-batches accumulated per optimizer step")
    ap.add_argument("--dropout", type=float, default=0.0, metavar="P",
                    help="train with dropout P (the pretraining configuration uses 0)")
    ap.add_argument("--fp16", action="store_true",
                    help="IEEE half precision with dynamic loss scaling instead of bf16")
    ap.add_argument("--fused-ce", type=int, default=None, choices=[0, 1], metavar="0|1",
                    help="GPT_OPT_FUSED_HEAD_CE: the cross-entropy fused into the tied head "
                         "(default: the library's default)")
    ap.add_argument("--probe", default=None, metavar="GROUP",
                    help="only launch one step's products of GROUP and a calibration copy "
                         "(counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library "
              f"runs one GPU per process and has no data-parallel gradient exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_lm_02_amd import binding as bd
    from transformer_lm_02_amd import synth

    dims = synth.WORKLOADS[args.workload]
    B, T = dims["batch"], dims["block_size"]
    headline = args.workload == WORKLOAD
    if args.decode:
        decode_bench(torch, bd, synth, synth.model_dims(dims), args.decode, 64, 448)
        return
    if args.probe:
        probe(torch, bd, B, T, dims, args.probe)
        return
    print(f"[bench] building model {args.workload} B={B} T={T}", file=sys.stderr, flush=True)
    params = synth.init_params(dims, seed=1337)
    model = bd.GPT(dims, bd.GPT_FP16 if args.fp16 else bd.GPT_BF16, max_batch=B,
                   init_params=params)
    if args.fused_ce is not None:
        model.set_option(bd.GPT_OPT_FUSED_HEAD_CE, args.fused_ce)
    model_fused = model.get_option(bd.GPT_OPT_FUSED_HEAD_CE) and not args.fp16
    nb = 4
    batches = []
    for i in range(nb):
        idx, tgt = synth.tokens(dims, seed=1338 + i)
        batches.append((torch.as_tensor(idx).cuda(), torch.as_tensor(tgt).cuda()))
    torch.cuda.synchronize()

    drop = (lambda i: (args.dropout, 1337, i)) if args.dropout > 0 else (lambda i: None)

    K = max(1, args.accum)

    def step(i):
        lr = bd.lr_at(i)  # warmup 715, cosine to 6e-5 at 19073
        for k in range(K):
            idx, tgt = batches[(i * K + k) % nb]
            if args.fp16:
                # scale, backward; after the micro-steps unscale, clip, step or skip, update
                model.forward(idx, tgt, loss_scale=1.0 / K, scaled=True, dropout=drop(i * K + k))
            else:
                model.forward(idx, tgt, loss_scale=1.0 / K, dropout=drop(i * K + k))
            model.backward(zero_first=(k == 0))
        if args.fp16:
            model.amp_step(lr=lr, max_norm=1.0)
        else:
            model.adamw_step(lr=lr, t=i + 1, max_norm=1.0)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    # one event per step boundary on the library's stream: no host sync inside
    # the timed window; per-step times give the spread
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(s)
    for i in range(args.steps):
        step(args.warmup + i)
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    pct = lambda q: per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]
    loss = float(model.scalars[0].item())
    norm = float(model.scalars[1].item())
    tokens = B * T * K
    value = tokens / (ms * 1e-3)
    fpt = flops_per_token(dims, T)
    mfu = fpt * tokens / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    print(f"[bench] {ms:.3f} ms/step (wall {wall / args.steps * 1e3:.3f}), loss {loss:.4f}, "
          f"norm {norm:.4f}, MFU {mfu:.4f}", file=sys.stderr, flush=True)
    scaler = model.scaler_state() if args.fp16 else None
    instep = None
    if not args.no_kernel_timing and headline:
        # the weight-gradient launches timed inside the step: HIP events the
        # library records on its stream around each of them.  The events cost
        # ~0.3 ms per step, so they run on further steps of the same workload
        # right after the timed ones, not inside them.
        n_ev = 10
        model.set_option(bd.GPT_OPT_TIME_WEIGHT_GRADIENTS, 1)
        for i in range(n_ev):
            step(args.warmup + args.steps + i)
        torch.cuda.synchronize()
        ev_ms, ev_n = model.read_timing()
        model.set_option(bd.GPT_OPT_TIME_WEIGHT_GRADIENTS, 0)
        # per backward (one micro-batch), as the groups are counted
        instep = {"ms_per_step": ev_ms / (n_ev * K), "launches_per_step": ev_n / (n_ev * K),
                  "steps": n_ev}
    roof = None
    model.close()
    del model
    torch.cuda.empty_cache()
    if not args.no_kernel_timing and headline:
        print("[bench] timing the step's matrix products by kernel", file=sys.stderr, flush=True)
        roof = roofline_from_groups(time_gemm_groups(torch, bd, B, T, dims, fp16=args.fp16),
                                    fp16=args.fp16, instep=instep)
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline and headline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(dims)
    prec = "fp16 (dynamic loss scaling)" if args.fp16 else "bf16"
    if args.dropout > 0:
        prec += f" dropout {args.dropout:g}"
    model_name = {"gpt2": "GPT-2 124M", "char": "character-level GPT (6x384)",
                  "gpt2_1p5b": "GPT-2 1.5B shape"}[args.workload]
    shape = f"B={B} T={T}" + (f" x {K} micro-batches" if K > 1 else "")
    out = {
        "metric": f"train tokens/sec + ms/step + MFU, {model_name} {prec} {shape}, 1 MI355X",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_per_step_p10_p50_p90": [round(pct(0.1), 4), round(pct(0.5), 4), round(pct(0.9), 4)],
        "mfu": round(mfu, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None if (args.fp16 or args.dropout > 0 or K > 1 or not headline)
        else round(value / A100_TOKENS_PER_S, 3),
        "baseline": "pages' 90 ms/step = ~182,000 tokens/s on one A100 SXM (context)",
        "dtype": "fp16" if args.fp16 else "bf16",
        "data": ("synthetic (Zipf(1.1) token ids; random-init weights)" if dims["tokens"] == "zipf"
                 else "synthetic (uniform token ids; random-init weights)"),
        "config": {"workload": f"{model_name} training step (fwd+bwd+clip+AdamW), vocab "
                               f"{dims['padded_vocab']} (pad masked), B={B}, T={T}"
                               + (f", {K} micro-batches per optimizer step" if K > 1 else ""),
                   "global_batch": B * K, "seq_len": T,
                   "fused_head_ce": bool(model_fused),
                   "flops_per_step": fpt * tokens, "loss": round(loss, 4), "grad_norm": round(norm, 4)},
        **({"loss_scaler": dict(zip(("scale", "growth_tracker", "updates", "last_skipped"), scaler)),
            "optimizer_steps_run": args.warmup + args.steps} if scaler else {}),
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
