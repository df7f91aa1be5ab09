"""Oracle runs fanned out over host processes for the full-size parity tests.

The forward and backward treat the sequences of a batch independently, and
the mean loss over B*T valid targets is the mean of the B per-sequence means
when every sequence has T of them.  So the gradients of a whole batch are the
sum over its sequences of loss_and_grads on that sequence alone with loss
scale 1/B ("Let's reproduce GPT-2 (124M)", chapter "Gradient Accumulation":
the same sum, taken in pieces).  Each worker runs the float64 oracle on one
sequence in a process of its own, single-threaded, so the pieces run side by
side on the host's cores.  Only the oracle and the seeded input generators
are used here.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _one_sequence(job):
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import gpt_oracle as O
    from transformer_lm_02_amd import synth

    dims, b, B, param_seed, data_seed, T = job
    cfg = O.Config(**{k: dims[k] for k in synth.MODEL_KEYS})
    with threadpool_limits(1):
        params = synth.init_params(dims, seed=param_seed)
        idx, tgt = synth.tokens(dims, seed=data_seed, batch=B, T=T)
        loss, g, _ = O.loss_and_grads(params, idx[b:b + 1], tgt[b:b + 1], cfg, loss_scale=1.0 / B)
    return b, float(loss), g.astype(np.float64)


def start_batch_grads(dims, B, param_seed, data_seed, T, workers=16):
    """Start the B per-sequence oracle runs; returns a handle for
    finish_batch_grads.  Spawned processes (not forked: the caller holds a
    GPU context and BLAS thread pools).  The runs start at once and go on
    while the caller uses the GPU."""
    ctx = mp.get_context("spawn")
    n = max(1, min(workers, B, os.cpu_count() or 1))
    pool = ctx.Pool(n)
    it = pool.imap(_one_sequence, [(dims, b, B, param_seed, data_seed, T) for b in range(B)])
    return pool, it, B


def finish_batch_grads(handle, timeout=900):
    """(mean loss over the batch, summed gradients) of a started run; the
    sequences are added in order as they arrive."""
    pool, it, B = handle
    loss, grads = 0.0, None
    try:
        for i in range(B):
            b, l, g = it.next(timeout=timeout)
            assert b == i
            loss += l
            if grads is None:
                grads = g
            else:
                grads += g
    finally:
        pool.terminate()
        pool.join()
    return loss / B, grads
