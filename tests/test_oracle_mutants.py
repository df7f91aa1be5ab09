"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant below is a plausible slip (a dropped term, a wrong sign, a
transposed operand, a wrong constant).  It is patched into the oracle module
on the CPU for the duration of one pin test, which must then fail.
"""
import math

import numpy as np
import pytest

from oracle import gpt_oracle as O
import tests.test_oracle_pins as pins


def _ln_unbiased(x, w, b, eps=O.LN_EPS):
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    return xhat * w + b, (xhat, rstd)


def _ln_bwd_no_mean_term(dy, w, cache):
    xhat, rstd = cache
    g = dy * w
    dx = rstd * (g - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    red = tuple(range(dy.ndim - 1))
    return dx, (dy * xhat).sum(axis=red), dy.sum(axis=red)


def _gelu_exact(u):
    from scipy.special import erf
    return 0.5 * u * (1 + erf(u / math.sqrt(2)))


def _gelu_bwd_sign(u):
    t = np.tanh(O.GELU_C * (u + O.GELU_A * u ** 3))
    return 0.5 * (1.0 + t) - 0.5 * u * (1.0 - t * t) * O.GELU_C * (1.0 + 3.0 * O.GELU_A * u * u)


def _attn_no_scale(q, k, v, z=None):
    T = q.shape[-2]
    s = q @ np.swapaxes(k, -1, -2)
    s = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, s)
    e = np.exp(s - s.max(-1, keepdims=True))
    p = e / e.sum(-1, keepdims=True)
    return (p if z is None else p * z) @ v, p


def _attn_mask_inclusive(q, k, v, z=None):
    # masks the diagonal too (off-by-one); row 0 then has no visible key, so
    # give it itself to stay finite
    T, hs = q.shape[-2], q.shape[-1]
    s = q @ np.swapaxes(k, -1, -2) / math.sqrt(hs)
    mask = np.triu(np.ones((T, T), bool), 0)
    mask[0, 0] = False
    s = np.where(mask, -np.inf, s)
    e = np.exp(s - s.max(-1, keepdims=True))
    p = e / e.sum(-1, keepdims=True)
    return (p if z is None else p * z) @ v, p


def _attn_bwd_transposed(dout, q, k, v, p, z=None):
    hs = q.shape[-1]
    dv = p @ dout
    dp = dout @ np.swapaxes(v, -1, -2)
    if z is not None:
        dp = dp * z
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    return ds @ k / math.sqrt(hs), np.swapaxes(ds, -1, -2) @ q / math.sqrt(hs), dv


def _ce_unmasked_pad(logits, targets, vocab_size, loss_scale=1.0):
    return _orig_ce(logits, targets, logits.shape[1], loss_scale)


def _ce_sum_not_mean(logits, targets, vocab_size, loss_scale=1.0):
    loss, d = _orig_ce(logits, targets, vocab_size, loss_scale)
    n = int((targets >= 0).sum())
    return loss * n, d * n


def _adamw_coupled(params, grads, m, v, mask, t, lr, beta1=0.9, beta2=0.95, eps=1e-8,
                   weight_decay=0.1, coef=1.0):
    g = grads * coef + weight_decay * mask * params  # L2 in the gradient, not decoupled
    return _orig_adamw(params, g, m, v, mask, t, lr, beta1, beta2, eps, 0.0, 1.0)


def _adamw_eps_inside(params, grads, m, v, mask, t, lr, beta1=0.9, beta2=0.95, eps=1e-8,
                      weight_decay=0.1, coef=1.0):
    g = grads * coef
    m = beta1 * m + (1 - beta1) * g
    v = beta2 * v + (1 - beta2) * g * g
    p = params * (1 - lr * weight_decay * mask)
    p = p - lr * (m / (1 - beta1 ** t)) / np.sqrt(v / (1 - beta2 ** t) + eps)
    return p, m, v


def _adamw_no_bias_correction(params, grads, m, v, mask, t, lr, beta1=0.9, beta2=0.95,
                              eps=1e-8, weight_decay=0.1, coef=1.0):
    g = grads * coef
    m = beta1 * m + (1 - beta1) * g
    v = beta2 * v + (1 - beta2) * g * g
    p = params * (1 - lr * weight_decay * mask)
    return p - lr * m / (np.sqrt(v) + eps), m, v


def _lr_warmup_from_zero(it, max_lr=6e-4, min_lr=None, warmup=715, decay_end=19073):
    if it < warmup:
        return max_lr * it / warmup
    return _orig_lr(it, max_lr, min_lr, warmup, decay_end)


def _clip_always(norm, max_norm):
    return max_norm / (norm + 1e-6)


def _decay_all(cfg, dtype=np.float64):
    return np.ones(O.num_params(cfg), dtype)


_orig_ce, _orig_adamw, _orig_lr = O.cross_entropy, O.adamw, O.get_lr


def _sample_drops_ties(logits_row, vocab_size, temperature, top_k, u, dtype=np.float64):
    z = np.asarray(logits_row, dtype=dtype)[:vocab_size] / temperature
    if 0 < top_k < vocab_size:
        cutoff = np.sort(z)[vocab_size - top_k]
        z = np.where(z <= cutoff, -np.inf, z)  # also removes the k-th largest
        if np.isinf(z).all():
            z[np.argmax(np.asarray(logits_row)[:vocab_size])] = 0.0
    p = np.exp(z - z.max())
    p = p / p.sum()
    return min(int(np.searchsorted(np.cumsum(p), u, side="right")), vocab_size - 1), p


def _sample_times_temperature(logits_row, vocab_size, temperature, top_k, u, dtype=np.float64):
    return _orig_sample(np.asarray(logits_row, dtype) * temperature * temperature, vocab_size,
                        temperature, top_k, u, dtype)


def _sample_left_boundary(logits_row, vocab_size, temperature, top_k, u, dtype=np.float64):
    z = np.asarray(logits_row, dtype=dtype)[:vocab_size] / temperature
    if 0 < top_k < vocab_size:
        z = np.where(z < np.sort(z)[vocab_size - top_k], -np.inf, z)
    p = np.exp(z - z.max())
    p = p / p.sum()
    return min(int(np.searchsorted(np.cumsum(p), u, side="left")), vocab_size - 1), p


def _sample_padded_vocab(logits_row, vocab_size, temperature, top_k, u, dtype=np.float64):
    return _orig_sample(logits_row, len(logits_row), temperature, top_k, u, dtype)


def _generate_first_position(flat_params, idx, cfg, n_new, temperature, top_k, us,
                             dtype=np.float64):
    idx = np.asarray(idx)
    steps = []
    for i in range(n_new):
        logits, _, _ = O.forward(flat_params, idx[:, -cfg.block_size:], None, cfg, dtype=dtype)
        last = logits[:, 0, :]
        steps.append(last)
        nxt = [_orig_sample(last[b], cfg.vocab_size, temperature, top_k, us[b, i], dtype)[0]
               for b in range(idx.shape[0])]
        idx = np.concatenate([idx, np.asarray(nxt, dtype=idx.dtype)[:, None]], axis=1)
    return idx, np.stack(steps)


_orig_sample = O.topk_sample


def _amp_no_unscale(params, scaled_grads, m, v, mask, state, lr, beta1=0.9, beta2=0.95,
                    eps=1e-8, weight_decay=0.1, max_norm=1.0, growth_factor=2.0,
                    backoff_factor=0.5, growth_interval=2000):
    return _orig_amp(params, scaled_grads, m, v, mask, O.LossScaler(1.0, state.growth_tracker,
                                                                     state.steps), lr, beta1,
                     beta2, eps, weight_decay, max_norm, growth_factor, backoff_factor,
                     growth_interval) | {"state": O.scaler_update(
                         state, not np.all(np.isfinite(scaled_grads)), growth_factor,
                         backoff_factor, growth_interval)}


def _amp_clip_before_unscale(params, scaled_grads, m, v, mask, state, lr, beta1=0.9, beta2=0.95,
                             eps=1e-8, weight_decay=0.1, max_norm=1.0, growth_factor=2.0,
                             backoff_factor=0.5, growth_interval=2000):
    norm = O.grad_norm(scaled_grads)
    g = scaled_grads * O.clip_coef(norm, max_norm) / state.scale
    return _orig_amp(params, g * state.scale, m, v, mask, state, lr, beta1, beta2, eps,
                     weight_decay, 0.0, growth_factor, backoff_factor, growth_interval)


def _scaler_counts_skips(state, found_inf, growth_factor=2.0, backoff_factor=0.5,
                         growth_interval=2000):
    out = _orig_update(state, found_inf, growth_factor, backoff_factor, growth_interval)
    return O.LossScaler(out.scale, out.growth_tracker, state.steps + 1)


def _scaler_grows_early(state, found_inf, growth_factor=2.0, backoff_factor=0.5,
                        growth_interval=2000):
    return _orig_update(state, found_inf, growth_factor, backoff_factor, growth_interval - 1)


def _scaler_backoff_keeps_count(state, found_inf, growth_factor=2.0, backoff_factor=0.5,
                                growth_interval=2000):
    if found_inf:
        return O.LossScaler(state.scale * backoff_factor, state.growth_tracker, state.steps)
    return _orig_update(state, found_inf, growth_factor, backoff_factor, growth_interval)


def _train_amp_unscaled_backward(params, m, v, state, micro_batches, cfg, lr, beta1=0.9,
                                 beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
                                 growth_factor=2.0, backoff_factor=0.5, growth_interval=2000,
                                 dtype=np.float64):
    # the loss is not multiplied by the scale before the backward pass
    k = len(micro_batches)
    grads = np.zeros(O.num_params(cfg), dtype=dtype)
    losses = []
    for idx, tgt in micro_batches:
        loss, g, _ = O.loss_and_grads(params, idx, tgt, cfg, 1.0 / k, dtype)
        grads += g
        losses.append(loss)
    out = O.amp_step(np.asarray(params, dtype), grads, np.asarray(m, dtype), np.asarray(v, dtype),
                     O.decay_mask(cfg, dtype), state, lr, beta1, beta2, eps, weight_decay,
                     max_norm, growth_factor, backoff_factor, growth_interval)
    out.update(loss=float(np.mean(losses)), grads=grads)
    return out


_orig_amp, _orig_update, _orig_train_amp = O.amp_step, O.scaler_update, O.train_step_amp


def _attn_drop_renormalised(q, k, v, z=None):
    # dropout whose kept probabilities are renormalised to sum to one
    out, p = _orig_attn_fwd(q, k, v)
    if z is None:
        return out, p
    pd = p * z
    pd = pd / pd.sum(axis=-1, keepdims=True).clip(1e-300)
    return pd @ v, p


def _attn_bwd_mask_only_on_dv(dout, q, k, v, p, z=None):
    # the mask is applied to dV but forgotten in dP
    dq, dk, dv = _orig_attn_bwd(dout, q, k, v, p)
    if z is None:
        return dq, dk, dv
    return dq, dk, np.swapaxes(p * z, -1, -2) @ dout


def _dropout_unscaled(dr, site, bh, rows, cols, dtype=np.float64):
    return (_orig_dmult(dr, site, bh, rows, cols, dtype) > 0).astype(dtype)


def _philox_bump_first(counter, key, width=32, mults=O.PHILOX_M32, weyl=O.PHILOX_W32, rounds=10):
    mask = (1 << width) - 1
    key = ((key[0] + weyl[0]) & mask, (key[1] + weyl[1]) & mask)
    return _orig_philox(counter, key, width, mults, weyl, rounds)


def _philox_hi_lo_swapped(counter, key, width=32, mults=O.PHILOX_M32, weyl=O.PHILOX_W32,
                          rounds=10):
    w = _orig_philox(counter, key, width, mults, weyl, rounds)
    return [w[1], w[0], w[3], w[2]]


def _philox32_multipliers_swapped(counter, key, width=32, mults=O.PHILOX_M32, weyl=O.PHILOX_W32,
                                  rounds=10):
    if width == 32:  # the 64-bit variant (checked against numpy) is left alone
        mults = (mults[1], mults[0])
    return _orig_philox(counter, key, width, mults, weyl, rounds)


_orig_attn_fwd, _orig_attn_bwd = O.causal_attention_fwd, O.causal_attention_bwd
_orig_dmult, _orig_philox = O.dropout_mult, O.philox

MUTANTS = [
    ("layernorm_fwd", _ln_unbiased),
    ("layernorm_bwd", _ln_bwd_no_mean_term),
    ("gelu_fwd", _gelu_exact),
    ("gelu_bwd", _gelu_bwd_sign),
    ("causal_attention_fwd", _attn_no_scale),
    ("causal_attention_fwd", _attn_mask_inclusive),
    ("causal_attention_bwd", _attn_bwd_transposed),
    ("cross_entropy", _ce_unmasked_pad),
    ("cross_entropy", _ce_sum_not_mean),
    ("adamw", _adamw_coupled),
    ("adamw", _adamw_eps_inside),
    ("adamw", _adamw_no_bias_correction),
    ("get_lr", _lr_warmup_from_zero),
    ("clip_coef", _clip_always),
    ("decay_mask", _decay_all),
    ("topk_sample", _sample_drops_ties),
    ("topk_sample", _sample_times_temperature),
    ("topk_sample", _sample_left_boundary),
    ("topk_sample", _sample_padded_vocab),
    ("generate", _generate_first_position),
    ("amp_step", _amp_no_unscale),
    ("amp_step", _amp_clip_before_unscale),
    ("scaler_update", _scaler_counts_skips),
    ("scaler_update", _scaler_grows_early),
    ("scaler_update", _scaler_backoff_keeps_count),
    ("train_step_amp", _train_amp_unscaled_backward),
    ("causal_attention_fwd", _attn_drop_renormalised),
    ("causal_attention_bwd", _attn_bwd_mask_only_on_dv),
    ("dropout_mult", _dropout_unscaled),
    ("philox", _philox_bump_first),
    ("philox", _philox_hi_lo_swapped),
    ("philox", _philox32_multipliers_swapped),
]

# the pins that should catch mistakes in the model and optimizer
PIN_TESTS = [
    lambda: pins.test_layernorm_brute_force_and_invariants(),
    lambda: pins.test_gelu_tanh_form_and_derivative(),
    lambda: pins.test_ops_match_pytorch_functional(),
    lambda: pins.test_attention_brute_force_loops(),
    lambda: pins.test_cross_entropy_against_logsumexp_and_invariants(),
    lambda: pins.test_model_matches_pytorch_autograd(pins.micro_cfg()),
    lambda: pins.test_finite_differences_every_tensor(),
    lambda: pins.test_adamw_first_step_closed_form(),
    lambda: pins.test_adamw_matches_torch_optimizer_over_steps(),
    lambda: pins.test_lr_schedule_matches_page_lab(),
    lambda: pins.test_lr_schedule_build_nanogpt_shape(),
    lambda: pins.test_clip_against_pytorch(),
    lambda: pins.test_decay_mask_groups(),
    lambda: pins.test_topk_sample_closed_forms(),
    lambda: pins.test_generate_repeats_last_token_in_an_identity_model(),
    lambda: pins.test_amp_step_matches_torch_grad_scaler(),
    lambda: pins.test_amp_scale_sequence_closed_form(),
    lambda: pins.test_amp_skipped_step_changes_nothing_and_keeps_the_step_count(),
    lambda: pins.test_train_step_amp_equals_unscaled_step(),
    lambda: pins.test_philox_round_structure_matches_numpy(),
    lambda: pins.test_philox32_known_answer_vectors(),
    lambda: pins.test_dropout_masks_keep_one_minus_p_and_are_independent(),
    lambda: pins.test_dropout_model_matches_pytorch_autograd(),
    lambda: pins.test_dropout_finite_differences(),
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f in MUTANTS])
def test_mutant_is_caught(name, fn, monkeypatch):
    monkeypatch.setattr(O, name, fn)
    caught = []
    for i, pin in enumerate(PIN_TESTS):
        try:
            pin()
        except AssertionError:
            caught.append(i)
            break
    assert caught, f"no pin fails when {name} is replaced by {fn.__name__}"
