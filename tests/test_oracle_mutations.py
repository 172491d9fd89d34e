"""Each plausible mistake in the differential-attention oracle fails at least
one of its pins (tests/test_oracle.py).  The mistakes are planted in the
oracle on the CPU, for the duration of one test, by replacing one of its
functions with a wrong copy; the oracle's own functions call each other
through the module, so the planted copy is used everywhere.
"""

import math

import numpy as np
import pytest

from oracle import diffattn_oracle as O

import test_oracle as pins

# every pin, with the parameters it runs under
PINS = [
    (pins.test_six_key_example_printed_values, {}),
    (pins.test_six_key_exact_closed_form, {}),
    (pins.test_lambda_closed_form, {}),
    *[(pins.test_rows_sum_to_one_minus_lambda, dict(lam=lam, causal=c))
      for lam in (-0.3, 0.0, 0.5, 1.0, 1.7) for c in (True, False)],
    (pins.test_key_permutation_invariance_noncausal, {}),
    (pins.test_shared_maps_reduce_to_scaled_attention, {}),
    (pins.test_large_logits_shift_invariance, {}),
    (pins.test_blocking_does_not_change_values, {}),
    *[(pins.test_lambda_zero_is_standard_attention, dict(causal=c)) for c in (True, False)],
    *[(pins.test_linearity_against_two_library_attentions, dict(d=d)) for d in (16, 64)],
    (pins.test_causal_row0_closed_form, {}),
    *[(pins.test_rmsnorm_constant_vector_closed_form, dict(c=c)) for c in (1.0, 1e-3, 0.0)],
    (pins.test_scale_is_one_minus_lambda_init_not_lambda, {}),
    *[(pins.test_brute_force_tiny, dict(n=n, causal=c)) for n, c in ((1, True), (5, True), (6, False))],
    (pins.test_forward_rows_matches_forward, {}),
    (pins.test_decode_equals_last_causal_prefill_row, {}),
    (pins.test_decode_empty_cache_gives_zeros, {}),
]

_attention_map = O.attention_map
_head_rmsnorm_scale = O.head_rmsnorm_scale
_visible = O._visible


def _scale_by_2d(q, k, causal, q_pos=None):
    # 1/sqrt(2d) (the value width) instead of 1/sqrt(d)
    q, k = O._f64(q), O._f64(k)
    s = (q @ k.T) / math.sqrt(2 * q.shape[-1])
    return O.softmax_rows(np.where(O._visible(q.shape[0], k.shape[0], causal, q_pos), s, -np.inf))


def _transposed_scores(q, k, causal, q_pos=None):
    # K Q^T read as if it were Q K^T (square heads only; rows and keys swap roles)
    q, k = O._f64(q), O._f64(k)
    s = (k @ q.T) / math.sqrt(q.shape[-1]) if q.shape[0] == k.shape[0] else (q @ k.T) / math.sqrt(q.shape[-1])
    return O.softmax_rows(np.where(O._visible(q.shape[0], k.shape[0], causal, q_pos), s, -np.inf))


def _strict_mask(nq, nk, causal, q_pos=None):
    # j < i: the diagonal hidden
    if not causal:
        return np.ones((nq, nk), dtype=bool)
    pos = np.arange(nq) if q_pos is None else np.asarray(q_pos)
    return np.arange(nk)[None, :] < pos[:, None]


def _no_max_subtraction(s):
    e = np.exp(s)
    return e / np.sum(e, axis=-1, keepdims=True)


def _lambda_sign_flipped(q1, k1, q2, k2, lam, causal, q_pos=None):
    return _attention_map(q1, k1, causal, q_pos) + float(lam) * _attention_map(q2, k2, causal, q_pos)


def _maps_swapped(q1, k1, q2, k2, lam, causal, q_pos=None):
    return _attention_map(q2, k2, causal, q_pos) - float(lam) * _attention_map(q1, k1, causal, q_pos)


def _eps_outside_root(y, weight, eps, lambda_init):
    y = O._f64(y)
    w = np.ones(y.shape[-1]) if weight is None else O._f64(weight)
    return (1.0 - float(lambda_init)) * (w * y) / (np.sqrt(np.mean(y * y, axis=-1, keepdims=True)) + float(eps))


def _fixed_scale(y, weight, eps, lambda_init):
    return _head_rmsnorm_scale(y, weight, eps, 0.8)


def _norm_over_tokens(y, weight, eps, lambda_init):
    y = O._f64(y)
    w = np.ones(y.shape[-1]) if weight is None else O._f64(weight)
    ms = np.mean(y * y, axis=-2, keepdims=True)
    return (1.0 - float(lambda_init)) * (w * y) / np.sqrt(ms + float(eps))


def _layernorm(y, weight, eps, lambda_init):
    y = O._f64(y)
    return _head_rmsnorm_scale(y - y.mean(axis=-1, keepdims=True), weight, eps, lambda_init)


def _exponentials_swapped(lq1, lk1, lq2, lk2, lambda_init):
    lq1, lk1, lq2, lk2 = (O._f64(v) for v in (lq1, lk1, lq2, lk2))
    return float(math.exp(float(np.dot(lq2, lk2))) - math.exp(float(np.dot(lq1, lk1))) + float(lambda_init))


def _lambda_init_dropped(lq1, lk1, lq2, lk2, lambda_init):
    lq1, lk1, lq2, lk2 = (O._f64(v) for v in (lq1, lk1, lq2, lk2))
    return float(math.exp(float(np.dot(lq1, lk1))) - math.exp(float(np.dot(lq2, lk2))))


def _scale_by_lambda(q1, k1, q2, k2, v, lam, lambda_init, weight=None, eps=1e-5, causal=True, norm=True, block=512):
    # (1 - lambda) where the pages fix (1 - lambda_init)
    q1, k1, q2, k2, v = (O._f64(t) for t in (q1, k1, q2, k2, v))
    B, H, N, _ = q1.shape
    out = np.empty(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            y = O.pre_norm(q1[b, h], k1[b, h], q2[b, h], k2[b, h], v[b, h], lam, causal)
            out[b, h] = _head_rmsnorm_scale(y, weight, eps, lam) if norm else y
    return out


MUTATIONS = {
    "scale_by_sqrt_2d": ("attention_map", _scale_by_2d),
    "transposed_scores": ("attention_map", _transposed_scores),
    "strict_causal_mask": ("_visible", _strict_mask),
    "no_max_subtraction": ("softmax_rows", _no_max_subtraction),
    "lambda_sign_flipped": ("diff_weights", _lambda_sign_flipped),
    "maps_swapped": ("diff_weights", _maps_swapped),
    "eps_outside_root": ("head_rmsnorm_scale", _eps_outside_root),
    "fixed_0p8_scale": ("head_rmsnorm_scale", _fixed_scale),
    "norm_over_tokens": ("head_rmsnorm_scale", _norm_over_tokens),
    "mean_subtracted": ("head_rmsnorm_scale", _layernorm),
    "lambda_exponentials_swapped": ("lambda_scalar", _exponentials_swapped),
    "lambda_init_dropped": ("lambda_scalar", _lambda_init_dropped),
    "scale_by_one_minus_lambda": ("forward", _scale_by_lambda),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    with np.errstate(all="ignore"):
        for pin, kw in PINS:
            try:
                pin(**kw)
            except (AssertionError, ValueError, FloatingPointError, OverflowError, pytest.fail.Exception):
                failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
    print(f"{name}: caught by {sorted(set(failed))}")


def test_unmutated_oracle_passes_every_pin():
    for pin, kw in PINS:
        pin(**kw)
