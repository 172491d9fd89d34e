"""Each plausible mistake in the projection oracle fails at least one of its
pins (tests/test_oracle_projection.py).  The mistakes are planted in the
oracle on the CPU, for the duration of one test.
"""

import numpy as np
import pytest

from oracle import projection_oracle as P

import test_oracle_projection as pins

PINS = [pins.test_in_projection_brute_force, pins.test_in_projection_selection_weights,
        pins.test_out_projection_identity_is_head_concatenation, pins.test_out_projection_brute_force,
        pins.test_against_torch_linear]

_in = P.in_projection


def _halves_swapped(x, w, H, d):
    q1, k1, q2, k2, v = _in(x, w, H, d)
    return q2, k2, q1, k1, v


def _split_by_map_first(x, w, H, d):
    # Q1 = the first H*d features of W_Q (map-major), not the first half of each head
    x, w = np.asarray(x, np.float64), np.asarray(w, np.float64)
    B, N, _ = x.shape
    width = H * 2 * d
    y = x @ w.T
    out = []
    for part in (0, 1):
        blk = y[..., part * width:(part + 1) * width]
        out.append([blk[..., m * H * d:(m + 1) * H * d].reshape(B, N, H, d).transpose(0, 2, 1, 3) for m in (0, 1)])
    v = y[..., 2 * width:].reshape(B, N, H, 2 * d).transpose(0, 2, 1, 3)
    return out[0][0], out[1][0], out[0][1], out[1][1], v


def _v_from_k(x, w, H, d):
    q1, k1, q2, k2, _ = _in(x, w, H, d)
    return q1, k1, q2, k2, np.concatenate([k1, k2], axis=-1)


def _channel_major_concat(o, w_o):
    o, w = np.asarray(o, np.float64), np.asarray(w_o, np.float64)
    B, H, N, dv = o.shape
    cat = o.transpose(0, 2, 3, 1).reshape(B, N, H * dv)
    return cat @ w.T


MUTATIONS = {
    "q_k_halves_swapped": ("in_projection", _halves_swapped),
    "split_by_map_first": ("in_projection", _split_by_map_first),
    "v_from_k": ("in_projection", _v_from_k),
    "channel_major_concat": ("out_projection", _channel_major_concat),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(P, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, pytest.fail.Exception):
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
