"""Each plausible mistake in the e4m3 oracle fails at least one of its pins.

The mistakes are planted in the oracle (on the CPU, by replacing a module
function or table for the duration of one test) and the pins of
tests/test_oracle_fp8.py are run against the mutated oracle; every mutation
must make at least one pin fail.
"""

import numpy as np
import pytest

from oracle import fp8_oracle as F

import test_oracle_fp8 as pins

PINS = [pins.test_spec_values, pins.test_binade_spacing, pins.test_round_trip_every_code,
        pins.test_midpoints_tie_to_even_and_neighbours, pins.test_saturation_and_sign,
        pins.test_against_torch_float8, pins.test_quantize_invariants, pins.test_quantize_zero_tensor]

_encode = F.encode


def _bias8_table():
    t = F._TABLE.copy()
    for code in range(256):
        e, m = (code >> 3) & 0xF, code & 7
        if not (e == 0xF and m == 7):
            sign = -1.0 if code & 0x80 else 1.0
            t[code] = sign * ((m / 8.0) * 2.0 ** -7 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 8))
    return t


def _ties_away(y):
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y).ravel()
    pos = F._POS
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, len(pos) - 1)
    lo = np.maximum(hi - 1, 0)
    code = np.where(pos[hi] - a <= a - pos[lo], hi, lo)
    code = np.where(a >= 448.0, 0x7E, code) | np.where(np.signbit(y.ravel()), 0x80, 0)
    return code.astype(np.uint8).reshape(y.shape)


def _no_saturation(y):
    c = _encode(np.where(np.abs(np.asarray(y, dtype=np.float64)) >= 448.0, 0.0, y))
    big = np.abs(np.asarray(y, dtype=np.float64)) >= 448.0
    return np.where(big, c | 0x7F, c).astype(np.uint8)


def _sign_lost_on_underflow(y):
    c = _encode(y)
    return np.where((c & 0x7F) == 0, 0, c).astype(np.uint8)


def _quantize_240(x):
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    if amax == 0:
        return F.encode(x32), np.float32(1.0)
    return F.encode((x32 * np.float32(np.float32(240.0) / amax)).astype(np.float32)), np.float32(amax / np.float32(240.0))


MUTATIONS = {
    "bias_8": ("_TABLE", _bias8_table),
    "ties_away_from_zero": ("encode", lambda: _ties_away),
    "no_saturation": ("encode", lambda: _no_saturation),
    "sign_lost_on_underflow": ("encode", lambda: _sign_lost_on_underflow),
    "absmax_to_240": ("quantize", lambda: _quantize_240),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(monkeypatch, name):
    attr, make = MUTATIONS[name]
    monkeypatch.setattr(F, attr, make())
    if attr == "_TABLE":
        monkeypatch.setattr(F, "_POS", F._TABLE[:0x7F])
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, pytest.fail.Exception):
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
