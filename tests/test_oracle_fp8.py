"""Pins of the e4m3 oracle (oracle/fp8_oracle.py) to facts outside it.

* decoded values that the OCP 8-bit floating point specification fixes for
  e4m3 (1.0 = 0x38, 448 = 0x7E, smallest subnormal 2^-9, NaN codes);
* closed forms: the spacing of the values inside each binade;
* a library routine: torch's float8_e4m3fn conversions (round to nearest
  even) agree with encode / decode wherever torch does not produce NaN;
* invariants of quantisation: the absmax element maps to +-448, the error of
  every element is at most half the local spacing times the scale.
"""

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as F

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_spec_values():
    v = F.decode(np.array([0x00, 0x01, 0x07, 0x08, 0x30, 0x38, 0x40, 0x44, 0x7E, 0xB8, 0xFE], np.uint8))
    assert list(v) == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 0.5, 1.0, 2.0, 3.0, 448.0, -1.0, -448.0]
    assert np.isnan(F.decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert np.signbit(F.decode(np.array([0x80], np.uint8)))[0]


def test_binade_spacing():
    pos = F.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    gaps = np.diff(pos)
    for i, g in enumerate(gaps):
        lo = pos[i]
        if lo < 2.0 ** -6:
            assert g == 2.0 ** -9
        else:
            e = np.floor(np.log2(lo))
            assert g == 2.0 ** (e - 3), (i, lo, g)


def test_round_trip_every_code():
    codes = np.array(FINITE, np.uint8)
    assert np.array_equal(F.encode(F.decode(codes)), codes)


def test_midpoints_tie_to_even_and_neighbours():
    pos = F.decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    got = F.encode(mids)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    step = np.diff(pos) * 1e-3
    assert np.array_equal(F.encode(mids - step), lo.astype(np.uint8))
    assert np.array_equal(F.encode(mids + step), (lo + 1).astype(np.uint8))


def test_saturation_and_sign():
    got = F.encode(np.array([448.0, 459.0, 464.0, 1e6, -500.0, -0.0, -1e-6]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80]
    with pytest.raises(ValueError):
        F.encode(np.array([np.inf]))


def test_against_torch_float8():
    # torch converts with round to nearest even; above the largest finite
    # value its result is NaN (where the oracle saturates), so only finite
    # in-range values are compared
    g = np.random.default_rng(5)
    y = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    y = y.astype(np.float32)
    y = y[np.abs(y) < 440.0]
    mine = F.encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    codes = torch.tensor(FINITE, dtype=torch.uint8)
    assert np.array_equal(codes.view(torch.float8_e4m3fn).to(torch.float64).numpy(),
                          F.decode(codes.numpy()))


def test_quantize_invariants():
    g = np.random.default_rng(6)
    x = (g.standard_normal((3, 257)) * 2.5).astype(np.float32)
    codes, scale = F.quantize(x)
    assert scale == np.float32(np.max(np.abs(x)) / np.float32(448.0))
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] in (0x7E, 0xFE)
    deq = F.dequantize(codes, scale)
    y = np.abs(x.astype(np.float64)) / float(scale)
    half_gap = np.where(y < 2.0 ** -6, 2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 4))
    # y itself carries the float32 rounding of x * (448 / amax): allow its few ulps
    assert np.all(np.abs(deq - x) <= (half_gap + 4 * y * 2.0 ** -24) * float(scale))
    assert np.array_equal(np.signbit(deq[codes != 0x80]), np.signbit(x[codes != 0x80]))


def test_quantize_zero_tensor():
    codes, scale = F.quantize(np.zeros(10, np.float32))
    assert scale == 1.0 and not codes.any()
