"""Oracle for the fp8 (e4m3) query/key path of the differential-attention forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call this module.  It shares no code with the HIP path and imports
nothing from the package.

What the pages say: the review page ("Differential Transformer" sample
peer review, reviewpaper.ai) notes in "Strengths" that the differential map
has far smaller attention-logit outliers (top-1 logits 38.8 against 318.0,
Table 5) and cites a 4-bit quantisation study of the attention LOGITS
(Fig. 8) as pointing to low-bit attention kernels; its "Questions" ask
whether that study's absmax quantisation is applied to each of the two logit
matrices separately, per head or per tensor.  The pages therefore quantise
logits, not queries and keys, and give no format.

This build's reading (an engineering one, not the pages'): the low-bit
attention kernel that gfx950's matrix cores make worthwhile quantises the
OPERANDS of the logit product, Q and K, to the 8-bit e4m3 format of the OCP
"8-bit floating point" specification (sign, 4 exponent bits with bias 7, 3
mantissa bits; subnormals at exponent field 0; no infinities; 0x7F / 0xFF
are NaN; largest finite value 448), so that the logits are formed by the fp8
product; the logits themselves stay fp32.

Readings taken where the pages are silent (listed in the design notes):

* one absmax scale per tensor: scale = max|x| / 448 (float32 division), and
  the values encoded are x * (448 / max|x|) (float32 division and product);
  an all-zero tensor takes scale 1;
* encoding rounds to the nearest e4m3 value, ties to the even code, and
  saturates magnitudes at or above 448 to 448; the code keeps the sign of its
  input (negative values that round to zero give 0x80);
* the attention then runs on the dequantised values code_value * scale: the
  fp8 path changes the inputs of Eq. 1, nothing after them.

``decode`` is the format's definition written out; ``encode`` picks the
nearest of the 127 finite non-negative values by search, not by bit
manipulation.  Pinned by ``tests/test_oracle_fp8.py``.
"""

from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "decode", "encode", "quantize", "dequantize"]

E4M3_MAX = 448.0


def _decode_table() -> np.ndarray:
    """Value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            t[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_TABLE = _decode_table()
_POS = _TABLE[:0x7F]  # codes 0x00..0x7E: increasing, finite, non-negative


def decode(codes) -> np.ndarray:
    """e4m3 codes (uint8 array) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y) -> np.ndarray:
    """float values -> nearest e4m3 codes (ties to even, saturating at 448).

    ``y`` must be finite.  Comparisons are made in float64, in which every
    float32 input and every e4m3 value is exact.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("e4m3 encoding takes finite values")
    a = np.abs(y).ravel()
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code | np.where(np.signbit(y.ravel()), 0x80, 0)
    return code.astype(np.uint8).reshape(y.shape)


def quantize(x):
    """Per-tensor absmax quantisation -> (codes uint8, scale float32).

    x: any float array whose values are exact in float32 (bf16 or fp32 data).
    """
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    if amax > 0:
        scale = np.float32(amax / np.float32(E4M3_MAX))
        inv = np.float32(np.float32(E4M3_MAX) / amax)
    else:
        scale = np.float32(1.0)
        inv = np.float32(1.0)
    y = (x32 * inv).astype(np.float32)
    return encode(y), scale


def dequantize(codes, scale) -> np.ndarray:
    """codes, scale -> float64 values code_value * scale."""
    return decode(codes) * np.float64(np.float32(scale))
