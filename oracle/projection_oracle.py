"""Oracle for the projections on either side of differential attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call this module.  It shares no code with the HIP path and imports
nothing from the package.  Plain NumPy in float64.

What the pages fix: each head's query and key projections are split into
two halves, Q1/K1 and Q2/K2, instead of being doubled (page 2 = "Differential
attention", datarekha.com, section "How it's wired"); heads are halved so
that h = d_model / 2d and the layer drops into a standard (LLaMA-style)
block (page 3 = "Differential Transformer" sample peer review, "Strengths").

Readings taken where the pages are silent (listed in the design notes):

* weights follow the linear-layer convention W[out_features, in_features]
  (y = x W^T); the in-projection weight is the row concatenation
  [W_Q; W_K; W_V], each [H*2d, d_model], with no bias;
* head h owns output features h*2d .. h*2d + 2d - 1 of each of W_Q, W_K,
  W_V; of a head's 2d query (key) features the first d are Q1 (K1) and the
  last d are Q2 (K2); V takes all 2d;
* the out-projection concatenates the heads' [N, 2d] outputs along the
  feature axis in head order and multiplies by W_O^T, W_O [d_out, H*2d],
  no bias.

Pinned by ``tests/test_oracle_projection.py``.
"""

from __future__ import annotations

import numpy as np

__all__ = ["in_projection", "out_projection"]


def _f64(t) -> np.ndarray:
    if hasattr(t, "detach"):
        t = t.detach().cpu().float().numpy()
    return np.asarray(t, dtype=np.float64)


def in_projection(x, w_qkv, H: int, d: int):
    """x [B, N, d_model], w_qkv [3*H*2d, d_model] -> (q1, k1, q2, k2 [B, H, N, d],
    v [B, H, N, 2d])."""
    x, w = _f64(x), _f64(w_qkv)
    B, N, _ = x.shape
    width = H * 2 * d
    assert w.shape[0] == 3 * width
    y = x @ w.T  # [B, N, 3 * H * 2d]
    q, k, v = y[..., :width], y[..., width:2 * width], y[..., 2 * width:]

    def heads(t):  # [B, N, H*2d] -> [B, H, N, 2d]
        return t.reshape(B, N, H, 2 * d).transpose(0, 2, 1, 3)

    q, k, v = heads(q), heads(k), heads(v)
    return (q[..., :d].copy(), k[..., :d].copy(), q[..., d:].copy(), k[..., d:].copy(), v.copy())


def out_projection(o, w_o):
    """o [B, H, N, 2d] (the attention's per-head output), w_o [d_out, H*2d] ->
    y [B, N, d_out]."""
    o, w = _f64(o), _f64(w_o)
    B, H, N, dv = o.shape
    cat = o.transpose(0, 2, 1, 3).reshape(B, N, H * dv)
    return cat @ w.T
