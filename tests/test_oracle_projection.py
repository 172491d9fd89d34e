"""Pins of the projection oracle (oracle/projection_oracle.py).

* brute force: scalar loops over (b, t, feature) with the head / half index
  arithmetic written out, on tiny shapes;
* special cases: selection weights (each output feature copies one input
  channel) make every head's Q1, Q2, K1, K2, V a known slice of x; an
  identity W_O makes the out-projection the head concatenation, built here
  by explicit per-head placement;
* a library routine: torch.nn.functional.linear in float64 on the flattened
  tokens for the unsplit products.
"""

import numpy as np
import torch

from oracle import projection_oracle as P


def _tiny(seed, B=2, N=3, H=2, d=2, dm=5):
    g = np.random.default_rng(seed)
    return g.standard_normal((B, N, dm)), g.standard_normal((3 * H * 2 * d, dm)), H, d


def test_in_projection_brute_force():
    x, w, H, d = _tiny(1)
    q1, k1, q2, k2, v = P.in_projection(x, w, H, d)
    B, N, dm = x.shape
    width = H * 2 * d
    for b in range(B):
        for t in range(N):
            for f in range(3 * width):
                val = sum(x[b, t, i] * w[f, i] for i in range(dm))
                part, r = divmod(f, width)
                h, c = divmod(r, 2 * d)
                if part == 2:
                    assert abs(v[b, h, t, c] - val) < 1e-12
                else:
                    half, j = divmod(c, d)
                    dst = [[q1, q2], [k1, k2]][part][half]
                    assert abs(dst[b, h, t, j] - val) < 1e-12


def test_in_projection_selection_weights():
    B, N, H, d = 2, 4, 3, 4
    dm = H * 2 * d
    x = np.random.default_rng(2).standard_normal((B, N, dm))
    perm = np.random.default_rng(3).permutation(dm)
    w = np.zeros((3 * dm, dm))
    for f in range(3 * dm):
        w[f, perm[f % dm] if f < dm else (f % dm)] = 1.0  # Q features permuted, K and V identity
    q1, k1, q2, k2, v = P.in_projection(x, w, H, d)
    for h in range(H):
        lo = 2 * d * h
        assert np.array_equal(q1[:, h], x[:, :, perm[lo:lo + d]])
        assert np.array_equal(q2[:, h], x[:, :, perm[lo + d:lo + 2 * d]])
        assert np.array_equal(k1[:, h], x[:, :, lo:lo + d])
        assert np.array_equal(k2[:, h], x[:, :, lo + d:lo + 2 * d])
        assert np.array_equal(v[:, h], x[:, :, lo:lo + 2 * d])


def test_out_projection_identity_is_head_concatenation():
    B, H, N, dv = 2, 3, 5, 4
    o = np.random.default_rng(4).standard_normal((B, H, N, dv))
    y = P.out_projection(o, np.eye(H * dv))
    for b in range(B):
        for t in range(N):
            row = np.empty(H * dv)
            for h in range(H):
                row[h * dv:(h + 1) * dv] = o[b, h, t]
            assert np.array_equal(y[b, t], row)


def test_out_projection_brute_force():
    B, H, N, dv, dout = 1, 2, 3, 4, 3
    g = np.random.default_rng(5)
    o, w = g.standard_normal((B, H, N, dv)), g.standard_normal((dout, H * dv))
    y = P.out_projection(o, w)
    for t in range(N):
        for f in range(dout):
            val = sum(o[0, h, t, c] * w[f, h * dv + c] for h in range(H) for c in range(dv))
            assert abs(y[0, t, f] - val) < 1e-12


def test_against_torch_linear():
    x, w, H, d = _tiny(6, B=3, N=7, H=2, d=4, dm=16)
    q1, k1, q2, k2, v = P.in_projection(x, w, H, d)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy()
    width = H * 2 * d
    # the V block of head 1 and the K2 half of head 0
    assert np.allclose(v[:, 1], ref[:, :, 2 * width + 2 * d:2 * width + 4 * d], rtol=0, atol=1e-12)
    assert np.allclose(k2[:, 0], ref[:, :, width + d:width + 2 * d], rtol=0, atol=1e-12)
    o = np.random.default_rng(7).standard_normal((3, H, 7, 2 * d))
    wo = np.random.default_rng(8).standard_normal((10, H * 2 * d))
    cat = torch.cat([torch.from_numpy(o[:, h]) for h in range(H)], dim=-1)
    assert np.allclose(P.out_projection(o, wo), torch.nn.functional.linear(cat, torch.from_numpy(wo)).numpy(),
                       rtol=0, atol=1e-12)
