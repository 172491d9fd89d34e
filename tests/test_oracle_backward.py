"""Pins for the oracle's gradients and per-map statistics (no GPU).

The backward is checked against things that do not come from its own
formulas: central finite differences of the (separately pinned) oracle
forward over every input entry of tiny cases, and float64 autograd through
library routines (torch's scaled_dot_product_attention and rms_norm).  A
dropped term of the RMSNorm Jacobian, a lambda sign, a transposed dS, a
missing 1/sqrt(d) or a wrong Eq. 2 chain factor fails these.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import diffattn_oracle as O


def _case(seed, B, H, N, d, lam_std=0.3, lambda_init=0.7):
    r = np.random.default_rng(seed)
    x = {k: r.standard_normal((B, H, N, d)) for k in ("q1", "k1", "q2", "k2")}
    x["v"] = r.standard_normal((B, H, N, 2 * d))
    for k in ("lq1", "lk1", "lq2", "lk2"):
        x[k] = lam_std * r.standard_normal(d)
    x["weight"] = 1.0 + 0.5 * r.standard_normal(2 * d)
    x["dout"] = r.standard_normal((B, H, N, 2 * d))
    x["lambda_init"] = lambda_init
    return x


def _loss(x, causal, eps):
    lam = O.lambda_scalar(x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"])
    out = O.forward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, x["lambda_init"],
                    weight=x["weight"], eps=eps, causal=causal)
    return float(np.sum(out * x["dout"]))


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_central_differences(causal):
    eps = 1e-3
    x = _case(7, 1, 2, 5, 3)
    g = O.backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"], x["lk2"],
                   x["lambda_init"], x["dout"], weight=x["weight"], eps=eps, causal=causal)
    h = 1e-6
    names = {"q1": "dq1", "k1": "dk1", "q2": "dq2", "k2": "dk2", "v": "dv", "weight": "dweight",
             "lq1": "dlq1", "lk1": "dlk1", "lq2": "dlq2", "lk2": "dlk2"}
    for name, gname in names.items():
        num = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            old = x[name][idx]
            x[name][idx] = old + h
            up = _loss(x, causal, eps)
            x[name][idx] = old - h
            dn = _loss(x, causal, eps)
            x[name][idx] = old
            num[idx] = (up - dn) / (2 * h)
        err = np.max(np.abs(num - g[gname]))
        assert err <= 1e-6 * max(1.0, np.max(np.abs(num))), (name, err)


def _torch_reference(x, causal, eps):
    """Autograd of the same forward composed from library routines."""
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in x.items() if isinstance(v, np.ndarray) and k != "dout"}
    lam = torch.exp(t["lq1"] @ t["lk1"]) - torch.exp(t["lq2"] @ t["lk2"]) + x["lambda_init"]
    y = (F.scaled_dot_product_attention(t["q1"], t["k1"], t["v"], is_causal=causal)
         - lam * F.scaled_dot_product_attention(t["q2"], t["k2"], t["v"], is_causal=causal))
    out = (1.0 - x["lambda_init"]) * F.rms_norm(y, (y.shape[-1],), weight=t["weight"], eps=eps)
    (out * torch.tensor(x["dout"])).sum().backward()
    return {k: v.grad.numpy() for k, v in t.items()}, float(lam.detach())


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [4, 16])
def test_backward_matches_library_autograd(causal, d):
    eps = 1e-5
    x = _case(11 + d, 2, 3, 37, d)
    ref, _ = _torch_reference(x, causal, eps)
    g = O.backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"], x["lk2"],
                   x["lambda_init"], x["dout"], weight=x["weight"], eps=eps, causal=causal)
    for k in ("q1", "k1", "q2", "k2", "v", "weight", "lq1", "lk1", "lq2", "lk2"):
        err = np.max(np.abs(ref[k] - g["d" + k]))
        assert err <= 1e-10 * max(1.0, np.max(np.abs(ref[k]))), (k, err)


def test_backward_lambda_zero_leaves_map2_without_gradient():
    """lambda = 0 (zero vectors, lambda_init 0): map 2 does not reach the
    output, so dQ2 = dK2 = 0, while dlambda (the slope in lambda) does not vanish."""
    x = _case(3, 1, 2, 9, 4, lam_std=0.0, lambda_init=0.0)
    g = O.backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"], x["lk2"],
                   0.0, x["dout"], weight=x["weight"], eps=1e-5, causal=True)
    assert np.max(np.abs(g["dq2"])) == 0.0 and np.max(np.abs(g["dk2"])) == 0.0
    assert abs(g["dlambda"]) > 1e-6
    # zero vectors: exp(0) = 1, so the Eq. 2 chain factors are the other vector (here 0)
    assert np.max(np.abs(g["dlq1"])) == 0.0


def test_map_stats_match_library_routines():
    x = _case(5, 1, 1, 23, 8)
    q1, k1, q2, k2, v = (x[k][0, 0] for k in ("q1", "k1", "q2", "k2", "v"))
    lse1, lse2, o1, o2 = O.map_stats(q1, k1, q2, k2, v, causal=True)
    for q, k, lse, o in ((q1, k1, lse1, o1), (q2, k2, lse2, o2)):
        s = torch.tensor(q @ k.T / math.sqrt(8))
        s = s.masked_fill(torch.ones(23, 23, dtype=torch.bool).triu(1), float("-inf"))
        assert np.max(np.abs(torch.logsumexp(s, -1).numpy() - lse)) < 1e-12
        ref = F.scaled_dot_product_attention(torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None],
                                             is_causal=True)[0].numpy()
        assert np.max(np.abs(ref - o)) < 1e-12
    lam = 0.37
    y = O.pre_norm(q1, k1, q2, k2, v, lam, causal=True)
    assert np.max(np.abs((o1 - lam * o2) - y)) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_backward_dq_rows_match_backward(causal):
    """The row-at-a-time dQ equals the full backward's dQ rows."""
    x = _case(23, 1, 1, 41, 8)
    g = O.backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"], x["lk2"],
                   x["lambda_init"], x["dout"], weight=x["weight"], eps=1e-5, causal=causal)
    rows = np.array([0, 1, 17, 40])
    sl = lambda k: x[k][0, 0]
    d1, d2 = O.backward_dq_rows(sl("q1"), sl("k1"), sl("q2"), sl("k2"), sl("v"), rows, x["lq1"], x["lk1"],
                                x["lq2"], x["lk2"], x["lambda_init"], x["dout"][0, 0][rows], weight=x["weight"],
                                eps=1e-5, causal=causal)
    assert np.max(np.abs(d1 - g["dq1"][0, 0][rows])) < 1e-12
    assert np.max(np.abs(d2 - g["dq2"][0, 0][rows])) < 1e-12


def test_backward_dk_sums_to_zero_over_keys():
    """Each row of dS sums to zero (softmax), so sum_j dK_k[j] = 0 per head:
    the property the long-sequence GPU test checks at full size."""
    x = _case(29, 2, 2, 33, 8)
    g = O.backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"], x["lk2"],
                   x["lambda_init"], x["dout"], weight=x["weight"], eps=1e-5, causal=True)
    for k in ("dk1", "dk2"):
        assert np.max(np.abs(g[k].sum(axis=2))) < 1e-12 * max(1.0, np.max(np.abs(g[k])))


@pytest.mark.parametrize("causal", [True, False])
def test_backward_dkv_keys_match_backward(causal):
    """The key-wise dK1, dK2, dV (each key's sum over the query rows that
    see it) equal the full backward's rows for those keys, at block sizes
    that split the rows unevenly, and summed over a split into row ranges."""
    x = _case(31, 1, 1, 53, 8)
    g = O.backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"], x["lk2"],
                   x["lambda_init"], x["dout"], weight=x["weight"], eps=1e-5, causal=causal)
    keys = np.array([0, 1, 7, 26, 51, 52])
    sl = lambda k: x[k][0, 0]
    args = (sl("q1"), sl("k1"), sl("q2"), sl("k2"), sl("v"), keys, x["lq1"], x["lk1"], x["lq2"], x["lk2"],
            x["lambda_init"], sl("dout"))
    for block in (5, 16, 64):
        dk1, dk2, dv = O.backward_dkv_keys(*args, weight=x["weight"], eps=1e-5, causal=causal, block=block)
        for got, name in ((dk1, "dk1"), (dk2, "dk2"), (dv, "dv")):
            ref = g[name][0, 0][keys]
            assert np.max(np.abs(got - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref))), (name, block)
    parts = [O.backward_dkv_keys(*args, weight=x["weight"], eps=1e-5, causal=causal, rows=r, block=7)
             for r in ((0, 20), (20, 33), (33, 53))]
    for i, name in enumerate(("dk1", "dk2", "dv")):
        got = sum(p[i] for p in parts)
        ref = g[name][0, 0][keys]
        assert np.max(np.abs(got - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref))), name


def test_backward_dkv_keys_last_key_sees_one_row():
    """Causal: the last key is seen by the last query row only, so its dV is
    D[N-1, N-1] dY_{N-1} -- checked against that row's own forward and dY
    written out from Eq. 3's Jacobian."""
    x = _case(37, 1, 1, 12, 4)
    sl = lambda k: x[k][0, 0]
    lam = O.lambda_scalar(x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"])
    _, _, dv = O.backward_dkv_keys(sl("q1"), sl("k1"), sl("q2"), sl("k2"), sl("v"), [11], x["lq1"], x["lk1"],
                                   x["lq2"], x["lk2"], x["lambda_init"], sl("dout"), weight=x["weight"],
                                   eps=1e-5, causal=True)
    dmap = O.diff_weights(sl("q1"), sl("k1"), sl("q2"), sl("k2"), lam, causal=True)
    y = dmap[11] @ sl("v")
    n = y.size
    r = math.sqrt(float(np.mean(y * y)) + 1e-5)
    g = (1 - x["lambda_init"]) * x["weight"] * sl("dout")[11]
    dy = g / r - y * float(np.dot(g, y)) / (n * r ** 3)
    assert np.max(np.abs(dv[0] - dmap[11, 11] * dy)) < 1e-12
