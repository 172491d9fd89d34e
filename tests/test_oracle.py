"""Pins for the CPU fp64 oracle (no GPU).

Each test checks the oracle against something that does not come from the
oracle itself: values printed on the pages, closed forms, invariants the
mathematics fixes, or library routines (torch's float64 CPU
scaled_dot_product_attention and rms_norm).  The cases are chosen so that a
plausible slip in the oracle -- a dropped or sign-flipped lambda term, the
wrong 1/sqrt scale, a transposed operand, an off-by-one causal mask, eps in the
wrong place, (1 - lambda) instead of (1 - lambda_init), the wrong norm axis --
fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import diffattn_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(q, k, v, causal):
    """Library attention in float64 on the CPU: softmax(q k^T / sqrt(E)) v."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal).numpy()


def _rand_heads(seed, B, H, N, d, scale=1.0):
    r = _rng(seed)
    q1, k1, q2, k2 = (scale * r.standard_normal((B, H, N, d)) for _ in range(4))
    v = r.standard_normal((B, H, N, 2 * d))
    return q1, k1, q2, k2, v


# ---------------------------------------------------------------------------
# values printed on the pages


def _six_key_inputs(fix):
    """Q, K chosen so that Q K^T / sqrt(d) equals the example's scores exactly.

    d = 4, q = [2,0,0,0], k_j = [s_j,0,0,0]  =>  q.k_j / sqrt(4) = s_j.
    V = [I_6 | 0] (6 x 2d) so that Y's first six channels are the weights.
    Every query row is the same q, non-causal, so every row of Y is the row
    the page prints.
    """
    s1 = np.array(fix["setup"]["scores_map1"])
    s2 = np.array(fix["setup"]["scores_map2"])
    n, d = len(s1), 4
    q = np.zeros((n, d))
    q[:, 0] = 2.0
    k1 = np.zeros((n, d))
    k1[:, 0] = s1
    k2 = np.zeros((n, d))
    k2[:, 0] = s2
    v = np.zeros((n, 2 * d))
    v[:, :n] = np.eye(n)
    return q, k1, q.copy(), k2, v


def test_six_key_example_printed_values():
    with open(os.path.join(GOLDEN, "six_key_example.json")) as f:
        fix = json.load(f)
    pr, dp = fix["printed"], fix["printed_decimals"]
    irr = fix["setup"]["irrelevant_keys"]
    q1, k1, q2, k2, v = _six_key_inputs(fix)
    z = np.zeros(4)
    lam = O.lambda_scalar(z, z, z, z, lambda_init=fix["setup"]["lambda"])
    assert lam == fix["setup"]["lambda"]

    a1 = O.attention_map(q1, k1, causal=False)
    assert np.array_equal(np.round(a1[0], dp), pr["standard_softmax_attn"])
    assert round(a1[0, irr].sum(), dp) == pr["standard_weight_on_irrelevant"]

    d = O.diff_weights(q1, k1, q2, k2, lam, causal=False)
    assert np.array_equal(np.round(d[0], dp) + 0.0, pr["differential_attn"])
    assert round(d[0, irr].sum(), dp) == pr["differential_weight_on_irrelevant"]

    # the same numbers through the whole multi-head path (Eq. 1 output, pre-norm)
    y = O.forward(*(t[None, None] for t in (q1, k1, q2, k2, v)), lam=lam, lambda_init=0.5,
                  causal=False, norm=False)[0, 0]
    for row in y:
        assert np.all(np.abs(row[:6] - np.array(pr["differential_attn"])) <= 5e-4)
        assert np.all(row[6:] == 0.0)
    # lambda = 0 recovers the printed standard map
    y0 = O.forward(*(t[None, None] for t in (q1, k1, q2, k2, v)), lam=0.0, lambda_init=0.0,
                   causal=False, norm=False)[0, 0]
    assert np.all(np.abs(y0[0, :6] - np.array(pr["standard_softmax_attn"])) <= 5e-4)


def test_six_key_exact_closed_form():
    # e^0.5 and e^3 written out: the map-1 weights are e^s / (5 e^0.5 + e^3)
    Z = 5 * math.exp(0.5) + math.exp(3.0)
    with open(os.path.join(GOLDEN, "six_key_example.json")) as f:
        fix = json.load(f)
    q1, k1, q2, k2, _ = _six_key_inputs(fix)
    d = O.diff_weights(q1, k1, q2, k2, 0.5, causal=False)[0]
    assert abs(d[1] - (math.exp(3.0) / Z - 0.5 / 6)) < 1e-15
    assert abs(d[0] - (math.exp(0.5) / Z - 0.5 / 6)) < 1e-15


# ---------------------------------------------------------------------------
# lambda (Eq. 2)


def test_lambda_closed_form():
    d = 8
    r = _rng(1)
    # lq1 . lk1 = ln 3 and lq2 . lk2 = ln 2 by construction (orthogonal noise added)
    lk1 = r.standard_normal(d)
    lq1 = math.log(3.0) * lk1 / np.dot(lk1, lk1)
    lk2 = r.standard_normal(d)
    lq2 = math.log(2.0) * lk2 / np.dot(lk2, lk2)
    assert abs(O.lambda_scalar(lq1, lk1, lq2, lk2, 0.8) - (3.0 - 2.0 + 0.8)) < 1e-12
    # swapping the two products flips the sign of the exponential difference
    assert abs(O.lambda_scalar(lq2, lk2, lq1, lk1, 0.8) - (2.0 - 3.0 + 0.8)) < 1e-12
    # all-zero vectors: exp(0) - exp(0) cancels
    z = np.zeros(d)
    assert O.lambda_scalar(z, z, z, z, 0.37) == 0.37


# ---------------------------------------------------------------------------
# invariants


@pytest.mark.parametrize("lam", [-0.3, 0.0, 0.5, 1.0, 1.7])
@pytest.mark.parametrize("causal", [True, False])
def test_rows_sum_to_one_minus_lambda(lam, causal):
    q1, k1, q2, k2, _ = _rand_heads(2, 1, 1, 37, 16)
    d = O.diff_weights(q1[0, 0], k1[0, 0], q2[0, 0], k2[0, 0], lam, causal)
    assert np.allclose(d.sum(-1), 1.0 - lam, atol=1e-13, rtol=0)
    if causal:
        assert np.all(d[np.triu_indices(37, 1)] == 0.0)


def test_key_permutation_invariance_noncausal():
    q1, k1, q2, k2, v = _rand_heads(3, 1, 1, 29, 16)
    perm = _rng(4).permutation(29)
    a = O.forward(q1, k1, q2, k2, v, 0.6, 0.8, causal=False)
    b = O.forward(q1, k1[..., perm, :], q2, k2[..., perm, :], v[..., perm, :], 0.6, 0.8, causal=False)
    assert np.allclose(a, b, atol=1e-13, rtol=0)


def test_shared_maps_reduce_to_scaled_attention():
    q, k, _, _, v = _rand_heads(5, 2, 3, 41, 16)
    lam = 0.3
    y = O.forward(q, k, q, k, v, lam, 0.8, causal=True, norm=False)
    assert np.allclose(y, (1 - lam) * _sdpa(q, k, v, True), atol=1e-12, rtol=0)


def test_large_logits_shift_invariance():
    # Logits near +-300 (the pages report trained top-1 logits of 318).  Adding
    # t*u to every key shifts each query's logits by the same per-row constant,
    # which softmax ignores; a missing max-subtraction overflows instead.
    q1, k1, q2, k2, v = _rand_heads(6, 1, 2, 33, 16)
    u = np.zeros(16)
    u[0] = 1.0
    q1[..., 0] = np.abs(q1[..., 0]) + 1.0
    base = O.forward(q1, k1, q2, k2, v, 0.4, 0.8)
    k1s = k1 + 1200.0 * u
    shifted = O.forward(q1, k1s, q2, k2, v, 0.4, 0.8)
    s = np.einsum("bhnd,bhmd->bhnm", q1, k1s) / 4.0
    assert s.max() > 300
    assert np.all(np.isfinite(shifted))
    assert np.allclose(base, shifted, atol=1e-9, rtol=0)


def test_blocking_does_not_change_values():
    q1, k1, q2, k2, v = _rand_heads(7, 1, 2, 50, 16)
    a = O.forward(q1, k1, q2, k2, v, 0.7, 0.8, block=512)
    b = O.forward(q1, k1, q2, k2, v, 0.7, 0.8, block=3)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# special cases that reduce to library routines


@pytest.mark.parametrize("causal", [True, False])
def test_lambda_zero_is_standard_attention(causal):
    q1, k1, q2, k2, v = _rand_heads(8, 2, 2, 45, 16)
    y = O.forward(q1, k1, q2, k2, v, 0.0, 0.0, causal=causal, norm=False)
    ref = _sdpa(q1, k1, v, causal)
    assert np.allclose(y, ref, atol=1e-12, rtol=0)
    out = O.forward(q1, k1, q2, k2, v, 0.0, 0.0, causal=causal, norm=True, eps=1e-5)
    refn = F.rms_norm(torch.from_numpy(ref), (v.shape[-1],), eps=1e-5).numpy()
    assert np.allclose(out, refn, atol=1e-12, rtol=0)


@pytest.mark.parametrize("d", [16, 64])
def test_linearity_against_two_library_attentions(d):
    q1, k1, q2, k2, v = _rand_heads(9 + d, 1, 2, 70, d)
    lam, lam_init, eps = 0.73, 0.35, 1e-5
    w = _rng(10).uniform(0.5, 1.5, 2 * d)
    y = O.forward(q1, k1, q2, k2, v, lam, lam_init, causal=True, norm=False)
    yref = _sdpa(q1, k1, v, True) - lam * _sdpa(q2, k2, v, True)
    assert np.allclose(y, yref, atol=1e-12, rtol=0)
    out = O.forward(q1, k1, q2, k2, v, lam, lam_init, weight=w, eps=eps, causal=True)
    outref = (1 - lam_init) * F.rms_norm(torch.from_numpy(yref), (2 * d,),
                                         weight=torch.from_numpy(w), eps=eps).numpy()
    assert np.allclose(out, outref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# closed forms


def test_causal_row0_closed_form():
    # row 0 sees only key 0, so D[0] = [1 - lambda, 0, ...] and Y[0] = (1 - lambda) V[0]
    q1, k1, q2, k2, v = _rand_heads(11, 1, 1, 12, 16)
    lam, lam_init, eps = 0.62, 0.2, 1e-5
    out = O.forward(q1, k1, q2, k2, v, lam, lam_init, eps=eps)[0, 0, 0]
    y0 = (1 - lam) * v[0, 0, 0]
    ref = (1 - lam_init) * y0 / math.sqrt(np.mean(y0 ** 2) + eps)
    assert np.allclose(out, ref, atol=1e-13, rtol=0)


@pytest.mark.parametrize("c", [1.0, 1e-3, 0.0])
def test_rmsnorm_constant_vector_closed_form(c):
    # a constant vector c: mean(y^2) = c^2, so out = (1 - lambda_init) w c / sqrt(c^2 + eps);
    # with c = 1e-3 the eps term is 10% of the denominator, so its placement matters.
    y = np.full((3, 32), c)
    w = np.linspace(0.5, 2.0, 32)
    out = O.head_rmsnorm_scale(y, w, 1e-5, 0.8)
    ref = 0.2 * w * c / math.sqrt(c * c + 1e-5)
    assert np.allclose(out, np.broadcast_to(ref, out.shape), atol=1e-15, rtol=1e-13)


def test_scale_is_one_minus_lambda_init_not_lambda():
    # V = ones: Y = (1 - lambda) everywhere, so the norm gives sign(1 - lambda) and the
    # output is exactly (1 - lambda_init) (1-lambda)/sqrt((1-lambda)^2 + eps)
    q1, k1, q2, k2, _ = _rand_heads(12, 1, 1, 20, 16)
    v = np.ones((1, 1, 20, 32))
    for lam in (-0.3, 0.5, 1.7):
        out = O.forward(q1, k1, q2, k2, v, lam, 0.8, eps=1e-5)
        ref = 0.2 * (1 - lam) / math.sqrt((1 - lam) ** 2 + 1e-5)
        assert np.allclose(out, ref, atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------
# brute force on tiny inputs


def _brute(q1, k1, q2, k2, v, lam, lam_init, eps, causal):
    """Scalar loops over one head, written without arrays or softmax helpers."""
    n, d = len(q1), len(q1[0])
    out = []
    for i in range(n):
        keys = [j for j in range(n) if (j <= i or not causal)]
        l1 = {j: sum(q1[i][t] * k1[j][t] for t in range(d)) / math.sqrt(d) for j in keys}
        l2 = {j: sum(q2[i][t] * k2[j][t] for t in range(d)) / math.sqrt(d) for j in keys}
        m1, m2 = max(l1.values()), max(l2.values())
        z1 = sum(math.exp(l1[j] - m1) for j in keys)
        z2 = sum(math.exp(l2[j] - m2) for j in keys)
        y = [0.0] * len(v[0])
        for j in keys:
            wgt = math.exp(l1[j] - m1) / z1 - lam * math.exp(l2[j] - m2) / z2
            for c in range(len(y)):
                y[c] += wgt * v[j][c]
        r = math.sqrt(sum(t * t for t in y) / len(y) + eps)
        out.append([(1 - lam_init) * t / r for t in y])
    return np.array(out)


@pytest.mark.parametrize("n,causal", [(1, True), (5, True), (6, False)])
def test_brute_force_tiny(n, causal):
    q1, k1, q2, k2, v = _rand_heads(13 + n, 1, 1, n, 4)
    got = O.forward(q1, k1, q2, k2, v, 0.45, 0.6, eps=1e-5, causal=causal)[0, 0]
    ref = _brute(*(t[0, 0].tolist() for t in (q1, k1, q2, k2, v)), 0.45, 0.6, 1e-5, causal)
    assert np.allclose(got, ref, atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------
# sampled rows and decode


def test_forward_rows_matches_forward():
    q1, k1, q2, k2, v = _rand_heads(14, 1, 1, 64, 16)
    full = O.forward(q1, k1, q2, k2, v, 0.5, 0.8)[0, 0]
    rows = np.array([0, 1, 17, 31, 32, 63])
    part = O.forward_rows(q1[0, 0], k1[0, 0], q2[0, 0], k2[0, 0], v[0, 0], rows, 0.5, 0.8)
    assert np.array_equal(part, full[rows])


def test_decode_equals_last_causal_prefill_row():
    q1, k1, q2, k2, v = _rand_heads(15, 3, 2, 40, 16)
    lens = np.array([40, 17, 1])
    dec = O.decode(q1[:, :, -1], q2[:, :, -1], k1, k2, v, None, 0.55, 0.8)
    pre = O.forward(q1, k1, q2, k2, v, 0.55, 0.8)[:, :, -1]
    assert np.allclose(dec, pre, atol=1e-13, rtol=0)
    # with shorter caches, sequence b equals the prefill of its first lens[b] tokens
    dec2 = O.decode(np.stack([q1[b, :, lens[b] - 1] for b in range(3)]),
                    np.stack([q2[b, :, lens[b] - 1] for b in range(3)]),
                    k1, k2, v, lens, 0.55, 0.8)
    for b in range(3):
        n = lens[b]
        pre_b = O.forward(q1[b:b + 1, :, :n], k1[b:b + 1, :, :n], q2[b:b + 1, :, :n],
                          k2[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.55, 0.8)[0, :, -1]
        assert np.allclose(dec2[b], pre_b, atol=1e-13, rtol=0)


def test_decode_empty_cache_gives_zeros():
    q1, k1, q2, k2, v = _rand_heads(16, 2, 2, 8, 16)
    out = O.decode(q1[:, :, 0], q2[:, :, 0], k1, k2, v, np.array([0, 8]), 0.5, 0.8)
    assert np.all(out[0] == 0.0)
    assert np.all(np.isfinite(out[1])) and np.any(out[1] != 0.0)


def test_bf16_inputs_upcast_exactly():
    x = torch.randn(4, 8).to(torch.bfloat16)
    assert np.array_equal(O._f64(x), x.float().numpy().astype(np.float64))
