"""GPU parity of the training entry points against the CPU fp64 oracle.

diffattn_fwd_train's saved statistics are compared with ``map_stats``; the
gradients of diffattn_bwd (+ diffattn_lambda_bwd) with ``backward``.

Tolerance (derived from the arithmetic): the kernels round the softmax
weights, dY, dS and the outputs to bf16 (relative 2^-9 each) and accumulate
in fp32, so each gradient is compared as
max|gpu - oracle| <= 2e-2 * scale over the whole tensor -- the forward's
bf16 tolerance, taken relative to the gradient's scale because gradients
carry no fixed unit (scale: see ``_compare``).  The saved per-map outputs o12 are bounded like the
forward's Y (2e-2 absolute) and the log2-sum-exp to LSE_TOL.
"""

import math

import numpy as np
import pytest
import torch

from oracle import diffattn_oracle as O
from transformer_attention_diffattn_amd import binding as da
from transformer_attention_diffattn_amd import workloads as W

pytestmark = pytest.mark.gpu

REL = 2e-2
# the row sum behind the saved log2-sum-exp adds bf16-rounded weights (each
# within a relative 2^-9), so |d log2 L| <= 2^-9 / ln 2 = 2.8e-3
LSE_TOL = 3e-3
# sum over keys of dK: rounding each dK to bf16 moves the sum by at most
# 2^-9 of sum |dK|; twice that leaves room for the bf16 rounding of dS
KEY_SUM_TOL = 4e-3


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _inputs(B, H, N, d, seed, weight=True):
    x = W.prefill_inputs(B, H, N, d, "bf16", seed=seed, lam_std=0.3)
    g = torch.Generator().manual_seed(seed + 1)
    x["dout"] = torch.randn((B, H, N, 2 * d), generator=g).to(torch.bfloat16)
    if weight:
        x["weight"] = (1.0 + 0.5 * torch.randn(2 * d, generator=g)).float()
    return x


def _run(x, dev, causal):
    g = {k: (t.to(dev) if torch.is_tensor(t) else t) for k, t in x.items()}
    lam_t = da.lam(g["lq1"], g["lk1"], g["lq2"], g["lk2"], g["lambda_init"])
    out, lse, o12 = da.fwd_train(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], lam_t, g["lambda_init"],
                                 weight=g["weight"], eps=g["eps"], causal=causal)
    gr = da.bwd(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], g["dout"], lse, o12, lam_t, g["lambda_init"],
                weight=g["weight"], eps=g["eps"], causal=causal)
    dl = da.lambda_bwd(g["lq1"], g["lk1"], g["lq2"], g["lk2"], gr["dlambda"])
    gr.update(dlq1=dl[0], dlk1=dl[1], dlq2=dl[2], dlk2=dl[3])
    torch.cuda.synchronize()
    plain = da.fwd(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], lam_t, g["lambda_init"], weight=g["weight"],
                   eps=g["eps"], causal=causal)
    torch.cuda.synchronize()
    return out, plain, lse, o12, {k: v.float().cpu().numpy() for k, v in gr.items()}


def _compare(gr, ref, keys):
    """max|gpu - oracle| <= REL * scale per tensor, where scale is the
    tensor's own max|oracle|.  Except for dweight, it is floored at a tenth of
    the largest of the five input gradients of the same call: a gradient
    whose exact value is near zero (dQ, dK with a single visible key, where
    dS = 0; dlambda and the lambda-vector gradients when the norm removes
    lambda's effect, as with one key) then carries the rounding noise of its
    neighbours, not an unbounded relative error."""
    inputs = ("dq1", "dk1", "dq2", "dk2", "dv")
    big = max(float(np.max(np.abs(ref[k]))) for k in inputs if k in ref)
    rows = []
    for k in keys:
        got = np.asarray(gr[k], np.float64).reshape(ref[k].shape)
        err = float(np.max(np.abs(got - ref[k]))) if np.size(ref[k]) else 0.0
        own = float(np.max(np.abs(ref[k]))) if np.size(ref[k]) else 0.0
        # dweight (a sum of sigma dout Y / r over every row, never near zero
        # as a whole) is held to its own scale; the others take the floor
        scale = own if k == "dweight" else max(own, 0.1 * big)
        rows.append((k, err, scale, err <= REL * scale))
    print("  ".join(f"{k}: {e:.2e}/{s:.2e}" for k, e, s, _ in rows), flush=True)
    assert all(ok for *_, ok in rows), [r for r in rows if not r[3]]


def _oracle(x, causal):
    return O.backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"], x["lk2"],
                      x["lambda_init"], x["dout"], weight=x["weight"], eps=x["eps"], causal=causal)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [1, 77, 200])
def test_backward_small(dev, d, causal, N):
    print(f"case bwd d={d} causal={causal} N={N}", flush=True)
    x = _inputs(2, 2, N, d, seed=500 + N + d)
    out, plain, lse, o12, gr = _run(x, dev, causal)
    # the training forward writes the same output as the plain forward
    assert torch.equal(out, plain)
    # saved statistics against the oracle's per-map rows
    lse = lse.cpu().numpy()
    o12 = o12.cpu().numpy()
    for b in range(2):
        for h in range(2):
            l1, l2, r1, r2 = O.map_stats(x["q1"][b, h], x["k1"][b, h], x["q2"][b, h], x["k2"][b, h], x["v"][b, h],
                                         causal=causal)
            assert np.max(np.abs(lse[0, b, h] - l1 / math.log(2))) < LSE_TOL
            assert np.max(np.abs(lse[1, b, h] - l2 / math.log(2))) < LSE_TOL
            assert np.max(np.abs(o12[0, b, h] - r1)) < 2e-2
            assert np.max(np.abs(o12[1, b, h] - r2)) < 2e-2
    ref = _oracle(x, causal)
    _compare(gr, ref, ("dq1", "dk1", "dq2", "dk2", "dv", "dweight", "dlq1", "dlk1", "dlq2", "dlk2"))
    assert abs(gr["dlambda"][0] - ref["dlambda"]) <= REL * max(1.0, abs(ref["dlambda"])), (gr["dlambda"], ref["dlambda"])


def test_backward_without_weight_and_lambda_zero(dev):
    """No norm weight (ones) and lambda = 0: map 2's gradients vanish."""
    x = _inputs(1, 2, 130, 64, seed=9, weight=False)
    for k in ("lq1", "lk1", "lq2", "lk2"):
        x[k] = torch.zeros_like(x[k])
    x["lambda_init"] = 0.0
    g = {k: (t.to(dev) if torch.is_tensor(t) else t) for k, t in x.items()}
    lam_t = da.lam(g["lq1"], g["lk1"], g["lq2"], g["lk2"], 0.0)
    _, lse, o12 = da.fwd_train(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], lam_t, 0.0, eps=g["eps"])
    gr = da.bwd(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], g["dout"], lse, o12, lam_t, 0.0, eps=g["eps"])
    torch.cuda.synchronize()
    assert float(gr["dq2"].abs().max()) == 0.0 and float(gr["dk2"].abs().max()) == 0.0
    ref = O.backward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"], x["lk2"], 0.0,
                     x["dout"], weight=None, eps=x["eps"], causal=True)
    _compare({k: gr[k].float().cpu().numpy() for k in ("dq1", "dk1", "dv", "dweight")}, ref,
             ("dq1", "dk1", "dv", "dweight"))


def test_training_forward_every_row_3b_shape(dev):
    """Every row of the training forward at the 3B layer's shape is written,
    with its saved per-map outputs and log-sum-exps (768 items of 128 rows:
    exactly three rounds of a 256-CU part, whose last three take the
    three-permutation order).  With V = ones each map's output O_k is 1 in
    every channel, and the normalised output is (1 - lambda_init) (1 - lambda)
    / sqrt((1 - lambda)^2 + eps) (weight ones)."""
    print("case fwd_train every-row B=2 H=12 N=4096 d=128", flush=True)
    x = W.prefill_inputs(2, 12, 4096, 128, "bf16", seed=85, device=dev)
    v = torch.ones_like(x["v"])
    lam = 0.37
    lam_t = torch.tensor([lam], dtype=torch.float32, device=dev)
    out, lse, o12 = da.fwd_train(x["q1"], x["k1"], x["q2"], x["k2"], v, lam_t, x["lambda_init"], eps=x["eps"])
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    assert (o12 - 1.0).abs().max().item() <= 1e-5
    y = 1.0 - lam
    want = (1.0 - x["lambda_init"]) * y / math.sqrt(y * y + x["eps"])
    assert (out.float() - want).abs().max().item() <= 4e-3


def test_backward_deterministic(dev):
    x = _inputs(1, 3, 300, 64, seed=21)
    a = _run(x, dev, True)[4]
    b = _run(x, dev, True)[4]
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_training_entry_points_reject_bad_arguments(dev):
    x = _inputs(1, 1, 8, 16, seed=3)
    g = {k: (t.to(dev) if torch.is_tensor(t) else t) for k, t in x.items()}
    lam_t = da.lam(g["lq1"], g["lk1"], g["lq2"], g["lk2"], g["lambda_init"])
    with pytest.raises(RuntimeError):  # d = 16 has no backward
        da.fwd_train(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], lam_t, 0.8)
    assert da.bwd_workspace_bytes(1, 1, 8, 16) == 0
    assert da.bwd_workspace_bytes(1, 1, 8, 64) > 0


@pytest.mark.parametrize("name", ["layer1p4b_bf16_b4h16n2048d64", "layer3b_bf16_b2h12n4096d128"])
def test_full_size_backward_sampled_heads(dev, name):
    """The full workload in one launch; two (batch, head) slices compared in
    full against the oracle (rows and keys of a head depend only on that head)."""
    print(f"case bwd full {name}", flush=True)
    w = W.WORKLOADS[name]
    x = W.workload_inputs(name)
    gen = torch.Generator().manual_seed(w.seed + 7)
    x["dout"] = torch.randn(x["v"].shape, generator=gen).to(torch.bfloat16)
    g = {k: (t.to(dev) if torch.is_tensor(t) else t) for k, t in x.items()}
    lam_t = da.lam(g["lq1"], g["lk1"], g["lq2"], g["lk2"], g["lambda_init"])
    _, lse, o12 = da.fwd_train(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], lam_t, g["lambda_init"], eps=g["eps"])
    gr = da.bwd(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], g["dout"], lse, o12, lam_t, g["lambda_init"],
                eps=g["eps"])
    torch.cuda.synchronize()
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        sl = lambda t: t[b:b + 1, h:h + 1]
        ref = O.backward(sl(x["q1"]), sl(x["k1"]), sl(x["q2"]), sl(x["k2"]), sl(x["v"]), x["lq1"], x["lk1"],
                         x["lq2"], x["lk2"], x["lambda_init"], sl(x["dout"]), weight=None, eps=x["eps"],
                         causal=True)
        got = {k: gr[k][b, h].float().cpu().numpy() for k in ("dq1", "dk1", "dq2", "dk2", "dv")}
        _compare(got, {k: ref[k][0, 0] for k in got}, tuple(got))


def test_longctx_backward_sampled_rows_and_key_sums(dev):
    """The 64K-token workload (needles included) in one launch.  The dense
    oracle backward does not fit this length, so: dQ1 and dQ2 on sampled rows
    (needle offsets, first and last rows) from the row-wise oracle, and for
    every head the property that each map's dK sums to zero over the keys
    (every row of dS sums to zero), to KEY_SUM_TOL of the sum of |dK|."""
    name = "longctx_bf16_b1h12n65536d128"
    print(f"case bwd full {name}", flush=True)
    w = W.WORKLOADS[name]
    x = W.workload_inputs(name)
    gen = torch.Generator().manual_seed(w.seed + 7)
    x["dout"] = torch.randn(x["v"].shape, generator=gen).to(torch.bfloat16)
    g = {k: (t.to(dev) if torch.is_tensor(t) else t) for k, t in x.items()}
    lam_t = da.lam(g["lq1"], g["lk1"], g["lq2"], g["lk2"], g["lambda_init"])
    _, lse, o12 = da.fwd_train(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], lam_t, g["lambda_init"], eps=g["eps"])
    gr = da.bwd(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], g["dout"], lse, o12, lam_t, g["lambda_init"],
                eps=g["eps"])
    torch.cuda.synchronize()
    rows = np.array([0, 6, 7, 311, 5003, 40009, 65534, 65535])
    for h in (0, w.H - 1):
        sl = lambda t: t[0, h]
        d1, d2 = O.backward_dq_rows(sl(x["q1"]), sl(x["k1"]), sl(x["q2"]), sl(x["k2"]), sl(x["v"]), rows,
                                    x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"],
                                    sl(x["dout"])[rows], eps=x["eps"])
        got = {"dq1": gr["dq1"][0, h][rows].float().cpu().numpy(), "dq2": gr["dq2"][0, h][rows].float().cpu().numpy()}
        _compare(got, {"dq1": d1, "dq2": d2, "dv": np.zeros(1)}, ("dq1", "dq2"))
    for k in ("dk1", "dk2"):
        t = gr[k][0].float()  # [H, N, d]
        s = t.sum(dim=1).abs().max().item()
        a = t.abs().sum(dim=1).max().item()
        print(f"{k}: max |sum_j dK| = {s:.3e}, max sum_j |dK| = {a:.3e}", flush=True)
        assert s <= KEY_SUM_TOL * a, (k, s, a)


def test_longctx_backward_sampled_keys(dev, tmp_path):
    """The 64K-token workload (needles included) in one launch: dK1, dK2 and
    dV compared element by element on sampled keys -- the first key (summed
    over all 65536 query rows), the needle offsets, the last keys and seeded
    random ones -- against the oracle's key-wise backward, which needs every
    row's own forward (computed over row ranges in parallel processes)."""
    from _oracle_pool import dkv_keys

    name = "longctx_bf16_b1h12n65536d128"
    print(f"case bwd keys {name}", flush=True)
    w = W.WORKLOADS[name]
    x = W.workload_inputs(name)
    gen = torch.Generator().manual_seed(w.seed + 7)
    x["dout"] = torch.randn(x["v"].shape, generator=gen).to(torch.bfloat16)
    g = {k: (t.to(dev) if torch.is_tensor(t) else t) for k, t in x.items()}
    lam_t = da.lam(g["lq1"], g["lk1"], g["lq2"], g["lk2"], g["lambda_init"])
    _, lse, o12 = da.fwd_train(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], lam_t, g["lambda_init"], eps=g["eps"])
    gr = da.bwd(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], g["dout"], lse, o12, lam_t, g["lambda_init"],
                eps=g["eps"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    keys = np.unique(np.concatenate([[0, 1, 7, 311, 5003, 40009, w.N - 8, w.N - 1],
                                     rng.integers(0, w.N, 8)]))
    lam_args = tuple(x[k].numpy() for k in ("lq1", "lk1", "lq2", "lk2")) + (x["lambda_init"],)
    for h in (0, w.H - 1):
        head = {k: x[k][0, h].float().numpy() for k in ("q1", "k1", "q2", "k2", "v", "dout")}
        d1, d2, dv = dkv_keys(str(tmp_path), head, keys, lam_args, eps=x["eps"])
        got = {k: gr[k][0, h][keys].float().cpu().numpy() for k in ("dk1", "dk2", "dv")}
        print(f"head {h}, keys {keys.tolist()}", flush=True)
        _compare(got, {"dk1": d1, "dk2": d2, "dv": dv}, ("dk1", "dk2", "dv"))


@pytest.mark.parametrize("d", [64, 128])
def test_backward_large_logits(dev, d):
    """Q and K scaled by 5 (logits with a spread of about 25 and maxima near
    100): the weights recomputed from the saved log2-sum-exp stay finite and
    the gradients keep the same bound."""
    x = W.prefill_inputs(1, 2, 150, d, "bf16", seed=77 + d, lam_std=0.3, qk_scale=5.0)
    gen = torch.Generator().manual_seed(78 + d)
    x["dout"] = torch.randn(x["v"].shape, generator=gen).to(torch.bfloat16)
    x["weight"] = torch.ones(2 * d)
    out, plain, lse, o12, gr = _run(x, dev, True)
    assert torch.equal(out, plain)
    for k in ("dq1", "dk1", "dq2", "dk2", "dv"):
        assert np.all(np.isfinite(gr[k])), k
    _compare(gr, _oracle(x, True), ("dq1", "dk1", "dq2", "dk2", "dv", "dweight"))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [31, 32, 33, 63, 64, 65, 127, 128, 129])
def test_backward_tile_boundaries(dev, d, N):
    """Lengths on each side of the 32-row tiles and the 64/128-row blocks of
    the dQ and dK/dV kernels."""
    print(f"case bwd boundary d={d} N={N}", flush=True)
    x = _inputs(1, 2, N, d, seed=4000 + N + d)
    out, plain, lse, o12, gr = _run(x, dev, True)
    assert torch.equal(out, plain)
    _compare(gr, _oracle(x, True), ("dq1", "dk1", "dq2", "dk2", "dv", "dweight"))
