"""GPU parity of the in- and out-projections (diffattn_in_proj,
diffattn_out_proj) against oracle/projection_oracle.py.

Bound per element, from the arithmetic: the inputs are bf16 (exact in the
oracle's float64), the kernel sums exact products in fp32 and rounds the
result to bf16, so |gpu - oracle| <= 2^-8 |oracle| (round to nearest) +
K 2^-24 sum_k |x_k w_k| (fp32 summation of K terms), with the magnitudes
summed by the oracle on |x| and |w|.
"""

import numpy as np
import pytest
import torch

from oracle import projection_oracle as P
from transformer_attention_diffattn_amd import binding as da
from transformer_attention_diffattn_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _check(got, ref, mag, K):
    got = got.float().cpu().numpy()
    tol = 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -24 * (1 + 2.0 ** -8) * mag + 1e-30
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    print(f"max err {err.max():.3e}; worst vs bound {err[worst]:.3e} / {tol[worst]:.3e}", flush=True)
    assert np.all(err <= tol)


def _abs(t):
    return t.float().abs().numpy()


IN_CASES = [(2, 77, 256, 2, 64), (1, 130, 200, 3, 32), (2, 33, 128, 1, 128), (1, 1, 64, 2, 16),
            (3, 129, 72, 4, 16)]


@pytest.mark.parametrize("B,N,dm,H,d", IN_CASES)
def test_in_proj(dev, B, N, dm, H, d):
    print(f"case in_proj B={B} N={N} d_model={dm} H={H} d={d}", flush=True)
    x = W.projection_inputs(B, N, dm, H, d, seed=900 + N)
    outs = da.in_proj(x["x"].to(dev), x["w_qkv"].to(dev), H, d)
    torch.cuda.synchronize()
    ref = P.in_projection(x["x"], x["w_qkv"], H, d)
    mag = P.in_projection(_abs(x["x"]), _abs(x["w_qkv"]), H, d)
    for g, r, m in zip(outs, ref, mag):
        _check(g, r, m, dm)


# reduction lengths H*2d of 32 and 96 leave the last 64-wide step half empty
OUT_CASES = [(2, 2, 77, 64, 256), (1, 3, 130, 32, 100), (2, 1, 33, 128, 4), (1, 4, 129, 16, 36),
             (1, 1, 50, 16, 8), (2, 3, 20, 16, 12)]


@pytest.mark.parametrize("B,H,N,d,dout", OUT_CASES)
def test_out_proj(dev, B, H, N, d, dout):
    print(f"case out_proj B={B} H={H} N={N} d={d} d_out={dout}", flush=True)
    x = W.projection_inputs(B, N, 64, H, d, seed=950 + N, d_out=dout)
    y = da.out_proj(x["o"].to(dev), x["w_o"].to(dev))
    torch.cuda.synchronize()
    _check(y, P.out_projection(x["o"], x["w_o"]), P.out_projection(_abs(x["o"]), _abs(x["w_o"])), H * 2 * d)


def test_projections_full_size_1p4b_layer_sampled(dev):
    # the benchmarked shapes: 4 x 2048 tokens, d_model 2048, 16 heads of 2d = 128;
    # every output feature of sampled tokens against the oracle
    B, N, dm, H, d = 4, 2048, 2048, 16, 64
    x = W.projection_inputs(B, N, dm, H, d, seed=20266, device=dev)
    outs = da.in_proj(x["x"], x["w_qkv"], H, d)
    y = da.out_proj(x["o"], x["w_o"])
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 1000, N - 2, N - 1])
    xs = x["x"][:, rows].cpu()
    ref = P.in_projection(xs, x["w_qkv"].cpu(), H, d)
    mag = P.in_projection(_abs(xs), _abs(x["w_qkv"].cpu()), H, d)
    for g, r, m in zip(outs, ref, mag):
        _check(g[:, :, rows], r, m, dm)
    os_ = x["o"][:, :, rows].cpu()
    _check(y[:, rows], P.out_projection(os_, x["w_o"].cpu()),
           P.out_projection(_abs(os_), _abs(x["w_o"].cpu())), H * 2 * d)


def test_projections_full_size_3b_layer_sampled(dev):
    # 2 x 4096 tokens, d_model 3072, 12 heads of 2d = 256 (d = 128)
    B, N, dm, H, d = 2, 4096, 3072, 12, 128
    x = W.projection_inputs(B, N, dm, H, d, seed=20267, device=dev)
    outs = da.in_proj(x["x"], x["w_qkv"], H, d)
    y = da.out_proj(x["o"], x["w_o"])
    torch.cuda.synchronize()
    rows = np.array([0, 127, 128, 2049, N - 1])
    xs = x["x"][:, rows].cpu()
    ref = P.in_projection(xs, x["w_qkv"].cpu(), H, d)
    mag = P.in_projection(_abs(xs), _abs(x["w_qkv"].cpu()), H, d)
    for g, r, m in zip(outs, ref, mag):
        _check(g[:, :, rows], r, m, dm)
    os_ = x["o"][:, :, rows].cpu()
    _check(y[:, rows], P.out_projection(os_, x["w_o"].cpu()),
           P.out_projection(_abs(os_), _abs(x["w_o"].cpu())), H * 2 * d)


def test_layer_chain_runs_on_device_layouts(dev):
    # in_proj -> diffattn_fwd -> out_proj with no copies between them: the
    # projection outputs are the attention's inputs as they stand
    B, N, dm, H, d = 1, 96, 256, 2, 64
    x = W.projection_inputs(B, N, dm, H, d, seed=31)
    q1, k1, q2, k2, v = da.in_proj(x["x"].to(dev), x["w_qkv"].to(dev), H, d)
    lam_t = torch.tensor([0.5], device=dev)
    o = da.fwd(q1, k1, q2, k2, v, lam_t, 0.8)
    y = da.out_proj(o, x["w_o"].to(dev))
    torch.cuda.synchronize()
    assert y.shape == (B, N, dm) and torch.isfinite(y.float()).all()


def test_projection_deterministic(dev):
    x = W.projection_inputs(2, 300, 512, 4, 64, seed=41, device=dev)
    a = da.in_proj(x["x"], x["w_qkv"], 4, 64)
    b = da.in_proj(x["x"], x["w_qkv"], 4, 64)
    for s, t in zip(a, b):
        assert torch.equal(s, t)
