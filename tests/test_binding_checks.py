"""The ctypes binding refuses caller-supplied outputs and workspaces that do
not match the call (wrong shape, dtype or device) before anything reaches
the library: the C ABI sees only pointers and sizes, so a short buffer would
otherwise be written past its end.  Every case raises before a launch."""

import pytest
import torch

from transformer_attention_diffattn_amd import binding as da

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _qkv(dev, B=1, H=2, N=8, d=64):
    t = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=dev)  # noqa: E731
    return t(B, H, N, d), t(B, H, N, d), t(B, H, N, d), t(B, H, N, d), t(B, H, N, 2 * d)


def test_fwd_out_must_match(dev):
    q1, k1, q2, k2, v = _qkv(dev)
    lam = torch.zeros(1, device=dev)
    for bad in (torch.empty(1, 2, 8, 64, dtype=torch.bfloat16, device=dev),  # half width
                torch.empty_like(v, dtype=torch.float32),
                torch.empty_like(v, device="cpu")):
        with pytest.raises(ValueError):
            da.fwd(q1, k1, q2, k2, v, lam, 0.8, out=bad)
    with pytest.raises(ValueError):
        da.fwd(q1, k1, q2, k2, v, lam, 0.8, weight=torch.ones(64, device=dev))


def test_decode_out_and_workspace_must_match(dev):
    B, H, L, d = 2, 2, 16, 64
    q = torch.zeros(B, H, 1, d, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(B, H, L, d, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros(B, H, L, 2 * d, dtype=torch.bfloat16, device=dev)
    lam = torch.zeros(1, device=dev)
    with pytest.raises(ValueError):
        da.decode(q, q, kc, kc, vc, lam, 0.8, out=torch.empty(B, H, 1, d, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        da.decode(q, q, kc, kc, vc, lam, 0.8, out=torch.empty(B, H, 1, 2 * d, device=dev))
    with pytest.raises(ValueError):
        da.decode(q, q, kc, kc, vc, lam, 0.8, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    # a device workspace is measured in bytes, whatever its dtype: one too small is refused by the library
    need = da.decode_workspace_bytes(B, H, L, d)
    with pytest.raises(RuntimeError, match="status 4"):
        da.decode(q, q, kc, kc, vc, lam, 0.8, workspace=torch.empty(need // 4 - 1, dtype=torch.float32,
                                                                    device=dev))


def test_training_outputs_and_workspace_must_match(dev):
    q1, k1, q2, k2, v = _qkv(dev)
    lam = torch.zeros(1, device=dev)
    lse = torch.zeros(2, 1, 2, 8, device=dev)
    o12 = torch.zeros(2, 1, 2, 8, 128, device=dev)
    with pytest.raises(ValueError):
        da.bwd(q1, k1, q2, k2, v, v, lse, o12, lam, 0.8, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    grads = dict(dq1=torch.empty_like(q1), dk1=torch.empty_like(k1), dq2=torch.empty_like(q2),
                 dk2=torch.empty_like(k2), dv=torch.empty_like(q1),  # dv must be [B,H,N,2d]
                 dlambda=torch.empty(1, device=dev), dweight=torch.empty(128, device=dev))
    with pytest.raises(ValueError):
        da.bwd(q1, k1, q2, k2, v, v, lse, o12, lam, 0.8, grads=grads)
    del grads["dv"]
    with pytest.raises(ValueError):
        da.bwd(q1, k1, q2, k2, v, v, lse, o12, lam, 0.8, grads=grads)


def test_projection_outputs_must_match(dev):
    B, N, dm, H, d = 1, 8, 64, 2, 64
    x = torch.zeros(B, N, dm, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(3 * H * 2 * d, dm, dtype=torch.bfloat16, device=dev)
    outs = list(_qkv(dev, B, H, N, d))
    with pytest.raises(ValueError):
        da.in_proj(x, w, H, d, outs=outs[:4])
    bad = list(outs)
    bad[4] = outs[0]  # v must be [B,H,N,2d]
    with pytest.raises(ValueError):
        da.in_proj(x, w, H, d, outs=bad)
    o = outs[4]
    w_o = torch.zeros(dm, H * 2 * d, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        da.out_proj(o, w_o, out=torch.empty(B, N, dm // 2, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        da.out_proj(o, w_o, out=torch.empty(B, N, dm, dtype=torch.float32, device=dev))


def test_quantiser_workspace_must_be_on_the_device(dev):
    x = torch.zeros(1024, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        da.quantize_fp8(x, workspace=torch.empty(4096, dtype=torch.uint8))
    with pytest.raises(ValueError):
        da.quantize_fp8_batch([x, x], codes=[torch.empty(1024, dtype=torch.uint8, device=dev)])
