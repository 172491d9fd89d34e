"""The C ABI without a GPU: the library loads, exports exactly what
include/diffattn.h declares, and rejects bad arguments before any HIP call.

Every call below fails validation (or is empty work), so nothing is launched.
Fake device pointers are plain integers that are never dereferenced.
"""

import ctypes
import os
import re
import subprocess

import pytest

from transformer_attention_diffattn_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffattn.h")

A16 = 0x100000  # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x100004  # a misaligned one


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"DIFFATTN_API\s+[\w\s\*]*?\b(diffattn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(b.LIB_PATH):
        pytest.skip("libdiffattn.so not built")
    return b.lib()


def test_header_declares_the_abi():
    assert declared_symbols() == sorted([
        "diffattn_abi_version", "diffattn_bwd", "diffattn_bwd_workspace_bytes", "diffattn_decode",
        "diffattn_decode_noalloc", "diffattn_decode_workspace_bytes", "diffattn_fwd", "diffattn_fwd_fp8qk", "diffattn_fwd_train",
        "diffattn_in_proj", "diffattn_lambda", "diffattn_lambda_bwd", "diffattn_out_proj", "diffattn_quantize_fp8", "diffattn_quantize_fp8_batch", "diffattn_quantize_fp8_workspace_bytes",
        "diffattn_strerror"])


def test_library_exports_every_declared_symbol(L):
    for name in declared_symbols():
        assert hasattr(L, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True, text=True)
    if nm.returncode == 0:
        exported = {ln.split()[-1] for ln in nm.stdout.splitlines() if " T " in ln}
        ours = {s for s in exported if s.startswith("diffattn")}
        assert ours == set(declared_symbols())


def test_version_and_strerror(L):
    assert L.diffattn_abi_version() == 5
    for code in range(5):
        assert L.diffattn_strerror(code)
    assert L.diffattn_strerror(99) == b"unknown status"


def _fwd(L, dt=b.BF16, ptrs=(A16,) * 6, B=1, H=1, N=8, d=64, lam=A16, w=None, eps=1e-5, flags=b.CAUSAL):
    return L.diffattn_fwd(dt, *ptrs, B, H, N, d, lam, 0.8, w, eps, flags, None)


def test_fwd_validation(L):
    assert _fwd(L, dt=5) == b.EUNSUPPORTED
    for d in (0, 8, 48, 96, 256):
        assert _fwd(L, d=d) == b.EUNSUPPORTED
    assert _fwd(L, B=-1) == b.EINVAL
    assert _fwd(L, N=-3) == b.EINVAL
    assert _fwd(L, flags=4) == b.EINVAL
    assert _fwd(L, eps=-1.0) == b.EINVAL
    assert _fwd(L, eps=float("nan")) == b.EINVAL
    for i in range(6):
        p = [A16] * 6
        p[i] = None
        assert _fwd(L, ptrs=p) == b.EINVAL
        p[i] = MIS
        assert _fwd(L, ptrs=p) == b.EINVAL
    assert _fwd(L, lam=None) == b.EINVAL
    assert _fwd(L, w=A16 + 2) == b.EINVAL
    # a query grid larger than a launch can hold
    assert _fwd(L, B=65535, H=65535, N=1 << 20) == b.EINVAL


def test_fwd_refuses_heads_past_32bit_offsets(L):
    """The bf16 kernel addresses a head's output rows with 32-bit byte
    offsets: N * 2d * 2 bytes must stay below 2^31.  The first N past that
    limit is refused before any launch, for every bf16 prefill entry point."""
    for d in (16, 32, 64, 128):
        n_bad = (1 << 31) // (4 * d)  # N * 2d * 2 == 2^31
        assert _fwd(L, d=d, N=n_bad) == b.EINVAL, d
        assert _fwd(L, d=d, N=(1 << 31) - 1) == b.EINVAL, d
        if d >= 32:
            assert _fwd_train(L, d=d, N=n_bad) == b.EINVAL, d
    assert _fp8(L, N=(1 << 31) // 512) == b.EINVAL


def test_fwd_empty_work_is_ok_without_launch(L):
    assert _fwd(L, B=0) == b.OK
    assert _fwd(L, H=0) == b.OK
    assert _fwd(L, N=0) == b.OK
    # empty tensors may carry null data pointers
    assert _fwd(L, N=0, ptrs=(None,) * 6, lam=None) == b.OK
    assert _fwd(L, N=0, d=48) == b.EUNSUPPORTED


def test_lambda_validation(L):
    assert L.diffattn_lambda(None, A16, A16, A16, 64, 0.8, A16, None) == b.EINVAL
    assert L.diffattn_lambda(A16, A16, A16, A16, 0, 0.8, A16, None) == b.EINVAL
    assert L.diffattn_lambda(A16, A16, A16, A16, 5000, 0.8, A16, None) == b.EINVAL
    assert L.diffattn_lambda(A16, A16, A16, A16, 64, float("inf"), A16, None) == b.EINVAL
    assert L.diffattn_lambda(A16, A16, A16, A16 + 1, 64, 0.8, A16, None) == b.EINVAL


def test_decode_workspace_bytes(L):
    assert L.diffattn_decode_workspace_bytes(0, 16, 100, 128) == 0
    assert L.diffattn_decode_workspace_bytes(2, 16, 100, 48) == 0
    n = L.diffattn_decode_workspace_bytes(64, 16, 32768, 128)
    rec = (4 + 4 * 128) * 4
    assert n > 0 and n % (64 * 16 * rec) == 0
    # an empty cache still needs one record per (b, h) for the zero output
    assert L.diffattn_decode_workspace_bytes(2, 3, 0, 16) == 2 * 3 * (4 + 64) * 4


def _dec(L, dt=b.BF16, d=128, B=2, H=2, Lmax=64, ws=A16, wsb=1 << 20, lens=None, ptrs=(A16,) * 6, eps=1e-5):
    q1, q2, k1, k2, v, out = ptrs
    return L.diffattn_decode(dt, q1, q2, k1, k2, v, lens, out, B, H, Lmax, d, A16, 0.8, None, eps, ws, wsb, None)


def test_decode_validation(L):
    assert _dec(L, dt=3) == b.EUNSUPPORTED
    assert _dec(L, d=100) == b.EUNSUPPORTED
    assert _dec(L, Lmax=-1) == b.EINVAL
    assert _dec(L, eps=-1e-3) == b.EINVAL
    assert _dec(L, ws=None) == b.EWORKSPACE
    assert _dec(L, wsb=16) == b.EWORKSPACE
    assert _dec(L, ws=A16 + 8) == b.EINVAL
    assert _dec(L, lens=A16 + 2) == b.EINVAL
    for i in range(6):
        p = [A16] * 6
        p[i] = MIS
        assert _dec(L, ptrs=p) == b.EINVAL
    assert _dec(L, B=0) == b.OK
    assert _dec(L, B=70000) == b.EINVAL


def _dec_na(L, dt=b.BF16, d=128, B=2, H=2, Lmax=64, lens=None, ptrs=(A16,) * 6, eps=1e-5):
    q1, q2, k1, k2, v, out = ptrs
    return L.diffattn_decode_noalloc(dt, q1, q2, k1, k2, v, lens, out, B, H, Lmax, d, A16, 0.8, None, eps, None)


def test_decode_noalloc_validation(L):
    """The allocation-free decode validates like diffattn_decode and refuses,
    before any HIP call, sizes whose split records exceed its fixed scratch."""
    assert _dec_na(L, dt=3) == b.EUNSUPPORTED
    assert _dec_na(L, d=100) == b.EUNSUPPORTED
    assert _dec_na(L, Lmax=-1) == b.EINVAL
    assert _dec_na(L, eps=-1e-3) == b.EINVAL
    assert _dec_na(L, lens=A16 + 2) == b.EINVAL
    for i in range(6):
        p = [A16] * 6
        p[i] = MIS
        assert _dec_na(L, ptrs=p) == b.EINVAL
    assert _dec_na(L, B=0) == b.OK
    assert _dec_na(L, B=70000) == b.EINVAL
    # 512 x 64 one-key caches: 32768 records of 2064 bytes > 32 MiB
    assert L.diffattn_decode_workspace_bytes(512, 64, 1, 128) > b.NOALLOC_SCRATCH_BYTES
    assert _dec_na(L, B=512, H=64, Lmax=1) == b.EWORKSPACE
    # the benchmarked decode (64 x 16 x 32768 keys) fits
    assert L.diffattn_decode_workspace_bytes(64, 16, 32768, 128) <= b.NOALLOC_SCRATCH_BYTES


def _fwd_train(L, dt=b.BF16, d=64, B=1, H=1, N=8, flags=b.CAUSAL, lse=A16, o12=A16, ptrs=(A16,) * 6):
    return L.diffattn_fwd_train(dt, *ptrs, B, H, N, d, A16, 0.8, None, 1e-5, flags, lse, o12, None)


def test_fwd_train_validation(L):
    assert _fwd_train(L, dt=b.FP32) == b.EUNSUPPORTED  # training takes bf16 only
    for d in (16, 48, 256):
        assert _fwd_train(L, d=d) == b.EUNSUPPORTED
    assert _fwd_train(L, flags=b.CAUSAL | b.NO_NORM) == b.EINVAL
    assert _fwd_train(L, lse=None) == b.EINVAL
    assert _fwd_train(L, o12=A16 + 4) == b.EINVAL
    assert _fwd_train(L, ptrs=(A16, A16, MIS, A16, A16, A16)) == b.EINVAL
    assert _fwd_train(L, N=-1) == b.EINVAL
    assert _fwd_train(L, N=0, lse=None, o12=None) == b.OK


def test_bwd_workspace_bytes(L):
    assert L.diffattn_bwd_workspace_bytes(0, 1, 8, 64) == 0
    assert L.diffattn_bwd_workspace_bytes(1, 1, 8, 16) == 0
    n = L.diffattn_bwd_workspace_bytes(4, 16, 2048, 64)
    # at least dY (bf16) and the two delta rows
    assert n >= 4 * 16 * 2048 * (128 * 2 + 2 * 4) and n % 256 == 0


def _bwd(L, dt=b.BF16, d=64, B=1, H=1, N=8, flags=b.CAUSAL, ws=0x200000, wsb=1 << 24, ptrs=(A16,) * 13,
         lam=A16, dlam=A16, dw=A16, eps=1e-5):
    q1, k1, q2, k2, v, dout, lse, o12, dq1, dk1, dq2, dk2, dv = ptrs
    return L.diffattn_bwd(dt, q1, k1, q2, k2, v, dout, lse, o12, B, H, N, d, lam, 0.8, None, eps, flags,
                          dq1, dk1, dq2, dk2, dv, dlam, dw, ws, wsb, None)


def test_bwd_validation(L):
    assert _bwd(L, dt=b.FP32) == b.EUNSUPPORTED
    assert _bwd(L, d=16) == b.EUNSUPPORTED
    assert _bwd(L, flags=b.NO_NORM) == b.EINVAL
    assert _bwd(L, eps=-1.0) == b.EINVAL
    assert _bwd(L, B=-1) == b.EINVAL
    for i in range(13):
        p = [A16] * 13
        p[i] = MIS
        assert _bwd(L, ptrs=p) == b.EINVAL, i
        p[i] = None
        assert _bwd(L, ptrs=p) == b.EINVAL, i
    assert _bwd(L, dlam=None) == b.EINVAL
    assert _bwd(L, dw=A16 + 2) == b.EINVAL
    assert _bwd(L, ws=None) == b.EWORKSPACE
    assert _bwd(L, wsb=256) == b.EWORKSPACE
    assert _bwd(L, ws=0x200000 + 16) == b.EINVAL  # the workspace must be 256-byte aligned
    # sizes whose 32-bit row offsets would overflow
    assert _bwd(L, B=1 << 12, H=1 << 12, N=1 << 6) == b.EINVAL
    assert _bwd(L, N=0) == b.OK


def _fp8(L, d=128, B=1, H=1, N=8, ptrs=(A16,) * 6, scale=A16, flags=b.CAUSAL, eps=1e-5):
    q1, k1, q2, k2, v, out = ptrs
    return L.diffattn_fwd_fp8qk(q1, k1, q2, k2, scale, v, out, B, H, N, d, A16, 0.8, None, eps, flags, None)


def test_fwd_fp8qk_validation(L):
    for d in (16, 32, 64, 256):
        assert _fp8(L, d=d) == b.EUNSUPPORTED  # the fp8 product is 128 deep
    assert _fp8(L, scale=None) == b.EINVAL
    assert _fp8(L, scale=A16 + 2) == b.EINVAL
    assert _fp8(L, flags=8) == b.EINVAL
    assert _fp8(L, eps=-1.0) == b.EINVAL
    assert _fp8(L, N=-1) == b.EINVAL
    for i in range(6):
        p = [A16] * 6
        p[i] = MIS
        assert _fp8(L, ptrs=p) == b.EINVAL, i
    assert _fp8(L, N=0, scale=None) == b.OK


def test_quantize_fp8_validation(L):
    assert L.diffattn_quantize_fp8_workspace_bytes(-1) == 0
    assert L.diffattn_quantize_fp8_workspace_bytes(1) == 4
    assert L.diffattn_quantize_fp8_workspace_bytes(1 << 40) == 1024
    q = L.diffattn_quantize_fp8
    assert q(A16, -1, A16, A16, A16, 4096, None) == b.EINVAL
    assert q(A16, 0, None, None, None, 0, None) == b.OK
    assert q(MIS, 100, A16, A16, A16, 4096, None) == b.EINVAL
    assert q(A16, 100, MIS, A16, A16, 4096, None) == b.EINVAL
    assert q(A16, 100, A16, None, A16, 4096, None) == b.EINVAL
    assert q(A16, 100, A16, A16, None, 4096, None) == b.EWORKSPACE
    assert q(A16, 1 << 30, A16, A16, A16, 16, None) == b.EWORKSPACE


def test_quantize_fp8_batch_validation(L):
    import ctypes

    arr = lambda *p: (ctypes.c_void_p * len(p))(*p)  # noqa: E731
    qb = L.diffattn_quantize_fp8_batch
    four = arr(A16, A16, A16, A16)
    assert qb(0, four, 100, four, A16, A16, 4096, None) == b.EINVAL
    assert qb(5, arr(*([A16] * 5)), 100, arr(*([A16] * 5)), A16, A16, 4096, None) == b.EINVAL
    assert qb(2, None, 100, four, A16, A16, 4096, None) == b.EINVAL
    assert qb(2, arr(A16, MIS), 100, four, A16, A16, 4096, None) == b.EINVAL
    assert qb(2, four, 100, arr(None, A16), A16, A16, 4096, None) == b.EINVAL
    assert qb(2, four, 100, four, None, A16, 4096, None) == b.EINVAL
    assert qb(2, four, 100, four, A16, A16, 4, None) == b.EWORKSPACE  # two tensors need 8 bytes
    assert qb(2, four, -1, four, A16, A16, 4096, None) == b.EINVAL
    assert qb(2, four, 0, four, A16, A16, 4096, None) == b.OK


def test_projection_validation(L):
    ip = lambda B=1, N=8, dm=64, H=2, d=64, ptrs=(A16,) * 7: L.diffattn_in_proj(  # noqa: E731
        ptrs[0], ptrs[1], B, N, dm, H, d, *ptrs[2:], None)
    assert ip(d=48) == b.EUNSUPPORTED
    assert ip(dm=60) == b.EINVAL  # d_model must be a multiple of 8
    assert ip(H=0) == b.EINVAL
    assert ip(B=-1) == b.EINVAL
    assert ip(B=65536, N=129) == b.EINVAL  # more token tiles than one grid dimension holds
    for i in range(7):
        p = [A16] * 7
        p[i] = MIS
        assert ip(ptrs=p) == b.EINVAL, i
    assert ip(N=0, ptrs=(None,) * 7) == b.OK
    op = lambda B=1, H=2, N=8, d=64, dout=64, ptrs=(A16,) * 3: L.diffattn_out_proj(  # noqa: E731
        ptrs[0], ptrs[1], B, H, N, d, dout, ptrs[2], None)
    assert op(d=8) == b.EUNSUPPORTED
    assert op(dout=6) == b.EINVAL  # d_out must be a multiple of 4
    assert op(H=0) == b.EINVAL
    for i in range(3):
        p = [A16] * 3
        p[i] = None
        assert op(ptrs=p) == b.EINVAL, i
    assert op(B=0, ptrs=(None,) * 3) == b.OK


def test_lambda_bwd_validation(L):
    p = [A16] * 9
    for i in range(9):
        q = list(p)
        q[i] = None
        assert L.diffattn_lambda_bwd(*q[:4], 64, *q[4:], None) == b.EINVAL
    assert L.diffattn_lambda_bwd(*p[:4], 0, *p[4:], None) == b.EINVAL


def test_training_bindings_refuse_host_tensors():
    """The ctypes layer refuses tensors that are not on a HIP device before
    anything reaches the library (no launch, no GPU needed)."""
    import torch

    t = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    v = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
    lam = torch.zeros(1)
    with pytest.raises(ValueError):
        b.fwd_train(t, t, t, t, v, lam, 0.8)
    with pytest.raises(ValueError):
        b.bwd(t, t, t, t, v, v, torch.zeros(2, 1, 1, 8), torch.zeros(2, 1, 1, 8, 128), lam, 0.8)
    with pytest.raises(ValueError):
        b.lambda_bwd(torch.zeros(64), torch.zeros(64), torch.zeros(64), torch.zeros(64), lam)
