"""ctypes binding of libdiffattn.so (C ABI in include/diffattn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch supplies device memory and the current stream.
There is no fallback: if the library is missing or the tensors are not on a
HIP device, these functions raise.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdiffattn.so")

OK, EINVAL, EUNSUPPORTED, EHIP, EWORKSPACE = 0, 1, 2, 3, 4
FP32, BF16 = 0, 1
CAUSAL, NO_NORM = 1, 2

_DT = {torch.float32: FP32, torch.bfloat16: BF16}
_lib = None

vp = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load the library once and declare the C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "or python -m transformer_attention_diffattn_amd.build_lib")
        L = ctypes.CDLL(LIB_PATH)
        i, f, u, sz = ctypes.c_int, ctypes.c_float, ctypes.c_uint, ctypes.c_size_t
        L.diffattn_lambda.argtypes = [vp, vp, vp, vp, i, f, vp, vp]
        L.diffattn_lambda.restype = i
        L.diffattn_fwd.argtypes = [i, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, f, vp, f, u, vp]
        L.diffattn_fwd.restype = i
        L.diffattn_decode_workspace_bytes.argtypes = [i, i, i, i]
        L.diffattn_decode_workspace_bytes.restype = sz
        L.diffattn_decode.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, f, vp, f, vp, sz, vp]
        L.diffattn_decode.restype = i
        L.diffattn_decode_noalloc.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, f, vp, f, vp]
        L.diffattn_decode_noalloc.restype = i
        L.diffattn_strerror.argtypes = [i]
        L.diffattn_strerror.restype = ctypes.c_char_p
        L.diffattn_fwd_train.argtypes = [i, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, f, vp, f, u, vp, vp, vp]
        L.diffattn_fwd_train.restype = i
        L.diffattn_bwd_workspace_bytes.argtypes = [i, i, i, i]
        L.diffattn_bwd_workspace_bytes.restype = sz
        L.diffattn_bwd.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, f, vp, f, u,
                                   vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.diffattn_bwd.restype = i
        L.diffattn_lambda_bwd.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, vp, vp]
        L.diffattn_lambda_bwd.restype = i
        L.diffattn_quantize_fp8_workspace_bytes.argtypes = [ctypes.c_longlong]
        L.diffattn_quantize_fp8_workspace_bytes.restype = sz
        L.diffattn_quantize_fp8.argtypes = [vp, ctypes.c_longlong, vp, vp, vp, sz, vp]
        L.diffattn_quantize_fp8.restype = i
        L.diffattn_quantize_fp8_batch.argtypes = [i, vp, ctypes.c_longlong, vp, vp, vp, sz, vp]
        L.diffattn_quantize_fp8_batch.restype = i
        L.diffattn_fwd_fp8qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, f, vp, f, u, vp]
        L.diffattn_fwd_fp8qk.restype = i
        L.diffattn_in_proj.argtypes = [vp, vp, i, i, i, i, i, vp, vp, vp, vp, vp, vp]
        L.diffattn_in_proj.restype = i
        L.diffattn_out_proj.argtypes = [vp, vp, i, i, i, i, i, vp, vp]
        L.diffattn_out_proj.restype = i
        L.diffattn_abi_version.argtypes = []
        L.diffattn_abi_version.restype = i
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != OK:
        msg = lib().diffattn_strerror(status).decode()
        raise RuntimeError(f"{what} failed: status {status} ({msg})")


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a tensor on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _like(t, name: str, shape, dtype, device) -> torch.Tensor:
    """A caller-supplied output: on the device, contiguous, exactly this
    shape and dtype (the C ABI cannot see buffer sizes)."""
    _dev(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)} on {device}")
    return t


def _workspace(ws, name: str, device) -> int:
    """A caller-supplied workspace on the device: returns its size in bytes."""
    _dev(ws, name)
    if ws.device != device:
        raise ValueError(f"{name} must be on {device}")
    return ws.numel() * ws.element_size()


def _weight(weight, d):
    if weight is not None:
        _dev(weight, "weight")
        if weight.dtype != torch.float32 or weight.shape != (2 * d,):
            raise ValueError("weight must be fp32 [2d]")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def lam(lq1, lk1, lq2, lk2, lambda_init: float, out: torch.Tensor | None = None) -> torch.Tensor:
    """lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init as a device fp32 [1]."""
    for n, t in (("lq1", lq1), ("lk1", lk1), ("lq2", lq2), ("lk2", lk2)):
        _dev(t, n)
        if t.dtype != torch.float32 or t.dim() != 1 or t.numel() != lq1.numel():
            raise ValueError(f"{n} must be fp32 [d]")
    if out is None:
        out = torch.empty(1, device=lq1.device, dtype=torch.float32)
    _check(lib().diffattn_lambda(_ptr(lq1), _ptr(lk1), _ptr(lq2), _ptr(lk2), lq1.numel(), float(lambda_init),
                                 _ptr(out), _stream(lq1.device)), "diffattn_lambda")
    return out


def fwd(q1, k1, q2, k2, v, lam_t, lambda_init: float, weight=None, eps: float = 1e-5,
        causal: bool = True, norm: bool = True, out=None) -> torch.Tensor:
    """Differential-attention prefill.  q1/k1/q2/k2 [B,H,N,d], v [B,H,N,2d] ->
    out [B,H,N,2d] (same dtype).  lam_t: device fp32 [1]."""
    for n, t in (("q1", q1), ("k1", k1), ("q2", q2), ("k2", k2), ("v", v), ("lambda", lam_t)):
        _dev(t, n)
    if q1.dtype not in _DT:
        raise ValueError("dtype must be float32 or bfloat16")
    B, H, N, d = q1.shape
    for n, t in (("k1", k1), ("q2", q2), ("k2", k2)):
        if t.shape != q1.shape or t.dtype != q1.dtype:
            raise ValueError(f"{n} must match q1 in shape and dtype")
    if v.shape != (B, H, N, 2 * d) or v.dtype != q1.dtype:
        raise ValueError("v must be [B,H,N,2d] of q1's dtype")
    if lam_t.dtype != torch.float32:
        raise ValueError("lambda must be fp32")
    _weight(weight, d)
    if out is None:
        out = torch.empty_like(v)
    else:
        _like(out, "out", v.shape, v.dtype, v.device)
    flags = (CAUSAL if causal else 0) | (0 if norm else NO_NORM)
    _check(lib().diffattn_fwd(_DT[q1.dtype], _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(out),
                              B, H, N, d, _ptr(lam_t), float(lambda_init), _ptr(weight), float(eps), flags,
                              _stream(q1.device)), "diffattn_fwd")
    return out


def decode_workspace_bytes(B: int, H: int, L: int, d: int) -> int:
    return int(lib().diffattn_decode_workspace_bytes(B, H, L, d))


def decode(q1, q2, k1c, k2c, vc, lam_t, lambda_init: float, cache_len=None, weight=None,
           eps: float = 1e-5, workspace=None, out=None) -> torch.Tensor:
    """One decode step.  q1/q2 [B,H,1,d]; caches k1c/k2c [B,H,L,d], vc [B,H,L,2d];
    cache_len: device int32 [B] or None -> out [B,H,1,2d]."""
    for n, t in (("q1", q1), ("q2", q2), ("k1c", k1c), ("k2c", k2c), ("vc", vc), ("lambda", lam_t)):
        _dev(t, n)
    if q1.dtype not in _DT:
        raise ValueError("dtype must be float32 or bfloat16")
    B, H, one, d = q1.shape
    L = k1c.shape[2]
    if one != 1 or q2.shape != q1.shape:
        raise ValueError("q1/q2 must be [B,H,1,d]")
    if k1c.shape != (B, H, L, d) or k2c.shape != (B, H, L, d) or vc.shape != (B, H, L, 2 * d):
        raise ValueError("caches must be [B,H,L,d] and [B,H,L,2d]")
    for t in (q2, k1c, k2c, vc):
        if t.dtype != q1.dtype:
            raise ValueError("all of q/k/v must share one dtype")
    if cache_len is not None:
        _dev(cache_len, "cache_len")
        if cache_len.dtype != torch.int32 or cache_len.shape != (B,):
            raise ValueError("cache_len must be int32 [B]")
    if weight is not None:
        _dev(weight, "weight")
        if weight.dtype != torch.float32 or weight.shape != (2 * d,):
            raise ValueError("weight must be fp32 [2d]")
    need = decode_workspace_bytes(B, H, L, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    ws_bytes = _workspace(workspace, "workspace", q1.device)
    if out is None:
        out = torch.empty((B, H, 1, 2 * d), dtype=q1.dtype, device=q1.device)
    _like(out, "out", (B, H, 1, 2 * d), q1.dtype, q1.device)
    _check(lib().diffattn_decode(_DT[q1.dtype], _ptr(q1), _ptr(q2), _ptr(k1c), _ptr(k2c), _ptr(vc),
                                 _ptr(cache_len), _ptr(out), B, H, L, d, _ptr(lam_t), float(lambda_init),
                                 _ptr(weight), float(eps), _ptr(workspace), ws_bytes,
                                 _stream(q1.device)), "diffattn_decode")
    return out


# bytes of the library's fixed scratch array used by decode_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_noalloc(q1, q2, k1c, k2c, vc, lam_t, lambda_init: float, out, cache_len=None, weight=None,
                   eps: float = 1e-5) -> torch.Tensor:
    """``decode`` through diffattn_decode_noalloc: no workspace, the split
    records go to the library's fixed device array (NOALLOC_SCRATCH_BYTES per
    GPU), so the call allocates nothing; ``out`` [B,H,1,2d] is required.
    Calls that overlap in time on one GPU share that array and must not be
    issued."""
    for n, t in (("q1", q1), ("q2", q2), ("k1c", k1c), ("k2c", k2c), ("vc", vc), ("lambda", lam_t)):
        _dev(t, n)
    if q1.dtype not in _DT:
        raise ValueError("dtype must be float32 or bfloat16")
    B, H, one, d = q1.shape
    L = k1c.shape[2]
    if one != 1 or q2.shape != q1.shape:
        raise ValueError("q1/q2 must be [B,H,1,d]")
    if k1c.shape != (B, H, L, d) or k2c.shape != (B, H, L, d) or vc.shape != (B, H, L, 2 * d):
        raise ValueError("caches must be [B,H,L,d] and [B,H,L,2d]")
    for t in (q2, k1c, k2c, vc):
        if t.dtype != q1.dtype:
            raise ValueError("all of q/k/v must share one dtype")
    if cache_len is not None:
        _dev(cache_len, "cache_len")
        if cache_len.dtype != torch.int32 or cache_len.shape != (B,):
            raise ValueError("cache_len must be int32 [B]")
    _weight(weight, d)
    _like(out, "out", (B, H, 1, 2 * d), q1.dtype, q1.device)
    need = decode_workspace_bytes(B, H, L, d)
    if need > NOALLOC_SCRATCH_BYTES:
        raise ValueError(f"these sizes need {need} bytes of split records, more than the "
                         f"{NOALLOC_SCRATCH_BYTES}-byte scratch of diffattn_decode_noalloc: use decode()")
    _check(lib().diffattn_decode_noalloc(_DT[q1.dtype], _ptr(q1), _ptr(q2), _ptr(k1c), _ptr(k2c), _ptr(vc),
                                         _ptr(cache_len), _ptr(out), B, H, L, d, _ptr(lam_t), float(lambda_init),
                                         _ptr(weight), float(eps), _stream(q1.device)), "diffattn_decode_noalloc")
    return out


def _check_qkv(q1, k1, q2, k2, v):
    for n, t in (("q1", q1), ("k1", k1), ("q2", q2), ("k2", k2), ("v", v)):
        _dev(t, n)
    if q1.dtype != torch.bfloat16:
        raise ValueError("training entry points take bfloat16 tensors")
    B, H, N, d = q1.shape
    for n, t in (("k1", k1), ("q2", q2), ("k2", k2)):
        if t.shape != q1.shape or t.dtype != q1.dtype:
            raise ValueError(f"{n} must match q1 in shape and dtype")
    if v.shape != (B, H, N, 2 * d) or v.dtype != q1.dtype:
        raise ValueError("v must be [B,H,N,2d] of q1's dtype")
    return B, H, N, d


def fwd_train(q1, k1, q2, k2, v, lam_t, lambda_init: float, weight=None, eps: float = 1e-5,
              causal: bool = True):
    """Training forward: returns (out [B,H,N,2d] bf16, lse [2,B,H,N] fp32 in
    log2 units, o12 [2,B,H,N,2d] fp32 per-map outputs)."""
    B, H, N, d = _check_qkv(q1, k1, q2, k2, v)
    _dev(lam_t, "lambda")
    if lam_t.dtype != torch.float32:
        raise ValueError("lambda must be fp32")
    _weight(weight, d)
    out = torch.empty_like(v)
    lse = torch.empty((2, B, H, N), dtype=torch.float32, device=q1.device)
    o12 = torch.empty((2, B, H, N, 2 * d), dtype=torch.float32, device=q1.device)
    _check(lib().diffattn_fwd_train(BF16, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(out),
                                    B, H, N, d, _ptr(lam_t), float(lambda_init), _ptr(weight), float(eps),
                                    CAUSAL if causal else 0, _ptr(lse), _ptr(o12), _stream(q1.device)),
           "diffattn_fwd_train")
    return out, lse, o12


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().diffattn_bwd_workspace_bytes(B, H, N, d))


def bwd(q1, k1, q2, k2, v, dout, lse, o12, lam_t, lambda_init: float, weight=None, eps: float = 1e-5,
        causal: bool = True, workspace=None, grads=None):
    """Backward of ``fwd_train``: returns a dict with dq1, dk1, dq2, dk2, dv
    (bf16) and dlambda [1], dweight [2d] (fp32)."""
    B, H, N, d = _check_qkv(q1, k1, q2, k2, v)
    for n, t in (("dout", dout), ("lse", lse), ("o12", o12), ("lambda", lam_t)):
        _dev(t, n)
    if dout.shape != v.shape or dout.dtype != v.dtype:
        raise ValueError("dout must match v")
    if lse.shape != (2, B, H, N) or o12.shape != (2, B, H, N, 2 * d):
        raise ValueError("lse / o12 must come from fwd_train on the same shapes")
    if lse.dtype != torch.float32 or o12.dtype != torch.float32 or lam_t.dtype != torch.float32:
        raise ValueError("lse, o12 and lambda must be fp32")
    _weight(weight, d)
    dev = q1.device
    if grads is None:
        grads = dict(dq1=torch.empty_like(q1), dk1=torch.empty_like(k1), dq2=torch.empty_like(q2),
                     dk2=torch.empty_like(k2), dv=torch.empty_like(v),
                     dlambda=torch.empty(1, dtype=torch.float32, device=dev),
                     dweight=torch.empty(2 * d, dtype=torch.float32, device=dev))
    for k, shape, dt in (("dq1", q1.shape, q1.dtype), ("dk1", q1.shape, q1.dtype), ("dq2", q1.shape, q1.dtype),
                         ("dk2", q1.shape, q1.dtype), ("dv", v.shape, v.dtype), ("dlambda", (1,), torch.float32),
                         ("dweight", (2 * d,), torch.float32)):
        if k not in grads:
            raise ValueError(f"grads must hold {k}")
        _like(grads[k], k, shape, dt, dev)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(B, H, N, d), 256), dtype=torch.uint8, device=dev)
    ws_bytes = _workspace(workspace, "workspace", dev)
    g = grads
    _check(lib().diffattn_bwd(BF16, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(dout), _ptr(lse),
                              _ptr(o12), B, H, N, d, _ptr(lam_t), float(lambda_init), _ptr(weight), float(eps),
                              CAUSAL if causal else 0, _ptr(g["dq1"]), _ptr(g["dk1"]), _ptr(g["dq2"]),
                              _ptr(g["dk2"]), _ptr(g["dv"]), _ptr(g["dlambda"]), _ptr(g["dweight"]),
                              _ptr(workspace), ws_bytes, _stream(dev)), "diffattn_bwd")
    return grads


def lambda_bwd(lq1, lk1, lq2, lk2, dlambda):
    """Eq. 2 backward: (dlq1, dlk1, dlq2, dlk2), fp32 [d] each."""
    for n, t in (("lq1", lq1), ("lk1", lk1), ("lq2", lq2), ("lk2", lk2), ("dlambda", dlambda)):
        _dev(t, n)
        if t.dtype != torch.float32:
            raise ValueError(f"{n} must be fp32")
    for n, t in (("lk1", lk1), ("lq2", lq2), ("lk2", lk2)):
        if t.shape != lq1.shape or lq1.dim() != 1:
            raise ValueError(f"{n} must be fp32 [d] like lq1")
    if dlambda.numel() != 1:
        raise ValueError("dlambda must be fp32 [1]")
    outs = [torch.empty_like(lq1) for _ in range(4)]
    _check(lib().diffattn_lambda_bwd(_ptr(lq1), _ptr(lk1), _ptr(lq2), _ptr(lk2), lq1.numel(), _ptr(dlambda),
                                     *[_ptr(o) for o in outs], _stream(lq1.device)), "diffattn_lambda_bwd")
    return tuple(outs)


def quantize_fp8_workspace_bytes(n: int) -> int:
    return int(lib().diffattn_quantize_fp8_workspace_bytes(n))


def quantize_fp8(x, codes=None, scale=None, workspace=None):
    """Per-tensor absmax e4m3 quantisation of a bf16 tensor: returns
    (codes uint8 of x's shape, scale fp32 [1]); scale may be a 1-element view
    of a larger fp32 tensor."""
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    n = x.numel()
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    else:
        _dev(codes, "codes")
        if codes.dtype != torch.uint8 or codes.numel() != n or codes.device != x.device:
            raise ValueError("codes must be uint8 with x's element count on x's device")
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    elif scale.dtype != torch.float32 or scale.numel() != 1 or scale.device != x.device:
        raise ValueError("scale must be one fp32 element on x's device")
    need = quantize_fp8_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=x.device)
    ws_bytes = _workspace(workspace, "workspace", x.device)
    _check(lib().diffattn_quantize_fp8(_ptr(x), n, _ptr(codes), _ptr(scale), _ptr(workspace),
                                       ws_bytes, _stream(x.device)),
           "diffattn_quantize_fp8")
    return codes, scale


def quantize_fp8_batch(xs, codes=None, scales=None, workspace=None):
    """diffattn_quantize_fp8 of 1..4 bf16 tensors of equal size in one pair of
    launches: returns (list of uint8 codes, scales fp32 [count])."""
    count = len(xs)
    if not 1 <= count <= 4:
        raise ValueError("one to four tensors")
    for k, x in enumerate(xs):
        _dev(x, f"x[{k}]")
        if x.dtype != torch.bfloat16 or x.numel() != xs[0].numel():
            raise ValueError("tensors must be bf16 with equal element counts")
    n = xs[0].numel()
    dev = xs[0].device
    if codes is None:
        codes = [torch.empty(x.shape, dtype=torch.uint8, device=dev) for x in xs]
    if len(codes) != count:
        raise ValueError("one codes tensor per input")
    for k, c in enumerate(codes):
        _dev(c, f"codes[{k}]")
        if c.dtype != torch.uint8 or c.numel() != n or c.device != dev:
            raise ValueError("codes must be uint8 with x's element count on x's device")
    if scales is None:
        scales = torch.empty(count, dtype=torch.float32, device=dev)
    _dev(scales, "scales")
    if scales.dtype != torch.float32 or scales.numel() != count or scales.device != dev:
        raise ValueError("scales must be fp32 [count] on x's device")
    need = count * quantize_fp8_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    ws_bytes = _workspace(workspace, "workspace", dev)
    xp = (ctypes.c_void_p * count)(*(x.data_ptr() for x in xs))
    cp = (ctypes.c_void_p * count)(*(c.data_ptr() for c in codes))
    _check(lib().diffattn_quantize_fp8_batch(count, xp, n, cp, _ptr(scales), _ptr(workspace),
                                             ws_bytes, _stream(dev)),
           "diffattn_quantize_fp8_batch")
    return codes, scales


def fwd_fp8qk(q1, k1, q2, k2, qk_scale, v, lam_t, lambda_init: float, weight=None, eps: float = 1e-5,
              causal: bool = True, norm: bool = True, out=None) -> torch.Tensor:
    """Prefill with e4m3 queries/keys (uint8 [B,H,N,128]) and their scales
    (device fp32 [4]: q1, k1, q2, k2); v bf16 [B,H,N,256] -> out bf16."""
    for n, t in (("q1", q1), ("k1", k1), ("q2", q2), ("k2", k2), ("qk_scale", qk_scale), ("v", v),
                 ("lambda", lam_t)):
        _dev(t, n)
    B, H, N, d = q1.shape
    for n, t in (("q1", q1), ("k1", k1), ("q2", q2), ("k2", k2)):
        if t.shape != q1.shape or t.dtype != torch.uint8:
            raise ValueError(f"{n} must be uint8 e4m3 codes of q1's shape")
    if qk_scale.dtype != torch.float32 or qk_scale.numel() != 4:
        raise ValueError("qk_scale must be fp32 [4]")
    if v.shape != (B, H, N, 2 * d) or v.dtype != torch.bfloat16:
        raise ValueError("v must be bf16 [B,H,N,2d]")
    if lam_t.dtype != torch.float32:
        raise ValueError("lambda must be fp32")
    _weight(weight, d)
    if out is None:
        out = torch.empty_like(v)
    else:
        _like(out, "out", v.shape, v.dtype, v.device)
    flags = (CAUSAL if causal else 0) | (0 if norm else NO_NORM)
    _check(lib().diffattn_fwd_fp8qk(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(qk_scale), _ptr(v), _ptr(out),
                                    B, H, N, d, _ptr(lam_t), float(lambda_init), _ptr(weight), float(eps),
                                    flags, _stream(q1.device)), "diffattn_fwd_fp8qk")
    return out


def in_proj(x, w_qkv, H: int, d: int, outs=None):
    """x bf16 [B,N,d_model], w_qkv bf16 [3*H*2d, d_model] -> (q1, k1, q2, k2
    [B,H,N,d], v [B,H,N,2d]), bf16, in the attention's layout."""
    _dev(x, "x")
    _dev(w_qkv, "w_qkv")
    if x.dtype != torch.bfloat16 or w_qkv.dtype != torch.bfloat16 or x.dim() != 3:
        raise ValueError("x must be bf16 [B,N,d_model] and w_qkv bf16")
    B, N, dm = x.shape
    if w_qkv.shape != (3 * H * 2 * d, dm):
        raise ValueError("w_qkv must be [3*H*2d, d_model]")
    if outs is None:
        outs = tuple(torch.empty((B, H, N, d), dtype=torch.bfloat16, device=x.device) for _ in range(4)) + (
            torch.empty((B, H, N, 2 * d), dtype=torch.bfloat16, device=x.device),)
    if len(outs) != 5:
        raise ValueError("outs must be (q1, k1, q2, k2, v)")
    for n, t in zip(("q1", "k1", "q2", "k2", "v"), outs):
        _like(t, n, (B, H, N, 2 * d if n == "v" else d), torch.bfloat16, x.device)
    if w_qkv.device != x.device:
        raise ValueError("w_qkv must be on x's device")
    _check(lib().diffattn_in_proj(_ptr(x), _ptr(w_qkv), B, N, dm, H, d, *(_ptr(t) for t in outs),
                                  _stream(x.device)), "diffattn_in_proj")
    return outs


def out_proj(o, w_o, out=None):
    """o bf16 [B,H,N,2d], w_o bf16 [d_out, H*2d] -> y bf16 [B,N,d_out]."""
    _dev(o, "o")
    _dev(w_o, "w_o")
    if o.dtype != torch.bfloat16 or w_o.dtype != torch.bfloat16 or o.dim() != 4:
        raise ValueError("o must be bf16 [B,H,N,2d] and w_o bf16")
    B, H, N, dv = o.shape
    if w_o.dim() != 2 or w_o.shape[1] != H * dv:
        raise ValueError("w_o must be [d_out, H*2d]")
    if w_o.device != o.device:
        raise ValueError("w_o must be on o's device")
    if out is None:
        out = torch.empty((B, N, w_o.shape[0]), dtype=torch.bfloat16, device=o.device)
    _like(out, "out", (B, N, w_o.shape[0]), torch.bfloat16, o.device)
    _check(lib().diffattn_out_proj(_ptr(o), _ptr(w_o), B, H, N, dv // 2, w_o.shape[0], _ptr(out),
                                   _stream(o.device)), "diffattn_out_proj")
    return out

