"""Benchmark of the differential-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = diffattn_lambda + diffattn_fwd over the 64K-token prefill (bf16,
B=1, H=12, N=65536, d=128, V width 256, causal, with needles): the largest
prefill workload that fits one GPU.  Prints ONE JSON line: the whole-step
throughput in TFLOP/s (12 d flops per causal query/key pair), the prefill
kernel's roofline fraction against the bf16 dense MFMA peak, the CPU fp64
oracle timed on a bounded sample of the same workload (sampled rows,
extrapolated per pair), and beside them: the 1.4B- and 3B-scale layer
prefills (each with its own roofline), a decode leg (diffattn_decode on 64
sequences x 16 heads x 32768 cached keys, d=128) in HBM GB/s against the
8 TB/s peak, a training leg (diffattn_fwd_train + diffattn_bwd on the 1.4B
layer), the fp8 query/key prefill and the projections.  Inputs are seeded
synthetic tensors already resident in HBM when timing starts.  Prefill steps
are replayed from HIP graphs (checked equal to the eager step) so that host
launch overhead does not idle the GPU; kernel durations come from HIP events
on the stream the kernels run on.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA (twice the bf16 rate)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "diff-attn fwd TFLOP/s & % bf16 MFMA peak (prefill); decode HBM GB/s & % peak"


# the prefill kernels and the host code that picks their schedule (which
# decides how the key tiles meet the L2 caches)
PREFILL_SOURCES = "prefill.hip,schedule.hip"


def _traffic(kind: str, src: str):
    """Per-launch HBM bytes from the committed counter summary, if it was
    taken on the current kernel source and headers; else None."""
    from transformer_attention_diffattn_amd.traffic_summary import source_hash

    path = os.path.join(ROOT, "profiles", f"{kind}_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except OSError:
        return None
    return t.get("bytes_per_launch") if t.get("source_sha256_16") == source_hash(src) else None


def _graph(fn, torch):
    """Capture fn (library launches on torch's current stream) into a HIP
    graph after one eager warm-up call on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _prewarm(replay, seconds, torch):
    """Untimed replays for about `seconds` of wall time (outside the timed
    region), so that the timed steps run at the sustained core clock rather
    than at the clock of an idle GPU."""
    if seconds <= 0:
        return
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(50):
            replay()
        torch.cuda.synchronize()


def _timed(replay, n, stream, torch):
    """Milliseconds for n back-to-back calls of replay(), from HIP events on
    the stream the work runs on."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def prefill_leg(w, x, steps, warmup, prewarm_s, stream, torch, da, W):
    """One prefill workload: diffattn_lambda + diffattn_fwd per step, replayed
    from a HIP graph of R consecutive steps (checked equal to the eager step),
    timed with HIP events on the stream the kernels run on.  Returns the
    leg's figures and the lambda launch's own time."""
    lam_t = torch.empty(1, device=x["q1"].device, dtype=torch.float32)
    out = torch.empty_like(x["v"])

    def step():
        da.lam(x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"], out=lam_t)
        da.fwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam_t, x["lambda_init"], eps=x["eps"],
               causal=w.causal, out=out)

    # One graph holds R consecutive steps (each exactly the eager step's two
    # library launches) and is replayed steps / R times, so one host launch
    # covers R steps and the host's per-call overhead does not idle the GPU.
    R = next(r for r in (20, 10, 8, 5, 4, 2, 1) if steps % r == 0)
    step()
    torch.cuda.synchronize()
    eager = out.clone()

    def lams_r():
        for _ in range(R):
            da.lam(x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"], out=lam_t)

    g_step = _graph(lambda: [step() for _ in range(R)], torch)
    g_lam = _graph(lams_r, torch)
    _prewarm(g_step.replay, prewarm_s, torch)
    for _ in range(-(-warmup // R)):
        g_step.replay()
    total_ms = _timed(g_step.replay, steps // R, stream, torch)
    if not torch.equal(out, eager):
        raise RuntimeError(f"graph replay of the {w.name} step differs from the eager step")
    # The dominant kernel's own time in the same launch configuration: the
    # step less its lambda launch, timed alone the same way.  (Forward
    # launches replayed back to back with nothing between them run slower:
    # each persistent grid then starts on compute units as the previous one
    # releases them, unevenly.)
    for _ in range(-(-warmup // R)):
        g_lam.replay()
    lam_ms = _timed(g_lam.replay, steps // R, stream, torch) / steps
    ms_step = total_ms / steps
    kern_ms = ms_step - lam_ms
    flops = 12.0 * w.d * w.pairs() * w.B * w.H
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    leg = {
        "value": round(value, 2), "ms_per_step": round(ms_step, 4), "steps_per_graph": R,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "v_width": 2 * w.d,
                   "causal": w.causal, "lambda_init": x["lambda_init"],
                   "flops_per_pair": 12 * w.d, "pairs_per_head": w.pairs(),
                   "needle_offsets": list(w.needle_offsets)},
        "roofline": {"bound": "mfma", "kernel": f"prefill_bf16_kernel<{w.d},{'causal' if w.causal else 'full'},norm>",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": (_traffic(W.PREFILL_TRAFFIC[w.name], PREFILL_SOURCES)
                                 if w.name in W.PREFILL_TRAFFIC else None),
                     # Q1, K1, Q2, K2 (4d) and V (2d) read once, out (2d) written once: 16 d bytes a row
                     "algorithmic_bytes": 16 * w.d * w.N * w.B * w.H,
                     "kernel_ms": round(kern_ms, 4), "lambda_ms": round(lam_ms, 5)},
    }
    del out
    return leg, lam_ms


def cpu_baseline(x, w, budget_s: float):
    """The oracle as it stands, on whole heads of the same inputs, until
    ``budget_s`` seconds of host time are spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import diffattn_oracle as O

    lam = O.lambda_scalar(x["lq1"].cpu(), x["lk1"].cpu(), x["lq2"].cpu(), x["lk2"].cpu(), x["lambda_init"])
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    if w.N > 8192:
        # long sequences: the dense oracle is far too slow for a whole head, so
        # evenly spaced query rows of the first head, each against its full
        # causal prefix, timed and priced by the pairs they cover; the rate is
        # extrapolated from that sample to the whole workload
        sl = lambda t: t[0, 0].cpu()
        pairs = 0
        h = {k: sl(x[k]) for k in ("q1", "k1", "q2", "k2", "v")}
        t0 = time.perf_counter()
        for r in np.linspace(0, w.N - 1, 4096).astype(np.int64):
            O.forward_rows(h["q1"], h["k1"], h["q2"], h["k2"], h["v"], [int(r)], lam, x["lambda_init"],
                           eps=x["eps"], causal=w.causal)
            pairs += int(r) + 1 if w.causal else w.N
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        return {"value": 12.0 * w.d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
                "kind": "oracle", "extrapolated": True,
                "sample": f"{done} evenly spaced query rows of head 0 with their full causal prefixes "
                          f"({pairs} pairs of the workload's {w.pairs() * w.B * w.H}), fp64 NumPy, {dt:.1f} s "
                          f"wall; rate extrapolated per pair"}
    for b, h in heads:
        sl = lambda t: t[b:b + 1, h:h + 1].cpu()
        O.forward(sl(x["q1"]), sl(x["k1"]), sl(x["q2"]), sl(x["k2"]), sl(x["v"]), lam, x["lambda_init"],
                  eps=x["eps"], causal=w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 12.0 * w.d * w.pairs() * done
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads of the same workload, every causal row, "
                      f"fp64 NumPy, {dt:.1f} s wall"}


def reference_gemm(torch, dev, n: int = 8192, seconds: float = 0.5):
    """Sustained rate of the vendor library's dense bf16 GEMM (torch.matmul,
    hipBLASLt) on this GPU in the same run: the practical matrix-pipe ceiling
    that the prefill rate can be read against.  Context only; no part of the
    differential-attention path uses it."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16).t().contiguous()
    c = a @ b
    torch.cuda.synchronize()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            c = a @ b
        torch.cuda.synchronize()
    k = 30
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(k):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / k
    del a, b, c
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def proj_leg(args, stream, torch, da, W):
    """The in- and out-projections of the 1.4B-scale layer (4 x 2048 tokens,
    d_model 2048, 16 heads of 2d = 128), each replayed from a graph of 10
    calls, with the vendor bf16 GEMM of the same shapes (plain products, no
    head split) timed beside them for context."""
    B, N, dm, H, d = 4, 2048, 2048, 16, 64
    dev = torch.device("cuda:0")
    x = W.projection_inputs(B, N, dm, H, d, seed=20266, device=dev)
    outs = da.in_proj(x["x"], x["w_qkv"], H, d)
    y = da.out_proj(x["o"], x["w_o"])
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs] + [y.clone()]
    R = 10
    steps = max(R, args.proj_steps // R * R)
    x2 = x["x"].reshape(B * N, dm)
    wq_t = x["w_qkv"].t().contiguous()
    o2 = x["o"].transpose(1, 2).reshape(B * N, H * 2 * d).contiguous()
    wo_t = x["w_o"].t().contiguous()
    ms = {}
    for name, fn in (("in", lambda: da.in_proj(x["x"], x["w_qkv"], H, d, outs=outs)),
                     ("out", lambda: da.out_proj(x["o"], x["w_o"], out=y)),
                     ("vendor_in", lambda: torch.matmul(x2, wq_t)),
                     ("vendor_out", lambda: torch.matmul(o2, wo_t))):
        g = _graph(lambda fn=fn: [fn() for _ in range(R)], torch)
        _prewarm(g.replay, min(0.3, args.prewarm_s), torch)
        ms[name] = _timed(g.replay, steps // R, stream, torch) / steps
    for a, b in zip(list(outs) + [y], eager):
        if not torch.equal(a, b):
            raise RuntimeError("graph replay of a projection differs from the eager call")
    M = B * N
    f_in, f_out = 2.0 * M * dm * 3 * H * 2 * d, 2.0 * M * H * 2 * d * dm
    t_in, t_out = f_in / (ms["in"] * 1e-3) / 1e12, f_out / (ms["out"] * 1e-3) / 1e12
    return {
        "shape": {"tokens": M, "d_model": dm, "H": H, "d": d},
        "in_proj": {"ms": round(ms["in"], 4), "tflops": round(t_in, 1),
                    "vendor_gemm_tflops": round(f_in / (ms["vendor_in"] * 1e-3) / 1e12, 1)},
        "out_proj": {"ms": round(ms["out"], 4), "tflops": round(t_out, 1),
                     "vendor_gemm_tflops": round(f_out / (ms["vendor_out"] * 1e-3) / 1e12, 1)},
        "roofline": {"bound": "mfma", "kernel": "proj256_kernel<in-projection>", "achieved": round(t_in, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(t_in / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic("proj_in_layer1p4b", "proj.hip"), "algorithmic_bytes": 159383552},
    }


def backward_leg(x, w, args, stream, torch, da):
    """diffattn_fwd_train and diffattn_bwd on the same workload, each replayed
    from a HIP graph (checked equal to the eager call).  The backward is priced
    at its algorithmic 20 d flops per causal pair (two QK^T products 4 d, dP 4 d,
    dV 4 d, dK1 + dK2 4 d, dQ1 + dQ2 4 d); the kernels execute 28 d, because
    the query-parallel dQ kernel evaluates S and dP again (32 d at d = 128,
where dV and dK are also computed apart)."""
    dev = x["q1"].device
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 7)
    dout = torch.randn(x["v"].shape, generator=gen, device=dev).to(torch.bfloat16)
    lam_t = da.lam(x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"])
    ws = torch.empty(da.bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    _, lse, o12 = da.fwd_train(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam_t, x["lambda_init"],
                               eps=x["eps"], causal=w.causal)
    grads = da.bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], dout, lse, o12, lam_t, x["lambda_init"],
                   eps=x["eps"], causal=w.causal, workspace=ws)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in grads.items()}

    def bstep():
        da.bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], dout, lse, o12, lam_t, x["lambda_init"],
               eps=x["eps"], causal=w.causal, workspace=ws, grads=grads)

    def fstep():
        da.fwd_train(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam_t, x["lambda_init"], eps=x["eps"],
                     causal=w.causal)

    R = 10
    n = max(R, args.bwd_steps // R * R)
    g_b = _graph(lambda: [bstep() for _ in range(R)], torch)
    _prewarm(g_b.replay, min(0.5, args.prewarm_s), torch)
    bms = _timed(g_b.replay, n // R, stream, torch) / n
    for k, v in grads.items():
        if not torch.equal(v, eager[k]):
            raise RuntimeError(f"graph replay of the backward differs from the eager call ({k})")
    g_f = _graph(lambda: [fstep() for _ in range(R)], torch)
    _prewarm(g_f.replay, min(0.3, args.prewarm_s), torch)
    fms = _timed(g_f.replay, n // R, stream, torch) / n
    flops = 20.0 * w.d * w.pairs() * w.B * w.H
    achieved = flops / (bms * 1e-3) / 1e12
    leg = {
        "workload": w.name, "ms_per_step": round(bms, 4), "flops_per_pair": 20 * w.d,
        "executed_flops_per_pair": 28 * w.d, "tflops": round(achieved, 2),
        "fwd_train_ms": round(fms, 4),
        "fwd_train_tflops": round(12.0 * w.d * w.pairs() * w.B * w.H / (fms * 1e-3) / 1e12, 2),
        # (at d <= 64 the dQ kernel also does the row-wise preparation)
        "roofline": {"bound": "mfma",
                     "kernel": ("" if w.d <= 64 else "bwd_prep + ") + "bwd_dq + bwd_reduce + bwd_dkv "
                               f"<{w.d},{'causal' if w.causal else 'full'}>",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": (_traffic("backward_layer1p4b", "backward.hip")
                                 if w.name == "layer1p4b_bf16_b4h16n2048d64" else None)},
    }
    if not args.no_cpu and w.N <= 8192:  # the oracle's backward holds dense N x N maps
        leg["cpu_baseline"] = cpu_backward(x, w, dout, budget_s=5.0)
    return leg


def fp8_leg(args, stream, torch, da, W):
    """The fp8 query/key prefill (diffattn_fwd_fp8qk) against the bf16 prefill
    on the same d = 128 workload, the quantiser that feeds it, and the layer
    step around it (in-projection, then either attention).  Its peak is that
    of its mix: per causal pair 4 d flops of QK^T at the fp8 rate and 8 d of
    PV at the bf16 rate."""
    w = W.WORKLOADS["layer3b_bf16_b2h12n4096d128"]
    dev = torch.device("cuda:0")
    x = W.workload_inputs(w.name, device=dev)
    lam_t = da.lam(x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"])
    names = ("q1", "k1", "q2", "k2")
    n = x["q1"].numel()
    codes = {k: torch.empty(x[k].shape, dtype=torch.uint8, device=dev) for k in names}
    scales = torch.empty(4, dtype=torch.float32, device=dev)
    qws = torch.empty(max(4, 4 * da.quantize_fp8_workspace_bytes(n)), dtype=torch.uint8, device=dev)
    out8 = torch.empty_like(x["v"])
    out16 = torch.empty_like(x["v"])

    xs = [x[k] for k in names]
    cl = [codes[k] for k in names]

    def quant():  # all four tensors in one pair of launches
        da.quantize_fp8_batch(xs, codes=cl, scales=scales, workspace=qws)

    def f8():
        da.fwd_fp8qk(codes["q1"], codes["k1"], codes["q2"], codes["k2"], scales, x["v"], lam_t,
                     x["lambda_init"], eps=x["eps"], causal=w.causal, out=out8)

    def f16():
        da.fwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam_t, x["lambda_init"], eps=x["eps"],
               causal=w.causal, out=out16)

    quant()
    f8()
    torch.cuda.synchronize()
    eager = out8.clone()
    R = 10
    steps = max(R, args.fp8_steps // R * R)
    ms = {}
    for name, fn, pre in (("quant", quant, 0.2), ("fp8", f8, min(0.5, args.prewarm_s)),
                          ("bf16", f16, min(0.5, args.prewarm_s))):
        g = _graph(lambda fn=fn: [fn() for _ in range(R)], torch)
        _prewarm(g.replay, pre, torch)
        ms[name] = _timed(g.replay, steps // R, stream, torch) / steps
    if not torch.equal(out8, eager):
        raise RuntimeError("graph replay of the fp8 prefill differs from the eager call")
    # the layer step the fp8 path sits in: the in-projection (B*N tokens x
    # d_model = H*2d -> Q1, K1, Q2, K2, V) then the attention, bf16 against
    # quantise + fp8 attention, each chain replayed from graphs like the rest
    p = W.projection_inputs(w.B, w.N, w.H * 2 * w.d, w.H, w.d, seed=w.seed + 11, device=dev)
    pq = da.in_proj(p["x"], p["w_qkv"], w.H, w.d)
    pcodes = [torch.empty(t.shape, dtype=torch.uint8, device=dev) for t in pq[:4]]
    pscales = torch.empty(4, dtype=torch.float32, device=dev)

    def proj():
        da.in_proj(p["x"], p["w_qkv"], w.H, w.d, outs=pq)

    def chain16():
        proj()
        da.fwd(pq[0], pq[1], pq[2], pq[3], pq[4], lam_t, x["lambda_init"], eps=x["eps"], causal=w.causal,
               out=out16)

    def chain8():
        proj()
        da.quantize_fp8_batch(list(pq[:4]), codes=pcodes, scales=pscales, workspace=qws)
        da.fwd_fp8qk(pcodes[0], pcodes[1], pcodes[2], pcodes[3], pscales, pq[4], lam_t, x["lambda_init"],
                     eps=x["eps"], causal=w.causal, out=out8)

    for name, fn in (("proj", proj), ("chain16", chain16), ("chain8", chain8)):
        g = _graph(lambda fn=fn: [fn() for _ in range(R)], torch)
        _prewarm(g.replay, min(0.3, args.prewarm_s), torch)
        ms[name] = _timed(g.replay, steps // R, stream, torch) / steps
    del p, pq, pcodes
    flops = 12.0 * w.d * w.pairs() * w.B * w.H
    peak = 12.0 / (4.0 / PEAK_FP8_TFLOPS + 8.0 / PEAK_BF16_TFLOPS)
    achieved = flops / (ms["fp8"] * 1e-3) / 1e12
    qbytes = 4 * 3 * n  # per tensor: n bf16 read, n codes written
    qgbs = qbytes / (ms["quant"] * 1e-3) / 1e9
    return {
        "workload": w.name, "ms_per_step": round(ms["fp8"], 4), "tflops": round(achieved, 2),
        "bf16_prefill_ms": round(ms["bf16"], 4),
        "bf16_prefill_tflops": round(flops / (ms["bf16"] * 1e-3) / 1e12, 2),
        "speedup_vs_bf16": round(ms["bf16"] / ms["fp8"], 3),
        "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel<128,causal,norm,fp8 QK^T>",
                     "achieved": round(achieved, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": _traffic("prefill_fp8qk_layer3b", PREFILL_SOURCES),
                     "peak_mix": "QK^T 4 d flops/pair at fp8 5033.2, PV 8 d at bf16 2516.6 TFLOP/s"},
        "layer_chain": {"what": "in-projection (%d tokens x %d -> %d) then attention" % (
                            w.B * w.N, w.H * 2 * w.d, 3 * w.H * 2 * w.d),
                        "in_proj_ms": round(ms["proj"], 4), "bf16_ms": round(ms["chain16"], 4),
                        "fp8_ms": round(ms["chain8"], 4),
                        "fp8_speedup": round(ms["chain16"] / ms["chain8"], 3)},
        "quantize": {"ms_per_call": round(ms["quant"], 4), "tensors": 4,
                     "end_to_end_ms": round(ms["quant"] + ms["fp8"], 4),
                     "roofline": {"bound": "hbm", "kernel": "amax_partial_kernel + quantize_kernel (4 tensors)",
                                  "achieved": round(qgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(qgbs / PEAK_HBM_GBS, 4),
                                  "traffic": _traffic("quant_fp8_layer3b", "quant.hip"),
                                  "algorithmic_bytes": qbytes}},
    }


def cpu_backward(x, w, dout, budget_s: float):
    """The oracle's backward as it stands, on whole heads of the same inputs,
    until ``budget_s`` seconds are spent; priced at 20 d flops per pair."""
    from threadpoolctl import threadpool_info

    from oracle import diffattn_oracle as O

    done = 0
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            sl = lambda t: t[b:b + 1, h:h + 1].cpu()
            O.backward(sl(x["q1"]), sl(x["k1"]), sl(x["q2"]), sl(x["k2"]), sl(x["v"]), x["lq1"].cpu(),
                       x["lk1"].cpu(), x["lq2"].cpu(), x["lk2"].cpu(), x["lambda_init"], sl(dout), eps=x["eps"],
                       causal=w.causal)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": 20.0 * w.d * w.pairs() * done / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{done} of {w.B * w.H} heads, dense fp64 NumPy, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-s", type=float, default=1.5,
                    help="seconds of untimed steps before the warmup steps: the GPU raises its "
                         "core clock only after some time under load")
    ap.add_argument("--decode-steps", type=int, default=10)
    ap.add_argument("--prefill-workload", default=None,
                    help="prefill workload to time instead of the headline one (a name in workloads.WORKLOADS)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg")
    ap.add_argument("--no-sublegs", action="store_true", help="skip the 1.4B / 3B layer prefill legs")
    ap.add_argument("--sub-steps", type=int, default=40, help="timed steps of each layer prefill leg")
    ap.add_argument("--no-bwd", action="store_true", help="skip the training (backward) leg")
    ap.add_argument("--bwd-steps", type=int, default=40)
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 query/key prefill leg")
    ap.add_argument("--no-proj", action="store_true", help="skip the projection leg")
    ap.add_argument("--proj-steps", type=int, default=40)
    ap.add_argument("--fp8-steps", type=int, default=40)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of CPU oracle time")
    ap.add_argument("--no-ref-gemm", action="store_true",
                    help="skip the vendor-GEMM reference rate (context for the roofline)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path has no multi-GPU leg "
              "(every (batch, head) is independent; sharding is described in the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from transformer_attention_diffattn_amd import binding as da
    from transformer_attention_diffattn_amd import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    # ---------------- prefill: the headline workload
    w = W.WORKLOADS[args.prefill_workload or W.HEADLINE_PREFILL]
    if w.kind != "prefill" or w.dtype != "bf16":
        raise SystemExit(f"{w.name}: the prefill leg times bf16 prefill workloads")
    x = W.workload_inputs(w.name, device=dev)
    leg, lam_ms = prefill_leg(w, x, args.steps, args.warmup, args.prewarm_s, stream, torch, da, W)
    res = {
        "metric": METRIC, "value": leg["value"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "prewarm_s": args.prewarm_s,
        "steps_per_graph": leg["steps_per_graph"], "ms_per_step": leg["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        # the same step priced at Eq. 1's 8 d flops per pair (two PV products only)
        "eq1_tflops": round(leg["value"] * 8.0 / 12.0, 2),
        "config": leg["config"],
        "roofline": leg["roofline"],
    }
    # cpu_baseline: the oracle on a bounded sample of the same workload
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(x, w, args.cpu_budget)
    del x

    # ---------------- the two model-layer prefills, each with its own roofline
    if not args.prefill_workload and not args.no_sublegs:
        res["prefill_layers"] = {}
        for name in W.PREFILL_SUBLEGS:
            ws = W.WORKLOADS[name]
            xs = W.workload_inputs(name, device=dev)
            sub, _ = prefill_leg(ws, xs, args.sub_steps, args.warmup, min(0.5, args.prewarm_s), stream, torch,
                                 da, W)
            res["prefill_layers"][name] = {k: sub[k] for k in ("ms_per_step", "value", "roofline", "config")}
            del xs

    # ---------------- decode leg
    if not args.no_decode:
        wd = W.WORKLOADS[W.HEADLINE_DECODE]
        y = W.workload_inputs(wd.name, device=dev)
        lam_d = da.lam(y["lq1"], y["lk1"], y["lq2"], y["lk2"], y["lambda_init"])
        ws = torch.empty(da.decode_workspace_bytes(wd.B, wd.H, wd.N, wd.d), dtype=torch.uint8, device=dev)
        outd = torch.empty((wd.B, wd.H, 1, 2 * wd.d), dtype=torch.bfloat16, device=dev)

        def dstep():
            da.decode(y["q1"], y["q2"], y["k1c"], y["k2c"], y["vc"], lam_d, y["lambda_init"],
                      cache_len=y["cache_len"], eps=y["eps"], workspace=ws, out=outd)

        for _ in range(2):
            dstep()
        dtotal = _timed(dstep, args.decode_steps, stream, torch)
        dms = dtotal / args.decode_steps
        nbytes = wd.B * wd.H * wd.N * 8 * wd.d  # K1 + K2 + V per cached key, bf16
        gbs = nbytes / (dms * 1e-3) / 1e9
        res["decode"] = {
            "workload": wd.name, "B": wd.B, "H": wd.H, "L": wd.N, "d": wd.d,
            "ms_per_step": round(dms, 4),
            "roofline": {"bound": "hbm", "kernel": "decode_split_kernel<bf16,128> + decode_merge_kernel",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": _traffic("decode_l32k", "decode.hip"),
                         "algorithmic_bytes": nbytes, "kernel_ms": round(dms, 4)},
        }
        del y, ws

    # ---------------- training leg: forward with saved statistics + backward
    if not args.no_bwd:
        # an error here must not cost the prefill and decode figures above:
        # it is reported in the leg's place (and on stderr)
        try:
            wb = W.WORKLOADS["layer1p4b_bf16_b4h16n2048d64"]
            res["backward"] = backward_leg(W.workload_inputs(wb.name, device=dev), wb, args, stream, torch, da)
        except Exception as e:  # noqa: BLE001
            print(f"training leg failed: {e!r}", file=sys.stderr, flush=True)
            res["backward"] = {"error": repr(e)}

    # ---------------- fp8 query/key prefill (d = 128)
    if not args.no_fp8:
        try:
            res["fp8_qk"] = fp8_leg(args, stream, torch, da, W)
        except Exception as e:  # noqa: BLE001
            print(f"fp8 leg failed: {e!r}", file=sys.stderr, flush=True)
            res["fp8_qk"] = {"error": repr(e)}

    # ---------------- projections either side of the attention
    if not args.no_proj:
        try:
            res["projections"] = proj_leg(args, stream, torch, da, W)
        except Exception as e:  # noqa: BLE001
            print(f"projection leg failed: {e!r}", file=sys.stderr, flush=True)
            res["projections"] = {"error": repr(e)}

    if not args.no_ref_gemm:
        g = reference_gemm(torch, dev)
        res["reference_gemm"] = {
            "what": "vendor bf16 GEMM 8192^3 (torch.matmul, hipBLASLt), sustained, same run; context only",
            "tflops": round(g, 1), "frac_of_peak": round(g / PEAK_BF16_TFLOPS, 4)}
        res["roofline"]["frac_of_reference_gemm"] = round(res["roofline"]["achieved"] / g, 4)
        for sub in res.get("prefill_layers", {}).values():
            sub["roofline"]["frac_of_reference_gemm"] = round(sub["roofline"]["achieved"] / g, 4)

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n

    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
