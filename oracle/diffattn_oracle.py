"""Oracle for the fused differential-attention forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call this module.  It shares no code with the HIP path and imports
nothing from the package.

Everything here is plain NumPy in float64: slow, obviously correct, written
straight from the definitions on the source pages.  Citations name the page
and the section / equation they follow:

* page 1 = "Differential Transformer: Canceling Context Noise with Differential
  Attention" (priorstack.com), section "Cancelling Context Noise Through
  Attention Map Subtraction" -- the DiffAttn formula (Eq. 1) and the lambda
  re-parameterisation (Eq. 2).
* page 2 = "Differential attention" (datarekha.com), section "The
  noise-canceling idea" -- the formula again, the numerically stable softmax of
  the worked six-key example, and the printed example values.
* page 3 = "Differential Transformer" sample peer review (reviewpaper.ai),
  "Summary" (Eq. 1, Eq. 2 and Eq. 3: per-head normalisation followed by the
  fixed (1 - lambda_init) factor) and "Weaknesses" (head-wise RMSNorm; rows of
  the differential map sum to 1 - lambda; lambda is unconstrained).

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* the per-head normaliser is RMSNorm over the 2d value channels, without mean
  subtraction or bias, with eps added inside the square root;
* the RMSNorm weight has shape [2d] and is shared by all heads;
* the 1/sqrt(d) scale uses the per-map query/key width d (not 2d);
* lambda is one scalar per call, shared by all heads and tokens;
* causal means key j is visible to query i iff j <= i (diagonal included);
* decode attends the first cache_len[b] cached keys; a sequence with
  cache_len 0 attends nothing and its output is defined as zero.

The gradients (``backward``) are those of the same definitions: training is
the pages' workload (page 3, "Summary": lambda is learnable through its
vectors, and the normalised outputs are trained end to end), and the
derivative of a composition of softmax, a matrix product and RMSNorm is fixed
by the forward.  lambda_init is a schedule constant and gets no gradient.

Every function below is pinned by ``tests/test_oracle.py`` against facts that
do not come from this file: the printed example values, closed forms,
invariants, and library routines (torch's scaled_dot_product_attention and
rms_norm, in float64 on the CPU).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "lambda_scalar",
    "softmax_rows",
    "attention_map",
    "diff_weights",
    "pre_norm",
    "head_rmsnorm_scale",
    "forward",
    "forward_rows",
    "decode",
    "map_stats",
    "backward",
    "backward_dq_rows",
    "backward_dkv_keys",
]


def _f64(x) -> np.ndarray:
    """Upcast to float64 exactly (bf16 and fp32 values are representable)."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32/float64 on the CPU
        x = x.detach().to("cpu")
        import torch  # local import: torch is only plumbing for readback

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def lambda_scalar(lq1, lk1, lq2, lk2, lambda_init: float) -> float:
    """lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init.

    Page 1, "Cancelling Context Noise Through Attention Map Subtraction" (the
    re-parameterisation); page 3, "Summary", Eq. 2.
    """
    lq1, lk1, lq2, lk2 = (_f64(v) for v in (lq1, lk1, lq2, lk2))
    return float(math.exp(float(np.dot(lq1, lk1))) - math.exp(float(np.dot(lq2, lk2))) + float(lambda_init))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax along the last axis, made stable by subtracting the row maximum.

    Page 2, "The noise-canceling idea": the example subtracts the maximum before
    exponentiating.  Entries equal to -inf (masked keys) get weight exactly 0.
    """
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _visible(nq: int, nk: int, causal: bool, q_pos=None) -> np.ndarray:
    """Boolean [nq, nk]: may query row r see key j?

    Causal reading: the query at absolute position p sees key j iff j <= p.
    ``q_pos`` gives each row's absolute position (default 0..nq-1).
    """
    if not causal:
        return np.ones((nq, nk), dtype=bool)
    pos = np.arange(nq) if q_pos is None else np.asarray(q_pos)
    return np.arange(nk)[None, :] <= pos[:, None]


def attention_map(q: np.ndarray, k: np.ndarray, causal: bool, q_pos=None) -> np.ndarray:
    """softmax(Q K^T / sqrt(d)) for one head.  q: [nq, d], k: [nk, d].

    Page 1 / page 2 (Eq. 1): each map is a softmax of scaled dot products; d is
    the query/key width of that map.
    """
    q, k = _f64(q), _f64(k)
    d = q.shape[-1]
    s = (q @ k.T) / math.sqrt(d)
    s = np.where(_visible(q.shape[0], k.shape[0], causal, q_pos), s, -np.inf)
    return softmax_rows(s)


def diff_weights(q1, k1, q2, k2, lam: float, causal: bool, q_pos=None) -> np.ndarray:
    """The differential map D = softmax(Q1 K1^T/sqrt d) - lambda softmax(Q2 K2^T/sqrt d).

    Page 1 and page 2, Eq. 1; page 3 "Summary", Eq. 1.  Entries may be
    negative and each row sums to 1 - lambda (page 3, "Weaknesses").
    """
    return attention_map(q1, k1, causal, q_pos) - float(lam) * attention_map(q2, k2, causal, q_pos)


def pre_norm(q1, k1, q2, k2, v, lam: float, causal: bool, q_pos=None) -> np.ndarray:
    """Y = D V for one head: the DiffAttn output before normalisation (Eq. 1)."""
    return diff_weights(q1, k1, q2, k2, lam, causal, q_pos) @ _f64(v)


def head_rmsnorm_scale(y, weight, eps: float, lambda_init: float) -> np.ndarray:
    """out = (1 - lambda_init) * w * y / sqrt(mean(y^2) + eps) over the last axis.

    Page 3, "Summary", Eq. 3 (per-head normalisation, then the fixed
    (1 - lambda_init) factor) and "Weaknesses" (head-wise RMSNorm).
    """
    y = _f64(y)
    w = np.ones(y.shape[-1]) if weight is None else _f64(weight)
    ms = np.mean(y * y, axis=-1, keepdims=True)
    return (1.0 - float(lambda_init)) * (w * y) / np.sqrt(ms + float(eps))


def forward(q1, k1, q2, k2, v, lam: float, lambda_init: float, weight=None,
            eps: float = 1e-5, causal: bool = True, norm: bool = True,
            block: int = 512) -> np.ndarray:
    """Multi-head differential attention forward.

    q1, k1, q2, k2: [B, H, N, d]; v: [B, H, N, 2d]  ->  out [B, H, N, 2d].
    With ``norm=False`` returns Y = D V (Eq. 1) instead of Eq. 3's output.
    Query rows are processed ``block`` at a time to bound memory; blocking
    does not change any value (each row is independent).
    """
    q1, k1, q2, k2, v = (_f64(t) for t in (q1, k1, q2, k2, v))
    B, H, N, _ = q1.shape
    out = np.empty(v.shape[:3] + (v.shape[-1],), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, block):
                rows = np.arange(r0, min(N, r0 + block))
                y = pre_norm(q1[b, h, rows], k1[b, h], q2[b, h, rows], k2[b, h], v[b, h],
                             lam, causal, q_pos=rows)
                out[b, h, rows] = head_rmsnorm_scale(y, weight, eps, lambda_init) if norm else y
    return out


def forward_rows(q1, k1, q2, k2, v, rows, lam: float, lambda_init: float,
                 weight=None, eps: float = 1e-5, causal: bool = True,
                 norm: bool = True) -> np.ndarray:
    """Outputs of the given query rows only, for one head.

    q1, k1, q2, k2: [N, d]; v: [N, 2d]; rows: 1-D int array.  Each row is
    computed against its full (causal) key prefix, exactly as in ``forward``.
    Used to check sampled outputs at sizes where the full oracle is too slow.
    """
    rows = np.asarray(rows)
    kmax = int(rows.max()) + 1 if causal else _f64(k1).shape[0]
    k1, k2, v = _f64(k1)[:kmax], _f64(k2)[:kmax], _f64(v)[:kmax]
    y = pre_norm(_f64(q1)[rows], k1, _f64(q2)[rows], k2, v, lam, causal, q_pos=rows)
    return head_rmsnorm_scale(y, weight, eps, lambda_init) if norm else y


def decode(q1, q2, k1c, k2c, vc, cache_len, lam: float, lambda_init: float,
           weight=None, eps: float = 1e-5, norm: bool = True) -> np.ndarray:
    """One query token per sequence against a KV cache.

    q1, q2: [B, H, d]; k1c, k2c: [B, H, L, d]; vc: [B, H, L, 2d];
    cache_len: [B] ints (None = L).  Sequence b attends cached keys
    [0, cache_len[b]) with no mask (the new token's keys are already in the
    cache).  Same maths as ``forward`` with one query row (Eq. 1-3).
    A sequence with cache_len 0 gives zeros (reading: nothing to attend to).
    """
    q1, q2 = _f64(q1), _f64(q2)
    B, H, d = q1.shape
    L = k1c.shape[2]
    dv = vc.shape[-1]
    lens = np.full(B, L) if cache_len is None else np.asarray(cache_len).astype(np.int64)
    out = np.zeros((B, H, dv))
    for b in range(B):
        n = int(min(max(lens[b], 0), L))
        if n == 0:
            continue
        for h in range(H):
            y = pre_norm(q1[b, h][None], _f64(k1c[b, h, :n]), q2[b, h][None], _f64(k2c[b, h, :n]),
                         _f64(vc[b, h, :n]), lam, causal=False)
            out[b, h] = (head_rmsnorm_scale(y, weight, eps, lambda_init) if norm else y)[0]
    return out


def map_stats(q1, k1, q2, k2, v, causal: bool = True):
    """Per-map row statistics of the forward, for one head.

    q1, k1, q2, k2: [N, d]; v: [N, 2d].  Returns (lse1, lse2, o1, o2):
    lse_k[i] = log sum_j exp(s_k[i, j]) over visible keys (natural log, with
    s_k = Q_k K_k^T / sqrt d) and o_k = softmax(s_k) V, the per-map outputs
    whose difference o1 - lambda o2 is Y (Eq. 1, by linearity).
    """
    q1, k1, q2, k2, v = (_f64(t) for t in (q1, k1, q2, k2, v))
    d = q1.shape[-1]
    vis = _visible(q1.shape[0], k1.shape[0], causal)
    res = []
    for q, k in ((q1, k1), (q2, k2)):
        s = np.where(vis, (q @ k.T) / math.sqrt(d), -np.inf)
        m = np.max(s, axis=-1, keepdims=True)
        lse = (m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True)))[:, 0]
        res.append((lse, softmax_rows(s) @ v))
    return res[0][0], res[1][0], res[0][1], res[1][1]


def backward(q1, k1, q2, k2, v, lq1, lk1, lq2, lk2, lambda_init: float, dout,
             weight=None, eps: float = 1e-5, causal: bool = True) -> dict:
    """Gradients of L = sum(out * dout) for the forward of ``forward``.

    q1, k1, q2, k2: [B, H, N, d]; v, dout: [B, H, N, 2d]; lambda vectors [d];
    weight [2d] or None (ones).  Chain rule through the definitions, step by
    step (sigma = 1 - lambda_init, n = 2d, per row i):

    * Eq. 3: out = sigma w Y / r with r = sqrt(mean(Y^2) + eps), so
      dw = sum over rows of sigma dout Y / r, and with g = sigma w dout,
      dY = g / r - Y (g . Y) / (n r^3);
    * Eq. 1: Y = A1 V - lambda A2 V, so dV = (A1 - lambda A2)^T dY,
      dA1 = dY V^T, dA2 = -lambda dY V^T, dlambda = -sum(A2 * dY V^T);
    * softmax: dS = A * (dA - rowsum(A * dA)), then with S = Q K^T / sqrt d,
      dQ = dS K / sqrt d and dK = dS^T Q / sqrt d;
    * Eq. 2: lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init, so
      dlq1 = dlambda exp(lq1.lk1) lk1, dlk1 = dlambda exp(lq1.lk1) lq1 and
      the map-2 pair with the opposite sign.

    Returns float64 arrays dq1, dk1, dq2, dk2, dv, dweight, dlq1, dlk1, dlq2,
    dlk2 and the scalar dlambda.
    """
    q1, k1, q2, k2, v, g_out = (_f64(t) for t in (q1, k1, q2, k2, v, dout))
    lq1, lk1, lq2, lk2 = (_f64(t) for t in (lq1, lk1, lq2, lk2))
    lam = lambda_scalar(lq1, lk1, lq2, lk2, lambda_init)
    sigma = 1.0 - float(lambda_init)
    B, H, N, d = q1.shape
    n = v.shape[-1]
    w = np.ones(n) if weight is None else _f64(weight)
    vis = _visible(N, N, causal)
    grads = {k: np.zeros_like(t) for k, t in (("dq1", q1), ("dk1", k1), ("dq2", q2), ("dk2", k2), ("dv", v))}
    dweight = np.zeros(n)
    dlam = 0.0
    for b in range(B):
        for h in range(H):
            a1 = softmax_rows(np.where(vis, (q1[b, h] @ k1[b, h].T) / math.sqrt(d), -np.inf))
            a2 = softmax_rows(np.where(vis, (q2[b, h] @ k2[b, h].T) / math.sqrt(d), -np.inf))
            y = (a1 - lam * a2) @ v[b, h]
            r = np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + float(eps))
            go = g_out[b, h]
            dweight += np.sum(sigma * go * y / r, axis=0)
            g = sigma * w * go
            dy = g / r - y * np.sum(g * y, axis=-1, keepdims=True) / (n * r ** 3)
            grads["dv"][b, h] = (a1 - lam * a2).T @ dy
            da = dy @ v[b, h].T  # dL/dA1; dL/dA2 = -lam * da
            dlam += -float(np.sum(a2 * da))
            for a, dak, q, k, dq, dk in ((a1, da, q1, k1, "dq1", "dk1"), (a2, -lam * da, q2, k2, "dq2", "dk2")):
                ds = a * (dak - np.sum(a * dak, axis=-1, keepdims=True))
                grads[dq][b, h] = ds @ k[b, h] / math.sqrt(d)
                grads[dk][b, h] = ds.T @ q[b, h] / math.sqrt(d)
    e1 = math.exp(float(np.dot(lq1, lk1)))
    e2 = math.exp(float(np.dot(lq2, lk2)))
    grads.update(dweight=dweight, dlambda=dlam,
                 dlq1=dlam * e1 * lk1, dlk1=dlam * e1 * lq1,
                 dlq2=-dlam * e2 * lk2, dlk2=-dlam * e2 * lq2)
    return grads


def backward_dq_rows(q1, k1, q2, k2, v, rows, lq1, lk1, lq2, lk2, lambda_init: float, dout_rows,
                     weight=None, eps: float = 1e-5, causal: bool = True):
    """dQ1 and dQ2 of the given query rows only, for one head.

    q1, k1, q2, k2: [N, d]; v: [N, 2d]; rows: 1-D ints; dout_rows: [len(rows), 2d],
    the output gradient of those rows.  The same chain rule as ``backward``,
    taken one row at a time: a row's dQ needs only that row's Y (its own
    forward row), its dY, and its scores against the keys it sees, so each
    row costs O(N d) and long sequences can be checked on sampled rows.
    Returns (dq1 [len(rows), d], dq2 [len(rows), d]).
    """
    q1, k1, q2, k2, v, g_out = (_f64(t) for t in (q1, k1, q2, k2, v, dout_rows))
    lam = lambda_scalar(lq1, lk1, lq2, lk2, lambda_init)
    sigma = 1.0 - float(lambda_init)
    d = q1.shape[-1]
    n = v.shape[-1]
    w = np.ones(n) if weight is None else _f64(weight)
    rows = np.asarray(rows)
    dq1 = np.zeros((len(rows), d))
    dq2 = np.zeros((len(rows), d))
    for r_i, i in enumerate(rows):
        kmax = int(i) + 1 if causal else k1.shape[0]
        a1 = softmax_rows((k1[:kmax] @ q1[i]) / math.sqrt(d))
        a2 = softmax_rows((k2[:kmax] @ q2[i]) / math.sqrt(d))
        y = (a1 - lam * a2) @ v[:kmax]
        r = math.sqrt(float(np.mean(y * y)) + float(eps))
        g = sigma * w * g_out[r_i]
        dy = g / r - y * float(np.dot(g, y)) / (n * r ** 3)
        da = v[:kmax] @ dy  # dL/dA1 for this row's keys; dL/dA2 = -lam * da
        ds1 = a1 * (da - float(np.dot(a1, da)))
        ds2 = a2 * (-lam * da - float(np.dot(a2, -lam * da)))
        dq1[r_i] = ds1 @ k1[:kmax] / math.sqrt(d)
        dq2[r_i] = ds2 @ k2[:kmax] / math.sqrt(d)
    return dq1, dq2


def backward_dkv_keys(q1, k1, q2, k2, v, keys, lq1, lk1, lq2, lk2, lambda_init: float, dout,
                      weight=None, eps: float = 1e-5, causal: bool = True, rows=None, block: int = 256):
    """dK1, dK2 and dV of the given keys only, for one head, summed over the
    query rows in ``rows`` (default: every row).

    q1, k1, q2, k2: [N, d]; v, dout: [N, 2d]; keys: 1-D ints; rows: a range of
    query rows (start, stop) or None.  The same chain rule as ``backward``,
    read column-wise: key j's gradients are sums over the query rows i that
    see it,

      dV[j]   = sum_i (A1[i,j] - lambda A2[i,j]) dY_i
      dK_k[j] = sum_i dS_k[i,j] Q_k[i] / sqrt d,
      dS_1[i,j] = A1[i,j] (dY_i . V_j - dY_i . O1_i),
      dS_2[i,j] = A2[i,j] (-lambda dY_i . V_j + lambda dY_i . O2_i),

    where each row's A_k, O_k = A_k V and dY come from that row's own forward
    against all the keys it sees.  A sum over rows splits exactly into sums
    over row ranges, so a long sequence can be covered range by range (in
    separate processes) and the partial results added.
    Returns (dk1 [len(keys), d], dk2 [len(keys), d], dv [len(keys), 2d]).
    """
    q1, k1, q2, k2, v, g_out = (_f64(t) for t in (q1, k1, q2, k2, v, dout))
    lam = lambda_scalar(lq1, lk1, lq2, lk2, lambda_init)
    sigma = 1.0 - float(lambda_init)
    N, d = q1.shape
    n = v.shape[-1]
    w = np.ones(n) if weight is None else _f64(weight)
    keys = np.asarray(keys)
    r_start, r_stop = (0, N) if rows is None else (int(rows[0]), int(rows[1]))
    if causal:  # rows before the first sampled key see none of them
        r_start = max(r_start, int(keys.min()))
    dk1 = np.zeros((len(keys), d))
    dk2 = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), n))
    for r0 in range(r_start, r_stop, block):
        rr = np.arange(r0, min(r_stop, r0 + block))
        kmax = int(rr[-1]) + 1 if causal else N
        vis = _visible(len(rr), kmax, causal, q_pos=rr)
        a1 = softmax_rows(np.where(vis, (q1[rr] @ k1[:kmax].T) / math.sqrt(d), -np.inf))
        a2 = softmax_rows(np.where(vis, (q2[rr] @ k2[:kmax].T) / math.sqrt(d), -np.inf))
        o1 = a1 @ v[:kmax]
        o2 = a2 @ v[:kmax]
        y = o1 - lam * o2
        r = np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + float(eps))
        g = sigma * w * g_out[rr]
        dy = g / r - y * np.sum(g * y, axis=-1, keepdims=True) / (n * r ** 3)
        sk = keys[keys < kmax]  # sampled keys inside this block's key range
        idx = np.nonzero(keys < kmax)[0]
        if len(sk) == 0:
            continue
        da = dy @ v[sk].T  # dL/dA1 at the sampled keys; dL/dA2 = -lambda da
        ds1 = a1[:, sk] * (da - np.sum(dy * o1, axis=-1, keepdims=True))
        ds2 = a2[:, sk] * (-lam * da + lam * np.sum(dy * o2, axis=-1, keepdims=True))
        dk1[idx] += ds1.T @ q1[rr] / math.sqrt(d)
        dk2[idx] += ds2.T @ q2[rr] / math.sqrt(d)
        dv[idx] += (a1[:, sk] - lam * a2[:, sk]).T @ dy
    return dk1, dk2, dv
