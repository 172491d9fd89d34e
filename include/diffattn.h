/*
 * diffattn.h -- C ABI of libdiffattn.so: the fused differential-attention
 * forward for AMD Instinct MI355X (gfx950).
 *
 * What is computed (per batch b, head h, query row i):
 *
 *   lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init            (Eq. 2)
 *   D      = softmax(Q1 K1^T / sqrt(d)) - lambda softmax(Q2 K2^T / sqrt(d))
 *   Y      = D V                                                     (Eq. 1)
 *   out    = (1 - lambda_init) * w * Y / sqrt(mean_{2d}(Y^2) + eps)   (Eq. 3)
 *
 * Sources: "Differential Transformer: Canceling Context Noise with
 * Differential Attention" (priorstack.com), section "Cancelling Context Noise
 * Through Attention Map Subtraction" (Eq. 1 and the lambda formula);
 * "Differential attention" (datarekha.com), section "The noise-canceling
 * idea" (Eq. 1, stable softmax) and "How it's wired" (Q/K split in halves, V
 * twice as wide); the "Differential Transformer" sample review
 * (reviewpaper.ai), "Summary" (Eq. 1-3: per-head normalisation and the fixed
 * (1 - lambda_init) factor) and "Weaknesses" (head-wise RMSNorm, V width 2d).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP), owned by the caller; the
 *    library allocates nothing and keeps no state between calls.
 *  - Tensors are dense, contiguous, row-major, in the shapes given, and each
 *    pointer is 16-byte aligned.  `dt` gives the element type of q/k/v/out
 *    and of the caches; lambda vectors, lambda, the norm weight are fp32.
 *  - d is the per-map query/key width and must be 16, 32, 64 or 128; the
 *    value width is exactly 2d.  The 1/sqrt(d) scale uses that d.
 *  - Arguments are validated before any HIP call.  A bad argument returns
 *    DIFFATTN_EINVAL / DIFFATTN_EUNSUPPORTED / DIFFATTN_EWORKSPACE and
 *    launches nothing.  A failed launch returns DIFFATTN_EHIP.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and runs asynchronously; faults surface at the caller's next sync.
 *  - Empty work (B, H or N equal to 0; for decode B or H) is valid: the call
 *    returns DIFFATTN_OK without inspecting pointers or launching anything.
 *  - Reads of the inputs and writes of the outputs never overlap: `out` must
 *    not alias any input.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIFFATTN_ABI_VERSION 5

#if defined(__GNUC__) || defined(__clang__)
#define DIFFATTN_API __attribute__((visibility("default")))
#else
#define DIFFATTN_API
#endif

typedef enum {
  DIFFATTN_OK = 0,
  DIFFATTN_EINVAL = 1,       /* null/misaligned pointer, negative size, bad flag  */
  DIFFATTN_EUNSUPPORTED = 2, /* d or dtype outside the supported set              */
  DIFFATTN_EHIP = 3,         /* a HIP launch or query failed                      */
  DIFFATTN_EWORKSPACE = 4    /* workspace missing or too small                    */
} diffattn_status;

typedef enum { DIFFATTN_FP32 = 0, DIFFATTN_BF16 = 1 } diffattn_dtype;

/* Key j is visible to query i iff j <= i (diagonal included). */
#define DIFFATTN_CAUSAL 1u
/* Emit Y = D V (Eq. 1 output) and skip the RMSNorm and the scale.  A testing
 * hook: lambda_init, norm_weight and eps are then ignored. */
#define DIFFATTN_NO_NORM 2u

/*
 * diffattn_lambda -- Eq. 2: lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init.
 *   lq1, lk1, lq2, lk2 : device fp32 [d], d in 1..4096.
 *   lambda_out         : device fp32 [1]; written by the kernel.
 * One scalar per call (per layer); it is shared by all heads and tokens and
 * is not clamped (it may be negative or exceed 1).
 */
DIFFATTN_API diffattn_status diffattn_lambda(const float* lq1, const float* lk1, const float* lq2,
                                const float* lk2, int d, float lambda_init,
                                float* lambda_out, void* stream);

/*
 * diffattn_fwd -- prefill: Eq. 1 for every query row, then Eq. 3.
 *   q1, k1, q2, k2 : [B, H, N, d]   of dtype dt
 *   v              : [B, H, N, 2d]  of dtype dt
 *   out            : [B, H, N, 2d]  of dtype dt (bf16 results are rounded to
 *                    nearest-even from fp32)
 *   lambda         : device fp32 [1] (e.g. from diffattn_lambda)
 *   lambda_init    : host scalar; the output is multiplied by (1 - lambda_init)
 *   norm_weight    : device fp32 [2d] shared by all heads, or NULL for ones
 *   eps            : added to mean(Y^2) inside the square root (>= 0)
 *   flags          : DIFFATTN_CAUSAL | DIFFATTN_NO_NORM
 * Softmax and all accumulation are fp32; for dt = BF16 the probabilities
 * enter the PV product rounded to bf16, except in rows that see no more
 * than one key tile of keys (32 at d = 128, 64 below: the first rows of a
 * causal head, every row of a sequence that short), where they enter as the
 * sum of two bf16 terms (relative 2^-17) because the norm can amplify their
 * rounding when the two maps nearly cancel.
 * Size limit (dt = BF16): a head's output rows are addressed with 32-bit byte
 * offsets, so N * 2d * 2 must stay below 2^31 (N < 4,194,304 at d = 128);
 * larger N returns DIFFATTN_EINVAL.  B * H must fit an int.
 */
DIFFATTN_API diffattn_status diffattn_fwd(diffattn_dtype dt, const void* q1, const void* k1, const void* q2,
                             const void* k2, const void* v, void* out, int B, int H, int N, int d,
                             const float* lambda, float lambda_init, const float* norm_weight,
                             float eps, unsigned flags, void* stream);

/*
 * diffattn_decode_workspace_bytes -- bytes of device scratch that
 * diffattn_decode needs for these sizes (0 if the sizes are invalid or
 * empty).  The caller allocates it; its contents need no initialisation.
 */
DIFFATTN_API size_t diffattn_decode_workspace_bytes(int B, int H, int L_max, int d);

/*
 * diffattn_decode -- one new query token per sequence against a KV cache.
 *   q1, q2    : [B, H, 1, d]
 *   k1c, k2c  : [B, H, L_max, d]
 *   vc        : [B, H, L_max, 2d]
 *   cache_len : device int32 [B]; sequence b attends cached keys
 *               [0, cache_len[b]) with no mask (the new token's keys are
 *               already in the cache).  NULL means L_max for all.  Values are
 *               clamped to [0, L_max]; a sequence with 0 keys outputs zeros.
 *   out       : [B, H, 1, 2d]
 *   lambda, lambda_init, norm_weight, eps: as for diffattn_fwd.
 *   workspace : device scratch of at least
 *               diffattn_decode_workspace_bytes(B, H, L_max, d) bytes,
 *               16-byte aligned; calls that share a workspace must be
 *               ordered on one stream.
 * The split over the cache is a fixed function of (B, H, L_max, d), and
 * partial results merge in a fixed order, so results are deterministic.
 */
DIFFATTN_API diffattn_status diffattn_decode(diffattn_dtype dt, const void* q1, const void* q2,
                                const void* k1c, const void* k2c, const void* vc,
                                const int* cache_len, void* out, int B, int H, int L_max, int d,
                                const float* lambda, float lambda_init, const float* norm_weight,
                                float eps, void* workspace, size_t workspace_bytes, void* stream);

/*
 * diffattn_decode_noalloc -- diffattn_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * results (bit for bit) and errors as diffattn_decode; the split records go
 * to a fixed device array inside the library, DIFFATTN_NOALLOC_SCRATCH_BYTES
 * bytes, one per GPU, held until the process ends.  The call allocates
 * nothing.
 *   Sizes whose diffattn_decode_workspace_bytes(B, H, L_max, d) exceeds
 *   DIFFATTN_NOALLOC_SCRATCH_BYTES return DIFFATTN_EWORKSPACE and launch
 *   nothing (64 sequences x 16 heads x 32768 keys at d = 128 need 16.9 MB).
 *   Every call on one GPU uses the same array: calls that overlap in time on
 *   one GPU (different streams, or different host threads without ordering)
 *   race and must not be issued; calls ordered on one stream are safe.
 *   The first call on each device looks the array's address up (no
 *   allocation); a failure there returns DIFFATTN_EHIP.
 */
#define DIFFATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
DIFFATTN_API diffattn_status diffattn_decode_noalloc(diffattn_dtype dt, const void* q1, const void* q2,
                                        const void* k1c, const void* k2c, const void* vc,
                                        const int* cache_len, void* out, int B, int H, int L_max,
                                        int d, const float* lambda, float lambda_init,
                                        const float* norm_weight, float eps, void* stream);

/*
 * Training: the gradients of the same forward.  The review page's "Summary"
 * describes the layer as trained end to end (lambda through its vectors,
 * Eq. 2; the per-head normalisation of Eq. 3); the derivatives follow from
 * Eq. 1-3 by the chain rule.  lambda_init is a schedule constant and gets no
 * gradient.  Supported: dt = BF16 and d in {32, 64, 128}; other values return
 * DIFFATTN_EUNSUPPORTED.
 *
 * diffattn_fwd_train -- diffattn_fwd (same arguments, NO_NORM not allowed)
 * that also keeps what the backward needs:
 *   lse : device fp32 [2, B, H, N]: per map k and row i, the log2-sum-exp
 *         log2(sum_j 2^(s_k[i,j] log2(e))) of the scaled scores
 *         s_k = Q_k K_k^T / sqrt(d) over the visible keys;
 *   o12 : device fp32 [2, B, H, N, 2d]: per map, softmax(s_k) V (so that
 *         Y = o12[0] - lambda o12[1]).
 * Both 16-byte aligned and written in full for rows < N.
 */
DIFFATTN_API diffattn_status diffattn_fwd_train(diffattn_dtype dt, const void* q1, const void* k1,
                                   const void* q2, const void* k2, const void* v, void* out, int B,
                                   int H, int N, int d, const float* lambda, float lambda_init,
                                   const float* norm_weight, float eps, unsigned flags, float* lse,
                                   float* o12, void* stream);

/*
 * diffattn_bwd_workspace_bytes -- device scratch bytes that diffattn_bwd
 * needs for these sizes (0 if they are invalid, empty or unsupported).
 */
DIFFATTN_API size_t diffattn_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * diffattn_bwd -- gradients of L = sum(out * dout) for one diffattn_fwd_train
 * call with the same inputs, lambda, lambda_init, norm_weight, eps and flags.
 *   q1..v, lambda, lambda_init, norm_weight, eps, flags : as for the forward
 *                    (flags: DIFFATTN_CAUSAL or 0)
 *   dout           : [B, H, N, 2d] of dtype dt
 *   lse, o12       : the training forward's outputs (read only)
 *   dq1, dk1, dq2, dk2 : [B, H, N, d] of dtype dt, written in full
 *   dv             : [B, H, N, 2d] of dtype dt, written in full
 *   dlambda        : device fp32 [1]: dL/dlambda (summed over all rows);
 *                    diffattn_lambda_bwd takes it to the lambda vectors
 *   dweight        : device fp32 [2d]: dL/dnorm_weight (written even when
 *                    norm_weight is NULL, as the gradient at ones)
 *   workspace      : at least diffattn_bwd_workspace_bytes(B, H, N, d) bytes,
 *                    256-byte aligned, no initialisation needed; calls that
 *                    share it must be ordered on one stream.
 * Products are bf16 matrix operations with fp32 accumulation; the softmax
 * weights and the gradient of Y enter them rounded to bf16.  dQ is computed
 * apart from dK/dV (no atomics), and the sums over rows (dweight, dlambda)
 * are added in a fixed order, so results are deterministic.  Outputs must
 * not alias inputs.
 */
DIFFATTN_API diffattn_status diffattn_bwd(diffattn_dtype dt, const void* q1, const void* k1, const void* q2,
                             const void* k2, const void* v, const void* dout, const float* lse,
                             const float* o12, int B, int H, int N, int d, const float* lambda,
                             float lambda_init, const float* norm_weight, float eps, unsigned flags,
                             void* dq1, void* dk1, void* dq2, void* dk2, void* dv, float* dlambda,
                             float* dweight, void* workspace, size_t workspace_bytes, void* stream);

/*
 * diffattn_lambda_bwd -- Eq. 2 backward: with e1 = exp(lq1 . lk1) and
 * e2 = exp(lq2 . lk2), dlq1 = g e1 lk1, dlk1 = g e1 lq1, dlq2 = -g e2 lk2,
 * dlk2 = -g e2 lq2, where g = dlambda[0] (device fp32, e.g. from
 * diffattn_bwd).  All vectors are device fp32 [d], d in 1..4096.
 */
DIFFATTN_API diffattn_status diffattn_lambda_bwd(const float* lq1, const float* lk1, const float* lq2,
                                    const float* lk2, int d, const float* dlambda, float* dlq1,
                                    float* dlk1, float* dlq2, float* dlk2, void* stream);

/*
 * fp8 (e4m3) query/key path.  The "Differential Transformer" sample peer
 * review ("Strengths", Table 5 and Fig. 8) reports smaller attention-logit
 * outliers and a 4-bit quantisation study of the attention logits, pointing
 * to low-bit attention kernels; it gives no format.  This path is an
 * engineering reading of that: the logit product's operands Q and K are
 * quantised (not the logits), to OCP e4m3 (bias 7, no infinities, largest
 * finite value 448), so that the fp8 matrix cores form the logits in fp32.
 *
 * diffattn_quantize_fp8_workspace_bytes -- device scratch bytes that
 * diffattn_quantize_fp8 needs for n values (at most 1024; 0 for n < 0).
 */
DIFFATTN_API size_t diffattn_quantize_fp8_workspace_bytes(long long n);

/*
 * diffattn_quantize_fp8 -- per-tensor absmax quantisation of n bf16 values:
 *   scale[0] = amax / 448 and codes[i] = e4m3(x[i] * (448 / amax)), with
 *   amax = max |x|, float32 division and product, round to nearest even and
 *   saturation at 448; an all-zero tensor gives scale 1 and zero codes.
 *   x         : device bf16 [n], 16-byte aligned, finite values
 *   codes     : device uint8 [n], 16-byte aligned, written in full
 *   scale     : device fp32 [1], written
 *   workspace : at least diffattn_quantize_fp8_workspace_bytes(n) bytes,
 *               4-byte aligned; calls sharing it must be ordered on one stream.
 * n = 0 launches nothing and leaves scale unwritten.
 */
DIFFATTN_API diffattn_status diffattn_quantize_fp8(const void* x, long long n, void* codes, float* scale,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * diffattn_quantize_fp8_batch -- diffattn_quantize_fp8 of count (1..4)
 * tensors of n values each in one pair of launches: x[t] -> codes[t] and
 * scales[t].  x and codes are HOST arrays of count device pointers (each
 * 16-byte aligned); scales is device fp32 [count]; the workspace holds at
 * least count * diffattn_quantize_fp8_workspace_bytes(n) bytes.  Results are
 * those of count separate diffattn_quantize_fp8 calls.
 */
DIFFATTN_API diffattn_status diffattn_quantize_fp8_batch(int count, const void* const* x, long long n,
                                            void* const* codes, float* scales, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * diffattn_fwd_fp8qk -- the prefill of diffattn_fwd (Eq. 1 then Eq. 3) with
 * e4m3 queries and keys: the logits are (q . k) * sq * sk / sqrt(d), the
 * products of e4m3 values summed exactly into fp32 by the fp8 matrix cores.
 *   q1, k1, q2, k2 : device e4m3 bytes [B, H, N, d], d = 128 only
 *   qk_scale       : device fp32 [4]: the scales of q1, k1, q2, k2 (e.g. from
 *                    diffattn_quantize_fp8)
 *   v, out         : device bf16 [B, H, N, 2d]
 *   the rest       : as for diffattn_fwd with dt = DIFFATTN_BF16
 */
DIFFATTN_API diffattn_status diffattn_fwd_fp8qk(const void* q1, const void* k1, const void* q2, const void* k2,
                                   const float* qk_scale, const void* v, void* out, int B, int H, int N,
                                   int d, const float* lambda, float lambda_init,
                                   const float* norm_weight, float eps, unsigned flags, void* stream);

/*
 * Projections either side of the attention ("Differential attention" page,
 * section "How it's wired": each head's query and key projections are split
 * into halves Q1/K1 and Q2/K2; "Differential Transformer" sample peer
 * review, "Strengths": heads halved, h = d_model / 2d).  Weights use the
 * linear-layer layout W[out_features, in_features] (y = x W^T), no bias.
 * bf16 inputs and outputs, fp32 accumulation, outputs rounded to nearest
 * even.  All pointers are device memory, 16-byte aligned, not aliased.
 *
 * diffattn_in_proj -- [Q | K | V] = x [W_Q; W_K; W_V]^T with the head split:
 *   x      : [B, N, d_model], d_model a multiple of 8
 *   w_qkv  : [3 * H * 2d, d_model]: rows of W_Q, then W_K, then W_V; head h
 *            owns rows h*2d .. h*2d + 2d - 1 of each, of which the first d of
 *            W_Q (W_K) give Q1 (K1) and the last d give Q2 (K2)
 *   q1, k1, q2, k2 : [B, H, N, d] written; v : [B, H, N, 2d] written
 *   d in {16, 32, 64, 128}; B * N <= 8388480.
 */
DIFFATTN_API diffattn_status diffattn_in_proj(const void* x, const void* w_qkv, int B, int N, int d_model, int H,
                                 int d, void* q1, void* k1, void* q2, void* k2, void* v, void* stream);

/*
 * diffattn_out_proj -- y = Concat_h(o[:, h]) W_O^T:
 *   o    : [B, H, N, 2d], the attention output (e.g. of diffattn_fwd)
 *   w_o  : [d_out, H * 2d]; d_out a multiple of 4
 *   y    : [B, N, d_out] written
 *   d in {16, 32, 64, 128}; B * N <= 8388480.
 */
DIFFATTN_API diffattn_status diffattn_out_proj(const void* o, const void* w_o, int B, int H, int N, int d, int d_out,
                                  void* y, void* stream);

/* Static English text for a status code (never NULL). */
DIFFATTN_API const char* diffattn_strerror(diffattn_status status);

/* DIFFATTN_ABI_VERSION of the built library. */
DIFFATTN_API int diffattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
