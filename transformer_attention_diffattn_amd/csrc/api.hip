// C ABI of libdiffattn.so (declared in include/diffattn.h): argument
// validation, dispatch and launch.  Validation happens before any HIP call;
// the library allocates nothing and holds no state.

#include <math.h>
#include <stdint.h>

#include "../../include/diffattn.h"
#include "device_common.h"
#include "kernels.h"

namespace diffattn {

// lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init   (Eq. 2 of the
// "Differential Transformer" sample review, "Summary"; the same formula in
// "Cancelling Context Noise Through Attention Map Subtraction").  One wave.
__global__ __launch_bounds__(64) void lambda_kernel(const float* __restrict__ lq1, const float* __restrict__ lk1,
                                                    const float* __restrict__ lq2, const float* __restrict__ lk2,
                                                    int d, float lambda_init, float* __restrict__ out) {
  float a = 0.f, b = 0.f;
  for (int i = threadIdx.x; i < d; i += 64) {
    a += lq1[i] * lk1[i];
    b += lq2[i] * lk2[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off);
    b += __shfl_xor(b, off);
  }
  if (threadIdx.x == 0) out[0] = expf(a) - expf(b) + lambda_init;
}

hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int d,
                         float lambda_init, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(lambda_kernel, dim3(1), dim3(64), 0, stream, lq1, lk1, lq2, lk2, d, lambda_init, out);
  return hipGetLastError();
}

}  // namespace diffattn

namespace diffattn {
// decode.hip: address of the allocation-free decode's fixed scratch array
// (DIFFATTN_NOALLOC_SCRATCH_BYTES) on the device that runs `stream`
hipError_t decode_scratch(hipStream_t stream, float** ptr);
// backward.hip: columns of per-workgroup partial sums diffattn_bwd writes
int bwd_partial_count(int BH, int N, int d);
}  // namespace diffattn

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
bool ok_ptr16(const void* p) { return p != nullptr && aligned(p, 16); }
bool ok_ptr4(const void* p) { return p != nullptr && aligned(p, 4); }
bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_bwd_d(int d) { return d == 32 || d == 64 || d == 128; }
bool finite_nonneg(float x) { return isfinite(x) && x >= 0.f; }

}  // namespace

extern "C" {

int diffattn_abi_version(void) { return DIFFATTN_ABI_VERSION; }

const char* diffattn_strerror(diffattn_status s) {
  switch (s) {
    case DIFFATTN_OK: return "ok";
    case DIFFATTN_EINVAL: return "invalid argument (null or misaligned pointer, negative size, bad flag or eps)";
    case DIFFATTN_EUNSUPPORTED: return "unsupported dtype or head width d (d must be 16, 32, 64 or 128)";
    case DIFFATTN_EHIP: return "HIP launch or runtime error";
    case DIFFATTN_EWORKSPACE: return "workspace missing or smaller than the size its *_workspace_bytes() call gives";
    default: return "unknown status";
  }
}

diffattn_status diffattn_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int d,
                                float lambda_init, float* lambda_out, void* stream) {
  if (!ok_ptr4(lq1) || !ok_ptr4(lk1) || !ok_ptr4(lq2) || !ok_ptr4(lk2) || !ok_ptr4(lambda_out))
    return DIFFATTN_EINVAL;
  if (d < 1 || d > 4096 || !isfinite(lambda_init)) return DIFFATTN_EINVAL;
  hipError_t e = diffattn::launch_lambda(lq1, lk1, lq2, lk2, d, lambda_init, lambda_out, (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

static diffattn_status fwd_impl(diffattn_dtype dt, const void* q1, const void* k1, const void* q2, const void* k2,
                                const void* v, void* out, int B, int H, int N, int d, const float* lambda,
                                float lambda_init, const float* norm_weight, float eps, unsigned flags,
                                float* lse, float* osave, void* stream, const float* qk_scale = nullptr) {
  if (dt != DIFFATTN_FP32 && dt != DIFFATTN_BF16) return DIFFATTN_EUNSUPPORTED;
  if (!supported_d(d)) return DIFFATTN_EUNSUPPORTED;
  if (qk_scale && (dt != DIFFATTN_BF16 || d != 128)) return DIFFATTN_EUNSUPPORTED;
  if (B < 0 || H < 0 || N < 0) return DIFFATTN_EINVAL;
  if (flags & ~(DIFFATTN_CAUSAL | DIFFATTN_NO_NORM)) return DIFFATTN_EINVAL;
  const bool norm = !(flags & DIFFATTN_NO_NORM);
  if (norm && (!finite_nonneg(eps) || !isfinite(lambda_init))) return DIFFATTN_EINVAL;
  if ((long long)B * H * N == 0) return DIFFATTN_OK;  // empty work: pointers are not inspected
  if (!ok_ptr16(q1) || !ok_ptr16(k1) || !ok_ptr16(q2) || !ok_ptr16(k2) || !ok_ptr16(v) || !ok_ptr16(out))
    return DIFFATTN_EINVAL;
  if (!ok_ptr4(lambda)) return DIFFATTN_EINVAL;
  if (norm_weight && !aligned(norm_weight, 4)) return DIFFATTN_EINVAL;
  if (qk_scale && !ok_ptr4(qk_scale)) return DIFFATTN_EINVAL;
  const long long BH = (long long)B * H;
  const bool bf16 = dt == DIFFATTN_BF16;
  const int bm = diffattn::prefill_block_rows(bf16, d);
  const long long qtiles = ((long long)N + bm - 1) / bm;
  // one workgroup per (query tile, head); a launch holds at most 2^32 - 1 work-items
  if (BH > INT32_MAX || qtiles * BH * diffattn::prefill_block_threads(bf16, d) > (long long)UINT32_MAX)
    return DIFFATTN_EINVAL;
  // the bf16 kernel stores a head's output rows through a buffer resource
  // with 32-bit byte offsets: the head's N x 2d bf16 outputs must stay below 2^31 bytes
  if (bf16 && (long long)N * 2 * d * 2 > (long long)INT32_MAX) return DIFFATTN_EINVAL;

  diffattn::PrefillArgs a;
  a.q1 = q1;
  a.k1 = k1;
  a.q2 = q2;
  a.k2 = k2;
  a.v = v;
  a.out = out;
  a.BH = (int)BH;
  a.N = N;
  a.n_qtiles = (int)qtiles;
  a.lambda = lambda;
  a.out_scale = 1.0f - lambda_init;
  a.norm_w = norm_weight;
  a.eps = eps;
  a.c = (float)(1.4426950408889634 / sqrt((double)d));
  a.lse = lse;
  a.osave = osave;
  a.qk_scale = qk_scale;
  const bool causal = (flags & DIFFATTN_CAUSAL) != 0;
  hipError_t e = qk_scale ? diffattn::launch_prefill_fp8qk(causal, norm, a, (hipStream_t)stream)
                          : diffattn::launch_prefill(bf16, d, causal, norm, a, (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

diffattn_status diffattn_fwd(diffattn_dtype dt, const void* q1, const void* k1, const void* q2, const void* k2,
                             const void* v, void* out, int B, int H, int N, int d, const float* lambda,
                             float lambda_init, const float* norm_weight, float eps, unsigned flags,
                             void* stream) {
  return fwd_impl(dt, q1, k1, q2, k2, v, out, B, H, N, d, lambda, lambda_init, norm_weight, eps, flags, nullptr,
                  nullptr, stream);
}

diffattn_status diffattn_fwd_fp8qk(const void* q1, const void* k1, const void* q2, const void* k2,
                                   const float* qk_scale, const void* v, void* out, int B, int H, int N, int d,
                                   const float* lambda, float lambda_init, const float* norm_weight, float eps,
                                   unsigned flags, void* stream) {
  if (d != 128) return DIFFATTN_EUNSUPPORTED;
  if ((long long)B * H * N > 0 && !ok_ptr4(qk_scale)) return DIFFATTN_EINVAL;
  return fwd_impl(DIFFATTN_BF16, q1, k1, q2, k2, v, out, B, H, N, d, lambda, lambda_init, norm_weight, eps, flags,
                  nullptr, nullptr, stream, qk_scale);
}

static int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}

// grid: feature tiles in x, token tiles in y (at most 65535 each, 128 per tile)
static bool proj_grid_ok(long long M, long long F) {
  return M <= 65535LL * 128 && F <= 65535LL * 128;
}

diffattn_status diffattn_in_proj(const void* x, const void* w_qkv, int B, int N, int d_model, int H, int d,
                                 void* q1, void* k1, void* q2, void* k2, void* v, void* stream) {
  if (!supported_d(d)) return DIFFATTN_EUNSUPPORTED;
  if (B < 0 || N < 0 || H < 1 || d_model < 8 || d_model % 8 != 0) return DIFFATTN_EINVAL;
  const long long M = (long long)B * N, F = 3LL * H * 2 * d;
  if (!proj_grid_ok(M, F)) return DIFFATTN_EINVAL;
  if (M == 0) return DIFFATTN_OK;
  if (!ok_ptr16(x) || !ok_ptr16(w_qkv) || !ok_ptr16(q1) || !ok_ptr16(k1) || !ok_ptr16(q2) || !ok_ptr16(k2) ||
      !ok_ptr16(v))
    return DIFFATTN_EINVAL;
  diffattn::ProjArgs a = {};
  a.w = w_qkv;
  a.x = x;
  a.q1 = q1;
  a.k1 = k1;
  a.q2 = q2;
  a.k2 = k2;
  a.v = v;
  a.M = M;
  a.K = d_model;
  a.F = (int)F;
  a.N = N;
  a.H = H;
  a.log2_dv = log2_exact(2 * d);
  hipError_t e = diffattn::launch_proj(0, a, (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

diffattn_status diffattn_out_proj(const void* o, const void* w_o, int B, int H, int N, int d, int d_out, void* y,
                                  void* stream) {
  if (!supported_d(d)) return DIFFATTN_EUNSUPPORTED;
  if (B < 0 || N < 0 || H < 1 || d_out < 4 || d_out % 4 != 0) return DIFFATTN_EINVAL;
  const long long M = (long long)B * N, K = (long long)H * 2 * d;
  if (!proj_grid_ok(M, d_out) || K > INT32_MAX) return DIFFATTN_EINVAL;
  if (M == 0) return DIFFATTN_OK;
  if (!ok_ptr16(o) || !ok_ptr16(w_o) || !ok_ptr16(y)) return DIFFATTN_EINVAL;
  diffattn::ProjArgs a = {};
  a.w = w_o;
  a.x = o;
  a.y = y;
  a.M = M;
  a.K = (int)K;
  a.F = d_out;
  a.N = N;
  a.H = H;
  a.log2_dv = log2_exact(2 * d);
  hipError_t e = diffattn::launch_proj(1, a, (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

size_t diffattn_quantize_fp8_workspace_bytes(long long n) {
  if (n < 0) return 0;
  return (size_t)diffattn::quant_partial_blocks(n) * sizeof(float);
}

diffattn_status diffattn_quantize_fp8(const void* x, long long n, void* codes, float* scale, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (n < 0) return DIFFATTN_EINVAL;
  if (n == 0) return DIFFATTN_OK;
  if (!ok_ptr16(x) || !ok_ptr16(codes) || !ok_ptr4(scale)) return DIFFATTN_EINVAL;
  if (workspace == nullptr || !aligned(workspace, 4) || workspace_bytes < diffattn_quantize_fp8_workspace_bytes(n))
    return DIFFATTN_EWORKSPACE;
  const void* xs[1] = {x};
  void* cs[1] = {codes};
  hipError_t e = diffattn::launch_quantize_fp8(1, xs, n, (float*)workspace, cs, scale, (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

diffattn_status diffattn_quantize_fp8_batch(int count, const void* const* x, long long n, void* const* codes,
                                            float* scales, void* workspace, size_t workspace_bytes, void* stream) {
  if (count < 1 || count > diffattn::kQuantBatch || x == nullptr || codes == nullptr || n < 0) return DIFFATTN_EINVAL;
  if (n == 0) return DIFFATTN_OK;
  for (int t = 0; t < count; ++t)
    if (!ok_ptr16(x[t]) || !ok_ptr16(codes[t])) return DIFFATTN_EINVAL;
  if (!ok_ptr4(scales)) return DIFFATTN_EINVAL;
  if (workspace == nullptr || !aligned(workspace, 4) ||
      workspace_bytes < (size_t)count * diffattn_quantize_fp8_workspace_bytes(n))
    return DIFFATTN_EWORKSPACE;
  hipError_t e = diffattn::launch_quantize_fp8(count, x, n, (float*)workspace, codes, scales, (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

diffattn_status diffattn_fwd_train(diffattn_dtype dt, const void* q1, const void* k1, const void* q2,
                                   const void* k2, const void* v, void* out, int B, int H, int N, int d,
                                   const float* lambda, float lambda_init, const float* norm_weight, float eps,
                                   unsigned flags, float* lse, float* o12, void* stream) {
  if (dt != DIFFATTN_BF16 || !supported_bwd_d(d)) return DIFFATTN_EUNSUPPORTED;
  if (flags & DIFFATTN_NO_NORM) return DIFFATTN_EINVAL;
  if (B < 0 || H < 0 || N < 0) return DIFFATTN_EINVAL;
  if ((long long)B * H * N == 0) return DIFFATTN_OK;
  if (!ok_ptr16(lse) || !ok_ptr16(o12)) return DIFFATTN_EINVAL;
  return fwd_impl(dt, q1, k1, q2, k2, v, out, B, H, N, d, lambda, lambda_init, norm_weight, eps, flags, lse, o12,
                  stream);
}

// workspace layout of diffattn_bwd: dY (bf16), delta (fp32), partial sums
static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
static void bwd_layout(int B, int H, int N, int d, size_t* off_delta, size_t* off_part, size_t* total) {
  const size_t rows = (size_t)B * H * N;
  const size_t dy = round256(rows * 2 * d * 2);
  const size_t delta = round256(rows * 2 * 4);
  const size_t part = round256((size_t)diffattn::bwd_partial_count(B * H, N, d) * (2 * d + 1) * 4);
  *off_delta = dy;
  *off_part = dy + delta;
  *total = dy + delta + part;
}

size_t diffattn_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || !supported_bwd_d(d)) return 0;
  size_t od, op, total;
  bwd_layout(B, H, N, d, &od, &op, &total);
  return total;
}

diffattn_status diffattn_bwd(diffattn_dtype dt, const void* q1, const void* k1, const void* q2, const void* k2,
                             const void* v, const void* dout, const float* lse, const float* o12, int B, int H,
                             int N, int d, const float* lambda, float lambda_init, const float* norm_weight,
                             float eps, unsigned flags, void* dq1, void* dk1, void* dq2, void* dk2, void* dv,
                             float* dlambda, float* dweight, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (dt != DIFFATTN_BF16 || !supported_bwd_d(d)) return DIFFATTN_EUNSUPPORTED;
  if (B < 0 || H < 0 || N < 0) return DIFFATTN_EINVAL;
  if (flags & ~DIFFATTN_CAUSAL) return DIFFATTN_EINVAL;
  if (!finite_nonneg(eps) || !isfinite(lambda_init)) return DIFFATTN_EINVAL;
  if ((long long)B * H * N == 0) return DIFFATTN_OK;  // empty work: pointers are not inspected
  const void* in16[] = {q1, k1, q2, k2, v, dout, lse, o12, dq1, dk1, dq2, dk2, dv};
  for (const void* p : in16)
    if (!ok_ptr16(p)) return DIFFATTN_EINVAL;
  if (!ok_ptr4(lambda) || !ok_ptr4(dlambda) || !ok_ptr4(dweight)) return DIFFATTN_EINVAL;
  if (norm_weight && !aligned(norm_weight, 4)) return DIFFATTN_EINVAL;
  const long long BH = (long long)B * H;
  // grids of (N / 64) x BH workgroups; the kernels address a head's rows and
  // the [2, B*H*N] statistics with 32-bit byte offsets
  if (BH * N > (1LL << 28) || (long long)N * 4 * d >= (1LL << 32)) return DIFFATTN_EINVAL;
  size_t od, op, total;
  bwd_layout(B, H, N, d, &od, &op, &total);
  if (workspace == nullptr || workspace_bytes < total) return DIFFATTN_EWORKSPACE;
  if (!aligned(workspace, 256)) return DIFFATTN_EINVAL;

  diffattn::BwdArgs a;
  a.q1 = q1;
  a.k1 = k1;
  a.q2 = q2;
  a.k2 = k2;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.osave = o12;
  a.dq1 = dq1;
  a.dk1 = dk1;
  a.dq2 = dq2;
  a.dk2 = dk2;
  a.dv = dv;
  a.dweight = dweight;
  a.dlambda = dlambda;
  a.dy = (uint16_t*)workspace;
  a.delta = (float*)((char*)workspace + od);
  a.partial = (float*)((char*)workspace + op);
  a.BH = (int)BH;
  a.N = N;
  a.lambda = lambda;
  a.out_scale = 1.0f - lambda_init;
  a.norm_w = norm_weight;
  a.eps = eps;
  a.c = (float)(1.4426950408889634 / sqrt((double)d));
  hipError_t e = diffattn::launch_bwd(d, (flags & DIFFATTN_CAUSAL) != 0, a, (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

diffattn_status diffattn_lambda_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int d,
                                    const float* dlambda, float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                                    void* stream) {
  const float* in4[] = {lq1, lk1, lq2, lk2, dlambda, dlq1, dlk1, dlq2, dlk2};
  for (const float* p : in4)
    if (!ok_ptr4(p)) return DIFFATTN_EINVAL;
  if (d < 1 || d > 4096) return DIFFATTN_EINVAL;
  hipError_t e = diffattn::launch_lambda_bwd(lq1, lk1, lq2, lk2, d, dlambda, dlq1, dlk1, dlq2, dlk2,
                                             (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

size_t diffattn_decode_workspace_bytes(int B, int H, int L_max, int d) {
  if (B <= 0 || H <= 0 || L_max < 0 || !supported_d(d)) return 0;
  int S = 1, chunk = 0;
  diffattn::decode_plan(B, H, L_max, d, &S, &chunk);
  return (size_t)B * H * S * diffattn::decode_record_floats(d) * sizeof(float);
}

// validation and arguments shared by the two decode entry points (without
// the workspace)
static diffattn_status decode_args(diffattn_dtype dt, const void* q1, const void* q2, const void* k1c,
                                   const void* k2c, const void* vc, const int* cache_len, void* out, int B, int H,
                                   int L_max, int d, const float* lambda, float lambda_init,
                                   const float* norm_weight, float eps, diffattn::DecodeArgs* a, bool* empty) {
  *empty = false;
  if (dt != DIFFATTN_FP32 && dt != DIFFATTN_BF16) return DIFFATTN_EUNSUPPORTED;
  if (!supported_d(d)) return DIFFATTN_EUNSUPPORTED;
  if (B < 0 || H < 0 || L_max < 0) return DIFFATTN_EINVAL;
  if (!finite_nonneg(eps) || !isfinite(lambda_init)) return DIFFATTN_EINVAL;
  if ((long long)B * H == 0) {  // empty work: pointers are not inspected
    *empty = true;
    return DIFFATTN_OK;
  }
  if (B > 65535 || H > 65535) return DIFFATTN_EINVAL;
  if (!ok_ptr16(q1) || !ok_ptr16(q2) || !ok_ptr16(out) || !ok_ptr4(lambda)) return DIFFATTN_EINVAL;
  if (L_max > 0 && (!ok_ptr16(k1c) || !ok_ptr16(k2c) || !ok_ptr16(vc))) return DIFFATTN_EINVAL;
  if (cache_len && !aligned(cache_len, 4)) return DIFFATTN_EINVAL;
  if (norm_weight && !aligned(norm_weight, 4)) return DIFFATTN_EINVAL;
  a->q1 = q1;
  a->q2 = q2;
  a->k1c = k1c;
  a->k2c = k2c;
  a->vc = vc;
  a->cache_len = cache_len;
  a->out = out;
  a->B = B;
  a->H = H;
  a->L = L_max;
  diffattn::decode_plan(B, H, L_max, d, &a->S, &a->chunk);
  a->lambda = lambda;
  a->out_scale = 1.0f - lambda_init;
  a->norm_w = norm_weight;
  a->eps = eps;
  a->c = (float)(1.4426950408889634 / sqrt((double)d));
  a->ws = nullptr;
  return DIFFATTN_OK;
}

diffattn_status diffattn_decode(diffattn_dtype dt, const void* q1, const void* q2, const void* k1c, const void* k2c,
                                const void* vc, const int* cache_len, void* out, int B, int H, int L_max, int d,
                                const float* lambda, float lambda_init, const float* norm_weight, float eps,
                                void* workspace, size_t workspace_bytes, void* stream) {
  diffattn::DecodeArgs a;
  bool empty = false;
  const diffattn_status st = decode_args(dt, q1, q2, k1c, k2c, vc, cache_len, out, B, H, L_max, d, lambda,
                                         lambda_init, norm_weight, eps, &a, &empty);
  if (st != DIFFATTN_OK || empty) return st;
  const size_t need = diffattn_decode_workspace_bytes(B, H, L_max, d);
  if (workspace == nullptr || workspace_bytes < need) return DIFFATTN_EWORKSPACE;
  if (!aligned(workspace, 16)) return DIFFATTN_EINVAL;
  a.ws = (float*)workspace;
  hipError_t e = diffattn::launch_decode(dt == DIFFATTN_BF16, d, true, a, (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

diffattn_status diffattn_decode_noalloc(diffattn_dtype dt, const void* q1, const void* q2, const void* k1c,
                                        const void* k2c, const void* vc, const int* cache_len, void* out, int B,
                                        int H, int L_max, int d, const float* lambda, float lambda_init,
                                        const float* norm_weight, float eps, void* stream) {
  diffattn::DecodeArgs a;
  bool empty = false;
  const diffattn_status st = decode_args(dt, q1, q2, k1c, k2c, vc, cache_len, out, B, H, L_max, d, lambda,
                                         lambda_init, norm_weight, eps, &a, &empty);
  if (st != DIFFATTN_OK || empty) return st;
  if (diffattn_decode_workspace_bytes(B, H, L_max, d) > DIFFATTN_NOALLOC_SCRATCH_BYTES) return DIFFATTN_EWORKSPACE;
  hipError_t e = diffattn::decode_scratch((hipStream_t)stream, &a.ws);
  if (e != hipSuccess) return DIFFATTN_EHIP;
  e = diffattn::launch_decode(dt == DIFFATTN_BF16, d, true, a, (hipStream_t)stream);
  return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

}  // extern "C"
