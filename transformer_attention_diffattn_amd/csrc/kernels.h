// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace diffattn {

struct PrefillArgs {
  const void* q1;
  const void* k1;
  const void* q2;
  const void* k2;
  const void* v;
  void* out;
  int BH;         // batch * heads
  int N;          // sequence length (>= 1)
  int n_qtiles;   // query tiles per head
  const float* lambda;  // device scalar
  float out_scale;      // 1 - lambda_init
  const float* norm_w;  // device [2d] or null (ones)
  float eps;
  float c;              // log2(e) / sqrt(d)
  float* lse;           // training forward: [2][BH][N] log2-sum-exp per map, or null
  float* osave;         // training forward: [2][BH][N][2d] per-map O / l, or null
  const float* qk_scale;  // fp8 queries/keys: device [4] scales of q1, k1, q2, k2; else null
};

struct DecodeArgs {
  const void* q1;
  const void* q2;
  const void* k1c;
  const void* k2c;
  const void* vc;
  const int* cache_len;  // device [B] or null
  void* out;
  int B, H, L;           // L = L_max (>= 0)
  int S;                 // splits per (b, h)
  int chunk;             // keys per split
  const float* lambda;
  float out_scale;
  const float* norm_w;
  float eps;
  float c;
  float* ws;             // [B*H*S] records of (4 + 4d) floats
};

struct BwdArgs {
  const void* q1;
  const void* k1;
  const void* q2;
  const void* k2;
  const void* v;
  const void* dout;     // [BH][N][2d] gradient of the output
  const float* lse;     // [2][BH][N] from the training forward (log2 units)
  const float* osave;   // [2][BH][N][2d] per-map O / l from the training forward
  void* dq1;
  void* dk1;
  void* dq2;
  void* dk2;
  void* dv;
  float* dweight;       // [2d]
  float* dlambda;       // [1]
  uint16_t* dy;         // workspace: [BH][N][2d] bf16 gradient of Y
  float* delta;         // workspace: [2][BH][N]
  float* partial;       // workspace: [prep workgroups][2d + 1]
  int BH;
  int N;
  const float* lambda;
  float out_scale;      // 1 - lambda_init
  const float* norm_w;  // [2d] or null (ones)
  float eps;
  float c;              // log2(e) / sqrt(d)
};

struct ProjArgs {
  const void* w;    // bf16 [F][K] (linear-layer layout: out x in)
  const void* x;    // in-projection: bf16 [M][K]; out-projection: bf16 [B][H][N][2d]
  void* q1;         // in-projection outputs: bf16 [B][H][N][d] (x4) and [B][H][N][2d]
  void* k1;
  void* q2;
  void* k2;
  void* v;
  void* y;          // out-projection output: bf16 [M][F]
  long long M;      // tokens, B * N
  int K;            // reduction length (multiple of 8)
  int F;            // output features (multiple of 4)
  int N, H;
  int log2_dv;      // log2(2d)
  int f_lo, f_hi;   // output features [f_lo, f_hi) of one launch (set by launch_proj)
};

// mode 0: in-projection, 1: out-projection
hipError_t launch_proj(int mode, const ProjArgs& a, hipStream_t stream);

// Query rows and threads per workgroup of the prefill kernels.
int prefill_block_rows(bool bf16, int d);
int prefill_block_threads(bool bf16, int d);

hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                         int d, float lambda_init, float* out, hipStream_t stream);

hipError_t launch_prefill(bool bf16, int d, bool causal, bool norm, const PrefillArgs& a,
                          hipStream_t stream);
// d = 128, e4m3 q1/k1/q2/k2 (a.qk_scale set), bf16 v and output
hipError_t launch_prefill_fp8qk(bool causal, bool norm, const PrefillArgs& a, hipStream_t stream);

// Per-tensor absmax e4m3 quantisation of `count` (1..kQuantBatch) bf16
// tensors of n values each: partial maxima of quant_partial_blocks(n)
// workgroups per tensor (partial: [count][P]), then each tensor's scale
// (scales[t]) and codes.
constexpr int kQuantBatch = 4;
struct QuantBatch {
  const uint16_t* x[kQuantBatch];
  uint8_t* codes[kQuantBatch];
  float* scale;
  float* partial;
  long long n;
  int P;
};
int quant_partial_blocks(long long n);
hipError_t launch_quantize_fp8(int count, const void* const* x, long long n, float* partial, void* const* codes,
                               float* scales, hipStream_t stream);

// Split plan for decode: number of splits and keys per split.
void decode_plan(int B, int H, int L, int d, int* S, int* chunk);
size_t decode_record_floats(int d);

hipError_t launch_decode(bool bf16, int d, bool norm, const DecodeArgs& a, hipStream_t stream);

// Backward: workgroups of the row-wise preparation kernel for `rows` rows
// (each writes one partial record), and the launch of all four kernels.
int bwd_prep_blocks(long long rows);
hipError_t launch_bwd(int d, bool causal, const BwdArgs& a, hipStream_t stream);
hipError_t launch_lambda_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int d,
                             const float* dlambda, float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                             hipStream_t stream);

}  // namespace diffattn
