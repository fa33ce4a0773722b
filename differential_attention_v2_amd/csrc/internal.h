// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace diffattn {

struct PrefillProblem {
  const void* q;
  const void* k;
  const void* v;
  const float* lam;
  void* out;
  int B, T, Hq, Hkv, d;
  int causal;
  int v1_rmsnorm;
  float eps;
  int window = 0;   // causal sliding window in keys, 0 = none (bf16 kernel)
  // training forward only (bf16, V2): the subtracted branch's output [B, T, P, d]
  // and the natural-log log-sum-exp of every row [B, T, Hq]; null otherwise
  void* o2 = nullptr;
  float* lse = nullptr;
};

struct DecodeProblem {
  const void* q;
  const void* k;
  const void* v;
  const float* lam;
  void* out;
  float* ws;
  int B, L, Hq, Hkv, d;
  int splits;       // number of key ranges per (b, KV head)
  int chunk;        // keys per range, a multiple of 32
  int v1_rmsnorm;
  float eps;
  const int* seq_lens = nullptr;   // valid cache rows per sequence (device), or null = L
  int window = 0;                  // keys before the query that stay visible, 0 = all
  int flat_ranges = 0;             // > 0: ragged caches split evenly into this many ranges per KV head
};

// Ragged-cache decode workspace: records [Hq][ranges + B][d+4] fp32, then the
// plan: B + 2 ints.
inline size_t decode_flat_record_floats(int B, int Hq, int d, int ranges) {
  return (size_t)Hq * (ranges + B) * (d + 4);
}
inline size_t decode_flat_workspace_bytes(int B, int Hq, int d, int ranges) {
  return decode_flat_record_floats(B, Hq, d, ranges) * sizeof(float) + (size_t)(B + 2) * sizeof(int);
}

// Decode in the layouts V2 is compared against: a standard transformer (H heads,
// one softmax each) or DIFF V1 (each head's q and k split into halves, one pass
// per branch over the full V).  q [B, H, d], caches [B, L, Hkv, d], lam [B, H]
// (V1), out [B, H, d]; ws holds one [B, H, splits, d+4] record array per pass.
struct CompareProblem {
  const void* q;
  const void* k;
  const void* v;
  const float* lam;
  void* out;
  float* ws;
  int B, L, H, Hkv, d;
  int splits, chunk;
  int v1_layout;
  int v1_rmsnorm;
  float eps;
};

// Backward pass (bf16, V2).  The workspace holds, in order: per-pair row
// statistics [B][P][5][Tpad] fp32 (log2-domain LSE of both heads, D_1, D_2,
// lambda; Tpad = T rounded up to 32), then fp32 dK and dV accumulators
// [B, T, Hkv, d] each.
struct BackwardProblem {
  const void* q;
  const void* k;
  const void* v;
  const float* lam;
  const void* out;
  const void* o2;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dlam;
  float* ws;
  int B, T, Hq, Hkv, d;
  int causal;
};
constexpr int kBackwardFields = 5;
inline int backward_tpad(int T) { return (T + 31) / 32 * 32; }
inline size_t backward_rs_floats(int B, int T, int Hq) {
  return (size_t)B * (Hq / 2) * kBackwardFields * backward_tpad(T);
}
inline size_t backward_workspace_floats(int B, int T, int Hq, int Hkv, int d) {
  return backward_rs_floats(B, T, Hq) + 2 * (size_t)B * T * Hkv * d;
}

// Floats per partial-state record in the decode workspace: acc[d], m, l, 2 pad
// (keeps every record 16-byte aligned).
inline int decode_record_floats(int d) { return d + 4; }

hipError_t launch_prefill_bf16(const PrefillProblem& p, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeProblem& p, hipStream_t s);
hipError_t launch_backward_bf16(const BackwardProblem& p, hipStream_t s);
hipError_t launch_decode_compare_bf16(const CompareProblem& p, hipStream_t s);
// Device address of the current device's fixed decode scratch
// (DIFFATTN_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned).
hipError_t decode_scratch(void** ptr);
hipError_t launch_lambda_proj(const void* x, const void* w, float* lam, int rows, int dm, int P, hipStream_t s);
// y [M, N] = a [M, K] @ w [K, N], row-major bf16, fp32 accumulation; K % 32 == 0, N % 8 == 0.
hipError_t launch_gemm_bf16(const void* a, const void* w, void* y, int M, int N, int K, hipStream_t s);
// fp32 path: rows of queries [B, Tq] over Tk keys; causal limit j <= i + (Tk - Tq).
hipError_t launch_rows_f32(const PrefillProblem& p, int Tq, int Tk, hipStream_t s);
hipError_t launch_v1_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                            float lambda_init, float* out, int P, int dl, int rows, hipStream_t s);

}  // namespace diffattn
