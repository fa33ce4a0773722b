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
};

// Floats per partial-state record in the decode workspace: acc[d], m, l, 2 pad
// (keeps every record 16-byte aligned).
inline int decode_record_floats(int d) { return d + 4; }

hipError_t launch_prefill_bf16(const PrefillProblem& p, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeProblem& p, hipStream_t s);
// fp32 path: rows of queries [B, Tq] over Tk keys; causal limit j <= i + (Tk - Tq).
hipError_t launch_rows_f32(const PrefillProblem& p, int Tq, int Tk, hipStream_t s);
hipError_t launch_v1_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                            float lambda_init, float* out, int P, int dl, int rows, hipStream_t s);

}  // namespace diffattn
