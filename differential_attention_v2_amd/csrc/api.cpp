// C-ABI entry points of libdiffattn: argument validation, split planning and
// dispatch to the gfx950 kernels.  Every check runs on the host before anything
// is enqueued, so an invalid call writes nothing and touches no device.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <cmath>

#include "diffattn.h"
#include "internal.h"

using namespace diffattn;

namespace {

constexpr int kVersion = 100;                    // 0.1.0
constexpr long long kMaxElems = 1LL << 40;       // per tensor
constexpr long long kMaxGrid = (1LL << 31) - 1;  // workgroups per launch
// Decode split target: two waves per CU of MI355X (256 CUs).  Each wave keeps its
// next step's cache rows in flight through two LDS stages, and fewer, longer cache
// streams read faster than more, shorter ones: on the device B=64 L=8192 reads
// 6.6 TB/s with 512 waves, 6.5 with 1024 (5.5 with 4096 before the LDS staging);
// ragged caches of the same shape take 183 us with 512 waves and 188 with 1024.
constexpr int kDecodeTargetWaves = 512;

bool aligned(const void* p, uintptr_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The kernels address the rows of a tile (up to 64 tokens) with 32-bit per-lane
// byte offsets from a 64-bit tile base, so 64 token strides of the widest row
// (q: Hq*d bf16 or fp32 values) must stay below 2^31 bytes.
constexpr long long kMaxHeadElems = 1LL << 22;   // Hq*d per token
constexpr int kMaxBackwardT = 1 << 26;
constexpr int kMaxModelDim = 1 << 24;            // lambda producer: 16 rows of x per 32-bit offset range

int check_heads(int Hq, int Hkv, int d) {
  if (Hkv < 1 || Hq < 2 || Hq % (2 * Hkv) != 0) return DIFFATTN_ERR_INVALID_ARG;
  if (d <= 0) return DIFFATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return DIFFATTN_ERR_UNSUPPORTED;
  if (Hq / (2 * Hkv) > 8) return DIFFATTN_ERR_UNSUPPORTED;
  if ((long long)Hq * d > kMaxHeadElems) return DIFFATTN_ERR_UNSUPPORTED;
  return DIFFATTN_OK;
}

int check_mode(int dtype, unsigned flags, float eps) {
  if (dtype != DIFFATTN_BF16 && dtype != DIFFATTN_FP32) return DIFFATTN_ERR_INVALID_ARG;
  if (flags & ~DIFFATTN_FLAG_V1_RMSNORM) return DIFFATTN_ERR_INVALID_ARG;
  if ((flags & DIFFATTN_FLAG_V1_RMSNORM) && !(std::isfinite(eps) && eps > 0.f)) return DIFFATTN_ERR_INVALID_ARG;
  return DIFFATTN_OK;
}

bool fits(long long a, long long b, long long c, long long d) {
  // a*b*c*d <= kMaxElems without overflowing (all >= 1)
  long long x = a;
  for (long long y : {b, c, d}) {
    if (x > kMaxElems / y) return false;
    x *= y;
  }
  return true;
}

// Key-range split of a decode problem: S ranges of `chunk` keys (a multiple of 32).
bool decode_plan(int B, int L, int Hkv, int num_splits, int* S, int* chunk) {
  if (B < 1 || L < 1 || Hkv < 1 || num_splits < 0) return false;
  const long long units = (long long)B * Hkv;
  const long long nblk = (L + 31) / 32;
  long long want = num_splits > 0 ? num_splits : (kDecodeTargetWaves + units - 1) / units;
  if (want > nblk) want = nblk;
  if (want < 1) want = 1;
  const long long per = (nblk + want - 1) / want;
  *chunk = (int)(per * 32);
  *S = (int)((L + *chunk - 1) / *chunk);
  return units * *S <= kMaxGrid;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP; }

}  // namespace

extern "C" {

int diffattn_prefill_fwd(const void* q, const void* k, const void* v, const float* lambda, void* out, int B, int T,
                         int Hq, int Hkv, int d, int causal, int dtype, unsigned flags, float rms_eps, void* stream) {
  if (B < 1 || T < 1) return DIFFATTN_ERR_INVALID_ARG;
  int st = check_heads(Hq, Hkv, d);
  if (st) return st;
  st = check_mode(dtype, flags, rms_eps);
  if (st) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lambda, 4))
    return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(B, T, Hq, d) || (long long)B * T * (Hq / 2) > kMaxGrid) return DIFFATTN_ERR_INVALID_ARG;

  PrefillProblem p{q, k, v, lambda, out, B, T, Hq, Hkv, d, causal ? 1 : 0,
                   (flags & DIFFATTN_FLAG_V1_RMSNORM) ? 1 : 0, rms_eps};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == DIFFATTN_FP32) return hip_status(launch_rows_f32(p, T, T, s));
  return hip_status(launch_prefill_bf16(p, s));
}

int diffattn_prefill_fwd_window(const void* q, const void* k, const void* v, const float* lambda, void* out,
                                int B, int T, int Hq, int Hkv, int d, int window, int dtype, unsigned flags,
                                float rms_eps, void* stream) {
  if (B < 1 || T < 1 || window < 0) return DIFFATTN_ERR_INVALID_ARG;
  int st = check_heads(Hq, Hkv, d);
  if (st) return st;
  st = check_mode(dtype, flags, rms_eps);
  if (st) return st;
  if (dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lambda, 4))
    return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(B, T, Hq, d) || (long long)B * T * (Hq / 2) > kMaxGrid) return DIFFATTN_ERR_INVALID_ARG;
  PrefillProblem p{q, k, v, lambda, out, B, T, Hq, Hkv, d, 1, (flags & DIFFATTN_FLAG_V1_RMSNORM) ? 1 : 0, rms_eps};
  p.window = window >= T ? 0 : window;   // a window covering the sequence is plain causal
  return hip_status(launch_prefill_bf16(p, static_cast<hipStream_t>(stream)));
}

int diffattn_prefill_fwd_train(const void* q, const void* k, const void* v, const float* lambda, void* out,
                               void* o2, float* lse, int B, int T, int Hq, int Hkv, int d, int causal,
                               void* stream) {
  if (B < 1 || T < 1) return DIFFATTN_ERR_INVALID_ARG;
  int st = check_heads(Hq, Hkv, d);
  if (st) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(o2, 16) ||
      !aligned(lambda, 4) || !aligned(lse, 4))
    return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(B, T, Hq, d) || (long long)B * T * (Hq / 2) > kMaxGrid) return DIFFATTN_ERR_INVALID_ARG;
  PrefillProblem p{q, k, v, lambda, out, B, T, Hq, Hkv, d, causal ? 1 : 0, 0, 0.f};
  p.o2 = o2;
  p.lse = lse;
  return hip_status(launch_prefill_bf16(p, static_cast<hipStream_t>(stream)));
}

size_t diffattn_prefill_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d) {
  if (B < 1 || T < 1 || check_heads(Hq, Hkv, d) != DIFFATTN_OK || !fits(B, T, Hq, d)) return 0;
  return backward_workspace_floats(B, T, Hq, Hkv, d) * sizeof(float);
}

int diffattn_prefill_bwd(const void* q, const void* k, const void* v, const float* lambda, const void* out,
                         const void* o2, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         float* dlambda, int B, int T, int Hq, int Hkv, int d, int causal, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (B < 1 || T < 1) return DIFFATTN_ERR_INVALID_ARG;
  int st = check_heads(Hq, Hkv, d);
  if (st) return st;
  for (const void* p16 : {q, k, v, out, o2, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                          static_cast<const void*>(dv)})
    if (!aligned(p16, 16)) return DIFFATTN_ERR_INVALID_ARG;
  if (!aligned(lambda, 4) || !aligned(lse, 4) || !aligned(dlambda, 4)) return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(B, T, Hq, d) || (long long)B * T * (Hq / 2) > kMaxGrid) return DIFFATTN_ERR_INVALID_ARG;
  // the dK/dV kernel reads the row statistics (5 fields of Tpad floats per pair)
  // through 32-bit per-lane offsets
  if (T > kMaxBackwardT) return DIFFATTN_ERR_UNSUPPORTED;
  const size_t need = backward_workspace_floats(B, T, Hq, Hkv, d) * sizeof(float);
  if (!aligned(workspace, 16) || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
  BackwardProblem p{q, k, v, lambda, out, o2, lse, dout, dq, dk, dv, dlambda, static_cast<float*>(workspace),
                    B, T, Hq, Hkv, d, causal ? 1 : 0};
  return hip_status(launch_backward_bf16(p, static_cast<hipStream_t>(stream)));
}

int diffattn_decode_num_splits(int B, int L, int Hq, int Hkv, int d) {
  if (check_heads(Hq, Hkv, d) != DIFFATTN_OK) return 0;
  int S, chunk;
  return decode_plan(B, L, Hkv, 0, &S, &chunk) ? S : 0;
}

size_t diffattn_decode_workspace_bytes(int B, int L, int Hq, int Hkv, int d, int num_splits) {
  if (check_heads(Hq, Hkv, d) != DIFFATTN_OK) return 0;
  int S, chunk;
  if (!decode_plan(B, L, Hkv, num_splits, &S, &chunk)) return 0;
  return (size_t)B * Hq * S * decode_record_floats(d) * sizeof(float);
}

int diffattn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, const float* lambda, void* out,
                        int B, int L, int Hq, int Hkv, int d, int dtype, unsigned flags, float rms_eps,
                        int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || L < 1 || num_splits < 0) return DIFFATTN_ERR_INVALID_ARG;
  int st = check_heads(Hq, Hkv, d);
  if (st) return st;
  st = check_mode(dtype, flags, rms_eps);
  if (st) return st;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(lambda, 4))
    return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(B, L, Hkv, d) || !fits(B, Hq, d, 1)) return DIFFATTN_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int v1 = (flags & DIFFATTN_FLAG_V1_RMSNORM) ? 1 : 0;

  if (dtype == DIFFATTN_FP32) {
    // one query row at position L-1: causal with Tq = 1 sees every cache row
    PrefillProblem p{q, k_cache, v_cache, lambda, out, B, L, Hq, Hkv, d, 1, v1, rms_eps};
    return hip_status(launch_rows_f32(p, 1, L, s));
  }
  int S, chunk;
  if (!decode_plan(B, L, Hkv, num_splits, &S, &chunk)) return DIFFATTN_ERR_INVALID_ARG;
  const size_t need = (size_t)B * Hq * S * decode_record_floats(d) * sizeof(float);
  if (!aligned(workspace, 16) || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
  DecodeProblem p{q, k_cache, v_cache, lambda, out, static_cast<float*>(workspace), B, L, Hq, Hkv, d, S, chunk,
                  v1, rms_eps};
  return hip_status(launch_decode_bf16(p, s));
}

int diffattn_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache, const float* lambda,
                                void* out, int B, int L, int Hq, int Hkv, int d, int dtype, unsigned flags,
                                float rms_eps, int num_splits, void* stream) {
  // the records' size is known only for a valid problem: validate like the
  // workspace entry point first, with a workspace that is never touched
  if (B < 1 || L < 1 || num_splits < 0) return DIFFATTN_ERR_INVALID_ARG;
  int st = check_heads(Hq, Hkv, d);
  if (st) return st;
  st = check_mode(dtype, flags, rms_eps);
  if (st) return st;
  int S, chunk;
  if (!decode_plan(B, L, Hkv, num_splits, &S, &chunk)) return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(B, Hq, S, decode_record_floats(d)) ||
      (size_t)B * Hq * S * decode_record_floats(d) * sizeof(float) > DIFFATTN_NOALLOC_SCRATCH_BYTES)
    return DIFFATTN_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(lambda, 4))
    return DIFFATTN_ERR_INVALID_ARG;
  void* scratch = nullptr;
  if (decode_scratch(&scratch) != hipSuccess) return DIFFATTN_ERR_HIP;
  return diffattn_decode_fwd(q, k_cache, v_cache, lambda, out, B, L, Hq, Hkv, d, dtype, flags, rms_eps, num_splits,
                             scratch, DIFFATTN_NOALLOC_SCRATCH_BYTES, stream);
}

namespace {
// ranges per KV head of the even split over ragged caches: the same wave target
int varlen_ranges(int Hkv, int num_splits) {
  return num_splits > 0 ? num_splits : (kDecodeTargetWaves + Hkv - 1) / Hkv;
}
}  // namespace

size_t diffattn_decode_varlen_workspace_bytes(int B, int L, int Hq, int Hkv, int d, int num_splits) {
  if (check_heads(Hq, Hkv, d) != DIFFATTN_OK || num_splits < 0) return 0;
  int S, chunk;
  if (!decode_plan(B, L, Hkv, num_splits, &S, &chunk)) return 0;
  const size_t split = (size_t)B * Hq * S * decode_record_floats(d) * sizeof(float);
  const long long ranges = varlen_ranges(Hkv, num_splits);
  if (ranges * Hkv > kMaxGrid) return 0;
  const size_t flat = decode_flat_workspace_bytes(B, Hq, d, (int)ranges);
  return split > flat ? split : flat;
}

int diffattn_decode_fwd_varlen(const void* q, const void* k_cache, const void* v_cache, const float* lambda,
                               void* out, const int* seq_lens, int B, int L, int Hq, int Hkv, int d, int window,
                               int dtype, unsigned flags, float rms_eps, int num_splits, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (B < 1 || L < 1 || num_splits < 0 || window < 0) return DIFFATTN_ERR_INVALID_ARG;
  int st = check_heads(Hq, Hkv, d);
  if (st) return st;
  st = check_mode(dtype, flags, rms_eps);
  if (st) return st;
  if (dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(lambda, 4) || (seq_lens != nullptr && !aligned(seq_lens, 4)))
    return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(B, L, Hkv, d) || !fits(B, Hq, d, 1)) return DIFFATTN_ERR_INVALID_ARG;
  int S, chunk;
  if (!decode_plan(B, L, Hkv, num_splits, &S, &chunk)) return DIFFATTN_ERR_INVALID_ARG;
  const long long ranges = varlen_ranges(Hkv, num_splits);
  if (ranges * Hkv > kMaxGrid) return DIFFATTN_ERR_INVALID_ARG;
  const size_t need = seq_lens != nullptr ? decode_flat_workspace_bytes(B, Hq, d, (int)ranges)
                                          : (size_t)B * Hq * S * decode_record_floats(d) * sizeof(float);
  if (!aligned(workspace, 16) || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
  DecodeProblem p{q, k_cache, v_cache, lambda, out, static_cast<float*>(workspace), B, L, Hq, Hkv, d, S, chunk,
                  (flags & DIFFATTN_FLAG_V1_RMSNORM) ? 1 : 0, rms_eps};
  p.seq_lens = seq_lens;
  p.window = window;
  p.flat_ranges = seq_lens != nullptr ? (int)ranges : 0;
  return hip_status(launch_decode_bf16(p, static_cast<hipStream_t>(stream)));
}

size_t diffattn_decode_compare_workspace_bytes(int B, int L, int H, int Hkv, int d, int num_splits) {
  if (B < 1 || L < 1 || Hkv < 1 || H < 1 || H % Hkv != 0 || H / Hkv > 16 || (d != 64 && d != 128) ||
      (long long)H * d > kMaxHeadElems)
    return 0;
  int S, chunk;
  if (!decode_plan(B, L, Hkv, num_splits, &S, &chunk)) return 0;
  return 2 * (size_t)B * H * S * decode_record_floats(d) * sizeof(float);
}

namespace {
int decode_compare(const void* q, const void* k_cache, const void* v_cache, const float* lambda, void* out, int B,
                   int L, int H, int Hkv, int d, int v1_layout, unsigned flags, float rms_eps, int num_splits,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || L < 1 || num_splits < 0 || H < 1 || Hkv < 1 || H % Hkv != 0) return DIFFATTN_ERR_INVALID_ARG;
  if (d <= 0) return DIFFATTN_ERR_INVALID_ARG;
  if ((d != 64 && d != 128) || H / Hkv > 16 || (long long)H * d > kMaxHeadElems) return DIFFATTN_ERR_UNSUPPORTED;
  int st = check_mode(DIFFATTN_BF16, flags, rms_eps);
  if (st) return st;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      (v1_layout && !aligned(lambda, 4)))
    return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(B, L, Hkv, d) || !fits(B, H, d, 1)) return DIFFATTN_ERR_INVALID_ARG;
  int S, chunk;
  if (!decode_plan(B, L, Hkv, num_splits, &S, &chunk)) return DIFFATTN_ERR_INVALID_ARG;
  const size_t need = (v1_layout ? 2 : 1) * (size_t)B * H * S * decode_record_floats(d) * sizeof(float);
  if (!aligned(workspace, 16) || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
  CompareProblem p{q, k_cache, v_cache, lambda, out, static_cast<float*>(workspace), B, L, H, Hkv, d, S, chunk,
                   v1_layout, (flags & DIFFATTN_FLAG_V1_RMSNORM) ? 1 : 0, rms_eps};
  return hip_status(launch_decode_compare_bf16(p, static_cast<hipStream_t>(stream)));
}
}  // namespace

int diffattn_decode_standard(const void* q, const void* k_cache, const void* v_cache, void* out, int B, int L, int H,
                             int Hkv, int d, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_compare(q, k_cache, v_cache, nullptr, out, B, L, H, Hkv, d, 0, 0u, 1e-5f, num_splits, workspace,
                        workspace_bytes, stream);
}

int diffattn_decode_v1_layout(const void* q, const void* k_cache, const void* v_cache, const float* lambda,
                              void* out, int B, int L, int H, int Hkv, int d, unsigned flags, float rms_eps,
                              int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_compare(q, k_cache, v_cache, lambda, out, B, L, H, Hkv, d, 1, flags, rms_eps, num_splits, workspace,
                        workspace_bytes, stream);
}

int diffattn_lambda_proj(const void* x, const void* w_lambda, float* lambda_out, int rows, int d_model, int P,
                         void* stream) {
  if (rows < 1 || d_model < 1 || P < 1) return DIFFATTN_ERR_INVALID_ARG;
  if (d_model % 512 != 0 || d_model > kMaxModelDim || P % 16 != 0 || P > 64) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w_lambda, 16) || !aligned(lambda_out, 4)) return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(rows, d_model, 1, 1) || !fits(rows, P, 1, 1)) return DIFFATTN_ERR_INVALID_ARG;
  return hip_status(launch_lambda_proj(x, w_lambda, lambda_out, rows, d_model, P, static_cast<hipStream_t>(stream)));
}

int diffattn_output_proj(const void* attn, const void* w_o, void* y, int rows, int in_dim, int out_dim,
                         void* stream) {
  if (rows < 1 || in_dim < 1 || out_dim < 1) return DIFFATTN_ERR_INVALID_ARG;
  // 32-wide k steps and 16-byte column chunks; 256 rows (32 k-rows) of the
  // operands are addressed with 32-bit per-lane offsets
  if (in_dim % 32 != 0 || out_dim % 8 != 0 || in_dim > kMaxModelDim || out_dim > kMaxModelDim)
    return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(attn, 16) || !aligned(w_o, 16) || !aligned(y, 16)) return DIFFATTN_ERR_INVALID_ARG;
  if (!fits(rows, in_dim, 1, 1) || !fits(in_dim, out_dim, 1, 1) || !fits(rows, out_dim, 1, 1))
    return DIFFATTN_ERR_INVALID_ARG;
  return hip_status(launch_gemm_bf16(attn, w_o, y, rows, out_dim, in_dim, static_cast<hipStream_t>(stream)));
}

int diffattn_v1_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2, float lambda_init,
                       float* lambda_out, int P, int d_lambda, int rows, void* stream) {
  if (P < 1 || d_lambda < 1 || rows < 1 || !std::isfinite(lambda_init)) return DIFFATTN_ERR_INVALID_ARG;
  if (!aligned(lq1, 4) || !aligned(lk1, 4) || !aligned(lq2, 4) || !aligned(lk2, 4) || !aligned(lambda_out, 4))
    return DIFFATTN_ERR_INVALID_ARG;
  if ((long long)rows * P > kMaxGrid * 256LL || !fits(P, d_lambda, 1, 1)) return DIFFATTN_ERR_INVALID_ARG;
  return hip_status(launch_v1_lambda(lq1, lk1, lq2, lk2, lambda_init, lambda_out, P, d_lambda, rows,
                                     static_cast<hipStream_t>(stream)));
}

const char* diffattn_status_string(int status) {
  switch (status) {
    case DIFFATTN_OK: return "ok";
    case DIFFATTN_ERR_INVALID_ARG: return "invalid argument";
    case DIFFATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case DIFFATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case DIFFATTN_ERR_HIP: return "HIP runtime or kernel launch failure";
    default: return "unknown status";
  }
}

int diffattn_version(void) { return kVersion; }

}  // extern "C"
