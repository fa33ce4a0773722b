// fp32 Differential Attention V2 (prefill and decode share it), plus the V1
// reference-mode lambda.
//
// The fp32 dtype serves small problems (parity-sized prefill, fp32 decode); its
// work is tiny, so the kernel is a direct row-per-wave form: one wave computes
// one (b, query row i, pair p), walking the visible keys with a running maximum
// and denominator for each of the pair's two heads (differential-attention
// lesson "差异性注意力 (V2)", section "差异性概念": out = A1 V - lambda A2 V with
// A_r = softmax(q_r K^T / sqrt(d)); V2 head layout per the dailytechsnack.ch
// article, section "Gemeinsamer KV-Cache statt Spezialkernel").  Scores are dot
// products reduced across the wave; exponentials use expf.
#include "dev_common.h"
#include "internal.h"

namespace diffattn {
namespace {

__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// q [B, Tq, Hq, D], k/v [B, Tk, Hkv, D], lam [B, Tq, P], out [B, Tq, P, D].
// Query row i sees keys j <= i + (Tk - Tq) when causal, else all Tk keys.
template <int D>
__global__ __launch_bounds__(64) void rows_f32_kernel(const float* q, const float* k, const float* v,
                                                      const float* lam, float* out, int B, int Tq, int Tk,
                                                      int Hq, int Hkv, int causal, int v1, float eps) {
  constexpr int E = D / 64;
  const int P = Hq / 2;
  const int G = Hq / (2 * Hkv);
  const int lane = threadIdx.x;
  const long long idx = blockIdx.x;
  const int p = (int)(idx % P);
  const int i = (int)((idx / P) % Tq);
  const int b = (int)(idx / ((long long)P * Tq));
  const int g = p / G;
  const float scale = 1.0f / sqrtf((float)D);

  float q1[E], q2[E], acc1[E], acc2[E];
  const float* qrow = q + (((size_t)b * Tq + i) * Hq + 2 * p) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q1[e] = qrow[lane + 64 * e];
    q2[e] = qrow[D + lane + 64 * e];
    acc1[e] = 0.f;
    acc2[e] = 0.f;
  }
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
  const int jmax = causal ? i + (Tk - Tq) : Tk - 1;
  for (int j = 0; j <= jmax; ++j) {
    const float* krow = k + (((size_t)b * Tk + j) * Hkv + g) * D;
    const float* vrow = v + (((size_t)b * Tk + j) * Hkv + g) * D;
    float d1 = 0.f, d2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float kv = krow[lane + 64 * e];
      d1 = fmaf(q1[e], kv, d1);
      d2 = fmaf(q2[e], kv, d2);
    }
    const float s1 = wave_sum(d1) * scale;
    const float s2 = wave_sum(d2) * scale;
    const float n1 = fmaxf(m1, s1), n2 = fmaxf(m2, s2);
    const float a1 = expf(m1 - n1), a2 = expf(m2 - n2);   // exp(-inf) = 0 on the first key
    const float e1 = expf(s1 - n1), e2 = expf(s2 - n2);
    l1 = l1 * a1 + e1;
    l2 = l2 * a2 + e2;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float vv = vrow[lane + 64 * e];
      acc1[e] = acc1[e] * a1 + e1 * vv;
      acc2[e] = acc2[e] * a2 + e2 * vv;
    }
    m1 = n1;
    m2 = n2;
  }
  const float lamv = lam[((size_t)b * Tq + i) * P + p];
  float x[E], ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] = acc1[e] / l1 - lamv * (acc2[e] / l2);
    ss += x[e] * x[e];
  }
  float r = 1.f;
  if (v1) r = 1.0f / sqrtf(wave_sum(ss) / (float)D + eps);
  float* orow = out + (((size_t)b * Tq + i) * P + p) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) orow[lane + 64 * e] = x[e] * r;
}

// lambda_out[r, p] = exp(lq1[p].lk1[p]) - exp(lq2[p].lk2[p]) + lambda_init
// (differential-attention lesson, section "差异性概念": V1 lambda re-parameterisation).
__global__ __launch_bounds__(256) void v1_lambda_kernel(const float* lq1, const float* lk1, const float* lq2,
                                                        const float* lk2, float lambda_init, float* out, int P,
                                                        int dl, long long total) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int p = (int)(t % P);
  float a = 0.f, c = 0.f;
  for (int j = 0; j < dl; ++j) {
    a = fmaf(lq1[(size_t)p * dl + j], lk1[(size_t)p * dl + j], a);
    c = fmaf(lq2[(size_t)p * dl + j], lk2[(size_t)p * dl + j], c);
  }
  out[t] = expf(a) - expf(c) + lambda_init;
}

}  // namespace

hipError_t launch_rows_f32(const PrefillProblem& pr, int Tq, int Tk, hipStream_t s) {
  const long long blocks = (long long)pr.B * Tq * (pr.Hq / 2);
  const float* q = static_cast<const float*>(pr.q);
  const float* k = static_cast<const float*>(pr.k);
  const float* v = static_cast<const float*>(pr.v);
  float* out = static_cast<float*>(pr.out);
  if (pr.d == 128)
    hipLaunchKernelGGL(rows_f32_kernel<128>, dim3((unsigned)blocks), dim3(64), 0, s, q, k, v, pr.lam, out, pr.B,
                       Tq, Tk, pr.Hq, pr.Hkv, pr.causal, pr.v1_rmsnorm, pr.eps);
  else
    hipLaunchKernelGGL(rows_f32_kernel<64>, dim3((unsigned)blocks), dim3(64), 0, s, q, k, v, pr.lam, out, pr.B,
                       Tq, Tk, pr.Hq, pr.Hkv, pr.causal, pr.v1_rmsnorm, pr.eps);
  return hipGetLastError();
}

hipError_t launch_v1_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                            float lambda_init, float* out, int P, int dl, int rows, hipStream_t s) {
  const long long total = (long long)rows * P;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(v1_lambda_kernel, dim3(blocks), dim3(256), 0, s, lq1, lk1, lq2, lk2, lambda_init, out, P, dl,
                     total);
  return hipGetLastError();
}

}  // namespace diffattn
