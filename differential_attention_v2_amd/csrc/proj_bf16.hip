// The projections on either side of the V2 attention core, gfx950.
//
// lambda producer: V2 projects a sigmoid-bounded lambda for every token and head
// (dailytechsnack.ch article "Differential Transformer V2 soll KI-Training
// stabiler machen", section "Weniger Ausreisser und Gradientenspitzen"):
//   lambda[r, p] = sigmoid(x[r] . w[p]),  x [rows, d_model] bf16, w [P, d_model] bf16.
// A workgroup of 16 waves owns 16 rows and every pair; each wave takes an equal
// slice of d_model and accumulates x w^T with v_mfma_f32_16x16x32_bf16 (A = 16
// rows of x, B = 16 projection vectors), issuing the loads of up to 8 k-steps
// before their products; the partial sums meet in LDS and the sigmoid is applied
// in fp32.  x is read from HBM exactly once; w (P x d_model, 256 KB for P = 32,
// d_model = 4096) stays in L2.
//
// Output projection: after the subtraction the P*d wide result is projected back
// to d_model by O_W (differential-attention lesson "差异性注意力 (V2)", section
// "V1 vs V2") -- a plain dense GEMM, run by rocBLAS (bf16 in and out, fp32
// accumulation).
#include <rocblas/rocblas.h>

#include "dev_common.h"
#include "internal.h"

namespace diffattn {
namespace {

constexpr int LP_ROWS = 16;
constexpr int LP_WAVES = 16;   // d_model split over 16 waves: 4 per SIMD, many loads in flight

// NCT = P / 16 column tiles of lambda.  All x and w loads of a group of
// LP_UNROLL k-steps (of 32 columns) issue before its products, so a workgroup
// keeps its 16 rows (d_model * 32 bytes) in flight from the start; the group is
// smaller for wide P so the operands fit 128 VGPRs.
template <int NCT, int LP_UNROLL = (NCT <= 2 ? 8 : 4)>
__global__ __launch_bounds__(64 * LP_WAVES) void lambda_proj_kernel(const bf16* x, const bf16* w, float* lam, int rows,
                                                                    int dm) {
  __shared__ f32x4 part[LP_WAVES][NCT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = blockIdx.x * LP_ROWS;
  const int kq = dm / LP_WAVES;            // this wave's slice of d_model (a multiple of 32)
  const int kbeg = wave * kq;
  const int row = min(r0 + (lane & 15), rows - 1);
  const bf16* xa = x + (size_t)row * dm + 8 * (lane >> 4);
  const bf16* wb = w + (size_t)(lane & 15) * dm + 8 * (lane >> 4);
  f32x4 acc[NCT];
#pragma unroll
  for (int t = 0; t < NCT; ++t) acc[t] = f32x4{};
  for (int k = kbeg; k < kbeg + kq; k += 32 * LP_UNROLL) {
    const int n = min(LP_UNROLL, (kbeg + kq - k) / 32);   // k-steps in this group
    bf16x8 av[LP_UNROLL], bv[LP_UNROLL][NCT];
#pragma unroll
    for (int u = 0; u < LP_UNROLL; ++u) {
      if (u < n) {
        av[u] = __builtin_bit_cast(bf16x8, ldg16(xa + k + 32 * u));
#pragma unroll
        for (int t = 0; t < NCT; ++t) bv[u][t] = __builtin_bit_cast(bf16x8, ldg16(wb + (size_t)16 * t * dm + k + 32 * u));
      }
    }
#pragma unroll
    for (int u = 0; u < LP_UNROLL; ++u)
      if (u < n)
#pragma unroll
        for (int t = 0; t < NCT; ++t) acc[t] = mfma16(av[u], bv[u][t], acc[t]);
  }
#pragma unroll
  for (int t = 0; t < NCT; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  // the 16 waves' partial sums meet in LDS; wave t (< NCT) finishes column tile t.
  // C layout: lane l, register i -> row 4 (l/16) + i, column l % 16
  if (wave >= NCT) return;
  const int t = wave;
  f32x4 z = part[0][t][lane];
#pragma unroll
  for (int wv = 1; wv < LP_WAVES; ++wv) z += part[wv][t][lane];
  const int P = NCT * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 4 * (lane >> 4) + i;
    if (r < rows) lam[(size_t)r * P + 16 * t + (lane & 15)] = 1.0f / (1.0f + __expf(-z[i]));
  }
}

// One rocBLAS handle per (thread, device), created on first use.
rocblas_handle blas_handle() {
  constexpr int kMaxDevices = 64;
  thread_local rocblas_handle handles[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (handles[dev] == nullptr && rocblas_create_handle(&handles[dev]) != rocblas_status_success) handles[dev] = nullptr;
  return handles[dev];
}

}  // namespace

hipError_t launch_lambda_proj(const void* x, const void* w, float* lam, int rows, int dm, int P, hipStream_t s) {
  const dim3 grid((rows + LP_ROWS - 1) / LP_ROWS), block(64 * LP_WAVES);
  const bf16* xb = static_cast<const bf16*>(x);
  const bf16* wb = static_cast<const bf16*>(w);
  switch (P / 16) {
    case 1: hipLaunchKernelGGL(lambda_proj_kernel<1>, grid, block, 0, s, xb, wb, lam, rows, dm); break;
    case 2: hipLaunchKernelGGL(lambda_proj_kernel<2>, grid, block, 0, s, xb, wb, lam, rows, dm); break;
    case 3: hipLaunchKernelGGL(lambda_proj_kernel<3>, grid, block, 0, s, xb, wb, lam, rows, dm); break;
    default: hipLaunchKernelGGL(lambda_proj_kernel<4>, grid, block, 0, s, xb, wb, lam, rows, dm); break;
  }
  return hipGetLastError();
}

// y [rows, out_dim] = attn [rows, in_dim] @ w_o [in_dim, out_dim], row-major bf16.
// In rocBLAS's column-major terms: y^T (out_dim x rows) = w_o^T (out_dim x in_dim)
// * attn^T (in_dim x rows), with each row-major matrix read as its transpose.
int run_output_proj(const void* attn, const void* w_o, void* y, int rows, int in_dim, int out_dim, hipStream_t s) {
  rocblas_handle h = blas_handle();
  if (h == nullptr) return 1;
  if (rocblas_set_stream(h, s) != rocblas_status_success) return 1;
  const float alpha = 1.0f, beta = 0.0f;
  const rocblas_status st =
      rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, out_dim, rows, in_dim, &alpha, w_o,
                      rocblas_datatype_bf16_r, out_dim, attn, rocblas_datatype_bf16_r, in_dim, &beta, y,
                      rocblas_datatype_bf16_r, out_dim, y, rocblas_datatype_bf16_r, out_dim,
                      rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? 0 : 1;
}

}  // namespace diffattn
