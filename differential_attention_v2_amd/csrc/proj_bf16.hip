// The lambda producer in front of the V2 attention core, gfx950.
//
// lambda producer: V2 projects a sigmoid-bounded lambda for every token and head
// (dailytechsnack.ch article "Differential Transformer V2 soll KI-Training
// stabiler machen", section "Weniger Ausreisser und Gradientenspitzen"):
//   lambda[r, p] = sigmoid(x[r] . w[p]),  x [rows, d_model] bf16, w [P, d_model] bf16.
// A workgroup of 16 waves owns 16 rows and every pair; each wave takes an equal
// slice of d_model, stages its 16 rows of that slice in LDS (whole row pieces per
// copy instruction) and accumulates x w^T with v_mfma_f32_16x16x32_bf16 (A = 16
// rows of x from LDS, B = 16 projection vectors from L2); the partial sums meet in
// LDS and the sigmoid is applied in fp32.  x is read from HBM exactly once; w
// (P x d_model, 256 KB for P = 32, d_model = 4096) stays in L2.
//
// The output projection O_W on the other side is the GEMM in gemm_bf16.hip.
#include "dev_common.h"
#include "internal.h"

namespace diffattn {
namespace {

constexpr int LP_ROWS = 16;
constexpr int LP_WAVES = 16;   // d_model split over 16 waves: 4 per SIMD, many loads in flight
constexpr int LP_CHUNK = 256;  // columns of a wave's slice staged at a time (16 rows x 512 bytes)

// Direct global -> LDS copy of 16 bytes per lane (lane l's bytes land at
// lds_addr + 16 l), scalar base plus per-lane byte offset, with the nontemporal
// hint (x is read exactly once); the caller waits on vmcnt.
__device__ __forceinline__ void dma16_lp(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  // one wait state between the M0 write and the copy that reads it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// NCT = P / 16 column tiles of lambda.  Each wave stages its 16 rows x 256
// columns of x in LDS with whole 512-byte row pieces per copy instruction (two
// rows per instruction; loaded straight into registers as MFMA operands, each
// instruction would touch 16 rows x 64 bytes, and the kernel measured 5 % slower),
// then accumulates x w^T over the staged columns with w read from L2, all w
// operands of a group of k-steps requested before their products.  The 16 waves'
// partial sums meet in LDS.
template <int NCT, int LP_UNROLL = (NCT <= 2 ? 8 : 4)>
__global__ __launch_bounds__(64 * LP_WAVES) void lambda_proj_kernel(const bf16* x, const bf16* w, float* lam, int rows,
                                                                    int dm) {
  // per wave: 16 rows x LP_CHUNK columns of x (row-major, 16-byte chunks XOR-
  // permuted by row so the operand reads hit distinct banks); after the products
  // the same memory holds the partial sums
  constexpr int STAGE = LP_ROWS * LP_CHUNK * 2;   // 8 KB per wave
  static_assert(LP_WAVES * NCT * 64 * 16 <= LP_WAVES * STAGE, "partial sums must fit the staging area");
  __shared__ __attribute__((aligned(16))) char smem[LP_WAVES * STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = blockIdx.x * LP_ROWS;
  const int kq = dm / LP_WAVES;            // this wave's slice of d_model (a multiple of 32)
  const int kbeg = wave * kq;
  char* stage = smem + wave * STAGE;
  const uint32_t stage_lds = (uint32_t)(uintptr_t)LDS_PTR(char, stage);
  // copy instruction u, lane l: row 2u + l/32, physical chunk l%32 of the row,
  // holding logical chunk (l%32) ^ (row%16); rows past the end repeat the last row
  const bf16* wb = w + (size_t)(lane & 15) * dm + 8 * (lane >> 4);
  f32x4 acc[NCT];
#pragma unroll
  for (int t = 0; t < NCT; ++t) acc[t] = f32x4{};
  for (int c0 = 0; c0 < kq; c0 += LP_CHUNK) {
    const int ncol = min(LP_CHUNK, kq - c0);   // columns in this chunk (a multiple of 32)
    const char* xs = reinterpret_cast<const char*>(x + (size_t)r0 * dm + kbeg + c0);
#pragma unroll
    for (int u = 0; u < LP_ROWS / 2; ++u) {
      const int row = 2 * u + (lane >> 5);
      const int lc = (lane & 31) ^ (row & 15);          // logical chunk this lane copies
      const int col = min(8 * lc, ncol - 8);           // chunks past the chunk end re-read its last one
      const uint32_t off = (uint32_t)((min(r0 + row, rows - 1) - r0) * dm + col) * 2;
      dma16_lp(xs, off, stage_lds + 1024 * u);
    }
    // k-steps of 32 columns in groups whose w operands are all requested before
    // their products (the first group's together with the x copies): A = rows
    // (lane % 16), logical chunk 4 ks + lane / 16
    for (int g0 = 0; g0 < ncol / 32; g0 += LP_UNROLL) {
      const int n = min(LP_UNROLL, ncol / 32 - g0);   // k-steps in this group
      bf16x8 bv[LP_UNROLL][NCT];
#pragma unroll
      for (int u = 0; u < LP_UNROLL; ++u)
        if (u < n)
#pragma unroll
          for (int t = 0; t < NCT; ++t)
            bv[u][t] = __builtin_bit_cast(bf16x8, ldg16(wb + (size_t)16 * t * dm + kbeg + c0 + 32 * (g0 + u)));
      if (g0 == 0) wait_vmcnt0();   // the staged x (and these w operands) have landed
#pragma unroll
      for (int u = 0; u < LP_UNROLL; ++u) {
        if (u < n) {
          const int lch = 4 * (g0 + u) + (lane >> 4), row = lane & 15;
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(stage + row * (LP_CHUNK * 2) + 16 * (lch ^ row));
#pragma unroll
          for (int t = 0; t < NCT; ++t) acc[t] = mfma16(av, bv[u][t], acc[t]);
        }
      }
    }
    if (c0 + LP_CHUNK < kq) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // staging reads done before the next copy
  }
  __syncthreads();   // every wave is done with its staged x: the memory now holds partial sums
  f32x4* part = reinterpret_cast<f32x4*>(smem);   // [LP_WAVES][NCT][64]
#pragma unroll
  for (int t = 0; t < NCT; ++t) part[(wave * NCT + t) * 64 + lane] = acc[t];
  __syncthreads();
  // wave t (< NCT) finishes column tile t.  C layout: lane l, register i -> row
  // 4 (l/16) + i, column l % 16
  if (wave >= NCT) return;
  const int t = wave;
  f32x4 z = part[t * 64 + lane];
#pragma unroll
  for (int wv = 1; wv < LP_WAVES; ++wv) z += part[(wv * NCT + t) * 64 + lane];
  const int P = NCT * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 4 * (lane >> 4) + i;
    if (r < rows) lam[(size_t)r * P + 16 * t + (lane & 15)] = 1.0f / (1.0f + __expf(-z[i]));
  }
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

}  // namespace diffattn
