// Output projection O_W of the V2 attention block, gfx950: after the
// subtraction the P*d wide result is projected back to the model width
// (differential-attention lesson "差异性注意力 (V2)", section "V1 vs V2"):
//     y [M, N] = attn [M, K] @ w_o [K, N],   row-major bf16, fp32 accumulation,
// M = tokens, K = P*d, N = d_model.  A plain dense contraction, so it runs on
// v_mfma_f32_32x32x16_bf16 at the MFMA roof.
//
// Workgroup = 8 waves (two per SIMD) = one 256 x 256 tile of y.  The K axis is
// walked in 32-wide steps through a 4-deep LDS ring (32 KB per step: the A tile
// [256 rows][32 k] and the B tile [32 k][256 n]), filled by direct global -> LDS
// copies (global_load_lds_dwordx4; scalar 64-bit base per step plus a per-lane
// 32-bit offset that never changes) and published by one barrier per step; the
// copy for step j+3 goes into the buffer of step j-1.  Wave (wm, wn) of the 2 x 4
// wave grid owns rows 128 wm .. +128 and columns 64 wn .. +64 of the tile: 4 x 2
// MFMA tiles, 16 products per step.
//
// Operands: a row of the A tile is 64 bytes (4 chunks of 16), the A operand of a
// row is one 16-byte read (ds_read_b128); chunks are XOR-permuted by bits 2-3 of
// the row, so 16 consecutive rows at one logical chunk hit 16 distinct bank
// groups.  The B tile is row-major in k (512-byte rows of n, as w_o is stored);
// its operand (lanes = columns, 8 consecutive k) comes from two transposing
// reads (ds_read_b64_tr_b16) of 4 k-rows each; chunks are XOR-permuted by
// 4 * (k % 4), so the 4 rows of a transposing read land in distinct banks.
// The products are issued as C^T = B^T A^T (the w_o operand in the A slot): the
// accumulator layout then gives each lane 4 consecutive output columns of one
// row, stored as 8-byte writes.
//
// Blocks map to tiles XCD by XCD: the 8 XCDs each take a contiguous run of
// tiles in an order that walks 4 tile-rows at a time, so the workgroups on one
// XCD share A rows and w_o columns in that XCD's L2.
#include "dev_common.h"
#include "internal.h"

namespace diffattn {
namespace {

constexpr int GM = 256, GN = 256, GK = 32;
constexpr int G_WAVES = 8;
constexpr int G_THREADS = 64 * G_WAVES;
constexpr int G_NS = 4;                       // LDS ring depth
constexpr int A_TILE = GM * GK * 2;           // 16 KB
constexpr int B_TILE = GK * GN * 2;           // 16 KB
constexpr int G_STAGE = A_TILE + B_TILE;
constexpr int A_LOADS = GM * GK / 8 / G_THREADS;   // copy instructions per thread per step (2)
constexpr int B_LOADS = GK * GN / 8 / G_THREADS;   // (2)
constexpr int G_LOADS = A_LOADS + B_LOADS;
constexpr int GROUP_M = 4;                    // tile-rows walked together

struct GemmArgs {
  const bf16* a;   // [M, K]
  const bf16* w;   // [K, N]
  bf16* y;         // [M, N]
  int M, N, K;
  int tiles_m, tiles_n;
};

__global__ __launch_bounds__(G_THREADS, 1) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) char smem[G_NS * G_STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- block -> tile: a contiguous run of tiles per XCD (block % 8 selects the
  // XCD), tiles ordered GROUP_M tile-rows at a time
  const int ntiles = g.tiles_m * g.tiles_n;
  int t = blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  const int per_group = GROUP_M * g.tiles_n;
  const int first_m = (t / per_group) * GROUP_M;
  const int gsz = min(g.tiles_m - first_m, GROUP_M);
  const int tm = first_m + (t % per_group) % gsz;
  const int tn = (t % per_group) / gsz;
  const int m0 = tm * GM, n0 = tn * GN;
  const int M = g.M, N = g.N, K = g.K;

  // ---- copy offsets (per lane, fixed for the whole K walk).  Slot s of a tile
  // (16 bytes each, instruction j of wave w covers slots (j*8 + w)*64 + lane):
  //   A: row s/4, physical chunk s%4 holds logical chunk (s%4) ^ ((row/4)%4);
  //      rows past M repeat row M-1.
  //   B: k-row s/32, physical chunk s%32 holds logical chunk (s%32) ^ 4 (k%4);
  //      chunks past N repeat the last chunk of the row.
  uint32_t aofs[A_LOADS], bofs[B_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int s = (j * G_WAVES + wave) * 64 + lane;
    const int r = s >> 2, lc = (s & 3) ^ ((r >> 2) & 3);
    aofs[j] = (uint32_t)(min(r, M - 1 - m0) * K + 8 * lc) * 2;
  }
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int s = (j * G_WAVES + wave) * 64 + lane;
    const int r = s >> 5, lc = (s & 31) ^ (4 * (r & 3));
    bofs[j] = (uint32_t)(r * N + min(8 * lc, N - 8 - n0)) * 2;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)LDS_PTR(const char, smem);
  const char* abase = reinterpret_cast<const char*>(g.a + (size_t)m0 * K);
  const char* wbase = reinterpret_cast<const char*>(g.w + n0);
  const size_t wstep = (size_t)GK * N * 2;
  auto copy_step = [&](int step, int buf) {
    const char* as = abase + (size_t)step * GK * 2;
    const char* ws = wbase + (size_t)step * wstep;
    const uint32_t dst = lds_base + buf * G_STAGE + wave * 1024;
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) dma16_saddr(as, aofs[j], dst + j * G_WAVES * 1024);
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) dma16_saddr(ws, bofs[j], dst + A_TILE + j * G_WAVES * 1024);
  };

  // ---- operand read offsets within a stage
  const int wm = wave >> 2, wn = wave & 3;
  uint32_t ard[4][2];   // A operand of row tile mt, k-substep ks
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = 128 * wm + 32 * mt + l32;
      ard[mt][ks] = (uint32_t)(r * GK * 2 + 16 * ((2 * ks + hi) ^ ((r >> 2) & 3)));
    }
  // B operand (transposing reads): 16-lane group q = lane/16 reads k-rows
  // 8 (q/2) + 4 h .. +3 at columns 16 (q%2) + 4 (i%4) .. +3 of its 32-column tile
  const int i16 = lane & 15, q16 = lane >> 4;
  uint32_t brd[2][2][2];   // [column tile nt][k-substep ks][half h]
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kr = 16 * ks + 8 * (q16 >> 1) + 4 * h + (i16 >> 2);
        const int col = 64 * wn + 32 * nt + 16 * (q16 & 1) + 4 * (i16 & 3);
        brd[nt][ks][h] = (uint32_t)(A_TILE + kr * GN * 2 + 16 * ((col >> 3) ^ (4 * (kr & 3))) + 2 * (col & 7));
      }

  f32x16 acc[2][4];   // [nt][mt], C^T tiles
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = f32x16{};

  auto load_ops = [&](const char* sb, int ks, bf16x8 (&ao)[4], bf16x8 (&bo)[2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ao[mt] = *reinterpret_cast<const bf16x8*>(sb + ard[mt][ks]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      bo[nt] = concat(lds_read_tr4(reinterpret_cast<const bf16*>(sb + brd[nt][ks][0])),
                      lds_read_tr4(reinterpret_cast<const bf16*>(sb + brd[nt][ks][1])));
  };

  const int nsteps = K / GK;
#pragma unroll
  for (int j = 0; j < G_NS - 1; ++j)
    if (j < nsteps) copy_step(j, j);
  // step 0's copies must have landed; the ones for steps 1 and 2 may stay in flight
  if (nsteps >= 3)
    wait_vmcnt<2 * G_LOADS>();
  else if (nsteps == 2)
    wait_vmcnt<G_LOADS>();
  else
    wait_vmcnt<0>();
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & (G_NS - 1);
    if (step + G_NS - 1 < nsteps) copy_step(step + G_NS - 1, (step + G_NS - 1) & (G_NS - 1));
    const char* sb = smem + buf * G_STAGE;
    bf16x8 ao[2][4], bo[2][2];
    load_ops(sb, 0, ao[0], bo[0]);
    load_ops(sb, 1, ao[1], bo[1]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = mfma32(bo[ks][nt], ao[ks][mt], acc[nt][mt]);
    // the copy for step+1 must have landed before the barrier that publishes it;
    // later copies may stay in flight
    const int ahead = min(G_NS - 2, nsteps - 2 - step);
    if (ahead >= 2)
      wait_vmcnt<2 * G_LOADS>();
    else if (ahead == 1)
      wait_vmcnt<G_LOADS>();
    else
      wait_vmcnt<0>();
    __syncthreads();
  }

  // ---- epilogue.  C^T layout: lane l, register i -> output row
  // m0 + 128 wm + 32 mt + l%32, column n0 + 64 wn + 32 nt + 8 (i/4) + 4 (l/32) + i%4
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = m0 + 128 * wm + 32 * mt + l32;
    if (row >= M) continue;
    bf16* yr = g.y + (size_t)row * N;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = n0 + 64 * wn + 32 * nt + 8 * i4 + 4 * hi;
        if (col >= N) continue;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)acc[nt][mt][4 * i4 + e];
        *reinterpret_cast<bf16x4*>(yr + col) = o;
      }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const void* a, const void* w, void* y, int M, int N, int K, hipStream_t s) {
  GemmArgs g{static_cast<const bf16*>(a), static_cast<const bf16*>(w), static_cast<bf16*>(y), M, N, K,
             (M + GM - 1) / GM, (N + GN - 1) / GN};
  const long long blocks = (long long)g.tiles_m * g.tiles_n;
  if (blocks > (1LL << 31) - 1) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)blocks), dim3(G_THREADS), 0, s, g);
  return hipGetLastError();
}

}  // namespace diffattn
