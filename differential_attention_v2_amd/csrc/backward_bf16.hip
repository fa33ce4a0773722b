// Backward pass of Differential Attention V2 prefill, bf16 in / fp32 accumulate, gfx950.
//
// The forward map (differential-attention lesson "差异性注意力 (V2)", section
// "差异性概念"; dailytechsnack.ch article, section "Gemeinsamer KV-Cache statt
// Spezialkernel") is out = O_1 - lambda O_2 with O_r = softmax(S_r) V,
// S_r = Q_r K^T / sqrt(d), both heads of pair p on KV head g = p / G.  Its
// derivative, per row i of pair p (dout given):
//   dO_1 = dout,  dO_2 = -lambda dout,  dlambda = -dout . O_2
//   D_1 = dout . O_1 = dout . out + lambda dout . O_2,   D_2 = dO_2 . O_2
//   dP   = dout V^T                         (one product serves both heads)
//   dS_1 = P_1 (dP - D_1),   dS_2 = P_2 (-lambda dP - D_2)
//   dV  += (P_1 - lambda P_2)^T dout        (one product per pair)
//   dK  += (dS_1^T Q_1 + dS_2^T Q_2) / sqrt(d),   dQ_r = dS_r K / sqrt(d)
// with P_r = exp(S_r - lse_r) rebuilt from the forward's log-sum-exp, so no
// T x T matrix is ever stored.
//
// Kernels, in launch order:
//   bwd_pre:   per (b, token, pair): D_1, D_2, dlambda and the log2-domain LSEs,
//              written as per-pair rows of 5 fields padded to Tpad tokens.
//   fill:      zero the fp32 dK/dV accumulators.
//   bwd_dkdv:  key-block outer.  A workgroup of 4 waves owns 128 keys of one
//              (b, g) (32 keys per wave, K and V held in registers as MFMA
//              operands) and one fixed 512-token chunk of queries; for every
//              32-token query tile and every pair of the group, Q_1, Q_2 and
//              dout tiles (and the row statistics) are staged in LDS by direct
//              global-to-LDS loads and read by all 4 waves.  Scores are computed
//              as S = Q K^T (lanes own keys), so P and dS feed the dV and dK
//              products straight from registers; the row-major Q and dout tiles
//              are transposed by the LDS transpose read.  Hidden scores are set
//              to -inf once per step, MFMA operands are read one product group
//              ahead.  Results are added to fp32 accumulators (the query chunks
//              of one key block run in different workgroups).
//   bwd_dq:    query-block outer, the forward's structure: 8 waves, each one
//              pair x 16 tokens (one 16-column MFMA tile per head), K/V tiles
//              streamed through a 4-deep LDS ring shared by the whole group.
//              Per 32-key half tile, in 16x16x32 tiles: S^T = K Q^T per head,
//              dP^T = V dout^T once for both heads (they share dout), dS^T in
//              registers, dQ^T += K^T dS^T with K^T from the transposing read.
//   convert:   fp32 dK/dV accumulators -> bf16.
// bwd_pre and the dQ kernel run on a side stream of the caller's stream, beside
// the zero fill, the dK/dV kernel and the conversions (see launch below).
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "dev_common.h"
#include "internal.h"

namespace diffattn {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int NF = kBackwardFields;   // row-statistics fields: lse2_1, lse2_2, D_1, D_2, lambda

// ---------------------------------------------------------------------------
// LDS tile layout shared by every tile here: unpadded row-major [row][d], the
// 16-byte chunks of a row XOR-permuted by a function of the row so that the MFMA
// operand reads hit distinct banks (rows 16 apart share the permutation).  The
// dK/dV kernel's Q / dout tiles use t_swz(row), which swaps the two low bit fields
// of the row index: ((row % 4) << 2) | (row / 4 % 4) for 16 chunks per row
// (((row % 4) << 1) | (row / 4 % 2) for 8); its reads (32 consecutive rows at one
// chunk, and transposing reads of 4 rows x 2 chunks per 16 lanes) are free of bank
// conflicts.  The dQ kernel's K / V tiles are read by 16x16x32 operand patterns
// (lanes 16g + i read row i at chunk 4s + g; transposing reads of rows 4g .. 4g + 3
// at one chunk pair per 16-lane group), which conflict under t_swz; they use
// q_swz(row) = ((row % 4) << 2) ^ (row / 4 % 2) << 1 ^ 11 (row / 8 % 2) for 16 chunks,
// chosen by measurement (rocprofv3 SQ_LDS_BANK_CONFLICT on the patterns alone).
template <int D>
__device__ __forceinline__ int t_swz(int row) {
  return D >= 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : (((row & 3) << 1) | ((row >> 2) & 1));
}
template <int D>
__device__ __forceinline__ int q_swz(int row) {
  return D >= 128 ? (((row & 3) << 2) ^ ((row & 4) >> 1) ^ ((row & 8) ? 11 : 0)) : t_swz<D>(row);
}
template <int D>
__device__ __forceinline__ int q_phys(int row, int col) {
  return row * D + ((((col >> 3) ^ q_swz<D>(row))) << 3) + (col & 7);
}
template <int D>
__device__ __forceinline__ int t_phys(int row, int col) {
  return row * D + ((((col >> 3) ^ t_swz<D>(row))) << 3) + (col & 7);
}

// ---------------------------------------------------------------------------
struct PreArgs {
  const bf16* out;
  const bf16* o2;
  const bf16* dout;
  const float* lam;
  const float* lse;
  float* rs;      // [B][P][NF][Tpad]
  float* dlam;    // [B][T][P]
  int B, T, P, Tpad;
};

// One group of D/8 lanes per row (b, t, p), rows ordered with p fastest so that
// a wave reads contiguous memory; padded rows t in [T, Tpad) get zeros.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(PreArgs a) {
  constexpr int LPR = D / 8;   // lanes per row
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = gtid / LPR;
  const int part = (int)(gtid % LPR);
  const long long nrows = (long long)a.B * a.Tpad * a.P;
  const bool in = row < nrows;
  const int p = in ? (int)(row % a.P) : 0;
  const long long bt = in ? row / a.P : 0;
  const int t = (int)(bt % a.Tpad);
  const int b = (int)(bt / a.Tpad);
  const bool valid = in && t < a.T;
  float s_out = 0.f, s_o2 = 0.f;
  if (valid) {
    const size_t base = (((size_t)b * a.T + t) * a.P + p) * D + 8 * part;
    const bf16x8 g = __builtin_bit_cast(bf16x8, ldg16(a.dout + base));
    const bf16x8 x = __builtin_bit_cast(bf16x8, ldg16(a.out + base));
    const bf16x8 y = __builtin_bit_cast(bf16x8, ldg16(a.o2 + base));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_out += (float)g[e] * (float)x[e];
      s_o2 += (float)g[e] * (float)y[e];
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) {
    s_out += __shfl_xor(s_out, off);
    s_o2 += __shfl_xor(s_o2, off);
  }
  if (!in || part != 0) return;
  float f[NF] = {0.f, 0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const float lamv = a.lam[((size_t)b * a.T + t) * a.P + p];
    const float* l = a.lse + ((size_t)b * a.T + t) * (2 * a.P) + 2 * p;
    f[0] = l[0] * LOG2E;
    f[1] = l[1] * LOG2E;
    f[2] = s_out + lamv * s_o2;   // dout . O_1
    f[3] = -lamv * s_o2;          // dO_2 . O_2
    f[4] = lamv;
    a.dlam[((size_t)b * a.T + t) * a.P + p] = -s_o2;
  }
  float* r = a.rs + ((size_t)b * a.P + p) * NF * a.Tpad + t;
#pragma unroll
  for (int k = 0; k < NF; ++k) r[(size_t)k * a.Tpad] = f[k];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* p, long long n4) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (long long)gridDim.x * blockDim.x)
    p[i] = float4{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(256) void convert_kernel(const float4* src, bf16x4* dst, long long n4) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (long long)gridDim.x * blockDim.x) {
    const float4 x = src[i];
    dst[i] = bf16x4{(bf16)x.x, (bf16)x.y, (bf16)x.z, (bf16)x.w};
  }
}

// ---------------------------------------------------------------------------
struct GradArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* rs;
  bf16* dq;
  float* dk_acc;
  float* dv_acc;
  int B, T, Hq, Hkv, G, P, Tpad;
  int causal;
  float scale_log2;   // log2(e) / sqrt(d)
  float rsqrt_d;
  // dK/dV grid
  int nkb;            // key blocks per (b, g)
  int nqt;            // 32-token query tiles
  int qtc;            // query tiles per chunk
  int nchunk;         // query chunks
  // dQ grid (the forward's decomposition)
  int ppw, nsub, chunks, ntb, units;
};

// ---- dK / dV -----------------------------------------------------------------
constexpr int A_WAVES = 4;
constexpr int A_THREADS = 64 * A_WAVES;
constexpr int A_KBLK = 32 * A_WAVES;   // keys per workgroup
constexpr int A_QT = 32;               // query tokens per tile
constexpr int A_NS = 3;                // staging ring depth (3 or 4)
static_assert(A_NS == 3 || A_NS == 4, "staging ring depth");
constexpr int PF_A = 1;                // k-steps the S-phase operand reads run ahead
constexpr int PF_B = 1;                // iterations the dV/dK operand reads run ahead

// Key blocks paired with query chunk c: those whose first key is at or before
// the chunk's last token (every key block without the causal mask).
__host__ __device__ inline int chunk_key_blocks(const GradArgs& a, int c) {
  if (!a.causal) return a.nkb;
  const int last_tile = min(a.nqt, (c + 1) * a.qtc) - 1;
  return min(a.nkb, last_tile * A_QT / A_KBLK + 1);
}

template <int D>
__global__ __launch_bounds__(A_THREADS, 1) void bwd_dkdv_kernel(GradArgs a) {
  constexpr int NCH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int TILE = A_QT * D * 2;                 // bytes of one [32][D] bf16 tile
  constexpr int RS_BYTES = A_THREADS * 16;           // one copy instruction per wave
  constexpr int STAGE = 3 * TILE + RS_BYTES;         // Q_1, Q_2, dout, row statistics
  constexpr int TLOADS = A_QT * NCH / A_THREADS;     // copy instructions per tile per thread
  constexpr int LOADS = 3 * TLOADS + 1;
  static_assert(TLOADS >= 1 && (A_QT * NCH) % A_THREADS == 0, "tile/thread mismatch");
  __shared__ __attribute__((aligned(16))) char smem[A_NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int T = a.T;

  // ---- workgroup -> ((b, g), query chunk, key block).  Chunks are fixed ranges
  // of qtc query tiles; chunk c pairs with every key block that has a visible
  // key in it (all of them without the causal mask).  Workgroups run from the
  // last chunk down, key blocks in order, so the workgroups that run together on
  // one XCD (same (b, g): blockIdx % units) stream the same query tiles and share
  // them through L2.
  const int units = a.B * a.Hkv;
  const int u = blockIdx.x % units;
  int idx = blockIdx.x / units;
  int qc = a.nchunk - 1;
  for (; qc >= 0; --qc) {
    const int n = chunk_key_blocks(a, qc);
    if (idx < n) break;
    idx -= n;
  }
  if (qc < 0) return;
  const int kb = idx;
  const int g = u % a.Hkv;
  const int b = u / a.Hkv;
  const int k0 = kb * A_KBLK;
  const int qt_first = a.causal ? k0 / A_QT : 0;
  const int qt0 = max(qc * a.qtc, qt_first);
  const int qt1 = min(a.nqt, (qc + 1) * a.qtc);
  if (qt0 >= qt1) return;
  const int nsteps = (qt1 - qt0) * a.G;

  // ---- this wave's 32 keys: K and V rows as the B operands of Q K^T and dout V^T
  const int kw0 = k0 + 32 * wave;
  const int key = kw0 + l32;
  bf16x8 kreg[KSTEPS], vreg[KSTEPS];
  {
    const bool ok = key < T;
    const size_t off = (((size_t)b * T + (ok ? key : 0)) * a.Hkv + g) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      kreg[s] = __builtin_bit_cast(bf16x8, ok ? ldg16(a.k + off + 16 * s) : u32x4{0, 0, 0, 0});
      vreg[s] = __builtin_bit_cast(bf16x8, ok ? ldg16(a.v + off + 16 * s) : u32x4{0, 0, 0, 0});
    }
  }
  f32x16 dk[DBLK], dv[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  // ---- staging copies.  Slot s of a tile = row s / NCH, physical chunk s % NCH,
  // holding logical chunk (s % NCH) ^ (row % NCH); rows past T repeat row T-1.
  const uint32_t qrow = (uint32_t)a.Hq * D * 2;   // bytes between tokens in q
  const uint32_t drow = (uint32_t)a.P * D * 2;    // ... in dout
  uint32_t qofs[TLOADS], dofs[TLOADS];
  int srow[TLOADS];
#pragma unroll
  for (int j = 0; j < TLOADS; ++j) {
    const int slot = (j * A_WAVES + wave) * 64 + lane;
    const int r = slot / NCH, pc = slot % NCH;
    srow[j] = r;
    qofs[j] = r * qrow + 16 * (pc ^ t_swz<D>(r));
    dofs[j] = r * drow + 16 * (pc ^ t_swz<D>(r));
  }
  // row statistics: 5 fields x 32 tokens = 40 chunks of 16 bytes; lanes past
  // them repeat the last chunk into the unused tail of the slot
  uint32_t rsofs;
  {
    const int cidx = min(wave * 64 + lane, NF * A_QT / 4 - 1);
    rsofs = (uint32_t)((cidx / 8) * a.Tpad * 4 + 16 * (cidx % 8));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)LDS_PTR(const char, smem);
  // Copy cursor: the (query tile, pair) of the next step to stage and its three
  // source rows, advanced by constant strides (steps run pair-fastest), so no
  // step recomputes a 64-bit address.
  int cp_t0 = qt0 * A_QT, cp_pp = 0;
  const char* cp_q = reinterpret_cast<const char*>(a.q) + (((size_t)b * T + cp_t0) * a.Hq + 2 * g * a.G) * D * 2;
  const char* cp_d = reinterpret_cast<const char*>(a.dout) + (((size_t)b * T + cp_t0) * a.P + g * a.G) * D * 2;
  const char* cp_r = reinterpret_cast<const char*>(a.rs) + (((size_t)b * a.P + g * a.G) * NF * a.Tpad + cp_t0) * 4;
  const long long rs_pair = (long long)NF * a.Tpad * 4;
  const long long q_tile = (long long)A_QT * a.Hq * D * 2 - (long long)a.G * 4 * D;
  const long long d_tile = (long long)A_QT * a.P * D * 2 - (long long)a.G * 2 * D;
  const long long r_tile = (long long)A_QT * 4 - a.G * rs_pair;
  auto stage_copy = [&](int st) {
    const bool tail = cp_t0 + A_QT > T;
    const uint32_t sbase = lds_base + st * STAGE;
#pragma unroll
    for (int j = 0; j < TLOADS; ++j) {
      uint32_t oq = qofs[j], od = dofs[j];
      if (tail) {
        const int back = max(0, cp_t0 + srow[j] - (T - 1));
        oq -= back * qrow;
        od -= back * drow;
      }
      const uint32_t dst = sbase + (j * A_WAVES + wave) * 1024;
      dma16_saddr(cp_q, oq, dst);
      dma16_saddr(cp_q + D * 2, oq, dst + TILE);
      dma16_saddr(cp_d, od, dst + 2 * TILE);
    }
    dma16_saddr(cp_r, rsofs, sbase + 3 * TILE + wave * 1024);
    cp_q += 4 * D;
    cp_d += 2 * D;
    cp_r += rs_pair;
    if (++cp_pp == a.G) {
      cp_pp = 0;
      cp_t0 += A_QT;
      cp_q += q_tile;
      cp_d += d_tile;
      cp_r += r_tile;
    }
  };

  // ---- per-lane LDS read offsets (bytes within a tile)
  uint32_t aofs[KSTEPS];   // rows as the A operand: row l32, d = 16 s + 8 hi
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) aofs[s] = 2 * t_phys<D>(l32, 16 * s + 8 * hi);
  // transposing reads: 16 lanes cover rows rr..rr+3 x 16 columns; lane = column
  const int i16 = lane & 15, g16 = lane >> 4;
  const int rr = 4 * (g16 >> 1) + (i16 >> 2);
  uint32_t tofs[DBLK][2];  // [d block][rows +0 / +8]; rows +16 ks keep the swizzle
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
      tofs[db][h8] = 2 * t_phys<D>(rr + 8 * h8, 32 * db + 16 * (g16 & 1) + 4 * (i16 & 3));

  const float c = a.scale_log2;

  auto compute = [&](int t0, auto st_c) {
    constexpr int ST = decltype(st_c)::value;
    const char* sb = smem + ST * STAGE;
    if (a.causal && t0 + A_QT - 1 < kw0) return;   // every key of this wave is in the future
    if (kw0 >= T) return;
    // S_1, S_2 = Q_r K^T and dP = dout V^T: rows (tokens) x this wave's keys
    // (A operands read one k-step ahead of their products)
    f32x16 s1 = f32x16{}, s2 = f32x16{}, dp = f32x16{};
    auto load_a = [&](int s, bf16x8 (&o)[3]) {
#pragma unroll
      for (int m = 0; m < 3; ++m) o[m] = *reinterpret_cast<const bf16x8*>(sb + m * TILE + aofs[s]);
    };
    bf16x8 aop[PF_A + 1][3];
#pragma unroll
    for (int s = 0; s < PF_A; ++s) load_a(s, aop[s]);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (s + PF_A < KSTEPS) load_a(s + PF_A, aop[(s + PF_A) % (PF_A + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      s1 = mfma32(aop[s % (PF_A + 1)][0], kreg[s], s1);
      s2 = mfma32(aop[s % (PF_A + 1)][1], kreg[s], s2);
      dp = mfma32(aop[s % (PF_A + 1)][2], vreg[s], dp);
    }
    // B operands of the dV / dK products (dout, Q_1, Q_2 read transposed), for
    // iteration it = (ks, db); read one iteration ahead of the products that use
    // them, the first before the softmax arithmetic, so that LDS latency hides
    // behind MFMA and VALU work
    constexpr int NIT = 2 * DBLK;
    auto load_b = [&](int it, bf16x8 (&o)[3]) {
      const int ks = it / DBLK, db = it % DBLK;
      const int ro = 16 * ks * D * 2;
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        const int tile = m == 0 ? 2 : m - 1;
        const char* p0 = sb + tile * TILE + tofs[db][0] + ro;
        const char* p1 = sb + tile * TILE + tofs[db][1] + ro;
        o[m] = concat(lds_read_tr4(reinterpret_cast<const bf16*>(p0)),
                      lds_read_tr4(reinterpret_cast<const bf16*>(p1)));
      }
    };
    bf16x8 bop[PF_B + 1][3];
#pragma unroll
    for (int it = 0; it < PF_B; ++it) load_b(it, bop[it]);
    __builtin_amdgcn_sched_barrier(0);
    // lane holds rows 8 (i/4) + 4 hi + i%4 of the tile for key l32.  Hidden
    // entries (future keys, rows or keys past T) get score -inf, so their P and dS
    // come out exactly 0 from the common arithmetic below; only tiles on the
    // diagonal or at the sequence end take this branch.
    if ((a.causal && t0 < kw0 + 31) || t0 + A_QT > T || kw0 + 32 > T) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = t0 + 8 * (i >> 2) + 4 * hi + (i & 3);
        const bool vis = tok < T && key < T && (!a.causal || key <= tok);
        s1[i] = vis ? s1[i] : -INFINITY;
        s2[i] = vis ? s2[i] : -INFINITY;
      }
    }
    bf16x8 pc[2], d1[2], d2[2];
    const float* rsl = reinterpret_cast<const float*>(sb + 3 * TILE);
    auto grad_group = [&](int gq) {
      const int r0 = 8 * gq + 4 * hi;
      const f32x4 L1 = *reinterpret_cast<const f32x4*>(rsl + 0 * A_QT + r0);
      const f32x4 L2 = *reinterpret_cast<const f32x4*>(rsl + 1 * A_QT + r0);
      const f32x4 D1 = *reinterpret_cast<const f32x4*>(rsl + 2 * A_QT + r0);
      const f32x4 D2 = *reinterpret_cast<const f32x4*>(rsl + 3 * A_QT + r0);
      const f32x4 LM = *reinterpret_cast<const f32x4*>(rsl + 4 * A_QT + r0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * gq + e;
        const float p1 = fast_exp2(__builtin_fmaf(s1[i], c, -L1[e]));
        const float p2 = fast_exp2(__builtin_fmaf(s2[i], c, -L2[e]));
        const float x1 = p1 * (dp[i] - D1[e]);
        const float x2 = -p2 * __builtin_fmaf(LM[e], dp[i], D2[e]);
        const float xc = __builtin_fmaf(-LM[e], p2, p1);
        pc[i >> 3][i & 7] = (bf16)xc;
        d1[i >> 3][i & 7] = (bf16)x1;
        d2[i >> 3][i & 7] = (bf16)x2;
      }
    };
    grad_group(0);
    grad_group(1);
    // dV += (P_1 - lambda P_2)^T dout,  dK += dS_1^T Q_1 + dS_2^T Q_2
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (it + PF_B < NIT) load_b(it + PF_B, bop[(it + PF_B) % (PF_B + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      const int ks = it / DBLK, db = it % DBLK;
      dv[db] = mfma32(pc[ks], bop[it % (PF_B + 1)][0], dv[db]);
      dk[db] = mfma32(d1[ks], bop[it % (PF_B + 1)][1], dk[db]);
      dk[db] = mfma32(d2[ks], bop[it % (PF_B + 1)][2], dk[db]);
      if (it < 2) grad_group(2 + it);   // rows 16..31 issue while the ks = 0 products run
    }
  };

  // ---- staging ring: step j uses stage j % A_NS; the copy for step j+A_NS-1
  // goes into the stage of step j-1, which every wave finished before the
  // barrier that closed step j-1.  After step j the copy for step j+1 must have
  // landed; the later ones may stay in flight.
#pragma unroll
  for (int j = 0; j < A_NS - 1; ++j)
    if (j < nsteps) stage_copy(j);
  wait_vmcnt0_builtin();
  __syncthreads();
  int ct0 = qt0 * A_QT, cpp = 0;   // compute cursor: query tile and pair of step j
  auto one = [&](int j, auto st_c) {
    constexpr int ST = decltype(st_c)::value;
    if (j + A_NS - 1 < nsteps) stage_copy((ST + A_NS - 1) % A_NS);
    compute(ct0, st_c);
    if (++cpp == a.G) {
      cpp = 0;
      ct0 += A_QT;
    }
    const int ahead = min(A_NS - 2, nsteps - 2 - j);   // copies allowed in flight
    if (A_NS > 3 && ahead >= 2)
      wait_vmcnt<2 * LOADS>();
    else if (ahead >= 1)
      wait_vmcnt<LOADS>();
    else
      wait_vmcnt<0>();
    __syncthreads();
  };
  for (int j = 0; j < nsteps; j += A_NS) {
    one(j, std::integral_constant<int, 0>{});
    if (j + 1 < nsteps) one(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 < nsteps) one(j + 2, std::integral_constant<int, 2>{});
    if constexpr (A_NS > 3)
      if (j + 3 < nsteps) one(j + 3, std::integral_constant<int, 3 % A_NS>{});
  }

  // ---- add this chunk's share to the fp32 accumulators.  C layout: lane l,
  // register i -> key kw0 + 8 (i/4) + 4 hi + i%4, d = 32 db + l32.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kk = kw0 + 8 * (i >> 2) + 4 * hi + (i & 3);
    if (kk >= T) continue;
    const size_t base = (((size_t)b * T + kk) * a.Hkv + g) * D + l32;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      unsafeAtomicAdd(a.dk_acc + base + 32 * db, dk[db][i] * a.rsqrt_d);
      unsafeAtomicAdd(a.dv_acc + base + 32 * db, dv[db][i]);
    }
  }
}

// ---- dQ ------------------------------------------------------------------------
constexpr int B_BN = 64;      // keys per LDS tile
constexpr int B_QT = 16;      // query tokens per wave
constexpr int B_WAVES = 8;
constexpr int B_THREADS = 64 * B_WAVES;

template <int D>
__global__ __launch_bounds__(B_THREADS, 1) void bwd_dq_kernel(GradArgs a) {
  constexpr int NCH = D / 8;
  constexpr int KS = D / 32;    // k-steps of the score products (32 d each)
  constexpr int DT = D / 16;    // 16-wide d tiles of dQ
  constexpr int LOADS = B_BN * NCH / B_THREADS;
  static_assert(LOADS >= 1 && (B_BN * NCH) % B_THREADS == 0, "tile/thread mismatch");
  constexpr int NBUF = 4;
  constexpr int TILE_BYTES = B_BN * D * 2;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * NBUF * B_BN * D];
  const char* lds = reinterpret_cast<const char*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15;   // MFMA column: query token i0 + i16 (both heads)
  const int g16 = lane >> 4;   // 16-lane group: which keys / d values of a tile

  // ---- workgroup -> (token block, b, g, pair chunk): the forward's order
  int tb, u;
  {
    const int idx = blockIdx.x;
    if ((a.units & 7) == 0) {
      const int upx = a.units >> 3;
      const int slot = idx >> 3;
      tb = a.ntb - 1 - slot / upx;
      u = (idx & 7) + 8 * (slot % upx);
    } else {
      tb = a.ntb - 1 - idx / a.units;
      u = idx % a.units;
    }
  }
  const int chunk = u % a.chunks;
  const int bg = u / a.chunks;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int tokens_wg = B_QT * a.nsub;
  const int tok0 = tb * tokens_wg;
  const int sub = wave / a.ppw;
  const int pig = chunk * a.ppw + (wave % a.ppw);
  const int p = g * a.G + pig;
  const int i0 = tok0 + sub * B_QT;
  const int T = a.T;
  const bool active = sub < a.nsub && pig < a.G && i0 < T;
  const int qtok = i0 + i16;

  const int kv_end = a.causal ? min(T, tok0 + tokens_wg) : T;
  const int ntiles = (kv_end + B_BN - 1) / B_BN;
  const bf16* kbase = a.k + ((size_t)b * T * a.Hkv + g) * D;
  const bf16* vbase = a.v + ((size_t)b * T * a.Hkv + g) * D;

  // ---- B operands in registers: Q^T of both heads and dout^T of this lane's
  // token, d = 32*s + 8*g16 + 0..7; row statistics of both heads
  bf16x8 qreg[2][KS], oreg[KS];
  float L2[2] = {0.f, 0.f}, Dr[2] = {0.f, 0.f}, sr[2] = {1.f, 0.f};
  {
    const bool ok = active && qtok < T;
    const int tq = ok ? qtok : 0;
    const bf16* qs = a.q + (((size_t)b * T + tq) * a.Hq + 2 * p) * D + 8 * g16;
    const bf16* os = a.dout + (((size_t)b * T + tq) * a.P + p) * D + 8 * g16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qreg[0][s] = __builtin_bit_cast(bf16x8, ok ? ldg16(qs + 32 * s) : u32x4{0, 0, 0, 0});
      qreg[1][s] = __builtin_bit_cast(bf16x8, ok ? ldg16(qs + D + 32 * s) : u32x4{0, 0, 0, 0});
      oreg[s] = __builtin_bit_cast(bf16x8, ok ? ldg16(os + 32 * s) : u32x4{0, 0, 0, 0});
    }
    if (ok) {
      const float* r = a.rs + ((size_t)b * a.P + p) * NF * a.Tpad + tq;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        L2[h] = r[(size_t)h * a.Tpad];
        Dr[h] = r[(size_t)(2 + h) * a.Tpad];
      }
      sr[1] = -r[(size_t)4 * a.Tpad];
    }
  }
  f32x4 o[DT][2];   // dQ^T tiles [d-tile][head]: lane holds d = 16*dt + 4*g16 + 0..3 of token qtok
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i][0] = o[i][1] = f32x4{};
  const float c = a.scale_log2;

  // ---- direct global -> LDS copies of K and V tiles (same swizzle for both)
  const uint32_t row_bytes = (uint32_t)a.Hkv * D * 2;
  uint32_t dofs[LOADS];
  int drow[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int slot = (j * B_WAVES + wave) * 64 + lane;
    const int r = slot / NCH, pc = slot % NCH;
    drow[j] = r;
    dofs[j] = r * row_bytes + 16 * (pc ^ q_swz<D>(r));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)LDS_PTR(const char, lds);
  auto dma_tile = [&](int t, int buf) {
    const char* kt = reinterpret_cast<const char*>(kbase) + (size_t)t * B_BN * row_bytes;
    const char* vt = reinterpret_cast<const char*>(vbase) + (size_t)t * B_BN * row_bytes;
    const bool tail = t * B_BN + B_BN > T;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      uint32_t of = dofs[j];
      if (tail) of -= max(0, t * B_BN + drow[j] - (T - 1)) * row_bytes;
      const uint32_t dst = lds_base + (j * B_WAVES + wave) * 1024;
      dma16_saddr(kt, of, dst + buf * TILE_BYTES);
      dma16_saddr(vt, of, dst + (NBUF + buf) * TILE_BYTES);
    }
  };

  // ---- per-lane LDS read offsets
  uint32_t aofs[2][KS];   // K (or V) rows as the A operand: key tile kt (row 16*kt + i16), k-step s
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int s = 0; s < KS; ++s) aofs[kt][s] = 2 * q_phys<D>(16 * kt + i16, 32 * s + 8 * g16);
  // K^T of d-tile dt: the lane's 8 k slots are keys 4*g16 + 0..3 and 16 + 4*g16 +
  // 0..3 (the keys its dS values cover); lane s of a 16-lane group addresses row
  // 4*g16 + s/4, columns 16*dt + 4*(s%4) .. +3 (rows 16 apart share the swizzle)
  uint32_t tofs[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) tofs[dt] = 2 * q_phys<D>(4 * g16 + (i16 >> 2), 16 * dt + 4 * (i16 & 3));

  auto compute_tile = [&](int t, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kbase_tok = t * B_BN + kb * 32;
      if (kbase_tok >= T) break;
      if (a.causal && kbase_tok > i0 + B_QT - 1) break;
      constexpr int KO = BUF * TILE_BYTES;
      constexpr int VO = (NBUF + BUF) * TILE_BYTES;
      const int ro = kb * 32 * D * 2;
      // S^T = K Q^T per head and dP^T = V dout^T (keys x tokens); lane -> keys
      // 16*kt + 4*g16 + i of token qtok.  K/V operands read one k-step ahead.
      f32x4 st[2][2], dpt[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) st[kt][0] = st[kt][1] = dpt[kt] = f32x4{};
      bf16x8 kva[2][2][2];   // [buffer][key tile][K, V]
      auto load_kv = [&](int s, bf16x8 (&ov)[2][2]) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          ov[kt][0] = *reinterpret_cast<const bf16x8*>(lds + KO + ro + aofs[kt][s]);
          ov[kt][1] = *reinterpret_cast<const bf16x8*>(lds + VO + ro + aofs[kt][s]);
        }
      };
      load_kv(0, kva[0]);
      // raised issue priority while these products issue, as in the forward: the
      // other wave of the SIMD then tends to run its dS and dQ work meanwhile
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) load_kv(s + 1, kva[(s + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          st[kt][0] = mfma16(kva[s & 1][kt][0], qreg[0][s], st[kt][0]);
          st[kt][1] = mfma16(kva[s & 1][kt][0], qreg[1][s], st[kt][1]);
          dpt[kt] = mfma16(kva[s & 1][kt][1], oreg[s], dpt[kt]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // hidden keys (future, or past T) get score -inf: P and dS come out 0
      if ((a.causal && kbase_tok + 31 > i0) || kbase_tok + 32 > T) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kbase_tok + 16 * kt + 4 * g16 + i;
            const bool vis = key < T && (!a.causal || key <= qtok);
            st[kt][0][i] = vis ? st[kt][0][i] : -INFINITY;
            st[kt][1][i] = vis ? st[kt][1][i] : -INFINITY;
          }
      }
      // dS^T of head h as the bf16 B operand: k slot e <-> key tile e/4, row 4*g16 + e%4
      bf16x8 ds[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = fast_exp2(__builtin_fmaf(st[e >> 2][h][e & 3], c, -L2[h]));
          ds[h][e] = (bf16)(pv * __builtin_fmaf(sr[h], dpt[e >> 2][e & 3], -Dr[h]));
        }
      // dQ^T += K^T dS^T (K^T operands read one d-tile ahead; each feeds both heads)
      auto load_kt = [&](int dt) {
        const char* p0 = lds + KO + ro + tofs[dt];
        return concat(lds_read_tr4(reinterpret_cast<const bf16*>(p0)),
                      lds_read_tr4(reinterpret_cast<const bf16*>(p0 + 16 * D * 2)));
      };
      bf16x8 ktr[2];
      ktr[0] = load_kt(0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if (dt + 1 < DT) ktr[(dt + 1) & 1] = load_kt(dt + 1);
        __builtin_amdgcn_sched_barrier(0);
        o[dt][0] = mfma16(ktr[dt & 1], ds[0], o[dt][0]);
        o[dt][1] = mfma16(ktr[dt & 1], ds[1], o[dt][1]);
      }
    }
  };

  dma_tile(0, 0);
  if (ntiles > 1) dma_tile(1, 1);
  if (ntiles > 2) dma_tile(2, 2);
  wait_vmcnt0_builtin();
  __syncthreads();
  auto tile = [&](int t, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    if (t + 3 < ntiles) dma_tile(t + 3, (BUF + 3) % NBUF);
    if (active) compute_tile(t, bufc);
    if (t + 3 < ntiles)
      wait_vmcnt<4 * LOADS>();
    else if (t + 2 < ntiles)
      wait_vmcnt<2 * LOADS>();
    else
      wait_vmcnt<0>();
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += NBUF) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < ntiles) tile(t + 2, std::integral_constant<int, 2>{});
    if (t + 3 < ntiles) tile(t + 3, std::integral_constant<int, 3>{});
  }

  if (!active || qtok >= T) return;
  // dQ^T tiles: lane -> token qtok, d = 16*dt + 4*g16 + 0..3
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    bf16* dst = a.dq + (((size_t)b * T + qtok) * a.Hq + 2 * p + h) * D + 4 * g16;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (bf16)(o[dt][h][e] * a.rsqrt_d);
      *reinterpret_cast<bf16x4*>(dst + 16 * dt) = w;
    }
  }
}

// A side stream per caller stream (and device), with the events that fork work
// onto it and join it back, created on first use and kept until the process ends.
// The dQ and dK/dV kernels read the same inputs and row statistics and write
// disjoint outputs; neither can share a CU with the other (LDS, registers), so on
// one stream each launch ends in a tail of idle CUs, and side by side the one
// fills the other's tail (T = 4096: 893-900 vs 924-928 us for the whole backward).
struct SideStream {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, pre = nullptr, join = nullptr;
};
std::mutex side_mu;   // guards side_streams and orders the enqueue sequences

// The entry for s (on the device s belongs to); side stays null if anything could
// not be created, once kMaxSideStreams caller streams have one, and while s is being
// captured into a graph (a stream that first meets the backward inside a capture
// runs it serially there; one that met it before forks and joins inside the capture
// too).  With a null side all launches go to s, in the same order of dependencies.
constexpr size_t kMaxSideStreams = 64;
SideStream& side_for(hipStream_t s) {
  static std::map<std::pair<int, hipStream_t>, SideStream> side_streams;
  static size_t created = 0;
  static SideStream none;
  int dev = -1;
  if (hipStreamGetDevice(s, &dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return none;
  }
  const auto key = std::make_pair(dev, s);
  auto it = side_streams.find(key);
  if (it != side_streams.end()) return it->second;
  if (created >= kMaxSideStreams) return none;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return none;
  }
  if (cs != hipStreamCaptureStatusNone) return none;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) {
    (void)hipGetLastError();
    return none;
  }
  if (cur != dev && hipSetDevice(dev) != hipSuccess) {   // the side stream lives on s's device
    (void)hipGetLastError();
    return none;
  }
  SideStream n;
  bool ok = hipStreamCreateWithFlags(&n.side, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&n.pre, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&n.join, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();   // clear the failed call's status
    if (n.join) (void)hipEventDestroy(n.join);
    if (n.pre) (void)hipEventDestroy(n.pre);
    if (n.fork) (void)hipEventDestroy(n.fork);
    if (n.side) (void)hipStreamDestroy(n.side);
  }
  if (cur != dev) (void)hipSetDevice(cur);
  if (!ok) return none;
  ++created;
  return side_streams.emplace(key, n).first->second;
}

template <int D>
hipError_t launch(const BackwardProblem& pr, hipStream_t s) {
  const int G = pr.Hq / (2 * pr.Hkv);
  const int P = pr.Hq / 2;
  const int Tpad = backward_tpad(pr.T);
  float* rs = pr.ws;
  float* dk_acc = rs + backward_rs_floats(pr.B, pr.T, pr.Hq);
  float* dv_acc = dk_acc + (size_t)pr.B * pr.T * pr.Hkv * D;
  const long long nkv = (long long)pr.B * pr.T * pr.Hkv * D;

  GradArgs a;
  a.q = static_cast<const bf16*>(pr.q);
  a.k = static_cast<const bf16*>(pr.k);
  a.v = static_cast<const bf16*>(pr.v);
  a.dout = static_cast<const bf16*>(pr.dout);
  a.rs = rs;
  a.dq = static_cast<bf16*>(pr.dq);
  a.dk_acc = dk_acc;
  a.dv_acc = dv_acc;
  a.B = pr.B;
  a.T = pr.T;
  a.Hq = pr.Hq;
  a.Hkv = pr.Hkv;
  a.G = G;
  a.P = P;
  a.Tpad = Tpad;
  a.causal = pr.causal ? 1 : 0;
  a.scale_log2 = LOG2E / sqrtf((float)D);
  a.rsqrt_d = 1.0f / sqrtf((float)D);
  a.nkb = (pr.T + A_KBLK - 1) / A_KBLK;
  a.nqt = (pr.T + A_QT - 1) / A_QT;
  a.qtc = 16;   // 512 query tokens per chunk
  a.nchunk = (a.nqt + a.qtc - 1) / a.qtc;
  a.ppw = G < B_WAVES ? G : B_WAVES;
  a.nsub = B_WAVES / a.ppw;
  a.chunks = (G + a.ppw - 1) / a.ppw;
  a.ntb = (pr.T + B_QT * a.nsub - 1) / (B_QT * a.nsub);
  a.units = pr.B * pr.Hkv * a.chunks;

  // grid sizes, checked before anything is enqueued: the dK/dV grid grows with T^2
  long long pairs = 0;   // (chunk, key block) pairs per (b, g)
  for (int c = 0; c < a.nchunk; ++c) pairs += chunk_key_blocks(a, c);
  const long long ga = (long long)pr.B * pr.Hkv * pairs;
  const long long gb = (long long)a.ntb * a.units;
  const long long gpre = ((long long)pr.B * Tpad * P * (D / 8) + 255) / 256;
  constexpr long long kMaxGrid = (1LL << 31) - 1;
  if (ga > kMaxGrid || gb > kMaxGrid || gpre > kMaxGrid) return hipErrorInvalidConfiguration;

  PreArgs pa{static_cast<const bf16*>(pr.out), static_cast<const bf16*>(pr.o2), static_cast<const bf16*>(pr.dout),
             pr.lam, pr.lse, rs, pr.dlam, pr.B, pr.T, P, Tpad};
  // s:    fill -> (wait pre) -> dK/dV -> convert dK, dV -> (wait dQ)
  // side: (wait for s) -> pre -> dQ
  // Everything the caller enqueues on s afterwards sees all outputs.  The lock keeps
  // another thread's calls on the same stream from interleaving with the event
  // records and waits.
  std::lock_guard<std::mutex> lock(side_mu);
  const SideStream& ss = side_for(s);
  const hipStream_t t = ss.side ? ss.side : s;
  hipError_t e = hipSuccess;
  auto chk = [&](hipError_t r) {
    if (e == hipSuccess) e = r;
  };
  if (ss.side) {
    chk(hipEventRecord(ss.fork, s));
    if (e == hipSuccess) chk(hipStreamWaitEvent(t, ss.fork, 0));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)gpre), dim3(256), 0, t, pa);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(2048), dim3(256), 0, s, reinterpret_cast<float4*>(dk_acc), 2 * nkv / 4);
  if (ss.side) {   // without this dependency the gradient kernels must not be enqueued
    chk(hipEventRecord(ss.pre, t));
    if (e == hipSuccess) chk(hipStreamWaitEvent(s, ss.pre, 0));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)ga), dim3(A_THREADS), 0, s, a);
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)gb), dim3(B_THREADS), 0, t, a);
  if (ss.side) chk(hipEventRecord(ss.join, t));
  hipLaunchKernelGGL(convert_kernel, dim3(2048), dim3(256), 0, s, reinterpret_cast<const float4*>(dk_acc),
                     static_cast<bf16x4*>(pr.dk), nkv / 4);
  hipLaunchKernelGGL(convert_kernel, dim3(2048), dim3(256), 0, s, reinterpret_cast<const float4*>(dv_acc),
                     static_cast<bf16x4*>(pr.dv), nkv / 4);
  if (ss.side && e == hipSuccess) chk(hipStreamWaitEvent(s, ss.join, 0));
  chk(hipGetLastError());
  return e;
}

}  // namespace

hipError_t launch_backward_bf16(const BackwardProblem& p, hipStream_t s) {
  return p.d == 128 ? launch<128>(p, s) : launch<64>(p, s);
}

}  // namespace diffattn
