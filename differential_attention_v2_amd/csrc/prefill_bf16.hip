// Tiled prefill kernel for Differential Attention V2, bf16 in / fp32 accumulate, gfx950.
//
// What it computes (sources: the Differential Transformer V2 web pages):
//   out[b,i,p,:] = softmax(q_{2p} K^T/sqrt(d)) V - lambda[b,i,p] * softmax(q_{2p+1} K^T/sqrt(d)) V
// over the keys j <= i (causal) or all keys, where both query heads of pair p
// read the same K/V head g = p / G -- differential-attention lesson "差异性注意力
// (V2)", section "差异性概念" (DiffAttn equation); dailytechsnack.ch article,
// section "Gemeinsamer KV-Cache statt Spezialkernel" (adjacent query heads of one
// GQA group share K/V and the head dim); attention-variants lesson, "步骤1"
// (causal mask).
//
// Work decomposition.  A workgroup of 8 waves (two per SIMD) owns one (batch b,
// KV head g) and a block of query tokens.  Each wave owns one differential pair
// p of that group and 16 query tokens: its 32 query rows (16 tokens x the pair's
// two heads) are the 32 columns of one MFMA tile, column n = 16*head + token, so
// the lambda-subtract pairs lanes l and l^16 in registers.  Every K/V tile of 64
// keys is copied from HBM/L2 into LDS once per workgroup and read by all waves:
// with G = 4 pairs per KV head, one staged byte serves all 8 query heads.  The
// copy uses the direct global-to-LDS loads (16 bytes per lane, no registers),
// issued three tiles ahead into a 4-deep ring.  The two waves of a SIMD
// interleave: one wave's softmax (VALU) issues while the other's MFMAs run.
//
// Per 32-key half tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (A = K from LDS, B = Q^T held in registers), so each lane holds the scores of
// one query row against 16 keys; lane l^32 holds the other 16.  P = exp2(S *
// log2(e)/sqrt(d) - m) is rounded to bf16 and fed straight from registers as the
// B operand of O^T += V^T P^T; the V^T operand comes from the row-major V tile
// via the transposing LDS read.  The running maximum m is raised only when a
// half tile's row sums could overflow (see the softmax step below).  The
// epilogue normalises each row, subtracts lambda * head 1 from head 0 of the
// same token, applies the optional V1 RMSNorm and stores bf16.
#include <type_traits>

#include "dev_common.h"
#include "internal.h"

namespace diffattn {
namespace {

constexpr int QT = 16;           // query tokens per wave (x 2 heads = 32 MFMA columns)
// Two tile shapes of one kernel.  SHAPE 0 (full prefill): 8 waves (two per SIMD),
// 64-key tiles in a 4-deep ring, a barrier in the middle of each tile.  SHAPE 1
// (sliding window): 4 waves, 32-key tiles in a 5-deep ring (80 KB), so two
// workgroups share a CU and their waves interleave on each SIMD without a common
// barrier; a window gives each workgroup only ~17 64-key tiles, and the second
// workgroup then hides the first one's prologue and tail (+7 % measured), while
// for full prefill the doubled tile staging makes it 2 % slower.
template <int SHAPE> struct Shape {
  static constexpr int WAVES = SHAPE == 0 ? 8 : 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BN = SHAPE == 0 ? 64 : 32;     // keys per LDS tile
  static constexpr int NBUF = SHAPE == 0 ? 4 : 5;     // ring depth
  static constexpr int WG_PER_CU = SHAPE == 0 ? 1 : 2;
};
constexpr float SUM_LIMIT = 65536.0f;  // per-lane half-tile row-sum bound (2^16)

struct Args {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const float* lam;
  bf16* out;
  bf16* o2;     // training forward: A_2 V per pair, or null
  float* lse;   // training forward: log-sum-exp per query row and head, or null
  int B, T, Hq, Hkv, G, P;
  int causal, v1;
  float eps, scale_log2;
  int window;  // causal sliding window in keys (0: none)
  int ppw;     // pairs per workgroup
  int nsub;    // 16-token sub-blocks per workgroup
  int chunks;  // workgroups needed to cover the G pairs of one KV head
  int ntb;     // token blocks
  int units;   // B * Hkv * chunks
};

// LDS layouts: tiles are row-major [key][d] without padding; 16-byte chunks of a
// row are XOR-permuted so that the MFMA operand reads hit distinct banks (K: chunk
// ^ (row % chunks per row); V: chunk ^ v_swz(row)).
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return (D >= 128) ? ((row & 3) << 2) : ((row & 1) << 2);
}
template <int D>
__device__ __forceinline__ int v_phys(int row, int col) {
  return row * D + ((((col >> 3) ^ v_swz<D>(row))) << 3) + (col & 7);
}

__device__ __forceinline__ float max16(const f32x16& x) {
  float m = fmaxf(fmaxf(x[0], x[1]), x[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) m = fmaxf(fmaxf(m, x[i]), x[i + 1]);
  return fmaxf(m, x[15]);
}

template <int D, int SHAPE>
__global__ __launch_bounds__(Shape<SHAPE>::THREADS, Shape<SHAPE>::WG_PER_CU) void prefill_kernel(Args a) {
  constexpr int WAVES = Shape<SHAPE>::WAVES;
  constexpr int THREADS = Shape<SHAPE>::THREADS;
  constexpr int BN = Shape<SHAPE>::BN;
  constexpr int HPT = BN / 32;             // 32-key half tiles per tile
  constexpr int NCH = D / 8;               // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;           // QK^T k-steps
  constexpr int DBLK = D / 32;             // PV output d-blocks
  constexpr int LOADS = BN * NCH / THREADS;  // 16-byte chunks per thread per tile (K or V)
  static_assert(LOADS >= 1 && (BN * NCH) % THREADS == 0, "tile/thread mismatch");
  // K/V tiles in a ring: tile t lives in buffer t % NBUF and is requested
  // NBUF-1 tiles ahead of its use, so its copy overlaps several tiles of compute.
  // The NBUF K buffers come first, then the NBUF V buffers, so every operand read
  // is a per-lane offset plus a compile-time immediate below 80 KB.
  constexpr int NBUF = Shape<SHAPE>::NBUF;
  constexpr int TILE_BYTES = BN * D * 2;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * NBUF * BN * D];
  const char* lds = reinterpret_cast<const char*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar, so everything derived from it (pair, first token,
  // masking decisions) stays wave-uniform and compiles to scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lo = lane < 32;
  const int l32 = lane & 31;   // MFMA column: query row 16*head + token

  // ---- workgroup -> (token block, b, g, pair chunk).  Token blocks run longest
  // first (causal work grows with the block index); when the (b, g, chunk) units
  // divide evenly over the 8 XCDs, all blocks of one unit land on one XCD so
  // its K/V stays in that XCD's L2.
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
  const int tokens_wg = QT * a.nsub;
  const int tok0 = tb * tokens_wg;
  const int sub = wave / a.ppw;
  const int pig = chunk * a.ppw + (wave % a.ppw);
  const bool active = sub < a.nsub && pig < a.G;
  const int p = g * a.G + pig;
  const int i0 = tok0 + sub * QT;          // first query token of this wave
  const int T = a.T;
  const int qtok = i0 + (l32 & 15);        // this lane's query token
  const int qhead = l32 >> 4;              // 0: positive branch, 1: subtracted branch

  // key tiles [t_first, t_first + nt): with a sliding window the tiles that end
  // before the window of the block's first token are never copied or read
  const int kv_end = a.causal ? min(T, tok0 + tokens_wg) : T;
  const int t_first = a.window > 0 ? max(0, tok0 - a.window + 1) / BN : 0;
  const int nt = (kv_end + BN - 1) / BN - t_first;
  const bf16* kbase = a.k + ((size_t)b * T * a.Hkv + g) * D;
  const bf16* vbase = a.v + ((size_t)b * T * a.Hkv + g) * D;

  // ---- Q^T operand in registers: lane -> query row l32, d = 16*s + 8*(lane/32) + 0..7
  bf16x8 qreg[KSTEPS];
  {
    const bool ok = active && qtok < T;
    const bf16* src = a.q + (((size_t)b * T + (ok ? qtok : 0)) * a.Hq + 2 * p + qhead) * D + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      u32x4 x = ok ? ldg16(src + 16 * s) : u32x4{0, 0, 0, 0};
      qreg[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};
  float m = -INFINITY;   // running maximum (log2 domain), uniform over lanes l, l^32
  float l = 0.f;         // this lane's share of the softmax denominator
  const float c = a.scale_log2;

  // ---- direct global -> LDS tile copy.  Wave-instruction j of wave w fills the
  // 64 consecutive 16-byte slots [(j*WAVES + w)*64, +64) of a tile; slot s holds
  // row s/NCH, physical chunk s%NCH, i.e. logical chunk (s%NCH) ^ swizzle(row).
  // Per lane the byte offset inside a tile of K (or V) rows is loop-invariant;
  // the tile's base is a scalar.  Rows past the sequence end (last tile only)
  // repeat the last row: finite data, always masked out.
  const uint32_t row_bytes = (uint32_t)a.Hkv * D * 2;
  uint32_t dofs_k[LOADS], dofs_v[LOADS];
  int drow[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int slot = (j * WAVES + wave) * 64 + lane;
    const int r = slot / NCH, pc = slot % NCH;
    drow[j] = r;
    dofs_k[j] = r * row_bytes + 16 * (pc ^ (r & (NCH - 1)));
    dofs_v[j] = r * row_bytes + 16 * (pc ^ v_swz<D>(r));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)LDS_PTR(const char, lds);
  auto dma_tile = [&](int t, int buf) {
    const char* kt = reinterpret_cast<const char*>(kbase) + (size_t)t * BN * row_bytes;
    const char* vt = reinterpret_cast<const char*>(vbase) + (size_t)t * BN * row_bytes;
    const bool tail = t * BN + BN > T;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      uint32_t ok = dofs_k[j], ov = dofs_v[j];
      if (tail) {   // clamp rows past the end to the last row
        const int back = max(0, t * BN + drow[j] - (T - 1));
        ok -= back * row_bytes;
        ov -= back * row_bytes;
      }
      const uint32_t dst = lds_base + (j * WAVES + wave) * 1024;
      dma16_saddr(kt, ok, dst + buf * TILE_BYTES);
      dma16_saddr(vt, ov, dst + (NBUF + buf) * TILE_BYTES);
    }
  };

  // ---- per-lane LDS read offsets (bytes), loop-invariant
  const int i16 = lane & 15, g16 = lane >> 4;
  uint32_t kofs[KSTEPS];   // K rows as the A operand of S^T: row l32, k-step s
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    kofs[s] = l32 * D * 2 + 16 * ((2 * s + (lane >> 5)) ^ (l32 & (NCH - 1)));
  uint32_t vofs[DBLK];     // transposing reads of V for output d-block db
  {
    const int vrow = 4 * (g16 >> 1) + (i16 >> 2);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int col = 32 * db + 16 * (g16 & 1) + 4 * (i16 & 3);
      vofs[db] = NBUF * TILE_BYTES + 2 * v_phys<D>(vrow, col);
    }
  }
  // (v_phys of row vrow + 16*ks + 8*r + 32*kb equals v_phys(vrow) + that many rows:
  // the V swizzle depends on row % 4 only.)

  // P = exp2(S*c - mb) as the bf16 B operand, and this lane's share of its row sum
  auto exp_rows = [&](const f32x16& sh, float mb, bf16x8 (&ph)[2], float& lt) {
    lt = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ph[i >> 3][i & 7] = (bf16)fast_exp2(__builtin_fmaf(sh[i], c, -mb));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 8; j += 2) lt = dot2_ones(bf16x2{ph[ks][j], ph[ks][j + 1]}, lt);
  };

  // Last 32-key half tile this wave reads; K operands are read one half tile
  // ahead into ka, right after the S products of the current one have issued.
  const int hl = active ? ((a.causal ? min(T, i0 + QT) : T) + 31) / 32 - 1 : -1;
  // first half tile this wave reads (the window of its first token)
  const int h_first = a.window > 0 ? max(0, i0 - a.window + 1) / 32 : 0;
  bf16x8 ka[KSTEPS];
  auto load_k = [&](int off) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) ka[s] = *reinterpret_cast<const bf16x8*>(lds + kofs[s] + off);
  };

  // half tile h = HPT t + KB, held in ring buffer BUF
  auto half = [&](int t, auto kb_c, auto buf_c) {
    constexpr int KB = decltype(kb_c)::value;
    constexpr int BUF = decltype(buf_c)::value;
    // LDS offset of the K half tile that follows this one
    constexpr int KNEXT = KB + 1 < HPT ? BUF * TILE_BYTES + (KB + 1) * 32 * D * 2 : ((BUF + 1) % NBUF) * TILE_BYTES;
    const int h = HPT * t + KB;
    if (h + 1 == h_first) load_k(KNEXT);   // the wave's first K operands
    if (h < h_first || h > hl) return;
    const int kbase_tok = 32 * h;

    // ---- V^T operands of this half tile
    bf16x8 va[2][DBLK];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const char* vp = lds + vofs[db] + BUF * TILE_BYTES + (KB * 32 + 16 * ks) * D * 2;
        va[ks][db] = concat(lds_read_tr4(reinterpret_cast<const bf16*>(vp)),
                            lds_read_tr4(reinterpret_cast<const bf16*>(vp + 8 * D * 2)));
      }
    // ---- S^T = K Q^T (keys x query rows)
    // raised issue priority while the S products issue: the other wave of the
    // SIMD then tends to run its softmax meanwhile instead of interleaving MFMAs
    f32x16 sc = f32x16{};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) sc = mfma32(ka[s], qreg[s], sc);
    __builtin_amdgcn_s_setprio(0);
    load_k(KNEXT);   // after the last half tile this reads unused (in-bounds) data
    const bool need_mask = (a.causal && kbase_tok + 31 > i0) || kbase_tok + 32 > T ||
                           (a.window > 0 && kbase_tok + a.window <= i0 + QT - 1);
    if (need_mask) {   // causal diagonal, sequence tail, window start
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase_tok + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const bool vis = key < T && (!a.causal || key <= qtok) && (a.window == 0 || key > qtok - a.window);
        if (!vis) sc[i] = -INFINITY;
      }
    }
    // ---- online softmax.  P = exp2(S*c - m) uses the current running maximum
    // m as is; the half tile's row sums bound every P value (a lane's 16 values
    // are non-negative), so if all sums stay <= 2^16 nothing overflows and m
    // needs no update.  Otherwise (and on the first half tile, where m = -inf
    // makes the sums infinite) a rare branch raises m to the true maximum,
    // rescales O and l, and recomputes P.  Either way numerator and denominator
    // share one reference, so the result is exact.
    bf16x8 pp[2];
    float lt;
    exp_rows(sc, m, pp, lt);
    if (__builtin_amdgcn_ballot_w64(!(lt <= SUM_LIMIT))) {
      float mx = max16(sc);
      mx = fmaxf(mx, partner32(mx, lo)) * c;
      const float nm = fmaxf(m, mx);
      const float alpha = (nm == -INFINITY) ? 1.f : fast_exp2(m - nm);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
      l *= alpha;
      m = nm;
      exp_rows(sc, nm == -INFINITY ? 0.f : nm, pp, lt);
    }
    l += lt;
    // ---- O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < DBLK; ++db) o[db] = mfma32(va[ks][db], pp[ks], o[db]);
  };

  // ---- tile loop, unrolled by NBUF so each buffer index is a constant.
  // SHAPE 0: tile t is read from the second half of tile t-1 (its first K half,
  // read ahead) to its own second half.  The barrier between the two halves of
  // tile t publishes tile t+1 (each wave waited for its own share of the copy)
  // and proves that every wave finished tile t-1, whose buffer then receives tile
  // t+3.  SHAPE 1: during tile t the waves read tiles t and t+1 (K one tile
  // ahead); the barrier after tile t publishes tile t+2 and proves every wave
  // finished tile t, so tile t+4 goes into the buffer of tile t-1.
  constexpr int FIRST = SHAPE == 0 ? 1 : 2;   // tiles published before the loop
  dma_tile(t_first, 0);
  if (FIRST > 1 && nt > 1) dma_tile(t_first + 1, 1);
  wait_vmcnt0_builtin();   // Q operands and the first tiles have landed
  __syncthreads();
#pragma unroll
  for (int j = FIRST; j < NBUF - 1; ++j)
    if (j < nt) dma_tile(t_first + j, j);
  load_k(0);
  // ring position r holds tile t_first + r in buffer r % NBUF
  auto tile = [&](int r, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int t = t_first + r;
    half(t, std::integral_constant<int, 0>{}, bufc);
    // the next tile to publish must have landed; one later copy may stay in flight
    if (r + NBUF - 2 < nt)
      wait_vmcnt<2 * LOADS>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (r + NBUF - 1 < nt) dma_tile(t + NBUF - 1, (BUF + NBUF - 1) % NBUF);
    if constexpr (HPT > 1) half(t, std::integral_constant<int, 1>{}, bufc);
  };
  for (int r = 0; r < nt; r += NBUF) {
    tile(r, std::integral_constant<int, 0>{});
    if (r + 1 < nt) tile(r + 1, std::integral_constant<int, 1>{});
    if (r + 2 < nt) tile(r + 2, std::integral_constant<int, 2>{});
    if (r + 3 < nt) tile(r + 3, std::integral_constant<int, 3>{});
    if constexpr (NBUF > 4)
      if (r + 4 < nt) tile(r + 4, std::integral_constant<int, 4 % NBUF>{});
  }

  if (!active) return;
  // ---- epilogue: normalise each row, subtract lambda * head 1 (columns 16-31,
  // lanes l^16) from head 0 (columns 0-15), optional RMSNorm, store head-0 lanes
  l += partner32(l, lo);
  if (a.lse != nullptr && lo && qtok < T)   // natural-log LSE of the row's scaled scores
    a.lse[((size_t)b * T + qtok) * a.Hq + 2 * p + qhead] = (m + __log2f(l)) * 0.6931471805599453f;
  const bool ok = qhead == 0 && qtok < T;
  const float lamv = ok ? a.lam[((size_t)b * T + qtok) * a.P + p] : 0.f;
  const float inv = 1.0f / l;
  float ss = 0.f;
  {
    // Both products are rounded before the subtraction (FMA contraction off), so
    // the two branches are treated alike and identical branches with lambda = 1
    // cancel exactly.  Head-1 lanes keep their own normalised row (A_2 V).
#pragma clang fp contract(off)
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float y = o[db][i] * inv;
        const float y1 = __shfl_xor(y, 16);
        const float x = qhead == 0 ? y - lamv * y1 : y;
        o[db][i] = x;
        ss += x * x;
      }
    }
  }
  auto store_rows = [&](bf16* base) {
    bf16* dst = base + (((size_t)b * T + qtok) * a.P + p) * D + 4 * (lane >> 5);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)o[db][4 * i4 + e];
        *reinterpret_cast<bf16x4*>(dst + 32 * db + 8 * i4) = w;
      }
    }
  };
  if (a.o2 != nullptr && qhead == 1 && qtok < T) store_rows(a.o2);
  if (a.v1) {
    ss += partner32(ss, lo);
    const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] *= r;
  }
  if (ok) store_rows(a.out);
}

template <int D, int SHAPE>
hipError_t launch(const PrefillProblem& pr, hipStream_t s) {
  constexpr int WAVES = Shape<SHAPE>::WAVES;
  Args a;
  a.q = static_cast<const bf16*>(pr.q);
  a.k = static_cast<const bf16*>(pr.k);
  a.v = static_cast<const bf16*>(pr.v);
  a.lam = pr.lam;
  a.out = static_cast<bf16*>(pr.out);
  a.o2 = static_cast<bf16*>(pr.o2);
  a.lse = pr.lse;
  a.B = pr.B;
  a.T = pr.T;
  a.Hq = pr.Hq;
  a.Hkv = pr.Hkv;
  a.G = pr.Hq / (2 * pr.Hkv);
  a.P = pr.Hq / 2;
  a.causal = pr.causal ? 1 : 0;
  a.v1 = pr.v1_rmsnorm ? 1 : 0;
  a.eps = pr.eps;
  a.window = pr.causal ? pr.window : 0;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  a.ppw = a.G < WAVES ? a.G : WAVES;
  a.nsub = WAVES / a.ppw;
  a.chunks = (a.G + a.ppw - 1) / a.ppw;
  const int tokens_wg = QT * a.nsub;
  a.ntb = (a.T + tokens_wg - 1) / tokens_wg;
  a.units = a.B * a.Hkv * a.chunks;
  const long long blocks = (long long)a.ntb * a.units;
  hipLaunchKernelGGL((prefill_kernel<D, SHAPE>), dim3((unsigned)blocks), dim3(Shape<SHAPE>::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillProblem& p, hipStream_t s) {
  const bool window = p.causal && p.window > 0;
  if (p.d == 128) return window ? launch<128, 1>(p, s) : launch<128, 0>(p, s);
  return window ? launch<64, 1>(p, s) : launch<64, 0>(p, s);
}

}  // namespace diffattn
