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
// p of that group and 16 query tokens; the pair's two heads are two 16-column
// MFMA tiles of the same tokens, so head 0 and head 1 of a token sit in the same
// lane and the lambda-subtract needs no lane exchange.  Every K/V tile of 64
// keys is copied from HBM/L2 into LDS once per workgroup and read by all waves:
// with G = 4 pairs per KV head, one staged byte serves all 8 query heads.  The
// copy uses the direct global-to-LDS loads (16 bytes per lane, no registers),
// issued three tiles ahead into a 4-deep ring.  The two waves of a SIMD
// interleave: one wave's softmax (VALU) issues while the other's MFMAs run.
//
// Per 32-key half tile a wave computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16
// as four independent 16 x 16 tiles (2 key tiles x 2 heads, each summed over D/32
// k-steps), so no product waits on the one before it; lane l then holds, for
// each head, the scores of query token l%16 against 8 of the 32 keys.  P =
// exp2(S * log2(e)/sqrt(d) - m) is rounded to bf16 and fed straight from
// registers as the B operand of O^T += V^T P^T (16 x 16 tiles, one product per
// d-tile and head); the V^T operand comes from the row-major V tile via the
// transposing LDS read, its k order matching the keys each lane holds.  The
// running maximum m is raised only when a half tile's row sums could overflow
// (see the softmax step below).  The epilogue normalises each row, subtracts
// lambda * head 1 from head 0 of the same token, applies the optional V1
// RMSNorm and stores bf16.
#include <atomic>
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
  int slot;    // persistent launches: work-queue slot (see prefill_kernel)
};

// LDS layouts: tiles are row-major [key][d] without padding; the 16-byte chunks
// of a row are XOR-permuted by a function of the row so that the MFMA operand
// reads hit distinct banks.  For d = 128 K and V share swz16(row) = ((row % 4) << 2)
// ^ (row / 4 % 2) << 1 ^ 11 (row / 8 % 2), chosen by measurement (rocprofv3
// SQ_LDS_BANK_CONFLICT on the two read patterns alone): it leaves both the K
// operand reads (ds_read_b128; lanes 16g + i read row i at chunk 4s + g) and the
// transposing V reads (16-lane group g reads rows 4g .. 4g + 3 at one chunk pair)
// free of bank conflicts, where chunk ^ (row % 16) conflicts on the V reads and
// chunk ^ 4 (row % 4) on both.  Rows 16 apart share the permutation.  d = 64 keeps
// K: chunk ^ (row % 8), V: chunk ^ 4 (row % 2).
__device__ __forceinline__ int swz16(int row) {
  return ((row & 3) << 2) ^ ((row & 4) >> 1) ^ ((row & 8) ? 11 : 0);
}
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return (D >= 128) ? swz16(row) : (row & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return (D >= 128) ? swz16(row) : ((row & 1) << 2);
}
template <int D>
__device__ __forceinline__ int v_phys(int row, int col) {
  return row * D + ((((col >> 3) ^ v_swz<D>(row))) << 3) + (col & 7);
}

// Work queues of the persistent schedule (long sequences, see prefill_kernel).  A
// launch takes one slot of QSLOTS, handed out round-robin by the host: 8 queue
// heads (one per XCD; queue q hands out the blocks idx = 8 j + q, j = 0, 1, ...) and
// a count of finished workgroups.  The last workgroup of a launch sets its slot back
// to zero, so the next launch that takes it starts from empty queues.
constexpr int QSLOTS = 1024;
constexpr int QSTRIDE = 16;   // ints per slot: 8 heads, the finished count, padding
__device__ int prefill_queue[QSLOTS * QSTRIDE];
// The persistent schedule pays for itself once the XCDs' different finish times,
// not the per-block claim overheads, dominate the tail: T = 32768 (32 blocks per
// CU) ran 4.5 % faster with it, T = 4096 (4 blocks per CU) 1.6 % slower.
constexpr int kPersistBlocksPerCu = 8;

template <int D, int SHAPE, bool PERSIST>
__global__ __launch_bounds__(Shape<SHAPE>::THREADS, Shape<SHAPE>::WG_PER_CU) void prefill_kernel(Args a) {
  constexpr int WAVES = Shape<SHAPE>::WAVES;
  constexpr int THREADS = Shape<SHAPE>::THREADS;
  constexpr int BN = Shape<SHAPE>::BN;
  constexpr int HPT = BN / 32;             // 32-key half tiles per tile
  constexpr int NCH = D / 8;               // 16-byte chunks per row
  constexpr int KS = D / 32;               // QK^T k-steps (32 d each)
  constexpr int DT = D / 16;               // PV output d-tiles
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

  // PERSIST: one workgroup per CU takes blocks from the launch's queues: first from
  // the queue of its own XCD (blockIdx % 8; the blocks of one (b, g) unit are all in
  // queue unit % 8, so its K/V stays in that XCD's L2), longest first, then from the
  // other queues once its own is empty, so that XCDs which run faster take over the
  // last blocks of slower ones (with one fixed share per XCD the XCDs finished up to
  // 4.5 % apart at T = 32768).  Otherwise one block per workgroup, placed on the XCDs
  // by the same rule through the block index.
  const long long nblk = (long long)a.ntb * a.units;
  int* const qctr = prefill_queue + (size_t)a.slot * QSTRIDE;
  const int xq = blockIdx.x & 7;            // this workgroup's own queue (its XCD)
  const long long qlen = nblk >> 3;         // blocks per queue
  __shared__ int s_next;
  // wave 0: claim a block from any queue that still has one (its lanes 0-7 read the
  // 8 queue heads, lane 0 claims from the fullest), or -1 when all are empty
  auto steal = [&]() -> int {
    const int ln = threadIdx.x & 63;
    for (;;) {
      const int h = ln < 8 ? __hip_atomic_load(qctr + ln, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
      long long left = ln < 8 ? qlen - h : 0;
      int best = ln;
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) {   // max over lanes 0-7 of (left, lane)
        const long long ol = __shfl_xor(left, off);
        const int ob = __shfl_xor(best, off);
        if (ol > left || (ol == left && ob < best)) { left = ol; best = ob; }
      }
      left = __shfl(left, 0);
      best = __shfl(best, 0);
      if (left <= 0) return -1;
      int got = -1;
      if (ln == 0) {
        const int j = __hip_atomic_fetch_add(qctr + best, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (j < qlen) got = j * 8 + best;
      }
      got = __shfl(got, 0);
      if (got >= 0) return got;
    }
  };
  if constexpr (PERSIST) {
    if (threadIdx.x < 64) {
      int got = -1;
      if (threadIdx.x == 0) {
        const int j = __hip_atomic_fetch_add(qctr + xq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (j < qlen) got = j * 8 + xq;
      }
      got = __shfl(got, 0);
      if (got < 0) got = steal();
      if (threadIdx.x == 0) s_next = got;
    }
  }
  for (int jblk = 0;; ++jblk) {
    int idx;
    if constexpr (PERSIST) {
      // publishes s_next, and every wave is done with the ring of the previous block
      // (each block's body passes barriers after reading s_next, so it is read before
      // it is written again)
      __syncthreads();
      idx = s_next;
      if (idx < 0) break;
    } else {
      if (jblk > 0) break;
      idx = blockIdx.x;
    }
    // the next block is claimed from the own queue while this block's first loads are
    // in flight (the claim returns with them); a steal, if needed, follows the prologue
    int jnext = 0;
    if constexpr (PERSIST)
      if (threadIdx.x == 0) jnext = __hip_atomic_fetch_add(qctr + xq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index as a scalar, so everything derived from it (pair, first token,
    // masking decisions) stays wave-uniform and compiles to scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i16 = lane & 15;   // MFMA column: query token i0 + i16 (both heads)
    const int g16 = lane >> 4;   // 16-lane group: which keys / d values of a tile

    // ---- block index -> (token block, b, g, pair chunk).  Token blocks run longest
    // first (causal work grows with the block index); when the (b, g, chunk) units
    // divide evenly over the 8 XCDs, all blocks of one unit have the same index % 8,
    // i.e. land on one XCD (hardware placement, or the queue above), so its K/V stays
    // in that XCD's L2.
    int tb, u;
    {
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
    const int qtok = i0 + i16;               // this lane's query token

    // key tiles [t_first, t_first + nt): with a sliding window the tiles that end
    // before the window of the block's first token are never copied or read
    const int kv_end = a.causal ? min(T, tok0 + tokens_wg) : T;
    const int t_first = a.window > 0 ? max(0, tok0 - a.window + 1) / BN : 0;
    const int nt = (kv_end + BN - 1) / BN - t_first;
    const bf16* kbase = a.k + ((size_t)b * T * a.Hkv + g) * D;
    const bf16* vbase = a.v + ((size_t)b * T * a.Hkv + g) * D;

    // ---- Q^T operands in registers: head h, k-step s -> lane holds token qtok,
    // d = 32*s + 8*g16 + 0..7 (the B layout of the 16x16x32 product)
    bf16x8 qreg[2][KS];
    {
      const bool ok = active && qtok < T;
      const bf16* src = a.q + (((size_t)b * T + (ok ? qtok : 0)) * a.Hq + 2 * p) * D + 8 * g16;
  #pragma unroll
      for (int h = 0; h < 2; ++h)
  #pragma unroll
        for (int s = 0; s < KS; ++s) {
          u32x4 x = ok ? ldg16(src + h * D + 32 * s) : u32x4{0, 0, 0, 0};
          qreg[h][s] = __builtin_bit_cast(bf16x8, x);
        }
    }

    f32x4 o[DT][2];   // O^T tiles [d-tile][head]: lane holds d = 16*dt + 4*g16 + 0..3 of token qtok
  #pragma unroll
    for (int i = 0; i < DT; ++i) o[i][0] = o[i][1] = f32x4{};
    float m[2] = {-INFINITY, -INFINITY};   // running maxima per head (log2 domain), uniform over the row's 4 lanes
    float l[2] = {0.f, 0.f};               // this lane's share of each head's softmax denominator
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
      dofs_k[j] = r * row_bytes + 16 * (pc ^ k_swz<D>(r));
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
    uint32_t kofs[2][KS];   // K rows as the A operand of S^T: key tile kt (row 16*kt + i16), k-step s
  #pragma unroll
    for (int kt = 0; kt < 2; ++kt)
  #pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int r = 16 * kt + i16;
        kofs[kt][s] = r * D * 2 + 16 * ((4 * s + g16) ^ k_swz<D>(r));
      }
    // V^T operand of d-tile dt: the lane's 8 k slots are keys 4*g16 + 0..3 and
    // 16 + 4*g16 + 0..3 (the keys its scores cover), read as two transposing
    // reads of 4 rows; lane s of a 16-lane group addresses row 4*g16 + s/4,
    // columns 16*dt + 4*(s%4) .. +3
    uint32_t vofs[DT];
  #pragma unroll
    for (int dt = 0; dt < DT; ++dt) vofs[dt] = NBUF * TILE_BYTES + 2 * v_phys<D>(4 * g16 + (i16 >> 2), 16 * dt + 4 * (i16 & 3));
    // (v_phys of row r + 16 equals v_phys(r) + 16 rows: the V swizzle depends on
    // row % 16 only.)

    // P = exp2(S*c - m) of head h as the bf16 B operand (k slot e <-> key tile e/4,
    // row 4*g16 + e%4), and this lane's share of its row sum
    auto exp_rows = [&](const f32x4 (&st)[2][2], int h, float mb, bf16x8& ph, float& lt) {
      lt = 0.f;
  #pragma unroll
      for (int e = 0; e < 8; ++e) ph[e] = (bf16)fast_exp2(__builtin_fmaf(st[e >> 2][h][e & 3], c, -mb));
  #pragma unroll
      for (int j = 0; j < 8; j += 2) lt = dot2_ones(bf16x2{ph[j], ph[j + 1]}, lt);
    };

    // Last 32-key half tile this wave reads; K operands are read one half tile
    // ahead into ka, right after the S products of the current one have issued.
    const int hl = active ? ((a.causal ? min(T, i0 + QT) : T) + 31) / 32 - 1 : -1;
    // first half tile this wave reads (the window of its first token)
    const int h_first = a.window > 0 ? max(0, i0 - a.window + 1) / 32 : 0;
    bf16x8 ka[2][KS];
    auto load_k = [&](int off) {
  #pragma unroll
      for (int kt = 0; kt < 2; ++kt)
  #pragma unroll
        for (int s = 0; s < KS; ++s) ka[kt][s] = *reinterpret_cast<const bf16x8*>(lds + kofs[kt][s] + off);
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
      bf16x8 va[DT];
  #pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const char* vp = lds + vofs[dt] + BUF * TILE_BYTES + KB * 32 * D * 2;
        va[dt] = concat(lds_read_tr4(reinterpret_cast<const bf16*>(vp)),
                        lds_read_tr4(reinterpret_cast<const bf16*>(vp + 16 * D * 2)));
      }
      // ---- S^T = K Q^T: tiles [key tile kt][head], lane -> keys 16*kt + 4*g16 + i
      // raised issue priority while the S products issue: the other wave of the
      // SIMD then tends to run its softmax meanwhile instead of interleaving MFMAs
      f32x4 st[2][2];
  #pragma unroll
      for (int kt = 0; kt < 2; ++kt) st[kt][0] = st[kt][1] = f32x4{};
      __builtin_amdgcn_s_setprio(1);
  #pragma unroll
      for (int s = 0; s < KS; ++s)
  #pragma unroll
        for (int kt = 0; kt < 2; ++kt)
  #pragma unroll
          for (int hh = 0; hh < 2; ++hh) st[kt][hh] = mfma16(ka[kt][s], qreg[hh][s], st[kt][hh]);
      __builtin_amdgcn_s_setprio(0);
      load_k(KNEXT);   // after the last half tile this reads unused (in-bounds) data
      const bool need_mask = (a.causal && kbase_tok + 31 > i0) || kbase_tok + 32 > T ||
                             (a.window > 0 && kbase_tok + a.window <= i0 + QT - 1);
      if (need_mask) {   // causal diagonal, sequence tail, window start
  #pragma unroll
        for (int kt = 0; kt < 2; ++kt)
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kbase_tok + 16 * kt + 4 * g16 + i;
            const bool vis = key < T && (!a.causal || key <= qtok) && (a.window == 0 || key > qtok - a.window);
            if (!vis) st[kt][0][i] = st[kt][1][i] = -INFINITY;
          }
      }
      // ---- online softmax.  P = exp2(S*c - m) uses the current running maximum
      // m as is; the half tile's row sums bound every P value (a lane's 8 values
      // of a row are non-negative), so if all sums stay <= 2^16 nothing overflows
      // and m needs no update.  Otherwise (and on the first half tile, where m =
      // -inf makes the sums infinite) a rare branch raises m to the true maximum
      // (over the row's 4 lanes), rescales O and l, and recomputes P.  Either way
      // numerator and denominator share one reference, so the result is exact.
      bf16x8 pp[2];
      float lt[2];
      exp_rows(st, 0, m[0], pp[0], lt[0]);
      exp_rows(st, 1, m[1], pp[1], lt[1]);
      if (__builtin_amdgcn_ballot_w64(!(lt[0] <= SUM_LIMIT) || !(lt[1] <= SUM_LIMIT))) {
  #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float mx = fmaxf(fmaxf(fmaxf(st[0][hh][0], st[0][hh][1]), fmaxf(st[0][hh][2], st[0][hh][3])),
                           fmaxf(fmaxf(st[1][hh][0], st[1][hh][1]), fmaxf(st[1][hh][2], st[1][hh][3])));
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
          const float nm = fmaxf(m[hh], mx);
          const float alpha = (nm == -INFINITY) ? 1.f : fast_exp2(m[hh] - nm);
  #pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt][hh] *= alpha;
          l[hh] *= alpha;
          m[hh] = nm;
          exp_rows(st, hh, nm == -INFINITY ? 0.f : nm, pp[hh], lt[hh]);
        }
      }
      l[0] += lt[0];
      l[1] += lt[1];
      // ---- O^T += V^T P^T
  #pragma unroll
      for (int dt = 0; dt < DT; ++dt)
  #pragma unroll
        for (int hh = 0; hh < 2; ++hh) o[dt][hh] = mfma16(va[dt], pp[hh], o[dt][hh]);
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
    if constexpr (PERSIST) {
      if (threadIdx.x < 64) {
        int got = (threadIdx.x == 0 && jnext < qlen) ? jnext * 8 + xq : -1;
        got = __shfl(got, 0);
        if (got < 0) got = steal();
        if (threadIdx.x == 0) s_next = got;
      }
    }
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

    if (active) {
    // ---- epilogue: each row's denominator is spread over the 4 lanes of its
    // token (g16 = 0..3); normalise, subtract lambda * head 1 from head 0 in the
    // lane, optional RMSNorm, store
  #pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      l[hh] += __shfl_xor(l[hh], 16);
      l[hh] += __shfl_xor(l[hh], 32);
    }
    const bool ok = qtok < T;
    if (a.lse != nullptr && g16 == 0 && ok) {   // natural-log LSE of each head's scaled scores
  #pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        a.lse[((size_t)b * T + qtok) * a.Hq + 2 * p + hh] = (m[hh] + __log2f(l[hh])) * 0.6931471805599453f;
    }
    const float lamv = ok ? a.lam[((size_t)b * T + qtok) * a.P + p] : 0.f;
    const float inv0 = 1.0f / l[0], inv1 = 1.0f / l[1];
    float ss = 0.f;
    {
      // Both products are rounded before the subtraction (FMA contraction off), so
      // the two branches are treated alike and identical branches with lambda = 1
      // cancel exactly.  o[.][1] keeps the normalised head-1 row (A_2 V).
  #pragma clang fp contract(off)
  #pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float y0 = o[dt][0][i] * inv0;
          const float y1 = o[dt][1][i] * inv1;
          const float x = y0 - lamv * y1;
          o[dt][0][i] = x;
          o[dt][1][i] = y1;
          ss += x * x;
        }
      }
    }
    auto store_rows = [&](bf16* base, int hh) {
      bf16* dst = base + (((size_t)b * T + qtok) * a.P + p) * D + 4 * g16;
  #pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x4 w;
  #pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)o[dt][hh][e];
        *reinterpret_cast<bf16x4*>(dst + 16 * dt) = w;
      }
    };
    if (a.o2 != nullptr && ok) store_rows(a.o2, 1);
    if (a.v1) {
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
  #pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][0] *= r;
    }
    if (ok) store_rows(a.out, 0);
    }
  }
  if constexpr (PERSIST) {
    if (threadIdx.x == 0) {   // the last workgroup to finish resets the slot for its next launch
      const int done = __hip_atomic_fetch_add(qctr + 8, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (done == (int)gridDim.x - 1)
        for (int q = 0; q <= 8; ++q) __hip_atomic_store(qctr + q, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// CUs of the current device (0 if the query fails), cached per device
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
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
  const int ncu = compute_units();
  a.slot = 0;
  if constexpr (SHAPE == 0) {
    if ((a.units & 7) == 0 && ncu > 0 && blocks >= (long long)kPersistBlocksPerCu * ncu) {
      static std::atomic<unsigned> next_slot{0};
      a.slot = (int)(next_slot.fetch_add(1, std::memory_order_relaxed) % QSLOTS);
      hipLaunchKernelGGL((prefill_kernel<D, SHAPE, true>), dim3((unsigned)ncu), dim3(Shape<SHAPE>::THREADS), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_kernel<D, SHAPE, false>), dim3((unsigned)blocks), dim3(Shape<SHAPE>::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillProblem& p, hipStream_t s) {
  const bool window = p.causal && p.window > 0;
  if (p.d == 128) return window ? launch<128, 1>(p, s) : launch<128, 0>(p, s);
  return window ? launch<64, 1>(p, s) : launch<64, 0>(p, s);
}

}  // namespace diffattn
