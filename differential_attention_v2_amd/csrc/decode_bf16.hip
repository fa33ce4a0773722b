// Split-KV decode for Differential Attention V2, bf16 cache / fp32 accumulate, gfx950.
//
// One new query token per sequence attends to a contiguous cache [B, L, Hkv, d]
// that already holds it.  Decode is bound by HBM bandwidth, and the V2 layout
// lets one pass over the cache serve both heads of every pair in a KV-head group
// (dailytechsnack.ch article, section "Gemeinsamer KV-Cache statt Spezialkernel":
// the KV cache does not grow and decoding runs at standard-transformer speed;
// differential-attention lesson, section "V1 vs V2": V2 loads the KV cache once
// per step and raises decode arithmetic intensity).
//
// Split kernel: one wave per (b, KV head g, key range s).  It streams its key
// range once, 32 keys per step: the step's K and V rows are copied global -> LDS
// directly (global_load_lds, nontemporal), each instruction moving whole 256-byte
// rows, one step ahead of the step being computed (two LDS stages).  Loading the
// K operand straight into registers would touch 16 rows x 64 bytes per
// instruction, which streams measurably slower than whole rows.  The scores of
// the group's 2G query heads are computed at once on v_mfma_f32_16x16x32_bf16
// (A = 16 cache keys read from LDS, B = the 2G query heads, padded to 16
// columns).  P^T stays in registers as the B operand of O^T += V^T P^T; the V^T
// operand comes from the row-major V rows in LDS with the transposing LDS read.
// Each wave writes, per query head, its partial softmax state (running max m in
// the log2 domain, denominator l and the unnormalised accumulator) to the
// workspace.
//
// Combine kernel: one wave per (b, pair).  For both heads of the pair it
// merges the partial states (M = max_s m_s, weights 2^(m_s - M)), normalises,
// forms o_1 - lambda * o_2 (optional V1 RMSNorm) and writes bf16.
//
// The split kernel is written for any number nq <= 16 of query heads per KV head
// and any dot-product slice [off, off + DK) of the q and k rows, so the same code
// also runs the two layouts V2 is compared against (differential-attention
// lesson, section "V1 vs V2"): a standard transformer (one softmax per head, H
// heads) and DIFF V1 (each head's q and k split into halves of d/2, one pass per
// branch, each pass reading the full V rows -- V is read twice per step).
#include "dev_common.h"
#include "internal.h"

namespace diffattn {
namespace {

constexpr int KSTEP = 32;   // keys per step
// ragged caches: largest batch whose waves plan their own rows (the c4-shaped ragged
// decode at B = 128-512 ran 0.6-0.9 % faster that way than with the plan kernel, at
// B = 1024 2 % slower)
constexpr int kPlanHereMaxB = 512;

struct Args {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const float* lam;
  bf16* out;
  float* ws;
  int B, L, Hq, Hkv, G, P;
  int S, chunk;
  int v1;
  float eps, scale_log2;
  const int* seq_lens;   // valid rows per sequence, or null (all L)
  int window;            // visible keys before and including the query, 0 = all
  int nq;                // query heads per KV head served by one wave (<= 16)
  int qoff, koff;        // start of the dot-product slice within q and k rows
  int* plan;             // ragged caches: row offsets per sequence, total, rows per range
  int nslot;             // ragged caches: record slots per query head
  int fuse;              // one key range per sequence: the split kernel writes out itself
  int plan_here;         // ragged caches: each wave derives its rows from seq_lens (the plan
                         // kernel is skipped; wave 0 of range 0 writes the plan for the combine)
};

// V rows in LDS: row-major [key][d], 16-byte chunks XOR-permuted per row so the
// transposing reads of 8 rows x 2 chunks hit distinct banks.
template <int D>
__device__ __forceinline__ int v_phys(int row, int col) {
  constexpr int NCH = D / 8;
  const int sw = (NCH >= 16) ? ((row & 7) << 1) : ((row & 3) << 1);
  return row * D + ((((col >> 3) ^ sw)) << 3) + (col & 7);
}

// Direct global -> LDS copy of 16 bytes per lane with the nontemporal hint (the
// cache is read exactly once): scalar base, per-lane byte offset, lane l's bytes
// land at lds_addr + 16 l.  Inline asm, so the compiler adds no waits of its own;
// the caller waits on vmcnt before reading the stage.
__device__ __forceinline__ void dma16_stream(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  // one wait state between the M0 write and the copy that reads it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds_addr), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}

// K-slice rows in LDS: [key][DK], 16-byte chunks XOR-permuted so that the MFMA
// operand reads (16 rows x one chunk per 16-lane group) hit distinct banks.
template <int KCH>
__device__ __forceinline__ int k_swz(int row) {
  constexpr int SH = KCH >= 16 ? 0 : (KCH == 8 ? 1 : 2);
  return (row >> SH) & (KCH - 1);
}

// LDS per wave: two stages of (32 K-slice rows, 32 V rows)
template <int D, int DK>
struct DecodeLds {
  static constexpr int KBYTES = KSTEP * DK * 2;
  static constexpr int VBYTES = KSTEP * D * 2;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int BYTES = 2 * STAGE;
};

// Attention of the nq query heads of KV head g of sequence b over the cache rows
// [k0, k1), streamed 32 rows per step.  Writes the partial state of query head
// n (n < nq) -- unnormalised acc[D], m (log2 domain), l -- to rec0 + n * hstride.
// Each step's K slice and V rows are copied global -> LDS directly, four or more
// whole rows per instruction, one step ahead of the one being computed; lds is
// this wave's DecodeLds<D, DK>::BYTES.
template <int D, int DK>
__device__ __forceinline__ void attend_range(const Args& a, char* lds, int b, int g, int k0, int k1, float* rec0,
                                             size_t hstride) {
  using LD = DecodeLds<D, DK>;
  constexpr int KS = DK / 32;                  // QK^T k-steps (k = 32 per MFMA)
  constexpr int DB = D / 16;                   // PV d-blocks (16 rows per MFMA)
  constexpr int NCH = D / 8;                   // 16-byte chunks per V row
  constexpr int KCH = DK / 8;                  // 16-byte chunks per K-slice row
  constexpr int KLOADS = KSTEP * KCH / 64;     // copy instructions per step
  constexpr int VLOADS = KSTEP * NCH / 64;
  constexpr int LOADS = KLOADS + VLOADS;
  const int lane = threadIdx.x;
  const int n = lane & 15;     // query column = head within the group
  const int grp = lane >> 4;   // 16-lane group
  const int nq = a.nq;

  // Q^T operand: column n = head g*nq + n, d = off + 32*ks + 8*grp + 0..7
  bf16x8 qr[KS];
  {
    const bool ok = n < nq;
    const bf16* src = a.q + ((size_t)b * a.Hq + g * nq + (ok ? n : 0)) * D + a.qoff + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = ok ? ldg16(src + 32 * ks) : u32x4{0, 0, 0, 0};
      qr[ks] = __builtin_bit_cast(bf16x8, x);
    }
    // q arrives before the first cache copy is issued: the compiler then has no
    // load of its own outstanding in the loop and inserts no wait there
    wait_vmcnt0_builtin();
  }
  const uint32_t row_bytes = (uint32_t)a.Hkv * D * 2;
  const char* kb0 = reinterpret_cast<const char*>(a.k + ((size_t)b * a.L * a.Hkv + g) * D);
  const char* vb0 = reinterpret_cast<const char*>(a.v + ((size_t)b * a.L * a.Hkv + g) * D);
  const float c = a.scale_log2;

  // copy instruction j, lane l fills LDS slot 64 j + l of the K (or V) stage:
  // row slot / CH, physical chunk slot % CH = logical chunk ^ swizzle(row)
  uint32_t kofs[KLOADS], vofs[VLOADS];
  int krow[KLOADS], vrow[VLOADS];
#pragma unroll
  for (int j = 0; j < KLOADS; ++j) {
    const int r = (64 * j + lane) / KCH, pc = lane % KCH;
    krow[j] = r;
    kofs[j] = r * row_bytes + 2 * a.koff + 16 * (pc ^ k_swz<KCH>(r));
  }
#pragma unroll
  for (int j = 0; j < VLOADS; ++j) {
    const int r = (64 * j + lane) / NCH, pc = lane % NCH;
    vrow[j] = r;
    vofs[j] = r * row_bytes + 2 * (v_phys<D>(r, 8 * pc) - r * D);   // v_phys permutes chunks within the row
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)LDS_PTR(const char, lds);
  // rows past k1 (last step only) repeat row k1 - 1: finite data, masked out
  auto issue = [&](int kk, int st) {
    const char* kt = kb0 + (size_t)kk * row_bytes;
    const char* vt = vb0 + (size_t)kk * row_bytes;
    const int last = k1 - 1 - kk;
    const uint32_t dst = lds_base + st * LD::STAGE;
#pragma unroll
    for (int j = 0; j < KLOADS; ++j)
      dma16_stream(kt, kofs[j] - (uint32_t)max(0, krow[j] - last) * row_bytes, dst + 1024 * j);
#pragma unroll
    for (int j = 0; j < VLOADS; ++j)
      dma16_stream(vt, vofs[j] - (uint32_t)max(0, vrow[j] - last) * row_bytes, dst + LD::KBYTES + 1024 * j);
  };

  // per-lane LDS read offsets: K operand of k-step ks for keys 16 h + n
  uint32_t krd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) krd[ks] = n * DK * 2 + 16 * ((4 * ks + grp) ^ k_swz<KCH>(n));

  f32x4 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x4{};
  float m = -INFINITY, l = 0.f;

  if (k0 < k1) issue(k0, 0);
  for (int kk = k0, st = 0; kk < k1; kk += KSTEP, st ^= 1) {
    if (kk + KSTEP < k1) {
      // the other stage was last read by the previous step: its reads are done
      // before the next copy into it is issued
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(kk + KSTEP, st ^ 1);
      wait_vmcnt<LOADS>();
    } else {
      wait_vmcnt0();
    }
    const char* ks_lds = lds + st * LD::STAGE;
    const bf16* vs = reinterpret_cast<const bf16*>(ks_lds + LD::KBYTES);
    // ---- S^T = K Q^T: lane -> query n, keys kk + 16*h + 4*grp + i
    f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(ks_lds + krd[ks]);
      const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(ks_lds + krd[ks] + 16 * DK * 2);
      s0 = mfma16(ka0, qr[ks], s0);
      s1 = mfma16(ka1, qr[ks], s1);
    }
    if (kk + KSTEP > k1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (kk + 4 * grp + i >= k1) s0[i] = -INFINITY;
        if (kk + 16 + 4 * grp + i >= k1) s1[i] = -INFINITY;
      }
    }
    // ---- online softmax over this step's 32 keys
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx * c);
    const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
    const float mb = (mn == -INFINITY) ? 0.f : mn;
    m = mn;
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = (bf16)fast_exp2(__builtin_fmaf(s0[i], c, -mb));
      pb[4 + i] = (bf16)fast_exp2(__builtin_fmaf(s1[i], c, -mb));
    }
    l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; j += 2) l = dot2_ones(bf16x2{pb[j], pb[j + 1]}, l);
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;

    // ---- O^T += V^T P^T, V^T read from LDS with the transposing read
    {
      const int r0 = 4 * grp + (n >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 16 * db + 4 * (n & 3);
        const bf16x4 va = lds_read_tr4(&vs[v_phys<D>(r0, col)]);
        const bf16x4 vb = lds_read_tr4(&vs[v_phys<D>(r0 + 16, col)]);
        o[db] = mfma16(concat(va, vb), pb, o[db]);
      }
    }
  }

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (a.fuse) {
    // The wave has seen every key of the sequence: each head's output is acc / l,
    // and the pair's two heads (head n of the group is branch n & 1 of pair
    // (g nq + n) / 2) sit in lanes n and n^1 with the same d, so o_1 - lambda o_2
    // (optional V1 RMSNorm) is finished here and no records are written.
    const bool head0 = (n & 1) == 0 && n < nq;
    const int p = (g * nq + n) >> 1;
    const float lamv = head0 ? a.lam[(size_t)b * a.P + p] : 0.f;
    float x[DB][4], ss = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = o[db][i] / l;
        const float y2 = __shfl_xor(y, 1);
        x[db][i] = y - lamv * y2;
        ss += x[db][i] * x[db][i];
      }
    if (a.v1) {   // lanes n, n^16, n^32, n^48 hold the pair's D values
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[db][i] *= r;
    }
    if (head0) {
      bf16* dst = a.out + ((size_t)b * a.P + p) * D + 4 * grp;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<bf16x4*>(dst + 16 * db) = bf16x4{(bf16)x[db][0], (bf16)x[db][1], (bf16)x[db][2], (bf16)x[db][3]};
    }
    return;
  }
  // ---- partial state per query head: acc[d] (unnormalised), m, l
  if (n >= nq) return;
  float* w = rec0 + n * hstride;
#pragma unroll
  for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(w + 16 * db + 4 * grp) = o[db];
  if (grp == 0) {
    w[D] = m;
    w[D + 1] = l;
  }
}

// One wave per (b, KV head g, key range s); KV head fastest so the Hkv waves of
// one (b, key range) are dispatched together and stream neighbouring 256-byte
// pieces of the same cache rows.
template <int D, int DK>
__global__ __launch_bounds__(64) void decode_split_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char lds[DecodeLds<D, DK>::BYTES];
  const int g = blockIdx.x % a.Hkv;
  const int s = (blockIdx.x / a.Hkv) % a.S;
  const int b = blockIdx.x / (a.Hkv * a.S);
  // keys this wave reads: its range of the cache, cut to the sequence's valid
  // rows [lo, Lb) (lengths outside [1, L] are clamped, so every read stays in
  // the cache); an empty range leaves m = -inf, l = 0, which the combine skips
  const int Lb = a.seq_lens ? min(a.L, max(1, a.seq_lens[b])) : a.L;
  const int lo = a.window > 0 ? max(0, Lb - a.window) : 0;
  const int k0 = max(s * a.chunk, lo);
  const int k1 = min(Lb, s * a.chunk + a.chunk);
  const int rec = D + 4;
  attend_range<D, DK>(a, lds, b, g, k0, k1, a.ws + ((size_t)(b * a.Hq + g * a.nq) * a.S + s) * rec,
                      (size_t)a.S * rec);
}

// ---- ragged caches: an even split of the whole batch's valid rows -----------
// plan[b] = rows of the sequences before b (their windows when a window is
// set), plan[B] = all rows, plan[B + 1] = rows per range (a multiple of 32).
__global__ __launch_bounds__(1024) void decode_plan_kernel(const int* seq_lens, int B, int L, int window, int nw,
                                                           int* plan) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += 1024) {
    const int b = c0 + t;
    int len = 0;
    if (b < B) {
      const int Lb = min(L, max(1, seq_lens[b]));
      len = window > 0 ? min(Lb, window) : Lb;
    }
    part[t] = len;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {   // inclusive scan
      const int v = t >= off ? part[t - off] : 0;
      __syncthreads();
      part[t] += v;
      __syncthreads();
    }
    if (b < B) plan[b] = carry + part[t] - len;
    carry += part[1023];
    __syncthreads();
  }
  if (t == 0) {
    plan[B] = carry;
    const int per = (carry + nw - 1) / nw;
    plan[B + 1] = max(32, (per + 31) / 32 * 32);
  }
}

// One wave per (range w, KV head g): the rows [w*Kw, (w+1)*Kw) of the batch's
// concatenated valid rows, one partial record per sequence the range touches,
// in slot w + b (unique: a later range never reaches back to an earlier sequence).
// Valid rows of sequence b: its length clamped to [1, L], the last `window` of them
// with a window.
__device__ __forceinline__ int valid_rows(const Args& a, int b) {
  const int Lb = min(a.L, max(1, a.seq_lens[b]));
  return a.window > 0 ? min(Lb, a.window) : Lb;
}

// Sum over the wave of v, in every lane.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Inclusive prefix sum over the wave (lane l: v of lanes 0..l).
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

template <int D, int DK>
__global__ __launch_bounds__(64) void decode_flat_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char lds[DecodeLds<D, DK>::BYTES];
  const int g = blockIdx.x % a.Hkv;
  const int w = blockIdx.x / a.Hkv;
  const int lane = threadIdx.x;
  int* const plan = a.plan;
  int total, Kw, b, pb;   // rows of the batch, rows per range, first sequence of this range and its first row
  if (a.plan_here) {
    // the plan kernel's arithmetic, per wave: total rows, rows per range, and the
    // sequence holding row w * Kw (wave 0 of range 0 also writes the plan).  All
    // lengths are requested at once (one memory round trip), then scanned from registers.
    constexpr int NCHUNK = kPlanHereMaxB / 64;
    int v[NCHUNK];
#pragma unroll
    for (int j = 0; j < NCHUNK; ++j) v[j] = 64 * j + lane < a.B ? valid_rows(a, 64 * j + lane) : 0;
    total = 0;
#pragma unroll
    for (int j = 0; j < NCHUNK; ++j)
      if (64 * j < a.B) total += wave_sum(v[j]);
    total = __builtin_amdgcn_readfirstlane(total);
    const int nw = a.nslot - a.B;
    const int per = (total + nw - 1) / nw;
    Kw = max(32, (per + 31) / 32 * 32);
    const int x0 = w * Kw;
    const bool writer = w == 0 && g == 0;
    b = -1;
    pb = 0;
    int carry = 0;
#pragma unroll
    for (int j = 0; j < NCHUNK; ++j) {
      const int c0 = 64 * j;
      if (c0 >= a.B || (b >= 0 && !writer)) break;
      const bool in = c0 + lane < a.B;
      const int incl = wave_scan(v[j], lane);
      if (writer && in) plan[c0 + lane] = carry + incl - v[j];
      const unsigned long long hit = __ballot(in && carry + incl > x0);
      if (b < 0 && hit != 0ull) {   // wave-uniform values, kept in scalar registers
        const int l = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
        b = c0 + l;
        pb = __builtin_amdgcn_readfirstlane(carry + __shfl(incl - v[j], l));
      }
      carry = __builtin_amdgcn_readfirstlane(carry + __shfl(incl, 63));
    }
    if (writer && lane == 0) {
      plan[a.B] = total;
      plan[a.B + 1] = Kw;
    }
    if (b < 0) return;   // this range starts past the last row
  } else {
    total = plan[a.B];
    Kw = plan[a.B + 1];
    const int x0 = w * Kw;
    if (x0 >= total) return;
    int lo_b = 0, hi_b = a.B - 1;   // last b with plan[b] <= x0
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if (plan[mid] <= x0) lo_b = mid; else hi_b = mid - 1;
    }
    b = lo_b;
    pb = plan[b];
  }
  int x = w * Kw;
  const int xend = min(total, x + Kw);
  if (x >= xend) return;
  const int rec = D + 4;
  const size_t hstride = (size_t)a.nslot * rec;
  while (x < xend) {
    const int n = valid_rows(a, b);            // rows of sequence b: [pb, pb + n) of the batch
    const int seg_end = min(xend, pb + n);
    if (seg_end > x) {
      const int Lb = min(a.L, max(1, a.seq_lens[b]));
      const int lo = a.window > 0 ? max(0, Lb - a.window) : 0;
      const int k0 = lo + (x - pb);
      attend_range<D, DK>(a, lds, b, g, k0, k0 + (seg_end - x),
                          a.ws + ((size_t)(g * a.nq) * a.nslot + w + b) * rec, hstride);
      x = seg_end;
    }
    pb += n;
    ++b;
  }
}

// Merge the S partial states of NH query heads (records at base[h]): lane owns
// D/64 consecutive columns of each normalised output.  Records are requested UNR
// key ranges at a time for all NH heads before any is used, with a running
// maximum raised per batch, so up to UNR ranges cost one memory round trip (and
// the result equals a merge against the true maximum computed first).
template <int D, int NH, int UNR>
__device__ __forceinline__ void merge_heads_n(const float* const (&base)[NH], int S, int lane, float (&o)[NH][D / 64]) {
  constexpr int E = D / 64;
  const int rec = D + 4;
  float M[NH], den[NH], acc[NH][E];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    M[h] = -INFINITY;
    den[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
  }
  for (int s0 = 0; s0 < S; s0 += UNR) {
    float ms[NH][UNR], ls[NH][UNR], av[NH][UNR][E];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float* r = base[h] + min(s0 + u, S - 1) * rec;
        ms[h][u] = r[D];
        ls[h][u] = r[D + 1];
#pragma unroll
        for (int e = 0; e < E; ++e) av[h][u][e] = r[E * lane + e];
      }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float mb = M[h];
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (s0 + u < S) mb = fmaxf(mb, ms[h][u]);
      if (mb != M[h]) {   // rescale what earlier batches gathered (nothing, for the first)
        const float r = M[h] == -INFINITY ? 0.f : fast_exp2(M[h] - mb);
        den[h] *= r;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] *= r;
        M[h] = mb;
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float wgt = (s0 + u >= S || ms[h][u] == -INFINITY) ? 0.f : fast_exp2(ms[h][u] - M[h]);
        den[h] += wgt * ls[h][u];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] += wgt * av[h][u][e];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) o[h][e] = acc[h][e] / den[h];
}

// batches of 4 key ranges for short merges (the split decode of a long batch
// has 2), 16 otherwise
template <int D, int NH>
__device__ __forceinline__ void merge_heads(const float* const (&base)[NH], int S, int lane, float (&o)[NH][D / 64]) {
  if (S <= 4)
    merge_heads_n<D, NH, 4>(base, S, lane, o);
  else
    merge_heads_n<D, NH, 16>(base, S, lane, o);
}

// One wave per (b, pair): o_1 - lambda o_2 (optional V1 RMSNorm), bf16 out.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(Args a) {
  constexpr int E = D / 64;            // columns per lane
  const int bp = blockIdx.x;
  const int b = bp / a.P, p = bp % a.P;
  const int lane = threadIdx.x;
  const int rec = D + 4;
  float o[2][E];
  const float* const base[2] = {a.ws + ((size_t)b * a.Hq + 2 * p) * a.S * rec, a.ws + ((size_t)b * a.Hq + 2 * p + 1) * a.S * rec};
  merge_heads<D, 2>(base, a.S, lane, o);
  const float lamv = a.lam[(size_t)b * a.P + p];
  float x[E], ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] = o[0][e] - lamv * o[1][e];
    ss += x[e] * x[e];
  }
  if (a.v1) {
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] *= r;
  }
  bf16* dst = a.out + ((size_t)b * a.P + p) * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = (bf16)x[e];
}

// Comparison layouts: one wave per (b, head).  Standard transformer: the head's
// merged output.  DIFF V1: (branch-1 output) - lambda[b, h] (branch-2 output),
// optional per-head RMSNorm; ws2 holds the second branch's records.
template <int D>
__global__ __launch_bounds__(64) void compare_combine_kernel(Args a, const float* ws2) {
  constexpr int E = D / 64;
  const int bh = blockIdx.x;
  const int lane = threadIdx.x;
  const int rec = D + 4;
  float x[E], ss = 0.f;
  if (ws2 != nullptr) {
    float o[2][E];
    const float* const base[2] = {a.ws + (size_t)bh * a.S * rec, ws2 + (size_t)bh * a.S * rec};
    merge_heads<D, 2>(base, a.S, lane, o);
    const float lamv = a.lam[bh];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = o[0][e] - lamv * o[1][e];
  } else {
    float o[1][E];
    const float* const base[1] = {a.ws + (size_t)bh * a.S * rec};
    merge_heads<D, 1>(base, a.S, lane, o);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = o[0][e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) ss += x[e] * x[e];
  if (a.v1) {
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] *= r;
  }
  bf16* dst = a.out + (size_t)bh * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = (bf16)x[e];
}

// Ragged caches: one wave per (b, pair); the records of sequence b sit in slots
// w + b for the ranges w that touch it.
template <int D>
__global__ __launch_bounds__(64) void decode_flat_combine_kernel(Args a) {
  constexpr int E = D / 64;
  const int bp = blockIdx.x;
  const int b = bp / a.P, p = bp % a.P;
  const int lane = threadIdx.x;
  const int rec = D + 4;
  const int Kw = a.plan[a.B + 1];
  const int w0 = a.plan[b] / Kw, w1 = (a.plan[b + 1] - 1) / Kw;
  float o[2][E];
  const float* const base[2] = {a.ws + ((size_t)(2 * p) * a.nslot + w0 + b) * rec,
                                a.ws + ((size_t)(2 * p + 1) * a.nslot + w0 + b) * rec};
  merge_heads<D, 2>(base, w1 - w0 + 1, lane, o);
  const float lamv = a.lam[(size_t)b * a.P + p];
  float x[E], ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] = o[0][e] - lamv * o[1][e];
    ss += x[e] * x[e];
  }
  if (a.v1) {
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] *= r;
  }
  bf16* dst = a.out + ((size_t)b * a.P + p) * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = (bf16)x[e];
}

template <int D>
hipError_t launch(const DecodeProblem& pr, hipStream_t st) {
  Args a;
  a.q = static_cast<const bf16*>(pr.q);
  a.k = static_cast<const bf16*>(pr.k);
  a.v = static_cast<const bf16*>(pr.v);
  a.lam = pr.lam;
  a.out = static_cast<bf16*>(pr.out);
  a.ws = pr.ws;
  a.B = pr.B;
  a.L = pr.L;
  a.Hq = pr.Hq;
  a.Hkv = pr.Hkv;
  a.G = pr.Hq / (2 * pr.Hkv);
  a.P = pr.Hq / 2;
  a.S = pr.splits;
  a.chunk = pr.chunk;
  a.v1 = pr.v1_rmsnorm ? 1 : 0;
  a.eps = pr.eps;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  a.seq_lens = pr.seq_lens;
  a.window = pr.window;
  a.nq = 2 * a.G;
  a.qoff = a.koff = 0;
  a.plan = nullptr;
  a.nslot = 0;
  a.fuse = 0;
  a.plan_here = 0;
  if (pr.flat_ranges > 0) {   // ragged caches: even split of the batch's valid rows
    int* plan = reinterpret_cast<int*>(pr.ws + decode_flat_record_floats(pr.B, pr.Hq, pr.d, pr.flat_ranges));
    // up to kPlanHereMaxB sequences every wave scans the lengths itself (a few
    // loads); beyond, one plan kernel scans them once for all waves
    a.plan_here = pr.B <= kPlanHereMaxB ? 1 : 0;
    if (!a.plan_here)
      hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, st, pr.seq_lens, pr.B, pr.L, pr.window,
                         pr.flat_ranges, plan);
    a.plan = plan;
    a.nslot = pr.flat_ranges + pr.B;
    hipLaunchKernelGGL((decode_flat_kernel<D, D>), dim3((unsigned)(pr.flat_ranges * a.Hkv)), dim3(64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_flat_combine_kernel<D>, dim3((unsigned)(a.B * a.P)), dim3(64), 0, st, a);
    return hipGetLastError();
  }
  const long long blocks = (long long)a.B * a.Hkv * a.S;
  a.fuse = a.S == 1 ? 1 : 0;
  hipLaunchKernelGGL((decode_split_kernel<D, D>), dim3((unsigned)blocks), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.fuse) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)(a.B * a.P)), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_compare(const CompareProblem& pr, hipStream_t st) {
  Args a{};
  a.q = static_cast<const bf16*>(pr.q);
  a.k = static_cast<const bf16*>(pr.k);
  a.v = static_cast<const bf16*>(pr.v);
  a.lam = pr.lam;
  a.out = static_cast<bf16*>(pr.out);
  a.ws = pr.ws;
  a.B = pr.B;
  a.L = pr.L;
  a.Hq = pr.H;
  a.Hkv = pr.Hkv;
  a.S = pr.splits;
  a.chunk = pr.chunk;
  a.v1 = pr.v1_rmsnorm ? 1 : 0;
  a.eps = pr.eps;
  a.seq_lens = nullptr;
  a.window = 0;
  a.nq = pr.H / pr.Hkv;
  const long long blocks = (long long)a.B * a.Hkv * a.S;
  float* ws2 = nullptr;
  if (!pr.v1_layout) {   // standard transformer: one pass, dot products over all D dims
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    a.qoff = a.koff = 0;
    hipLaunchKernelGGL((decode_split_kernel<D, D>), dim3((unsigned)blocks), dim3(64), 0, st, a);
  } else {               // DIFF V1: one pass per branch over its half of q and k, V in full each time
    constexpr int DH = D / 2;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
    a.qoff = a.koff = 0;
    hipLaunchKernelGGL((decode_split_kernel<D, DH>), dim3((unsigned)blocks), dim3(64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    Args a2 = a;
    ws2 = pr.ws + (size_t)pr.B * pr.H * pr.splits * (D + 4);
    a2.ws = ws2;
    a2.qoff = a2.koff = DH;
    hipLaunchKernelGGL((decode_split_kernel<D, DH>), dim3((unsigned)blocks), dim3(64), 0, st, a2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compare_combine_kernel<D>, dim3((unsigned)(a.B * a.Hq)), dim3(64), 0, st, a,
                     static_cast<const float*>(ws2));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeProblem& p, hipStream_t s) {
  return p.d == 128 ? launch<128>(p, s) : launch<64>(p, s);
}

hipError_t launch_decode_compare_bf16(const CompareProblem& p, hipStream_t s) {
  return p.d == 128 ? launch_compare<128>(p, s) : launch_compare<64>(p, s);
}

}  // namespace diffattn
