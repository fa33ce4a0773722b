/*
 * libdiffattn -- Differential Attention V2 forward pass for AMD MI355X (gfx950).
 *
 * The operation (sources: the web pages on Differential Transformer V2):
 *   For each batch b, differential pair p and query token i, with the pair's two
 *   query heads h1 = 2p and h2 = 2p+1 sharing one K/V head g = p / G
 *   (G = Hq / (2*Hkv) pairs per KV head):
 *       A_r = softmax(q[b,i,h_r] . K[b,:,g]^T / sqrt(d))     r = 1, 2
 *       out[b,i,p,:] = A_1 V[b,:,g] - lambda[b,i,p] * A_2 V[b,:,g]
 *   -- the differential map (A1 - lambda A2) V: lesson "差异性注意力 (V2)"
 *   (AI Engineering from Scratch, phase 10), section "概念 / 差异性概念", computed
 *   as A1 V - lambda A2 V; the V2 head layout (query heads doubled, adjacent query
 *   heads of one GQA group share K/V and the head dim, KV heads unchanged): article
 *   "Differential Transformer V2 soll KI-Training stabiler machen"
 *   (dailytechsnack.ch), section "Gemeinsamer KV-Cache statt Spezialkernel";
 *   lambda per token and head, sigmoid-bounded: same article, section "Weniger
 *   Ausreisser und Gradientenspitzen"; causal mask j <= i: lesson "注意 变量"
 *   (phase 7, attention variants), "建立它 / 步骤1".
 *   V1 reference mode (flag DIFFATTN_FLAG_V1_RMSNORM): out = x / sqrt(mean_c x_c^2 + eps)
 *   per output head, applied after the difference -- differential-attention lesson,
 *   "关键词" (per-head RMSNorm).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory owned by the caller; the library
 *     never allocates, frees, or keeps them, and never synchronises.  Work is
 *     enqueued on `stream` (a hipStream_t; NULL = the legacy default stream) and
 *     completes asynchronously (the backward forks part of it onto a side stream
 *     of `stream` and joins it back, see Thread safety).  Outputs must not alias
 *     inputs.
 *   - Element types: dtype DIFFATTN_BF16 (q/k/v/out are bf16, fp32 accumulation)
 *     or DIFFATTN_FP32 (q/k/v/out are fp32).  lambda is always fp32.
 *   - Layouts are row-major with the head dim fastest ("BTHD").
 *   - Supported: d in {64, 128}; Hq a multiple of 2*Hkv; G = Hq/(2*Hkv) <= 8;
 *     Hq*d <= 2^22 per token (tile rows are addressed with 32-bit offsets);
 *     larger head counts return DIFFATTN_ERR_UNSUPPORTED.
 *   - Errors: arguments are validated on the host before anything is enqueued;
 *     on error nothing is written and a nonzero diffattn_status_t is returned.
 *     Device pointers must be non-NULL and 16-byte aligned.  A failed kernel
 *     launch returns DIFFATTN_ERR_HIP; faults inside a kernel surface at the
 *     caller's next synchronisation, as with any HIP call.
 *   - Thread safety: concurrent calls are safe, with two pieces of device state
 *     the library keeps: the fixed scratch of diffattn_decode_fwd_noalloc (see
 *     there), and the work queues of long prefills.  A prefill (plain, V1 mode or
 *     training forward; not the sliding window) with at least 8 token blocks per
 *     CU (e.g. T >= 8192 at Hkv = 8, G = 4) runs as one workgroup per CU taking its
 *     blocks from queues in a static device array of 1024 slots, one slot per call,
 *     handed out round-robin; the call's last workgroup empties its slot again.
 *     So at most 1024 such calls may be in flight on one device at once, and two
 *     instances of one captured graph that contains such a call must not run
 *     concurrently (they share its slot).  The backward also keeps state: it runs
 *     its row statistics and dQ kernel on a side stream of `stream` (one per
 *     stream, on that stream's device, with three events, created on its first
 *     call on that stream outside graph capture and kept until the process ends;
 *     at most 64 of them), forked off and joined back with events, so work
 *     enqueued on `stream` after the call still sees every output; a capture of
 *     `stream` holds the fork and the join.  A stream whose first backward call
 *     is captured, and every stream past the 64th, runs it serially instead.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIFFATTN_OK = 0,
  DIFFATTN_ERR_INVALID_ARG = 1, /* NULL/misaligned pointer, non-positive size, bad ratio, overflow */
  DIFFATTN_ERR_UNSUPPORTED = 2, /* valid but not built: head dim, group size, dtype */
  DIFFATTN_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  DIFFATTN_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} diffattn_status_t;

typedef enum { DIFFATTN_BF16 = 0, DIFFATTN_FP32 = 1 } diffattn_dtype_t;

/* V1 reference mode: per-head RMSNorm (no gain) of the differential output. */
#define DIFFATTN_FLAG_V1_RMSNORM 0x1u

/*
 * Prefill: differential attention over a whole sequence.
 *   q      device [B, T, Hq, d]   (dtype)
 *   k, v   device [B, T, Hkv, d]  (dtype)
 *   lambda device [B, T, P] fp32, P = Hq/2; used as given (V2 callers pass
 *          sigmoid outputs; any real value is accepted, as V1's lambda may be < 0)
 *   out    device [B, T, P, d]    (dtype), fully overwritten
 *   causal nonzero: key j visible to query i iff j <= i; zero: all T keys visible
 *   flags  0 or DIFFATTN_FLAG_V1_RMSNORM; rms_eps used only with that flag (> 0)
 * Returns a diffattn_status_t.
 */
int diffattn_prefill_fwd(const void* q, const void* k, const void* v, const float* lambda, void* out,
                         int B, int T, int Hq, int Hkv, int d, int causal,
                         int dtype, unsigned flags, float rms_eps, void* stream);

/*
 * Prefill with a causal sliding window (attention-variants lesson, "建立它 /
 * 步骤2", swa_mask): key j is visible to query i iff max(0, i - window + 1) <= j
 * <= i.  Key tiles wholly before a query block's window are neither copied nor
 * read.  window = 0 or window >= T is the plain causal prefill.
 *   q, k, v, lambda, out, flags, rms_eps   as diffattn_prefill_fwd; bf16 only
 *   window  >= 0
 * Returns a diffattn_status_t (fp32 -> DIFFATTN_ERR_UNSUPPORTED).
 */
int diffattn_prefill_fwd_window(const void* q, const void* k, const void* v, const float* lambda, void* out,
                                int B, int T, int Hq, int Hkv, int d, int window, int dtype, unsigned flags,
                                float rms_eps, void* stream);

/*
 * Training forward (bf16, V2 map, no RMSNorm): the prefill above, plus what the
 * backward needs -- the subtracted branch's output and each row's log-sum-exp.
 *   q, k, v, lambda, out, causal   as diffattn_prefill_fwd (bf16 only)
 *   o2     device [B, T, P, d] bf16: A_2 V for every pair (head 2p+1's attention
 *          output before lambda), fully overwritten
 *   lse    device [B, T, Hq] fp32: log sum_j exp(q_h . k_j / sqrt(d)) over the
 *          visible keys of each row and query head (natural log)
 * Returns a diffattn_status_t.
 */
int diffattn_prefill_fwd_train(const void* q, const void* k, const void* v, const float* lambda, void* out,
                               void* o2, float* lse, int B, int T, int Hq, int Hkv, int d, int causal,
                               void* stream);

/*
 * Backward of the prefill map for training (the pages report pretraining
 * results and motivate V2 by training stability: dailytechsnack.ch article,
 * section "Weniger Ausreisser und Gradientenspitzen").  Gradients of
 * L = sum(dout * out) with out = A_1 V - lambda A_2 V (differential-attention
 * lesson "差异性注意力 (V2)", section "差异性概念"), bf16 V2 map only.
 *   q, k, v, lambda, causal   the forward's inputs
 *   out, o2, lse              the training forward's outputs for those inputs
 *   dout   device [B, T, P, d] bf16
 *   dq     device [B, T, Hq, d] bf16 (out)      dk, dv  device [B, T, Hkv, d] bf16 (out)
 *   dlambda device [B, T, P] fp32 (out)
 *   workspace  device scratch >= diffattn_prefill_bwd_workspace_bytes(...) bytes,
 *              16-byte aligned; contents on entry are ignored
 * Outputs are fully overwritten and must not alias any input.  dk and dv are
 * summed over query chunks with fp32 atomics, so their last bits can vary from
 * run to run; dq and dlambda are deterministic.
 * Returns a diffattn_status_t; T > 2^26 returns DIFFATTN_ERR_UNSUPPORTED, and
 * sizes whose dK/dV grid (growing with T^2) would exceed 2^31-1 workgroups return
 * DIFFATTN_ERR_HIP with nothing enqueued.
 */
int diffattn_prefill_bwd(const void* q, const void* k, const void* v, const float* lambda, const void* out,
                         const void* o2, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         float* dlambda, int B, int T, int Hq, int Hkv, int d, int causal, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Workspace bytes diffattn_prefill_bwd needs (host only; 0 on invalid sizes). */
size_t diffattn_prefill_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d);

/*
 * Decode: one new query token per sequence against a contiguous KV cache that
 * already holds that token (the query sits at position L-1 and sees all L rows).
 * Each cache byte is read from HBM once per KV-head group (both heads of every
 * pair in the group share it), split over `num_splits` key ranges whose partial
 * softmax states are merged by a second kernel; with one range per sequence the
 * first kernel finishes the output itself and the workspace is not touched.
 *   q        device [B, Hq, d]       (dtype)
 *   k_cache  device [B, L, Hkv, d]   (dtype)
 *   v_cache  device [B, L, Hkv, d]   (dtype)
 *   lambda   device [B, P] fp32
 *   out      device [B, P, d]        (dtype), fully overwritten
 *   num_splits  key-range splits per (b, KV head); 0 = library's choice
 *               (diffattn_decode_num_splits); clamped to [1, ceil(L/32)]
 *   workspace   device scratch, >= diffattn_decode_workspace_bytes(...) bytes,
 *               16-byte aligned; contents on entry are ignored
 * Returns a diffattn_status_t.
 */
int diffattn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, const float* lambda,
                        void* out, int B, int L, int Hq, int Hkv, int d,
                        int dtype, unsigned flags, float rms_eps, int num_splits,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and kernels as diffattn_decode_fwd
 * minus the workspace: the key-range records live in a fixed device array of
 * DIFFATTN_NOALLOC_SCRATCH_BYTES bytes inside the library, one per device, held
 * from the first call on that device until the process ends.  The call never
 * allocates or frees device memory.
 *   - Problems whose records need more than DIFFATTN_NOALLOC_SCRATCH_BYTES
 *     (B * Hq * splits * (d + 4) * 4 bytes when splits > 1) return
 *     DIFFATTN_ERR_WORKSPACE with nothing enqueued; use diffattn_decode_fwd.
 *   - Every call on a device shares that device's array: calls that overlap in
 *     time on one device (different streams, or threads without ordering) race
 *     and may corrupt each other's output.  Calls ordered on one stream are safe.
 *   - The array keeps the last call's records; nothing in it needs to start at
 *     zero, since each call writes every record it reads.
 *   - The first call on a device looks up the array's device address (a HIP
 *     runtime call, DIFFATTN_ERR_HIP on failure) and must run with that device
 *     current; make that first call outside graph capture.
 * Returns a diffattn_status_t.
 */
#define DIFFATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int diffattn_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache, const float* lambda,
                                void* out, int B, int L, int Hq, int Hkv, int d,
                                int dtype, unsigned flags, float rms_eps, int num_splits, void* stream);

/*
 * Decode over ragged caches: sequence b holds seq_lens[b] valid rows of a cache
 * allocated for L (its query is the token at row seq_lens[b]-1), and with
 * window > 0 only its last `window` rows are visible.  Serving engines batch
 * sequences of different lengths this way (the differential-attention lesson,
 * "用它", notes V2 integration into serving engines).  With seq_lens, the
 * batch's valid rows are split evenly over num_splits ranges per KV head (0 =
 * library's choice, about one wave per SIMD) by a plan computed on the device,
 * so long and short sequences cost in proportion to their rows.
 *   seq_lens  device int32 [B], values in [1, L] (values outside are clamped),
 *             or NULL: every sequence has L rows (then as diffattn_decode_fwd)
 *   window    >= 0, 0 = every valid row visible
 *   workspace >= diffattn_decode_varlen_workspace_bytes(...) bytes, 16-byte aligned
 *   other arguments as diffattn_decode_fwd; bf16 only
 * Returns a diffattn_status_t (fp32 -> DIFFATTN_ERR_UNSUPPORTED).
 */
int diffattn_decode_fwd_varlen(const void* q, const void* k_cache, const void* v_cache, const float* lambda,
                               void* out, const int* seq_lens, int B, int L, int Hq, int Hkv, int d, int window,
                               int dtype, unsigned flags, float rms_eps, int num_splits, void* workspace,
                               size_t workspace_bytes, void* stream);
/* Workspace bytes for diffattn_decode_fwd_varlen (host only; 0 on invalid sizes). */
size_t diffattn_decode_varlen_workspace_bytes(int B, int L, int Hq, int Hkv, int d, int num_splits);

/*
 * Decode in the layouts V2 is measured against (differential-attention lesson,
 * section "V1 vs V2": V1 halves the per-branch head dim and must load the value
 * cache twice per decode step, once per softmax branch, so it decodes slower
 * than a standard transformer; V2 loads the KV cache once and matches it).
 * Both use the same cache geometry as diffattn_decode_fwd and its split plan.
 *
 * diffattn_decode_standard: standard transformer decode, H query heads over Hkv
 * KV heads (GQA), out[b,h] = softmax(q_h k^T / sqrt(d)) v.
 *   q device [B, H, d] bf16, caches [B, L, Hkv, d] bf16, out [B, H, d] bf16
 * diffattn_decode_v1_layout: DIFF V1 decode; head h's q and k rows split into
 * halves (q1 | q2), (k1 | k2) of d/2, A_r = softmax(q_r k_r^T / sqrt(d/2)),
 * out = (A_1 - lambda[b,h] A_2) v with the full d-dim v, then the per-head
 * RMSNorm when flags has DIFFATTN_FLAG_V1_RMSNORM.  Runs one pass per branch,
 * each reading its half of K and all of V.
 *   lambda device [B, H] fp32
 * Constraints: H % Hkv == 0, H / Hkv <= 16, d in {64, 128}; bf16 only.
 * workspace >= diffattn_decode_compare_workspace_bytes(...) bytes, 16-byte aligned.
 * Return a diffattn_status_t.
 */
int diffattn_decode_standard(const void* q, const void* k_cache, const void* v_cache, void* out, int B, int L, int H,
                             int Hkv, int d, int num_splits, void* workspace, size_t workspace_bytes, void* stream);
int diffattn_decode_v1_layout(const void* q, const void* k_cache, const void* v_cache, const float* lambda,
                              void* out, int B, int L, int H, int Hkv, int d, unsigned flags, float rms_eps,
                              int num_splits, void* workspace, size_t workspace_bytes, void* stream);
/* Workspace bytes for either comparison decode (host only; 0 on invalid sizes). */
size_t diffattn_decode_compare_workspace_bytes(int B, int L, int H, int Hkv, int d, int num_splits);

/* Split count the library picks for a decode problem (host only; no GPU call).
 * Returns 0 on invalid sizes. */
int diffattn_decode_num_splits(int B, int L, int Hq, int Hkv, int d);

/* Workspace bytes diffattn_decode_fwd needs for these sizes and num_splits
 * (0 = library's choice).  Host only; returns 0 on invalid sizes. */
size_t diffattn_decode_workspace_bytes(int B, int L, int Hq, int Hkv, int d, int num_splits);

/*
 * V1 reference-mode lambda, one value per differential pair, broadcast over rows:
 *   lambda_out[r, p] = exp(lq1[p].lk1[p]) - exp(lq2[p].lk2[p]) + lambda_init
 * (differential-attention lesson, "概念 / 差异性概念": the lambda re-parameterisation;
 * lambda_init a small positive number such as 0.8).
 *   lq1, lk1, lq2, lk2  device [P, d_lambda] fp32
 *   lambda_out          device [rows, P] fp32 (rows = B*T for prefill, B for decode)
 * Returns a diffattn_status_t.
 */
int diffattn_v1_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                       float lambda_init, float* lambda_out, int P, int d_lambda, int rows,
                       void* stream);

/*
 * lambda producer: V2 projects a sigmoid-bounded lambda for every token and head
 * (dailytechsnack.ch article, section "Weniger Ausreisser und Gradientenspitzen"):
 *   lambda_out[r, p] = 1 / (1 + exp(-(x[r] . w_lambda[p])))
 *   x          device [rows, d_model] bf16 (rows = B*T: the attention block's input)
 *   w_lambda   device [P, d_model] bf16, one projection vector per pair
 *   lambda_out device [rows, P] fp32 -- the `lambda` input of the prefill calls
 * Constraints: d_model % 512 == 0, d_model <= 2^24, P % 16 == 0, P <= 64.
 * Returns a diffattn_status_t.
 */
int diffattn_lambda_proj(const void* x, const void* w_lambda, float* lambda_out, int rows, int d_model, int P,
                         void* stream);

/*
 * Output projection O_W: the P*d wide differential output projected back to the
 * model width (differential-attention lesson, section "V1 vs V2").
 *   y [rows, out_dim] = attn [rows, in_dim] @ w_o [in_dim, out_dim], all bf16
 *   row-major, fp32 accumulation; attn is the prefill's out viewed as [B*T, P*d].
 * A dense GEMM on bf16 MFMA (the library's own kernel, 256 x 256 output tiles);
 * like every entry point here it allocates nothing.
 * Constraints: in_dim % 32 == 0 and out_dim % 8 == 0 (in_dim = P*d always is a
 * multiple of 64), both <= 2^24; otherwise DIFFATTN_ERR_UNSUPPORTED.
 * Returns a diffattn_status_t.
 */
int diffattn_output_proj(const void* attn, const void* w_o, void* y, int rows, int in_dim, int out_dim,
                         void* stream);

/* Static description of a status code (never NULL). */
const char* diffattn_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int diffattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
