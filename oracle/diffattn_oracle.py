"""fp64 CPU oracle for the Differential Attention V2 forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library; inputs come
from the seeded generator as exact bytes and are widened to fp64 here.

What it computes is the plain definition, written out (sources are the five web
pages on Differential Transformer V2; each function names its passage):

* softmax attention weights w_j = exp(q.k_j/sqrt(d)) / sum_j' exp(q.k_j'/sqrt(d)),
  stabilised by subtracting the row maximum -- lesson "差异性注意力 (V2)"
  (AI Engineering from Scratch, phase 10), section "概念 / 软max的噪音地板" and
  "建立它 / 步骤1" (stable softmax);
* the differential map DiffAttn = (A1 - lambda*A2) V with A_r = softmax(Q_r K^T/sqrt(d))
  -- same lesson, "概念 / 差异性概念" (the DiffAttn equation) and "步骤3";
  lesson "注意 变量" (phase 7, attention variants), "建立它 / 步骤4" (diff_attention);
* the causal mask, key j visible to query i iff j <= i -- attention-variants
  lesson, "建立它 / 步骤1" (causal_mask);
* the V2 head layout: query heads come in adjacent pairs inside one GQA group and
  share that group's K/V head and head dim -- dailytechsnack.ch article
  "Differential Transformer V2 soll KI-Training stabiler machen", section
  "Gemeinsamer KV-Cache statt Spezialkernel"; lambda is a per-token, per-head
  sigmoid-bounded factor -- same article, "Weniger Ausreisser und Gradientenspitzen";
* the causal sliding-window mask: key j visible to query i iff
  max(0, i - window + 1) <= j <= i (window >= the sequence length restores the
  full causal mask, window = 1 leaves each token only itself) -- attention-variants
  lesson, "建立它 / 步骤2" (swa_mask); the same lesson's "用它" notes hybrids that
  alternate DIFF attention with sliding-window layers, and serving engines are
  integrating V2 (differential-attention lesson, "用它"), hence per-sequence cache
  lengths in decode;
* V1 reference mode: lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init and a
  per-head RMSNorm after the difference -- differential-attention lesson,
  "差异性概念" and "关键词" (lambda, per-head RMSNorm).

Readings taken where the pages are silent (each is pinned by a test):
  pair p = query heads (2p, 2p+1); head 2p is the positive branch A1, head 2p+1
  is subtracted (A2); pair p reads KV head p // G with G = Hq / (2 Hkv); the
  score scale is 1/sqrt(d) with d the shared head dim; lambda is consumed as given
  (layout [B, T, P] in prefill, [B, P] in decode); decode's single query sits at
  cache position L-1 and sees all L rows; RMSNorm has no gain and eps is explicit.

The softmax is two-pass over a fully materialised score row (max, then
exp-normalise) -- deliberately not the online/tiled form the kernels use.
Rows are independent, so callers may ask for any subset of query rows.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "softmax_rows", "attention_weights", "diffattn_prefill", "diffattn_decode",
    "v1_lambda", "rmsnorm", "snr", "DEFAULT_RMS_EPS", "standard_decode", "v1_layout_decode",
]

DEFAULT_RMS_EPS = 1e-5


def softmax_rows(scores: np.ndarray) -> np.ndarray:
    """Row-wise stable softmax (max-subtract, exponentiate, normalise) in fp64.

    Differential-attention lesson, "建立它 / 步骤1": subtract the row max before
    exponentiating.  Entries equal to -inf (masked) get weight exactly 0.
    """
    s = np.asarray(scores, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _pair_heads(p: int, G: int) -> tuple[int, int, int]:
    """Pair p -> (positive head, subtracted head, KV head).  V2 layout reading."""
    return 2 * p, 2 * p + 1, p // G


def attention_weights(q_rows: np.ndarray, k: np.ndarray, row_pos: np.ndarray,
                      causal: bool, window: int = 0) -> np.ndarray:
    """Softmax(q k^T / sqrt(d)) for the given query rows of one head.

    q_rows [R, d] (fp64), k [N, d] (fp64), row_pos [R] = position of each query
    row in the key sequence.  Causal: key j visible iff j <= row_pos (the
    attention-variants lesson's causal_mask); window > 0 (causal only) further
    requires j >= row_pos - window + 1 (its swa_mask).  Returns A [R, N].
    """
    d = q_rows.shape[-1]
    s = (q_rows @ k.T) / math.sqrt(d)
    j = np.arange(k.shape[0])[None, :]
    if causal:
        s = np.where(j <= row_pos[:, None], s, -np.inf)
    if window > 0:
        assert causal, "the sliding window is a causal mask"
        s = np.where(j >= row_pos[:, None] - window + 1, s, -np.inf)
    return softmax_rows(s)


def rmsnorm(x: np.ndarray, eps: float = DEFAULT_RMS_EPS) -> np.ndarray:
    """V1 per-head RMSNorm over the head dim, no gain: x / sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def v1_lambda(lq1, lk1, lq2, lk2, lambda_init: float = 0.8) -> np.ndarray:
    """V1 re-parameterised lambda per pair: exp(lq1.lk1) - exp(lq2.lk2) + lambda_init.

    Differential-attention lesson, "差异性概念" (lambda formula; lambda_init is a
    small positive number such as 0.8).  Inputs [P, d_lambda]; returns [P] fp64.
    """
    a = np.sum(np.asarray(lq1, np.float64) * np.asarray(lk1, np.float64), axis=-1)
    b = np.sum(np.asarray(lq2, np.float64) * np.asarray(lk2, np.float64), axis=-1)
    return np.exp(a) - np.exp(b) + float(lambda_init)


def diffattn_prefill(q, k, v, lam, causal: bool = True, v1_rmsnorm: bool = False,
                     eps: float = DEFAULT_RMS_EPS, rows=None, row_block: int = 512,
                     window: int = 0) -> np.ndarray:
    """Differential attention over a whole sequence (prefill), fp64.

    q [B, T, Hq, d], k/v [B, T, Hkv, d], lam [B, T, P] (any real numbers, used as
    given), all already widened to fp64 (or castable exactly).  For each batch b,
    pair p and query row i:
        o_r = softmax(q[b,i,h_r] . k[b,:,g]^T / sqrt(d)) @ v[b,:,g]   (r = 1, 2)
        x   = o_1 - lam[b,i,p] * o_2
        out = x                      (V2)   or   rmsnorm(x, eps)   (V1 mode)
    Returns out [B, R, P, d] for the requested rows (all T rows by default).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    assert Hq % (2 * Hkv) == 0, "Hq must be a multiple of 2*Hkv"
    G = Hq // (2 * Hkv)
    P = Hq // 2
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, rows.size, P, d), dtype=np.float64)
    for b in range(B):
        for p in range(P):
            h1, h2, g = _pair_heads(p, G)
            kk = k[b, :, g, :]
            vv = v[b, :, g, :]
            for r0 in range(0, rows.size, row_block):
                rr = rows[r0:r0 + row_block]
                n = int(rr.max()) + 1 if causal else T
                a1 = attention_weights(q[b, rr, h1, :], kk[:n], rr, causal, window)
                a2 = attention_weights(q[b, rr, h2, :], kk[:n], rr, causal, window)
                x = a1 @ vv[:n] - lam[b, rr, p][:, None] * (a2 @ vv[:n])
                out[b, r0:r0 + rr.size, p, :] = rmsnorm(x, eps) if v1_rmsnorm else x
    return out


def diffattn_decode(q, k_cache, v_cache, lam, v1_rmsnorm: bool = False,
                    eps: float = DEFAULT_RMS_EPS, batches=None, pairs=None,
                    seq_lens=None, window: int = 0) -> np.ndarray:
    """Differential attention for one new query token per sequence over a KV cache.

    q [B, Hq, d], k_cache/v_cache [B, L, Hkv, d], lam [B, P].  Sequence b holds
    seq_lens[b] valid cache rows (all L if None); its query is the token at
    position seq_lens[b]-1 and sees rows max(0, seq_lens[b] - window) ..
    seq_lens[b]-1 (all of them if window = 0).  Same per-pair arithmetic as
    ``diffattn_prefill``.  Returns out [len(batches), len(pairs), d].
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    assert Hq % (2 * Hkv) == 0
    G = Hq // (2 * Hkv)
    P = Hq // 2
    batches = np.arange(B) if batches is None else np.asarray(batches)
    pairs = np.arange(P) if pairs is None else np.asarray(pairs)
    out = np.empty((batches.size, pairs.size, d), dtype=np.float64)
    for bi, b in enumerate(batches):
        kv_cache = {}
        for pi, p in enumerate(pairs):
            h1, h2, g = _pair_heads(int(p), G)
            if g not in kv_cache:
                Lb = k_cache.shape[1] if seq_lens is None else int(seq_lens[b])
                lo = max(0, Lb - window) if window > 0 else 0
                kv_cache = {g: (np.asarray(k_cache[b, lo:Lb, g, :], dtype=np.float64),
                                np.asarray(v_cache[b, lo:Lb, g, :], dtype=np.float64))}
            kk, vv = kv_cache[g]
            qq = np.asarray(q[b, [h1, h2], :], dtype=np.float64)
            a = attention_weights(qq, kk, np.array([kk.shape[0] - 1] * 2), causal=False)
            o = a @ vv
            x = o[0] - float(lam[b, p]) * o[1]
            out[bi, pi] = rmsnorm(x[None], eps)[0] if v1_rmsnorm else x
    return out


def standard_decode(q, k_cache, v_cache, batches=None) -> np.ndarray:
    """Baseline transformer decode: one softmax per query head, GQA.

    q [B, H, d], k_cache/v_cache [B, L, Hkv, d]; head h reads KV head h // (H / Hkv);
    out[b, h] = softmax(q k^T / sqrt(d)) v over all L rows (the standard attention
    of the differential-attention lesson, "软max的噪音地板").  Returns [len(batches), H, d].
    """
    q = np.asarray(q)
    B, H, d = q.shape
    Hkv = k_cache.shape[2]
    assert H % Hkv == 0
    batches = np.arange(B) if batches is None else np.asarray(batches)
    out = np.empty((batches.size, H, d))
    for bi, b in enumerate(batches):
        for g in range(Hkv):
            kk = np.asarray(k_cache[b, :, g], np.float64)
            vv = np.asarray(v_cache[b, :, g], np.float64)
            hs = np.arange(g * (H // Hkv), (g + 1) * (H // Hkv))
            a = attention_weights(np.asarray(q[b, hs], np.float64), kk, np.zeros(hs.size, np.int64), causal=False)
            out[bi, hs] = a @ vv
    return out


def v1_layout_decode(q, k_cache, v_cache, lam, v1_rmsnorm: bool = True, eps: float = DEFAULT_RMS_EPS,
                     batches=None) -> np.ndarray:
    """DIFF V1 decode: each head's query and key are split into halves (Q1, Q2),
    (K1, K2) of d/2 dims, A_r = softmax(Q_r K_r^T / sqrt(d/2)), out = (A1 - lam A2) V
    with the head's full d-dim V, then the per-head RMSNorm -- differential-attention
    lesson, "差异性概念" (split Q, K into two halves; the DiffAttn equation) and
    "V1 vs V2" (V1 halves the per-branch head dim and applies per-head RMSNorm).
    The scale uses the dot-product dimension d/2 (reading: the equation's d is the
    dimension of the vectors in the dot product, as in the noise-floor formula).

    q [B, H, d], k_cache/v_cache [B, L, Hkv, d], lam [B, H].  Returns [len(batches), H, d].
    """
    q = np.asarray(q)
    B, H, d = q.shape
    Hkv = k_cache.shape[2]
    h2 = d // 2
    batches = np.arange(B) if batches is None else np.asarray(batches)
    out = np.empty((batches.size, H, d))
    for bi, b in enumerate(batches):
        for g in range(Hkv):
            kk = np.asarray(k_cache[b, :, g], np.float64)
            vv = np.asarray(v_cache[b, :, g], np.float64)
            for h in range(g * (H // Hkv), (g + 1) * (H // Hkv)):
                qh = np.asarray(q[b, h], np.float64)
                z = np.zeros(1, np.int64)
                a1 = attention_weights(qh[None, :h2], kk[:, :h2], z, causal=False)
                a2 = attention_weights(qh[None, h2:], kk[:, h2:], z, causal=False)
                x = (a1 - float(lam[b, h]) * a2) @ vv
                out[bi, h] = (rmsnorm(x, eps) if v1_rmsnorm else x)[0]
    return out


def snr(weights: np.ndarray, signal: np.ndarray, visible: int) -> float:
    """Signal-to-noise ratio of one attention row.

    Differential-attention lesson, "关键词" (signal-to-noise ratio): weight on the
    signal positions divided by the average weight on unrelated positions.
    Reading: mean weight over the signal set / signed mean weight over the other
    visible positions [0, visible).
    """
    w = np.asarray(weights, dtype=np.float64)[:visible]
    mask = np.zeros(visible, dtype=bool)
    mask[np.asarray(signal)] = True
    return float(np.mean(w[mask]) / np.mean(w[~mask]))
