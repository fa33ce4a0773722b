"""fp64 CPU oracle for the backward pass of Differential Attention V2 (prefill).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/`` and ``bench.py``'s CPU-baseline leg may use it.  It
shares no code with the HIP library.

The pages give the forward map only (differential-attention lesson "差异性注意力
(V2)", section "差异性概念": DiffAttn = (A1 - lambda A2) V with
A_r = softmax(Q_r K^T / sqrt(d)); dailytechsnack.ch article, section "Gemeinsamer
KV-Cache statt Spezialkernel": the two heads of a pair share their GQA group's
K/V; section "Weniger Ausreisser und Gradientenspitzen": lambda is a per-token,
per-head factor and the method is about training stability).  The backward is
the derivative of that map, written out with the chain rule, densely, per
(batch, pair):

    x      = O_1 - lam * O_2,  O_r = A_r V             (V1 mode: y = x / rms(x))
    dx     = dout                                      (V1: dx = (dy - y mean(dy y)) / rms)
    dO_1   = dx,   dO_2 = -lam dx,   dlam = -sum_c dx O_2
    dA_r   = dO_r V^T
    dS_r   = A_r * (dA_r - rowsum(A_r * dA_r))         (softmax Jacobian)
    dQ_r   = dS_r K / sqrt(d)
    dK    += dS_r^T Q_r / sqrt(d)      (summed over every head of the group)
    dV    += A_r^T dO_r

S_r is the scaled score matrix with the causal mask (j <= i) applied before the
softmax; masked entries get weight and gradient exactly 0.  Everything is
materialised (T x T per head) in fp64; there is no tiling, no online softmax
and no recomputation.

``prefill_saved`` returns what a training forward keeps for the backward: the
output, O_2 (the subtracted branch's attention output) and the natural-log
log-sum-exp of each row's scaled scores, per query head.

Pins (tests/test_backward_oracle.py): central finite differences of
L = sum(dout * out) on tiny shapes (V2 and V1, causal and not), an independent
torch fp64 autograd implementation of the forward, lambda = 0 and Q2 = Q1 special
cases, and the shift-invariance identities sum_j dK_j = 0 and
sum_j dV_j = sum over pairs and rows of (1 - lam) dx.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["prefill_saved", "diffattn_prefill_bwd"]


def _scores(qh: np.ndarray, kk: np.ndarray, causal: bool) -> np.ndarray:
    """Scaled scores q k^T / sqrt(d) of one head, causal entries j > i set to -inf."""
    d = qh.shape[-1]
    s = (qh @ kk.T) / math.sqrt(d)
    if causal:
        T = s.shape[0]
        s = np.where(np.arange(T)[None, :] <= np.arange(T)[:, None], s, -np.inf)
    return s


def _softmax(s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Row softmax of s and the natural-log log-sum-exp of each row."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def _f64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def prefill_saved(q, k, v, lam, causal: bool = True):
    """Forward values a training step keeps: (out [B,T,P,d], o2 [B,T,P,d], lse [B,T,Hq]).

    out = A_1 V - lam A_2 V (V2), o2 = A_2 V, lse[b,i,h] = log sum_j exp(s_ij) over
    the visible keys of row i of head h (natural log, scaled scores).
    """
    q, k, v, lam = _f64(q, k, v, lam)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // (2 * Hkv)
    P = Hq // 2
    out = np.empty((B, T, P, d))
    o2 = np.empty((B, T, P, d))
    lse = np.empty((B, T, Hq))
    for b in range(B):
        for p in range(P):
            g = p // G
            a1, lse[b, :, 2 * p] = _softmax(_scores(q[b, :, 2 * p], k[b, :, g], causal))
            a2, lse[b, :, 2 * p + 1] = _softmax(_scores(q[b, :, 2 * p + 1], k[b, :, g], causal))
            o1 = a1 @ v[b, :, g]
            o2[b, :, p] = a2 @ v[b, :, g]
            out[b, :, p] = o1 - lam[b, :, p][:, None] * o2[b, :, p]
    return out, o2, lse


def diffattn_prefill_bwd(q, k, v, lam, dout, causal: bool = True, v1_rmsnorm: bool = False,
                         eps: float = 1e-5, groups=None):
    """Gradients (dq, dk, dv, dlam) of L = sum(dout * out) for the prefill map.

    q [B,T,Hq,d], k/v [B,T,Hkv,d], lam [B,T,P], dout [B,T,P,d].  Returns fp64
    dq [B,T,Hq,d], dk/dv [B,T,Hkv,d], dlam [B,T,P].  ``groups``: optional list of
    KV heads to compute (the other entries are left as NaN), for large shapes.
    """
    q, k, v, lam, dout = _f64(q, k, v, lam, dout)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    assert Hq % (2 * Hkv) == 0
    G = Hq // (2 * Hkv)
    P = Hq // 2
    sc = 1.0 / math.sqrt(d)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    dlam = np.full(lam.shape, np.nan)
    groups = range(Hkv) if groups is None else groups
    for b in range(B):
        for g in groups:
            kk, vv = k[b, :, g], v[b, :, g]
            dk_g = np.zeros((T, d))
            dv_g = np.zeros((T, d))
            for p in range(g * G, (g + 1) * G):
                h1, h2 = 2 * p, 2 * p + 1
                a1, _ = _softmax(_scores(q[b, :, h1], kk, causal))
                a2, _ = _softmax(_scores(q[b, :, h2], kk, causal))
                o1, o2 = a1 @ vv, a2 @ vv
                lp = lam[b, :, p][:, None]
                dy = dout[b, :, p]
                if v1_rmsnorm:
                    x = o1 - lp * o2
                    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
                    y = x / r
                    dx = (dy - y * np.mean(dy * y, axis=-1, keepdims=True)) / r
                else:
                    dx = dy
                dlam[b, :, p] = -np.sum(dx * o2, axis=-1)
                for h, a, do in ((h1, a1, dx), (h2, a2, -lp * dx)):
                    da = do @ vv.T
                    ds = a * (da - np.sum(a * da, axis=-1, keepdims=True))
                    dq[b, :, h] = (ds @ kk) * sc
                    dk_g += (ds.T @ q[b, :, h]) * sc
                    dv_g += a.T @ do
            dk[b, :, g] = dk_g
            dv[b, :, g] = dv_g
    return dq, dk, dv, dlam
