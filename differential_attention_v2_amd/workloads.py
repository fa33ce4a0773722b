"""Seeded synthetic inputs for the Differential Attention V2 forward pass.

This module only *draws* inputs: normal samples, their rounding to the input
dtype, the sigmoid that maps a logit to a post-sigmoid lambda, and the planting
recipe of the signal-plus-noise workload.  It holds none of the attention
arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path consume the
exact same bytes from here without sharing any computation.

Layouts (row-major, head dim fastest):
  prefill  q [B, T, Hq, d], k/v [B, T, Hkv, d], lambda [B, T, P] (P = Hq // 2)
  decode   q [B, Hq, d], k/v cache [B, L, Hkv, d], lambda [B, P]
bf16 tensors are returned as ``uint16`` bit patterns; ``bf16_to_f32`` widens them.

Generation is chunked along the leading (batch x sequence) axis, one independent
``SeedSequence`` child per fixed-size chunk, so the bytes do not depend on the
number of threads used, and chunks are drawn in parallel (numpy's Generator
releases the GIL while filling an array).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# Elements per independently seeded chunk.  Part of the input definition:
# changing it changes every drawn value.
_CHUNK_ELEMS = 1 << 22

# Stream indices under each workload seed.
_S_Q, _S_K, _S_V, _S_LAM, _S_PLAN, _S_V1 = range(6)


# ----------------------------------------------------------------------------
# dtype helpers
# ----------------------------------------------------------------------------
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even); returns uint16 bit patterns.

    Inputs here are finite normals, so the NaN special case is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of an input tensor as handed to the GPU."""
    if dtype == "bf16":
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# chunked, seeded normal draws
# ----------------------------------------------------------------------------
def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal(seed_seq: np.random.SeedSequence, n: int, scale: float, dtype: str) -> np.ndarray:
    """n normals N(0, scale^2) as fp32 (dtype 'fp32') or bf16 bits (dtype 'bf16')."""
    nchunks = max(1, -(-n // _CHUNK_ELEMS))
    children = seed_seq.spawn(nchunks)
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fill(i: int) -> None:
        lo = i * _CHUNK_ELEMS
        hi = min(n, lo + _CHUNK_ELEMS)
        x = np.random.default_rng(children[i]).standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[lo:hi] = f32_to_bf16(x) if dtype == "bf16" else x

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _sigmoid_f32(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float32)
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-z))).astype(np.float32)


# ----------------------------------------------------------------------------
# workload definitions
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "prefill" | "decode"
    dtype: str         # "bf16" | "fp32"
    B: int
    T: int             # sequence length (prefill) or KV-cache length L (decode)
    Hq: int
    Hkv: int
    d: int
    qkv_scale: float = 1.0
    causal: bool = True
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def P(self) -> int:
        return self.Hq // 2

    @property
    def G(self) -> int:
        return self.Hq // (2 * self.Hkv)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    # Algorithmic work, counted as the path defines it.
    def prefill_flops(self, window: int = 0) -> float:
        """4*d flops per visible (query, key, head): QK^T and PV, 2*d each.  With a
        causal sliding window, query i sees min(i + 1, window) keys."""
        T = self.T
        if window > 0 and window < T:
            pairs = window * (window + 1) / 2 + (T - window) * window
        else:
            pairs = T * (T + 1) / 2 if self.causal else T * T
        return 4.0 * self.d * self.Hq * self.B * pairs

    def prefill_bwd_flops(self) -> float:
        """8*d flops per visible (query, key, head): the four gradient products
        dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q (2*d each), without the
        score recomputation."""
        return 2.0 * self.prefill_flops()

    def decode_kv_bytes(self) -> float:
        """K and V cache bytes, each byte counted once per KV-head group."""
        esize = 2 if self.dtype == "bf16" else 4
        return 2.0 * self.B * self.T * self.Hkv * self.d * esize


# The five workloads the hot path is measured and checked on.
TINY_PREFILL_FP32 = Workload("prefill_fp32_T128", "prefill", "fp32", B=1, T=128, Hq=2, Hkv=1, d=64,
                             qkv_scale=1.0, seed=1001)
PREFILL_T4096 = Workload("prefill_T4096", "prefill", "bf16", B=1, T=4096, Hq=64, Hkv=8, d=128,
                         qkv_scale=1.0 / math.sqrt(2.0), seed=1002)
PREFILL_T32768 = Workload("prefill_T32768", "prefill", "bf16", B=1, T=32768, Hq=64, Hkv=8, d=128,
                          qkv_scale=1.0 / math.sqrt(2.0), seed=1003)
DECODE_B64_L8192 = Workload("decode_B64_L8192", "decode", "bf16", B=64, T=8192, Hq=64, Hkv=8, d=128,
                            qkv_scale=1.0, seed=1004)
DECODE_B8_L131072 = Workload("decode_B8_L131072", "decode", "bf16", B=8, T=131072, Hq=64, Hkv=8, d=128,
                             qkv_scale=1.0, seed=1005)
WORKLOADS = (TINY_PREFILL_FP32, PREFILL_T4096, PREFILL_T32768, DECODE_B64_L8192, DECODE_B8_L131072)


def _streams(seed: int) -> list[np.random.SeedSequence]:
    return np.random.SeedSequence(seed).spawn(6)


def make_prefill(w: Workload) -> dict:
    """q, k, v (uint16 bf16 bits or fp32) and lambda fp32 [B, T, P]."""
    assert w.kind == "prefill"
    s = _streams(w.seed)
    q = _normal(s[_S_Q], w.B * w.T * w.Hq * w.d, w.qkv_scale, w.dtype).reshape(w.B, w.T, w.Hq, w.d)
    k = _normal(s[_S_K], w.B * w.T * w.Hkv * w.d, w.qkv_scale, w.dtype).reshape(w.B, w.T, w.Hkv, w.d)
    v = _normal(s[_S_V], w.B * w.T * w.Hkv * w.d, w.qkv_scale, w.dtype).reshape(w.B, w.T, w.Hkv, w.d)
    z = _normal(s[_S_LAM], w.B * w.T * w.P, 1.0, "fp32").reshape(w.B, w.T, w.P)
    return dict(q=q, k=k, v=v, lam=_sigmoid_f32(z))


def make_dout(w: Workload) -> np.ndarray:
    """Output gradient for the backward pass: N(0, 1) in the workload's dtype, [B, T, P, d],
    from a stream independent of the forward inputs."""
    assert w.kind == "prefill"
    s = np.random.SeedSequence([w.seed, 7])
    return _normal(s, w.B * w.T * w.P * w.d, 1.0, w.dtype).reshape(w.B, w.T, w.P, w.d)


def make_decode(w: Workload) -> dict:
    """q [B, Hq, d], k/v cache [B, L, Hkv, d], lambda [B, P]."""
    assert w.kind == "decode"
    s = _streams(w.seed)
    q = _normal(s[_S_Q], w.B * w.Hq * w.d, w.qkv_scale, w.dtype).reshape(w.B, w.Hq, w.d)
    k = _normal(s[_S_K], w.B * w.T * w.Hkv * w.d, w.qkv_scale, w.dtype).reshape(w.B, w.T, w.Hkv, w.d)
    v = _normal(s[_S_V], w.B * w.T * w.Hkv * w.d, w.qkv_scale, w.dtype).reshape(w.B, w.T, w.Hkv, w.d)
    z = _normal(s[_S_LAM], w.B * w.P, 1.0, "fp32").reshape(w.B, w.P)
    return dict(q=q, k=k, v=v, lam=_sigmoid_f32(z))


def make_compare_decode(B: int, L: int, H: int, Hkv: int, d: int, seed: int) -> dict:
    """Inputs for the decode layout comparison: q [B, H, d], caches [B, L, Hkv, d]
    (bf16 bits, N(0, 1)) and a per-head lambda [B, H] uniform in [-0.3, 0.9]
    (V1's lambda may be negative)."""
    s = _streams(seed)
    q = _normal(s[_S_Q], B * H * d, 1.0, "bf16").reshape(B, H, d)
    k = _normal(s[_S_K], B * L * Hkv * d, 1.0, "bf16").reshape(B, L, Hkv, d)
    v = _normal(s[_S_V], B * L * Hkv * d, 1.0, "bf16").reshape(B, L, Hkv, d)
    lam = np.random.default_rng(s[_S_LAM]).uniform(-0.3, 0.9, (B, H)).astype(np.float32)
    return dict(q=q, k=k, v=v, lam=lam)


def make_projections(rows: int, d_model: int, P: int, in_dim: int, out_dim: int, seed: int = 6001) -> dict:
    """Inputs of the projections around the attention core, bf16 bits: x [rows, d_model]
    ~ N(0, 1), w_lambda [P, d_model] ~ N(0, 1/d_model), attn [rows, in_dim] ~ N(0, 1),
    w_o [in_dim, out_dim] ~ N(0, 1/in_dim) (unit-variance outputs at initialisation)."""
    s = _streams(seed)
    return dict(x=_normal(s[0], rows * d_model, 1.0, "bf16").reshape(rows, d_model),
                w_lambda=_normal(s[1], P * d_model, 1.0 / math.sqrt(d_model), "bf16").reshape(P, d_model),
                attn=_normal(s[2], rows * in_dim, 1.0, "bf16").reshape(rows, in_dim),
                w_o=_normal(s[3], in_dim * out_dim, 1.0 / math.sqrt(in_dim), "bf16").reshape(in_dim, out_dim))


def ragged_lengths(B: int, L: int, seed: int = 4242) -> np.ndarray:
    """Per-sequence cache lengths for ragged decode: uniform in [1, L], int32 [B]."""
    return np.random.default_rng(seed).integers(1, L + 1, size=B, dtype=np.int32)


def make_v1_lambda_vectors(P: int, d_lambda: int = 128, std: float = 0.1, seed: int = 2005) -> dict:
    """V1 reference-mode re-parameterisation vectors lq1, lk1, lq2, lk2 ~ N(0, std^2), fp32 [P, d_lambda]."""
    ss = np.random.SeedSequence(seed).spawn(4)
    out = {}
    for name, s in zip(("lq1", "lk1", "lq2", "lk2"), ss):
        out[name] = (np.random.default_rng(s).standard_normal((P, d_lambda), dtype=np.float32)
                     * np.float32(std)).astype(np.float32)
    return out


def plant_signal(w: Workload, inputs: dict, probes_per_pair: int = 8, n_signal: int = 16,
                 magnitude: float = 4.0, noise_scale: float = 1.0) -> dict:
    """Signal-plus-noise variant of a bf16 prefill workload (modifies k in place).

    Non-planted key rows are redrawn N(0, noise_scale^2).  For every (b, KV head g)
    and every pair p of that group, ``probes_per_pair`` probe query rows are drawn
    from [T/2, T); each probe gets ``n_signal`` distinct, not yet planted key
    positions j <= i, and those key rows are set to magnitude * q/||q|| of the
    probe's first-branch head (2p), computed in fp32 from the bf16 q and rounded
    to bf16.  Returns the plan: probe rows and their planted positions.
    """
    assert w.kind == "prefill" and w.dtype == "bf16"
    s = _streams(w.seed)
    k = _normal(s[_S_PLAN], w.B * w.T * w.Hkv * w.d, noise_scale, "bf16").reshape(w.B, w.T, w.Hkv, w.d)
    rng = np.random.default_rng(np.random.SeedSequence(w.seed + 7919))
    q = inputs["q"]
    plan = []   # (b, p, probe_row, positions[n_signal])
    for b in range(w.B):
        for g in range(w.Hkv):
            taken = np.zeros(w.T, dtype=bool)
            for pl in range(w.G):
                p = g * w.G + pl
                probes = rng.choice(np.arange(w.T // 2, w.T), size=probes_per_pair, replace=False)
                for i in np.sort(probes):
                    free = np.flatnonzero(~taken[: i + 1])
                    pos = np.sort(rng.choice(free, size=n_signal, replace=False))
                    taken[pos] = True
                    qi = bf16_to_f32(q[b, i, 2 * p]).astype(np.float32)
                    unit = qi / np.float32(np.sqrt(np.sum(qi * qi, dtype=np.float32)))
                    k[b, pos, g] = f32_to_bf16(np.float32(magnitude) * unit)[None, :]
                    plan.append((b, p, int(i), pos.astype(np.int64)))
    inputs = dict(inputs)
    inputs["k"] = k
    inputs["plan"] = plan
    return inputs


def signal_indicator_v(w: Workload, plan: list) -> tuple[np.ndarray, dict]:
    """Value rows that make a prefill's output read out attention mass directly.

    For the signal-plus-noise variant's plan (from ``plant_signal``): within each
    (b, KV head g), probe number c (in plan order) owns column c of V, which is 1
    on that probe's planted key rows and 0 elsewhere; column ``n_probes`` is 1 on
    every row; all other columns are 0.  With these values, output column c of the
    probe's own row and pair is the mass its attention map puts on the planted
    keys, and the all-ones column is the map's row sum.  Returns (v as bf16 bits
    [B, T, Hkv, d], {(b, p, row): column}) and requires more columns than probes
    per KV head.
    """
    assert w.kind == "prefill"
    v = np.zeros((w.B, w.T, w.Hkv, w.d), dtype=np.uint16)
    one = np.uint16(0x3F80)           # bf16 1.0
    column, count = {}, {}
    for b, p, i, pos in plan:
        g = p // w.G
        c = count.get((b, g), 0)
        count[(b, g)] = c + 1
        v[b, pos, g, c] = one
        column[(b, p, i)] = c
    ones_col = max(count.values())
    assert ones_col < w.d, "more probes per KV head than value columns"
    v[:, :, :, ones_col] = one
    column["ones"] = ones_col
    return v, column
