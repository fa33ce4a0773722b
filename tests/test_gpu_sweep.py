"""Seeded random sweep of small shapes through the C ABI vs the fp64 oracle (needs an
MI355X): prefill (causal, non-causal, sliding window), decode over a contiguous cache
with several key-range splits, decode over ragged caches, and the backward pass.

The shapes are drawn once from a fixed seed: batch 1-3, lengths 1-600 (ragged ends
at every tile size), GQA group sizes G in {1, 2, 3, 4, 8} (2G query heads per KV head,
up to 64), head dim 64 or 128.  Forward bar as everywhere (max-abs <= 2e-2, mean-abs <=
2e-3, rel-L2 <= 1e-2); gradients relative to their own scale, as in the backward tests.
"""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_v2_amd import binding as bd
from differential_attention_v2_amd import workloads as W

from _helpers import assert_parity, errors, from_device, to_device

pytestmark = pytest.mark.gpu


def _draw(n, seed, max_T=600):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 3, 4, 8]))
        Hkv = int(rng.choice([1, 2, 4] if G <= 4 else [1, 2]))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, max_T + 1))
        out.append((B, T, 2 * G * Hkv, Hkv, d, int(rng.integers(0, 1 << 30))))
    return out


PREFILL = _draw(16, 9101)
DECODE = _draw(8, 9102, max_T=900)
BACKWARD = _draw(6, 9103, max_T=300)


def _ids(cases):
    return [f"B{B}_T{T}_Hq{Hq}_Hkv{Hkv}_d{d}" for B, T, Hq, Hkv, d, _ in cases]


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", PREFILL, ids=_ids(PREFILL))
def test_prefill_sweep(gpu_device, B, T, Hq, Hkv, d, seed):
    w = W.Workload("sweep_prefill", "prefill", "bf16", B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, qkv_scale=1.0 / np.sqrt(2.0),
                   seed=seed % 100000)
    inp = W.make_prefill(w)
    q, k, v = (to_device(inp[n], "bf16", gpu_device) for n in ("q", "k", "v"))
    lam = torch.from_numpy(inp["lam"]).to(gpu_device)
    f = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    window = int(np.random.default_rng(seed).integers(1, T + 1))
    for causal, win in ((True, 0), (False, 0), (True, window)):
        got = from_device(bd.prefill_window(q, k, v, lam, win) if win else bd.prefill(q, k, v, lam, causal=causal))
        ref = oracle.diffattn_prefill(f["q"], f["k"], f["v"], inp["lam"], causal=causal, window=win)
        assert_parity(got, ref, f"sweep prefill B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} causal={causal} window={win}")


@pytest.mark.parametrize("B,L,Hq,Hkv,d,seed", DECODE, ids=_ids(DECODE))
def test_decode_sweep(gpu_device, B, L, Hq, Hkv, d, seed):
    w = W.Workload("sweep_decode", "decode", "bf16", B=B, T=L, Hq=Hq, Hkv=Hkv, d=d, seed=seed % 100000)
    inp = W.make_decode(w)
    q, k, v = (to_device(inp[n], "bf16", gpu_device) for n in ("q", "k", "v"))
    lam = torch.from_numpy(inp["lam"]).to(gpu_device)
    f = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    ref = oracle.diffattn_decode(f["q"], f["k"], f["v"], inp["lam"])
    for splits in (0, 1, 3):
        got = from_device(bd.decode(q, k, v, lam, num_splits=splits))
        assert_parity(got, ref, f"sweep decode B={B} L={L} Hq={Hq} Hkv={Hkv} d={d} splits={splits}")
    rng = np.random.default_rng(seed)
    lens_np = rng.integers(1, L + 1, B).astype(np.int32)
    lens = torch.from_numpy(lens_np).to(gpu_device)
    window = int(rng.integers(0, L + 1))
    ref = oracle.diffattn_decode(f["q"], f["k"], f["v"], inp["lam"], seq_lens=lens_np, window=window)
    got = from_device(bd.decode_varlen(q, k, v, lam, seq_lens=lens, window=window))
    assert_parity(got, ref, f"sweep ragged decode B={B} L={L} lengths={lens_np.tolist()} window={window}")


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", BACKWARD, ids=_ids(BACKWARD))
def test_backward_sweep(gpu_device, B, T, Hq, Hkv, d, seed):
    causal = bool(seed & 1)
    w = W.Workload("sweep_bwd", "prefill", "bf16", B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, qkv_scale=1.0 / np.sqrt(2.0),
                   causal=causal, seed=seed % 100000)
    inp = W.make_prefill(w)
    dout_np = W.make_dout(w)
    q, k, v = (to_device(inp[n], "bf16", gpu_device) for n in ("q", "k", "v"))
    lam = torch.from_numpy(inp["lam"]).to(gpu_device)
    dout = to_device(dout_np, "bf16", gpu_device)
    out, o2, lse = bd.prefill_train(q, k, v, lam, causal=causal)
    grads = [from_device(t) for t in bd.prefill_backward(q, k, v, lam, out, o2, lse, dout, causal=causal)]
    f = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    refs = oracle.diffattn_prefill_bwd(f["q"], f["k"], f["v"], inp["lam"], W.to_f64(dout_np, "bf16"), causal=causal)
    for name, got, ref in zip(("dq", "dk", "dv", "dlambda"), grads, refs):
        e = errors(got, ref)
        scale_max, scale_mean = float(np.max(np.abs(ref))), float(np.mean(np.abs(ref)))
        print(f"[parity] sweep backward B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} causal={causal} {name}: "
              f"max_abs={e['max_abs']:.3e} (ref max {scale_max:.3e}) rel_l2={e['rel_l2']:.3e}", flush=True)
        assert e["nonfinite"] == 0, (name, e)
        assert e["max_abs"] <= 2e-2 * max(scale_max, 1.0), (name, e)
        assert e["mean_abs"] <= 1e-2 * max(scale_mean, 0.1), (name, e)
