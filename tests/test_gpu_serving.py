"""Serving variants through the C ABI vs the fp64 oracle (needs an MI355X): the
causal sliding-window prefill and decode over ragged caches (per-sequence
lengths, optional window).  Bar as for the plain path: max-abs <= 2e-2 and
mean-abs <= 2e-3 (bf16 in, fp32 accumulate)."""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_v2_amd import binding as bd
from differential_attention_v2_amd import workloads as W

from _helpers import assert_parity, from_device, to_device

pytestmark = pytest.mark.gpu


def _prefill_inputs(w, dev):
    inp = W.make_prefill(w)
    t = [to_device(inp[n], "bf16", dev) for n in ("q", "k", "v")]
    return inp, t + [torch.from_numpy(inp["lam"]).to(dev)]


def _case(B, T, Hq, Hkv, d, seed):
    return W.Workload(f"swa_B{B}_T{T}_Hq{Hq}_Hkv{Hkv}_d{d}", "prefill", "bf16", B=B, T=T, Hq=Hq, Hkv=Hkv, d=d,
                      qkv_scale=1.0 / np.sqrt(2.0), seed=seed)


@pytest.mark.parametrize("shape,windows", [
    ((1, 300, 16, 2, 128), [1, 17, 64, 100, 299]),
    ((2, 1000, 8, 1, 64), [130]),
    ((1, 700, 4, 2, 128), [1, 200, 333]),      # G = 1: 128-token blocks, waves start in later tiles
    ((1, 257, 16, 1, 64), [50]),              # G = 8
])
def test_prefill_window_parity(gpu_device, shape, windows):
    w = _case(*shape, seed=8000 + shape[1])
    inp, (q, k, v, lam) = _prefill_inputs(w, gpu_device)
    f = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    for win in windows:
        got = from_device(bd.prefill_window(q, k, v, lam, win))
        ref = oracle.diffattn_prefill(f["q"], f["k"], f["v"], inp["lam"], causal=True, window=win)
        assert_parity(got, ref, f"{w.name} window={win}")


def test_prefill_window_covering_sequence_is_plain_causal(gpu_device):
    w = _case(1, 200, 8, 2, 128, seed=8100)
    _, (q, k, v, lam) = _prefill_inputs(w, gpu_device)
    plain = bd.prefill(q, k, v, lam).view(torch.int16)
    for win in (0, 200, 5000):
        assert torch.equal(bd.prefill_window(q, k, v, lam, win).view(torch.int16), plain), win


def test_prefill_window_v1_mode(gpu_device):
    w = _case(1, 160, 8, 2, 128, seed=8200)
    inp, (q, k, v, lam) = _prefill_inputs(w, gpu_device)
    f = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    got = from_device(bd.prefill_window(q, k, v, lam, 40, v1_rmsnorm=True))
    ref = oracle.diffattn_prefill(f["q"], f["k"], f["v"], inp["lam"], causal=True, window=40, v1_rmsnorm=True)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"[parity] V1 window 40: rel_l2={rel:.3e}", flush=True)
    assert rel <= 1e-2


def test_prefill_window_T4096_sampled_rows(gpu_device):
    """B=1, T=4096, Hq=64, Hkv=8, d=128 with the lesson's 1024-key window, 200 rows checked."""
    w = W.PREFILL_T4096
    inp, (q, k, v, lam) = _prefill_inputs(w, gpu_device)
    out = from_device(bd.prefill_window(q, k, v, lam, 1024))
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(0, 8), [1023, 1024, 1025, 4095], rng.choice(4096, 188, False)]))
    ref = oracle.diffattn_prefill(*(W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")), inp["lam"], causal=True,
                                  window=1024, rows=rows)
    assert_parity(out[:, rows], ref, "prefill T=4096 window=1024 sampled rows")


# --------------------------------------------------------------------------------- decode
def _decode_case(B, L, Hq, Hkv, d, seed):
    return W.Workload(f"varlen_B{B}_L{L}_Hq{Hq}_Hkv{Hkv}_d{d}", "decode", "bf16", B=B, T=L, Hq=Hq, Hkv=Hkv, d=d,
                      seed=seed)


def _decode_inputs(w, dev):
    inp = W.make_decode(w)
    t = [to_device(inp[n], "bf16", dev) for n in ("q", "k", "v")]
    return inp, t + [torch.from_numpy(inp["lam"]).to(dev)]


@pytest.mark.parametrize("d", [128, 64])
def test_decode_varlen_parity(gpu_device, d):
    w = _decode_case(8, 1000, 16, 2, d, seed=8300 + d)
    inp, (q, k, v, lam) = _decode_inputs(w, gpu_device)
    lens_np = np.array([1, 1000, 33, 999, 512, 2, 700, 64], dtype=np.int32)
    lens = torch.from_numpy(lens_np).to(gpu_device)
    f = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    for window in (0, 1, 7, 64, 2000):
        ref = oracle.diffattn_decode(f["q"], f["k"], f["v"], inp["lam"], seq_lens=lens_np, window=window)
        for splits in (0, 1, 5, 32):
            got = from_device(bd.decode_varlen(q, k, v, lam, seq_lens=lens, window=window, num_splits=splits))
            assert_parity(got, ref, f"{w.name} window={window} splits={splits}")


def test_decode_varlen_full_lengths_equal_plain_decode(gpu_device):
    """No lengths: the plain decode, bit for bit.  All lengths = L: the even split
    over the batch's rows, which partitions the keys differently, agrees closely."""
    w = _decode_case(4, 777, 16, 2, 128, seed=8400)
    _, (q, k, v, lam) = _decode_inputs(w, gpu_device)
    plain = bd.decode(q, k, v, lam)
    assert torch.equal(bd.decode_varlen(q, k, v, lam).view(torch.int16), plain.view(torch.int16))
    full = torch.full((4,), 777, dtype=torch.int32, device=gpu_device)
    assert_parity(from_device(bd.decode_varlen(q, k, v, lam, seq_lens=full)), from_device(plain),
                  "even split, full lengths vs plain decode", max_abs=1e-2, mean_abs=1e-3)


def test_decode_varlen_many_short_sequences(gpu_device):
    """1500 sequences of 1-40 rows: ranges cross many sequences (a plan kernel scans
    the lengths once: B > 512)."""
    w = _decode_case(1500, 64, 8, 2, 64, seed=8450)
    inp, (q, k, v, lam) = _decode_inputs(w, gpu_device)
    lens_np = np.random.default_rng(8).integers(1, 41, size=1500).astype(np.int32)
    lens = torch.from_numpy(lens_np).to(gpu_device)
    f = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    for splits in (0, 3):
        got = from_device(bd.decode_varlen(q, k, v, lam, seq_lens=lens, num_splits=splits))
        sel = np.arange(0, 1500, 37)
        ref = oracle.diffattn_decode(f["q"], f["k"], f["v"], inp["lam"], batches=sel, seq_lens=lens_np)
        assert_parity(got[sel], ref, f"1500 short sequences splits={splits}")


@pytest.mark.parametrize("B", [512, 513])
def test_decode_varlen_plan_paths(gpu_device, B):
    """Up to 512 sequences every wave scans the lengths itself (8 chunks of 64 at
    B = 512); from 513 on a plan kernel scans them once.  Both against the oracle,
    with and without a window."""
    w = _decode_case(B, 48, 8, 2, 64, seed=8460 + B)
    inp, (q, k, v, lam) = _decode_inputs(w, gpu_device)
    lens_np = np.random.default_rng(B).integers(1, 49, size=B).astype(np.int32)
    lens = torch.from_numpy(lens_np).to(gpu_device)
    f = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    sel = np.unique(np.concatenate([np.arange(0, B, 41), [B - 2, B - 1]]))
    for window in (0, 16):
        got = from_device(bd.decode_varlen(q, k, v, lam, seq_lens=lens, window=window))
        ref = oracle.diffattn_decode(f["q"], f["k"], f["v"], inp["lam"], batches=sel, seq_lens=lens_np, window=window)
        assert_parity(got[sel], ref, f"{B} short sequences window={window}")


def test_decode_varlen_clamps_out_of_range_lengths(gpu_device):
    """Lengths outside [1, L] read only the cache: 0 and negatives act as 1, > L as L."""
    w = _decode_case(3, 100, 8, 2, 128, seed=8500)
    inp, (q, k, v, lam) = _decode_inputs(w, gpu_device)
    got = from_device(bd.decode_varlen(q, k, v, lam, seq_lens=torch.tensor([0, -5, 1000], dtype=torch.int32,
                                                                            device=gpu_device)))
    f = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    ref = oracle.diffattn_decode(f["q"], f["k"], f["v"], inp["lam"], seq_lens=np.array([1, 1, 100]))
    assert_parity(got, ref, "clamped lengths")


def test_decode_varlen_B64_L8192_sampled(gpu_device):
    """B=64, L=8192, Hq=64, Hkv=8, d=128 with lengths uniform in [1, 8192]; 8 sequences checked."""
    w = W.DECODE_B64_L8192
    inp, (q, k, v, lam) = _decode_inputs(w, gpu_device)
    lens_np = W.ragged_lengths(w.B, w.T)
    lens = torch.from_numpy(lens_np).to(gpu_device)
    got = from_device(bd.decode_varlen(q, k, v, lam, seq_lens=lens))
    bsel = np.array([0, 1, 13, 31, 32, 47, 62, 63])
    ref = oracle.diffattn_decode(*(W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")), inp["lam"], batches=bsel,
                                 seq_lens=lens_np)
    assert_parity(got[bsel], ref, "decode B=64 L=8192 ragged lengths (8 sequences)")
