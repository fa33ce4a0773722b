"""The prefill's persistent schedule for long sequences (needs an MI355X).

From 8 token blocks per CU on (T >= 8192 with 8 KV heads and G = 4), one workgroup
per CU takes its blocks from per-XCD work queues in a static device array, one slot
per launch (round-robin over 1024 slots), which the launch's last workgroup sets back
to zero.  These tests check that every block is computed exactly once and that the
queues are reset for the next launch: against the sliding-window prefill with a window
covering the sequence (another kernel shape that never uses the queues, bitwise equal
by construction of the per-block arithmetic), over more launches than there are slots,
on two streams at once, under graph replay, and against the oracle on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_v2_amd import binding as bd
from differential_attention_v2_amd import workloads as W

from _helpers import assert_parity, from_device, to_device

pytestmark = pytest.mark.gpu


def _inputs(B, T, Hq, Hkv, d, seed, dev):
    w = W.Workload(f"persist_B{B}_T{T}_Hq{Hq}_Hkv{Hkv}_d{d}", "prefill", "bf16", B=B, T=T, Hq=Hq, Hkv=Hkv, d=d,
                   qkv_scale=1.0 / np.sqrt(2.0), seed=seed)
    inp = W.make_prefill(w)
    q, k, v = (to_device(inp[n], "bf16", dev) for n in ("q", "k", "v"))
    return w, inp, (q, k, v, torch.from_numpy(inp["lam"]).to(dev))


def _nan_out(w, dev):
    return torch.full((w.B, w.T, w.P, w.d), float("nan"), dtype=torch.bfloat16, device=dev)


@pytest.mark.parametrize("B,T,Hq,Hkv,d,v1", [
    (1, 8192, 64, 8, 128, False),
    (2, 8192, 32, 4, 128, False),    # units from two batches
    (1, 8192, 64, 8, 64, False),
    (1, 9000, 64, 8, 128, True),     # ragged last block, V1 mode
])
def test_every_block_once_against_window_shape(gpu_device, B, T, Hq, Hkv, d, v1):
    w, _, (q, k, v, lam) = _inputs(B, T, Hq, Hkv, d, seed=9500 + T + d, dev=gpu_device)
    out = _nan_out(w, gpu_device)   # a block left out would keep its NaNs
    bd.prefill(q, k, v, lam, v1_rmsnorm=v1, out=out)
    ref = bd.prefill_window(q, k, v, lam, T, v1_rmsnorm=v1)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_sampled_rows_against_oracle(gpu_device):
    w, inp, (q, k, v, lam) = _inputs(2, 8192, 32, 4, 128, seed=9600, dev=gpu_device)
    got = from_device(bd.prefill(q, k, v, lam))
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(8152, 8192), rng.choice(8192, 120, False)]))
    ref = oracle.diffattn_prefill(*(W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")), inp["lam"], rows=rows)
    assert_parity(got[:, rows], ref, "persistent prefill B=2 T=8192 sampled rows")


def test_more_launches_than_slots(gpu_device):
    """1100 launches in a row cycle through every queue slot and reuse some: each
    starts from empty queues only if the previous user of its slot reset it."""
    w, _, (q, k, v, lam) = _inputs(1, 8192, 64, 8, 128, seed=9700, dev=gpu_device)
    first = bd.prefill(q, k, v, lam).view(torch.int16).clone()
    out = torch.empty_like(first).view(torch.bfloat16)
    for i in range(1100):
        bd.prefill(q, k, v, lam, out=out)
        if i % 250 == 0 or i == 1099:
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), first), i
            out.fill_(float("nan"))


def test_two_streams_at_once(gpu_device):
    """Launches on two streams overlap on the device; each takes its own slot."""
    cases = [_inputs(1, 8192, 64, 8, 128, seed=9800 + i, dev=gpu_device) for i in range(4)]
    refs = []
    for w, _, (q, k, v, lam) in cases:
        refs.append(bd.prefill(q, k, v, lam).view(torch.int16).clone())
    torch.cuda.synchronize()
    outs = [_nan_out(w, gpu_device) for w, _, _ in cases]
    streams = [torch.cuda.Stream(device=gpu_device) for _ in range(2)]   # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for i, (w, _, (q, k, v, lam)) in enumerate(cases):
            with torch.cuda.stream(streams[i % 2]):
                bd.prefill(q, k, v, lam, out=outs[i])
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(len(cases)):
        assert torch.equal(outs[i].view(torch.int16), refs[i]), i


def test_graph_replays(gpu_device):
    w, _, (q, k, v, lam) = _inputs(1, 8192, 64, 8, 128, seed=9900, dev=gpu_device)
    out = torch.empty((w.B, w.T, w.P, w.d), dtype=torch.bfloat16, device=gpu_device)
    side = torch.cuda.Stream(device=gpu_device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bd.prefill(q, k, v, lam, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bd.prefill(q, k, v, lam, out=out)
    for rep in range(1, 4):
        fresh = _inputs(1, 8192, 64, 8, 128, seed=9900 + rep, dev=gpu_device)[2]
        for dst, src in zip((q, k, v, lam), fresh):
            dst.copy_(src)
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        ref = bd.prefill(q, k, v, lam)   # eager, between the replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep


def test_training_forward_uses_the_same_schedule(gpu_device):
    w, inp, (q, k, v, lam) = _inputs(1, 8192, 64, 8, 128, seed=9950, dev=gpu_device)
    out, o2, lse = bd.prefill_train(q, k, v, lam)
    plain = bd.prefill(q, k, v, lam)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    # A_2 V on sampled rows: the difference of two oracle maps, lambda = 0 and lambda = 1
    rows = np.array([0, 1, 63, 64, 4095, 4096, 8190, 8191])
    f = [W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")]
    zero, one = np.zeros_like(inp["lam"]), np.ones_like(inp["lam"])
    ref_o2 = oracle.diffattn_prefill(*f, zero, rows=rows) - oracle.diffattn_prefill(*f, one, rows=rows)
    assert_parity(from_device(o2)[:, rows], ref_o2, "persistent training forward o2 sampled rows")
    assert bool(torch.isfinite(lse).all())
