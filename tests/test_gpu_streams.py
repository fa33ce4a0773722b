"""Stream and graph semantics of the C ABI (needs an MI355X).

Every entry point enqueues its kernels on the stream it is given (the backward
forks part of them onto a side stream of it and joins them back), allocates
nothing and never synchronises (include/diffattn.h).  So the same calls
(1) give bitwise the same results on a side stream as on the default stream, and
(2) can be captured into a HIP graph and replayed: each replay, with new inputs
copied into the captured buffers, must equal eager calls on those inputs, with
eager work and synchronisations between the replays.  dK and dV are summed with
fp32 atomics (their last bits may differ from run to run); every other output is
compared bitwise.
"""
import numpy as np
import pytest
import torch

from differential_attention_v2_amd import binding as bd
from differential_attention_v2_amd import workloads as W

from _helpers import to_device

pytestmark = pytest.mark.gpu

# prefill: several 64-key tiles and a ragged tail, G = 4; decode: ragged lengths
PRE = W.Workload("stream_prefill", "prefill", "bf16", B=1, T=700, Hq=16, Hkv=2, d=128, qkv_scale=1 / np.sqrt(2),
                 seed=9100)
DEC = W.Workload("stream_decode", "decode", "bf16", B=3, T=1500, Hq=16, Hkv=2, d=128, qkv_scale=1 / np.sqrt(2),
                 seed=9200)
WINDOW = 200


# projections either side of the core: lambda from x [T, 512] (16 pairs), O_W of the
# prefill's output [T, P*d] back to 512
PROJ_DM, PROJ_P = 512, 16


def _host_inputs(seed_offset: int) -> dict:
    pre = W.make_prefill(PRE.with_(seed=PRE.seed + seed_offset))
    dec = W.make_decode(DEC.with_(seed=DEC.seed + seed_offset))
    proj = W.make_projections(PRE.B * PRE.T, PROJ_DM, PROJ_P, PRE.P * PRE.d, PROJ_DM, seed=9400 + seed_offset)
    return dict(q=pre["q"], k=pre["k"], v=pre["v"], lam=pre["lam"],
                dout=W.make_dout(PRE.with_(seed=PRE.seed + seed_offset)),
                qd=dec["q"], kc=dec["k"], vc=dec["v"], lamd=dec["lam"],
                lens=W.ragged_lengths(DEC.B, DEC.T, seed=9300 + seed_offset),
                xl=proj["x"], wl=proj["w_lambda"], wo=proj["w_o"])


def _to_device(h: dict, dev) -> dict:
    out = {}
    for n, x in h.items():
        if n in ("lam", "lamd"):
            out[n] = torch.from_numpy(x).to(dev)
        elif n == "lens":
            out[n] = torch.from_numpy(x).to(dev)
        else:
            out[n] = to_device(x, "bf16", dev)
    return out


def _buffers(dev) -> dict:
    """Outputs and workspaces, allocated once (a captured graph keeps their addresses)."""
    B, T, Hq, Hkv, d, P = PRE.B, PRE.T, PRE.Hq, PRE.Hkv, PRE.d, PRE.P
    bf = dict(dtype=torch.bfloat16, device=dev)
    n_bwd = bd.diffattn_prefill_bwd_workspace_bytes(B, T, Hq, Hkv, d)
    n_var = bd.diffattn_decode_varlen_workspace_bytes(DEC.B, DEC.T, DEC.Hq, DEC.Hkv, DEC.d)
    return dict(pre=torch.empty((B, T, P, d), **bf), win=torch.empty((B, T, P, d), **bf),
                dec=torch.empty((DEC.B, DEC.P, DEC.d), **bf), var=torch.empty((DEC.B, DEC.P, DEC.d), **bf),
                dq=torch.empty((B, T, Hq, d), **bf), dk=torch.empty((B, T, Hkv, d), **bf),
                dv=torch.empty((B, T, Hkv, d), **bf), dlam=torch.empty((B, T, P), dtype=torch.float32, device=dev),
                ws_dec=bd.decode_workspace(DEC.B, DEC.T, DEC.Hq, DEC.Hkv, DEC.d, device=dev),
                ws_var=torch.empty(n_var, dtype=torch.uint8, device=dev),
                ws_bwd=torch.empty(n_bwd, dtype=torch.uint8, device=dev),
                lp=torch.empty((B * T, PROJ_P), dtype=torch.float32, device=dev),
                y=torch.empty((B * T, PROJ_DM), **bf),
                dna=torch.empty((DEC.B, DEC.P, DEC.d), **bf))


def _run_all(x: dict, o: dict) -> dict:
    """Every attention entry point once, on the current stream, into the buffers o."""
    bd.prefill(x["q"], x["k"], x["v"], x["lam"], out=o["pre"])
    bd.prefill_window(x["q"], x["k"], x["v"], x["lam"], WINDOW, out=o["win"])
    bd.decode(x["qd"], x["kc"], x["vc"], x["lamd"], workspace=o["ws_dec"], out=o["dec"])
    bd.decode_varlen(x["qd"], x["kc"], x["vc"], x["lamd"], seq_lens=x["lens"], workspace=o["ws_var"], out=o["var"])
    out, o2, lse = bd.prefill_train(x["q"], x["k"], x["v"], x["lam"])
    bd.prefill_backward(x["q"], x["k"], x["v"], x["lam"], out, o2, lse, x["dout"], workspace=o["ws_bwd"],
                        grads=(o["dq"], o["dk"], o["dv"], o["dlam"]))
    bd.lambda_proj(x["xl"], x["wl"], out=o["lp"])
    bd.output_proj(o["pre"].view(PRE.B * PRE.T, PRE.P * PRE.d), x["wo"], out=o["y"])
    # the decode without a workspace, over 4 key ranges (its records go through the
    # library's fixed scratch); its first call on the device ran before any capture
    bd.decode_noalloc(x["qd"], x["kc"], x["vc"], x["lamd"], num_splits=4, out=o["dna"])
    return dict(train_out=out, o2=o2, lse=lse)


RESULTS = ("pre", "win", "dec", "var", "dq", "dk", "dv", "dlam", "lp", "y", "dna")
ATOMIC = ("dk", "dv")


def _compare(got: dict, ref: dict, what: str):
    for n in ref:
        a, b = got[n], ref[n]
        if n in ATOMIC:   # fp32 atomics in any order, then one rounding to bf16
            err = (a.float() - b.float()).abs().max().item()
            tol = 1e-2 * max(1.0, b.float().abs().max().item())
            assert err <= tol, (what, n, err, tol)
        else:
            assert torch.equal(a, b), (what, n, (a.float() - b.float()).abs().max().item())


def _snapshot(o: dict, extra: dict) -> dict:
    r = {n: o[n].clone() for n in RESULTS}
    r.update({n: t.clone() for n, t in extra.items()})
    return r


def test_side_stream_matches_default_stream(gpu_device):
    x = _to_device(_host_inputs(0), gpu_device)
    o_ref = _buffers(gpu_device)
    ref = _snapshot(o_ref, _run_all(x, o_ref))
    torch.cuda.synchronize()

    o_side = _buffers(gpu_device)
    side = torch.cuda.Stream(device=gpu_device)   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        extra = _run_all(x, o_side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _compare(_snapshot(o_side, extra), ref, "side stream")


def test_graph_capture_replays_match_eager(gpu_device):
    x = _to_device(_host_inputs(0), gpu_device)     # captured input buffers
    o = _buffers(gpu_device)                          # captured output buffers
    side = torch.cuda.Stream(device=gpu_device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # one warm-up pass before capture
        _run_all(x, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured_extra = _run_all(x, o)

    o_eager = _buffers(gpu_device)
    prev = None
    for rep in range(1, 4):
        fresh = _to_device(_host_inputs(rep), gpu_device)
        for n in x:
            x[n].copy_(fresh[n])
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(o, captured_extra)
        # eager calls on the same inputs, between the replays
        ref = _snapshot(o_eager, _run_all(x, o_eager))
        torch.cuda.synchronize()
        _compare(got, ref, f"replay {rep}")
        # each replay read the inputs copied in before it
        if prev is not None:
            assert not torch.equal(got["pre"], prev) and not torch.equal(got["var"], prev_var)
        prev, prev_var = got["pre"], got["var"]


GRADS = ("dq", "dk", "dv", "dlam")


def test_backward_fork_join_inside_capture(gpu_device):
    """The backward runs its row statistics and dQ kernel on a side stream of the
    caller's stream, forked off and joined back with events.  On a stream that has
    run the backward eagerly (its side stream exists), a capture holds the fork and
    the join: every replay, with new inputs, equals eager calls, and copies of the
    gradients captured after the call on the same stream see their final values."""
    x = _to_device(_host_inputs(0), gpu_device)
    o = _buffers(gpu_device)
    s = torch.cuda.Stream(device=gpu_device)   # default priority
    s.wait_stream(torch.cuda.current_stream())

    def step(bufs):
        out, o2, lse = bd.prefill_train(x["q"], x["k"], x["v"], x["lam"])
        bd.prefill_backward(x["q"], x["k"], x["v"], x["lam"], out, o2, lse, x["dout"], workspace=bufs["ws_bwd"],
                            grads=tuple(bufs[n] for n in GRADS))
        return {n: bufs[n].clone() for n in GRADS}   # enqueued right after the call, no synchronisation

    with torch.cuda.stream(s):
        step(o)                                     # eager first: creates the side stream of s
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        copies = step(o)

    o_eager = _buffers(gpu_device)
    for rep in range(1, 4):
        fresh = _to_device(_host_inputs(rep), gpu_device)
        for n in x:
            x[n].copy_(fresh[n])
        for n in GRADS:
            copies[n].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {n: copies[n].clone() for n in GRADS}
        ref = step(o_eager)
        torch.cuda.synchronize()
        _compare(got, ref, f"backward replay {rep}")


def test_backward_on_many_streams(gpu_device):
    """One side stream per caller stream, at most 64: calls on 70 streams (the last
    ones past the cap run serially) all give the same gradients, each read right
    after its call on its own stream."""
    w = W.Workload("many_streams_bwd", "prefill", "bf16", B=1, T=96, Hq=8, Hkv=2, d=64, qkv_scale=1 / np.sqrt(2),
                   seed=9250)
    h = W.make_prefill(w)
    q, k, v = (to_device(h[n], "bf16", gpu_device) for n in ("q", "k", "v"))
    lam = torch.from_numpy(h["lam"]).to(gpu_device)
    dout = to_device(W.make_dout(w), "bf16", gpu_device)
    out, o2, lse = bd.prefill_train(q, k, v, lam)
    ref = bd.prefill_backward(q, k, v, lam, out, o2, lse, dout)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=gpu_device) for _ in range(70)]
    got = []
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            g = bd.prefill_backward(q, k, v, lam, out, o2, lse, dout)
            got.append(tuple(t.clone() for t in g))   # on s, right after the call
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i, g in enumerate(got):
        _compare(dict(zip(GRADS, g)), dict(zip(GRADS, ref)), f"stream {i}")
