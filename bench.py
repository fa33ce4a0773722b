#!/usr/bin/env python3
"""Benchmark of the Differential Attention V2 forward hot path on one MI355X.

A step is one pass of the whole path over synthetic inputs already resident in
HBM: one causal bf16 prefill (B=1, T=4096, Hq=64, Hkv=8, d=128) followed by one
bf16 split-KV decode (B=64, L=8192, Hq=64, Hkv=8, d=128).  The prefill and
decode launches are each bracketed by HIP events on the stream they run on;
`value` is the prefill's algorithmic TFLOP/s (4*d flops per visible
query-key-head, causal) over its mean launch time, and the decode's KV-cache
GB/s (every K/V byte once) is reported beside it.  Rank 0 prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 50] [--settle-ms 300] [--no-cpu-baseline]

Before the warmup steps the path runs for --settle-ms of wall time: MI355X's
clock ramps from about 1.9 to 2.35 GHz over the first tens of ms of sustained
load, and the timed steps are meant to see the sustained clock.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "DiffAttn-V2 fwd: prefill TFLOP/s & decode KV GB/s, % of MI355X peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _kernel_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "differential_attention_v2_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _traffic(kind: str, launches_per_record: int = 1):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kind]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != _kernel_hash(rec["sources"]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(budget_s: float) -> dict:
    """The fp64 oracle on a bounded sample of the prefill workload: whole pairs, all 4096 rows."""
    import numpy as np
    import oracle
    from differential_attention_v2_amd import workloads as W
    try:
        import threadpoolctl
        threads = sum(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info() if i["user_api"] == "blas")
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    w = W.PREFILL_T4096
    inp = W.make_prefill(w)
    q, k, v = (W.to_f64(inp[n], "bf16") for n in ("q", "k", "v"))
    G = w.G
    # whole pairs (all rows, both heads), cycling over the P pairs until the budget is spent
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        p = done % w.P
        g = p // G
        oracle.diffattn_prefill(q[:, :, 2 * p:2 * p + 2], k[:, :, g:g + 1], v[:, :, g:g + 1],
                                inp["lam"][:, :, p:p + 1])
        done += 1
    dt = time.perf_counter() - t0
    flops = w.prefill_flops() * done / w.P
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads or 1), "kind": "oracle",
            "sample": f"T={w.T} prefill, {done} pair passes ({w.P} pairs in the workload) x all {w.T} rows, "
                      f"fp64 numpy (OpenBLAS), {dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50, help="untimed steps after the clock settle phase")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed wall time of steps before the warmup steps (clock ramp-up); 0 skips it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--only", choices=["prefill", "decode", "backward", "serving", "layouts", "projections", "long"],
                    default=None,
                    help="time one part (for profiler runs); backward = training forward + backward, "
                         "serving = windowed prefill + ragged decode")
    ap.add_argument("--no-backward", action="store_true", help="skip the training forward / backward timing")
    ap.add_argument("--no-serving", action="store_true", help="skip the serving-variant timing")
    ap.add_argument("--no-projections", action="store_true", help="skip the lambda producer / O_W timing")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long configurations (T=32768 prefill, B=8 L=131072 decode)")
    ap.add_argument("--no-layouts", action="store_true",
                    help="skip the decode layout comparison (standard transformer, DIFF V1, V2)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (x5) to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU sharding or collectives)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from differential_attention_v2_amd import binding as bd
    from differential_attention_v2_amd import workloads as W

    if not os.path.exists(bd.LIB_PATH):
        from differential_attention_v2_amd import build_lib
        build_lib.build()
    dev = torch.device("cuda:0")

    def dev_bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    wp, wd = W.PREFILL_T4096, W.DECODE_B64_L8192
    do_p = args.only in (None, "prefill")
    do_d = args.only in (None, "decode")
    do_b = args.only == "backward" or (args.only is None and not args.no_backward)
    do_s = args.only == "serving" or (args.only is None and not args.no_serving)
    do_l = args.only == "layouts" or (args.only is None and not args.no_layouts)
    do_j = args.only == "projections" or (args.only is None and not args.no_projections)
    do_g = args.only == "long" or (args.only is None and not args.no_long)
    if do_p:
        ip = W.make_prefill(wp)
        pq, pk, pv = dev_bf16(ip["q"]), dev_bf16(ip["k"]), dev_bf16(ip["v"])
        plam = torch.from_numpy(ip["lam"]).to(dev)
        pout = torch.empty((wp.B, wp.T, wp.P, wp.d), dtype=torch.bfloat16, device=dev)
        del ip
    if do_d:
        idc = W.make_decode(wd)
        dq, dk, dv = dev_bf16(idc["q"]), dev_bf16(idc["k"]), dev_bf16(idc["v"])
        dlam = torch.from_numpy(idc["lam"]).to(dev)
        dout = torch.empty((wd.B, wd.P, wd.d), dtype=torch.bfloat16, device=dev)
        dws = bd.decode_workspace(wd.B, wd.T, wd.Hq, wd.Hkv, wd.d, 0, dev)
        del idc
    stream = torch.cuda.current_stream()

    def settle(fn, ms):
        """Run fn for `ms` of wall time (untimed) so the clock is at its sustained level."""
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()

    def step(evs=None):
        if do_p:
            if evs: evs[0].record(stream)
            bd.prefill(pq, pk, pv, plam, out=pout)
            if evs: evs[1].record(stream)
        if do_d:
            if evs: evs[2].record(stream)
            bd.decode(dq, dk, dv, dlam, workspace=dws, out=dout)
            if evs: evs[3].record(stream)

    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_pre = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) if do_p else None
    ms_dec = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) if do_d else None

    bwd = None
    if do_b:
        # training step of the attention core: training forward (out, o2, lse) and
        # backward, timed after the main step, on the same T=4096 prefill inputs
        if not do_p:
            ip = W.make_prefill(wp)
            pq, pk, pv = dev_bf16(ip["q"]), dev_bf16(ip["k"]), dev_bf16(ip["v"])
            plam = torch.from_numpy(ip["lam"]).to(dev)
            del ip
        bdout = dev_bf16(W.make_dout(wp))
        tout, to2, tlse = bd.prefill_train(pq, pk, pv, plam)
        bws = torch.empty(bd.diffattn_prefill_bwd_workspace_bytes(wp.B, wp.T, wp.Hq, wp.Hkv, wp.d),
                          dtype=torch.uint8, device=dev)
        grads = (torch.empty_like(pq), torch.empty_like(pk), torch.empty_like(pv), torch.empty_like(plam))

        def bstep(ev=None):
            if ev: ev[0].record(stream)
            bd.prefill_train(pq, pk, pv, plam)
            if ev: ev[1].record(stream)
            bd.prefill_backward(pq, pk, pv, plam, tout, to2, tlse, bdout, workspace=bws, grads=grads)
            if ev: ev[2].record(stream)

        settle(bstep, min(args.settle_ms, 100.0))
        for _ in range(max(3, args.warmup // 5)):
            bstep()
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            bstep(bev[i])
        torch.cuda.synchronize()
        ms_tf = float(np.mean([e[0].elapsed_time(e[1]) for e in bev]))
        ms_bw = float(np.mean([e[1].elapsed_time(e[2]) for e in bev]))
        bw_tf = wp.prefill_bwd_flops() / (ms_bw * 1e-3) / 1e12
        bwd = {"value": bw_tf, "unit": "TFLOP/s", "frac": bw_tf / PEAK_BF16_TFLOPS, "ms_per_launch": ms_bw,
               "algorithmic_flops_per_launch": wp.prefill_bwd_flops(),
               "flop_count": "8*d per visible (query, key, head): dP, dV, dQ, dK products, no recompute",
               "kernels": "bwd_pre + fill_zero + bwd_dkdv_kernel<128> + bwd_dq_kernel<128> + 2 x convert",
               "traffic": _traffic("backward"),
               "train_forward_ms": ms_tf,
               "train_forward_tflops": wp.prefill_flops() / (ms_tf * 1e-3) / 1e12,
               "workload": f"{wp.name} causal bf16, dout ~ N(0,1)"}

    serving = None
    if do_s:
        # serving variants on the same shapes: the T=4096 prefill with a 1024-key causal
        # window, and the B=64, L=8192 decode over caches with lengths uniform in [1, 8192]
        SWA = 1024
        if not (do_p or do_b):
            ip = W.make_prefill(wp)
            pq, pk, pv = dev_bf16(ip["q"]), dev_bf16(ip["k"]), dev_bf16(ip["v"])
            plam = torch.from_numpy(ip["lam"]).to(dev)
            del ip
        if not do_d:
            idc = W.make_decode(wd)
            dq, dk, dv = dev_bf16(idc["q"]), dev_bf16(idc["k"]), dev_bf16(idc["v"])
            dlam = torch.from_numpy(idc["lam"]).to(dev)
            dws = bd.decode_workspace(wd.B, wd.T, wd.Hq, wd.Hkv, wd.d, 0, dev)
            del idc
        sout = torch.empty((wp.B, wp.T, wp.P, wp.d), dtype=torch.bfloat16, device=dev)
        lens_np = W.ragged_lengths(wd.B, wd.T)
        lens = torch.from_numpy(lens_np).to(dev)
        vout = torch.empty((wd.B, wd.P, wd.d), dtype=torch.bfloat16, device=dev)
        vws = torch.empty(bd.diffattn_decode_varlen_workspace_bytes(wd.B, wd.T, wd.Hq, wd.Hkv, wd.d, 0),
                          dtype=torch.uint8, device=dev)

        def sstep(ev=None):
            if ev: ev[0].record(stream)
            bd.prefill_window(pq, pk, pv, plam, SWA, out=sout)
            if ev: ev[1].record(stream)
            bd.decode_varlen(dq, dk, dv, dlam, seq_lens=lens, workspace=vws, out=vout)
            if ev: ev[2].record(stream)

        settle(sstep, min(args.settle_ms, 100.0))
        for _ in range(max(3, args.warmup // 2)):
            sstep()
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            sstep(sev[i])
        torch.cuda.synchronize()
        ms_sw = float(np.mean([e[0].elapsed_time(e[1]) for e in sev]))
        ms_vl = float(np.mean([e[1].elapsed_time(e[2]) for e in sev]))
        vl_bytes = 2.0 * float(lens_np.sum()) * wd.Hkv * wd.d * 2
        serving = {
            "prefill_window": {"value": wp.prefill_flops(SWA) / (ms_sw * 1e-3) / 1e12, "unit": "TFLOP/s",
                               "ms_per_launch": ms_sw, "window": SWA,
                               "algorithmic_flops_per_launch": wp.prefill_flops(SWA),
                               "kernel": "prefill_kernel<128, 1>", "traffic": _traffic("prefill_window"),
                               "frac": wp.prefill_flops(SWA) / (ms_sw * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                               "workload": f"{wp.name} causal, window {SWA}"},
            "decode_varlen": {"value": vl_bytes / (ms_vl * 1e-3) / 1e9, "unit": "GB/s", "ms_per_launch": ms_vl,
                              "traffic": _traffic("decode_varlen"),
                              "algorithmic_bytes_per_launch": vl_bytes,
                              "frac": vl_bytes / (ms_vl * 1e-3) / 1e9 / PEAK_HBM_GBS,
                              "workload": f"{wd.name} with lengths uniform in [1, {wd.T}] (mean "
                                          f"{float(lens_np.mean()):.0f})"}}

    layouts = None
    if do_l:
        # decode-speed claim of the pages: on the B=64, L=8192 cache geometry (
        # Hkv=8, d=128) time a standard transformer with H=32 heads, DIFF V1 with
        # the same 32 heads (q, k halves per branch, V read once per branch) and V2
        # (64 query heads = 32 pairs, the bench's decode)
        H = wd.P
        ic = W.make_compare_decode(wd.B, wd.T, H, wd.Hkv, wd.d, seed=9300)
        cq, ck, cv = dev_bf16(ic["q"]), dev_bf16(ic["k"]), dev_bf16(ic["v"])
        clam = torch.from_numpy(ic["lam"]).to(dev)
        del ic
        if not do_d:
            idc = W.make_decode(wd)
            dq, dk, dv = dev_bf16(idc["q"]), dev_bf16(idc["k"]), dev_bf16(idc["v"])
            dlam = torch.from_numpy(idc["lam"]).to(dev)
            dws = bd.decode_workspace(wd.B, wd.T, wd.Hq, wd.Hkv, wd.d, 0, dev)
            del idc
        cws = torch.empty(bd.diffattn_decode_compare_workspace_bytes(wd.B, wd.T, H, wd.Hkv, wd.d, 0),
                          dtype=torch.uint8, device=dev)
        cout = torch.empty((wd.B, H, wd.d), dtype=torch.bfloat16, device=dev)
        v2out = torch.empty((wd.B, wd.P, wd.d), dtype=torch.bfloat16, device=dev)
        runs = {"standard": lambda: bd.decode_standard(cq, ck, cv, workspace=cws, out=cout),
                "v1_layout": lambda: bd.decode_v1_layout(cq, ck, cv, clam, workspace=cws, out=cout),
                "v2": lambda: bd.decode(dq, dk, dv, dlam, workspace=dws, out=v2out)}
        cache = wd.B * wd.T * wd.Hkv * wd.d * 2
        bytes_read = {"standard": 2.0 * cache, "v1_layout": 3.0 * cache, "v2": 2.0 * cache}
        layouts = {}
        for name, fn in runs.items():
            settle(fn, min(args.settle_ms, 100.0))
            for _ in range(max(3, args.warmup // 2)):
                fn()
            lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
            torch.cuda.synchronize()
            for i in range(args.steps):
                lev[i][0].record(stream)
                fn()
                lev[i][1].record(stream)
            torch.cuda.synchronize()
            ms = float(np.mean([e[0].elapsed_time(e[1]) for e in lev]))
            layouts[name] = {"ms_per_launch": ms, "cache_bytes_read": bytes_read[name],
                             "GB_per_s": bytes_read[name] / (ms * 1e-3) / 1e9}
        for name in ("v1_layout", "v2"):
            layouts[name]["time_vs_standard"] = layouts[name]["ms_per_launch"] / layouts["standard"]["ms_per_launch"]
        layouts["workload"] = (f"B={wd.B} L={wd.T} Hkv={wd.Hkv} d={wd.d} bf16 cache; standard and V1: {H} heads; "
                               f"V2: {wd.Hq} query heads ({wd.P} pairs)")

    projections = None
    if do_j:
        # the steps either side of the T=4096 attention core: lambda for 4096 tokens x 32
        # pairs from d_model = 4096, and O_W from P*d = 4096 back to d_model = 4096
        rows, dm, kin = wp.B * wp.T, wp.P * wp.d, wp.P * wp.d
        ij = W.make_projections(rows, dm, wp.P, kin, dm)
        jx, jw = dev_bf16(ij["x"]), dev_bf16(ij["w_lambda"])
        ja, jo = dev_bf16(ij["attn"]), dev_bf16(ij["w_o"])
        del ij
        jl = torch.empty((rows, wp.P), dtype=torch.float32, device=dev)
        jy = torch.empty((rows, dm), dtype=torch.bfloat16, device=dev)
        jruns = {"lambda_proj": lambda: bd.lambda_proj(jx, jw, out=jl),
                 "output_proj": lambda: bd.output_proj(ja, jo, out=jy)}
        jt = {}
        for name, fn in jruns.items():
            settle(fn, min(args.settle_ms, 100.0))
            for _ in range(max(3, args.warmup // 2)):
                fn()
            jev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
            torch.cuda.synchronize()
            for i in range(args.steps):
                jev[i][0].record(stream)
                fn()
                jev[i][1].record(stream)
            torch.cuda.synchronize()
            jt[name] = float(np.mean([e[0].elapsed_time(e[1]) for e in jev]))
        lp_bytes = rows * dm * 2.0 + wp.P * dm * 2.0 + rows * wp.P * 4.0
        op_flops = 2.0 * rows * kin * dm
        projections = {
            "lambda_proj": {"value": lp_bytes / (jt["lambda_proj"] * 1e-3) / 1e9, "unit": "GB/s",
                            "ms_per_launch": jt["lambda_proj"], "algorithmic_bytes_per_launch": lp_bytes,
                            "frac": lp_bytes / (jt["lambda_proj"] * 1e-3) / 1e9 / PEAK_HBM_GBS, "bound": "hbm",
                            "workload": f"x [{rows}, {dm}] bf16, w [{wp.P}, {dm}] -> lambda [{rows}, {wp.P}] fp32"},
            "output_proj": {"value": op_flops / (jt["output_proj"] * 1e-3) / 1e12, "unit": "TFLOP/s",
                            "ms_per_launch": jt["output_proj"], "algorithmic_flops_per_launch": op_flops,
                            "frac": op_flops / (jt["output_proj"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                            "bound": "mfma", "engine": "rocBLAS gemm_ex (bf16, fp32 accumulate)",
                            "workload": f"[{rows}, {kin}] x [{kin}, {dm}] bf16"}}

    long_cfg = None
    if do_g:
        # the long configurations, timed only (their parity runs in the GPU tests):
        # T=32768 causal prefill and the B=8, L=131072 decode, V2 and V1 mode.
        # Inputs are drawn on the device from a seeded generator with the same
        # distributions as the host generator (host generation of 4.3 GB of cache
        # would take minutes).
        w3, w5 = W.PREFILL_T32768, W.DECODE_B8_L131072
        gen = torch.Generator(device=dev)
        gen.manual_seed(3000 + 3)

        def rnd(shape, scale=1.0):
            return (torch.randn(shape, generator=gen, device=dev, dtype=torch.bfloat16) * scale).contiguous()

        lq = rnd((w3.B, w3.T, w3.Hq, w3.d), 0.7071)
        lk = rnd((w3.B, w3.T, w3.Hkv, w3.d), 0.7071)
        lv = rnd((w3.B, w3.T, w3.Hkv, w3.d), 0.7071)
        llam = torch.sigmoid(torch.randn((w3.B, w3.T, w3.P), generator=gen, device=dev))
        lout = torch.empty((w3.B, w3.T, w3.P, w3.d), dtype=torch.bfloat16, device=dev)

        def time_fn(fn, steps):
            for _ in range(2):
                fn()
            lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
            torch.cuda.synchronize()
            for i in range(steps):
                lev[i][0].record(stream)
                fn()
                lev[i][1].record(stream)
            torch.cuda.synchronize()
            return float(np.mean([e[0].elapsed_time(e[1]) for e in lev]))

        lsteps = max(3, min(args.steps, 10))
        settle(lambda: bd.prefill(lq, lk, lv, llam, out=lout), min(args.settle_ms, 100.0))
        ms3 = time_fn(lambda: bd.prefill(lq, lk, lv, llam, out=lout), lsteps)
        del lq, lk, lv, llam, lout
        gen.manual_seed(3000 + 5)
        cq = rnd((w5.B, w5.Hq, w5.d))
        ck = rnd((w5.B, w5.T, w5.Hkv, w5.d))
        cv = rnd((w5.B, w5.T, w5.Hkv, w5.d))
        clam = torch.sigmoid(torch.randn((w5.B, w5.P), generator=gen, device=dev))
        cout5 = torch.empty((w5.B, w5.P, w5.d), dtype=torch.bfloat16, device=dev)
        cws = bd.decode_workspace(w5.B, w5.T, w5.Hq, w5.Hkv, w5.d, 0, dev)
        settle(lambda: bd.decode(cq, ck, cv, clam, workspace=cws, out=cout5), min(args.settle_ms, 100.0))
        ms5 = time_fn(lambda: bd.decode(cq, ck, cv, clam, workspace=cws, out=cout5), args.steps)
        ms5v1 = time_fn(lambda: bd.decode(cq, ck, cv, clam, v1_rmsnorm=True, eps=1e-5, workspace=cws, out=cout5),
                        args.steps)
        del cq, ck, cv, clam, cout5, cws
        f3, b5 = w3.prefill_flops(), w5.decode_kv_bytes()
        long_cfg = {
            "prefill": {"value": f3 / (ms3 * 1e-3) / 1e12, "unit": "TFLOP/s", "ms_per_launch": ms3,
                        "frac": f3 / (ms3 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "algorithmic_flops_per_launch": f3,
                        "traffic": _traffic("prefill_long"),
                        "workload": f"{w3.name}: B={w3.B} T={w3.T} Hq={w3.Hq} Hkv={w3.Hkv} d={w3.d} causal bf16"},
            "decode": {"value": b5 / (ms5 * 1e-3) / 1e9, "unit": "GB/s", "ms_per_launch": ms5,
                       "frac": b5 / (ms5 * 1e-3) / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": b5,
                       "traffic": _traffic("decode_long"),
                       "splits": bd.diffattn_decode_num_splits(w5.B, w5.T, w5.Hq, w5.Hkv, w5.d),
                       "workload": f"{w5.name}: B={w5.B} L={w5.T} Hq={w5.Hq} Hkv={w5.Hkv} d={w5.d} bf16"},
            "decode_v1_mode": {"value": b5 / (ms5v1 * 1e-3) / 1e9, "unit": "GB/s", "ms_per_launch": ms5v1,
                               "frac": b5 / (ms5v1 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                               "workload": f"{w5.name}, V1 reference mode (RMSNorm after the difference)"},
            "inputs": "drawn on the device: torch bf16 normals (q, k, v scaled 1/sqrt(2) for the prefill), "
                      "lambda = sigmoid(N(0,1)), seeded"}

    src_p = ["prefill_bf16.hip", "dev_common.h"]
    src_d = ["decode_bf16.hip", "dev_common.h"]
    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms_total / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded normals; no dataset)"}
    if do_p:
        tflops = wp.prefill_flops() / (ms_pre * 1e-3) / 1e12
        res.update(value=tflops, unit="TFLOP/s")
        res["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": tflops / PEAK_BF16_TFLOPS, "traffic": _traffic("prefill"),
                           "kernel": "prefill_kernel<128, 0>", "ms_per_launch": ms_pre,
                           "algorithmic_flops_per_launch": wp.prefill_flops()}
    if do_d:
        gbs = wd.decode_kv_bytes() / (ms_dec * 1e-3) / 1e9
        res["decode"] = {"value": gbs, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "ms_per_launch": ms_dec,
                         "workload": f"{wd.name}: B={wd.B} L={wd.T} Hq={wd.Hq} Hkv={wd.Hkv} d={wd.d} bf16",
                         "splits": bd.diffattn_decode_num_splits(wd.B, wd.T, wd.Hq, wd.Hkv, wd.d)}
        res["roofline_decode"] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": gbs / PEAK_HBM_GBS, "traffic": _traffic("decode"),
                                  "kernel": ("decode_split_kernel<128, 128>" if bd.diffattn_decode_num_splits(
                                      wd.B, wd.T, wd.Hq, wd.Hkv, wd.d) == 1 else
                                             "decode_split_kernel<128, 128> + decode_combine_kernel<128>"),
                                  "algorithmic_bytes_per_launch": wd.decode_kv_bytes()}
        if not do_p:
            res.update(value=gbs, unit="GB/s")
    if serving is not None:
        res["serving"] = serving
    if layouts is not None:
        res["decode_layouts"] = layouts
    if projections is not None:
        res["projections"] = projections
    if long_cfg is not None:
        res["long_configs"] = long_cfg
    if bwd is not None:
        res["backward"] = bwd
        if not (do_p or do_d):
            res.update(value=bwd["value"], unit="TFLOP/s")
    res["config"] = {"workload": (f"{wp.name}: B={wp.B} T={wp.T} Hq={wp.Hq} Hkv={wp.Hkv} d={wp.d} causal bf16"
                                  if do_p else None),
                     "decode_workload": wd.name if do_d else None,
                     "global_batch": wp.B, "seq_len": wp.T, "parallelism": "none (1 GPU)"}
    if not args.no_cpu_baseline and do_p:
        res["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    order = ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
             "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "decode", "roofline_decode",
             "backward", "serving", "decode_layouts", "projections", "long_configs", "cpu_baseline"]
    print(json.dumps({k: res[k] for k in order if k in res}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
