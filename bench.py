#!/usr/bin/env python3
"""Benchmark of the Differential Attention V2 forward hot path on one MI355X.

A step is one pass of the whole path over synthetic inputs already resident in
HBM, on the largest single-GPU workloads: one causal bf16 prefill (B=1,
T=32768, Hq=64, Hkv=8, d=128) followed by one bf16 split-KV decode (B=8,
L=131072, Hq=64, Hkv=8, d=128; key ranges merged by the combine kernel).  Both
use the seeded host generator's exact bytes, the ones the parity tests check.
Each launch is bracketed by HIP events on the stream it runs on; `value` is the
prefill's algorithmic TFLOP/s (4*d flops per visible query-key-head, causal)
over its median launch time, and the decode's KV-cache GB/s (every K/V byte
once) is reported beside it.  Rank 0 prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 50] [--settle-ms 300] [--no-cpu-baseline]

After the main step the same line carries, each timed on its own (medians over
--steps launches): the T=4096 prefill and B=64, L=8192 decode, the decode in V1
reference mode, the training forward + backward, the serving variants, the
decode layout comparison, the projections either side of the core, the SNR of
the signal-plus-noise variant read from the device's outputs, and the fp64
oracle timed on the host's cores.

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
SECTIONS = ("main", "short", "backward", "serving", "layouts", "projections", "snr")
BACKWARD_KERNELS = "bwd_pre + fill_zero + bwd_dkdv_kernel<128> + bwd_dq_kernel<128> + 2 x convert"
OUTPUT_PROJ_ENGINES = {"output_proj": "gemm_bf16_kernel (this library: 256x256 tiles, bf16 MFMA, fp32 accumulate)",
                       "output_proj_library": "torch.matmul (hipBLASLt, bf16, fp32 accumulate): baseline"}


def _kernel_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "differential_attention_v2_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _traffic(kind: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kind]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != _kernel_hash(rec["sources"]):
        return None
    return rec.get("bytes_per_launch")


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


# ----------------------------------------------------------------------------
# the oracle on the host's cores
# ----------------------------------------------------------------------------
def progress(section: str) -> None:
    """One line on stderr per finished section (the JSON result goes to stdout)."""
    print(f"bench.py: section {section} done", file=sys.stderr, flush=True)


def cpu_baseline() -> dict:
    """The fp64 oracle, as it stands, on each workload: in full where it takes
    seconds, otherwise on a labelled sample extrapolated to the whole workload."""
    import numpy as np
    import oracle
    from differential_attention_v2_amd import workloads as W
    blas_threads, vendor = os.cpu_count(), "unknown"
    try:
        import threadpoolctl
        blas = [i for i in threadpoolctl.threadpool_info() if i["user_api"] == "blas"]
        if blas:
            blas_threads = sum(i.get("num_threads", 0) for i in blas)
            vendor = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in blas)
    except Exception:  # noqa: BLE001
        pass
    f32 = W.bf16_to_f32
    per = {}

    def clock(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # T=128 fp32 prefill and T=4096 bf16 prefill: every row of every pair
    for w in (W.TINY_PREFILL_FP32, W.PREFILL_T4096):
        inp = W.make_prefill(w)
        q, k, v = ((f32(inp[n]) if w.dtype == "bf16" else inp[n]) for n in ("q", "k", "v"))
        dt = clock(lambda: oracle.diffattn_prefill(q, k, v, inp["lam"], causal=w.causal))
        per[w.name] = {"seconds": dt, "sample": "full", "value": w.prefill_flops() / dt / 1e12,
                       "unit": "TFLOP/s"}
    # B=64, L=8192 decode: every (sequence, pair)
    w = W.DECODE_B64_L8192
    inp = W.make_decode(w)
    q, k, v = (f32(inp[n]) for n in ("q", "k", "v"))
    del inp["k"], inp["v"]
    dt = clock(lambda: oracle.diffattn_decode(q, k, v, inp["lam"]))
    per[w.name] = {"seconds": dt, "sample": "full", "value": w.decode_kv_bytes() / dt / 1e9, "unit": "GB/s"}
    del q, k, v
    # B=8, L=131072 decode: 2 of the 8 sequences (all pairs), scaled by 4
    w = W.DECODE_B8_L131072
    ws = w.with_(B=2)
    inp = W.make_decode(ws)
    q, k, v = (f32(inp[n]) for n in ("q", "k", "v"))
    del inp["k"], inp["v"]
    dt = clock(lambda: oracle.diffattn_decode(q, k, v, inp["lam"]))
    full = dt * w.B / ws.B
    per[w.name] = {"seconds": full, "measured_seconds": dt, "extrapolated": True,
                   "sample": f"{ws.B} of {w.B} sequences (same shapes and distributions), all pairs; "
                             f"time x {w.B // ws.B}",
                   "value": w.decode_kv_bytes() / full / 1e9, "unit": "GB/s"}
    del q, k, v
    # T=32768 prefill: four runs of 64 consecutive query rows ending at T/4, T/2,
    # 3T/4 and T, all pairs; a row costs in proportion to its visible keys, so the
    # full run (all T rows) is extrapolated by sum_i (i + 1) over the sampled sum
    w = W.PREFILL_T32768
    inp = W.make_prefill(w)
    q, k, v = (f32(inp[n]) for n in ("q", "k", "v"))
    lam = inp["lam"]
    del inp
    blocks = [np.arange(e - 64, e) for e in (w.T // 4, w.T // 2, 3 * w.T // 4, w.T)]
    dt = sum(clock(lambda r=r: oracle.diffattn_prefill(q, k, v, lam, rows=r)) for r in blocks)
    keys_sampled = float(sum(64 * (int(r[-1]) + 1) for r in blocks))   # the oracle's block spans keys 0..last row
    keys_full = w.T * (w.T + 1) / 2.0
    full = dt * keys_full / keys_sampled
    per[w.name] = {"seconds": full, "measured_seconds": dt, "extrapolated": True,
                   "sample": "4 runs of 64 consecutive query rows ending at T/4, T/2, 3T/4, T, all 32 pairs; "
                             "time x (sum over all rows of visible keys) / (keys the sampled runs scored)",
                   "value": w.prefill_flops() / full / 1e12, "unit": "TFLOP/s"}
    head = per[w.name]
    return {"value": head["value"], "unit": "TFLOP/s", "cores": int(blas_threads or 1), "kind": "oracle",
            "sample": f"{w.name} (the headline workload): " + head["sample"] + f"; {head['measured_seconds']:.1f} s "
                      f"measured, {full:.0f} s extrapolated for the whole prefill",
            "host_cpu_count": os.cpu_count(), "blas_threads": blas_threads, "blas_vendor": vendor,
            "cores_note": "cores = the BLAS threads the oracle's matrix products run on; its elementwise "
                          "softmax steps run on one thread",
            "per_workload": per}


# ----------------------------------------------------------------------------
# device side
# ----------------------------------------------------------------------------
def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50, help="untimed steps after the clock settle phase")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed wall time of steps before the warmup steps (clock ramp-up); 0 skips it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=SECTIONS, default=None,
                    help="time one part (for profiler runs): main = T=32768 prefill + B=8 L=131072 decode; "
                         "short = T=4096 prefill + B=64 L=8192 decode; backward = training forward + backward; "
                         "serving = windowed prefill + ragged decode; snr = signal-plus-noise SNR")
    for s in SECTIONS[1:]:
        ap.add_argument(f"--no-{s}", action="store_true", help=f"skip the {s} section")
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
    if args.steps < 1:
        print("bench.py: --steps must be >= 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from differential_attention_v2_amd import binding as bd
    from differential_attention_v2_amd import workloads as W

    if not os.path.exists(bd.LIB_PATH):
        from differential_attention_v2_amd import build_lib
        build_lib.build()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    do = {s: (args.only == s) or (args.only is None and not getattr(args, f"no_{s}", False)) for s in SECTIONS}

    def dev_bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    def settle(fn, ms):
        """Run fn for `ms` of wall time (untimed) so the clock is at its sustained level."""
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()

    def time_parts(fn, nparts, steps, warm):
        """Median ms of each of the nparts event-bracketed parts of fn(ev) over `steps` calls."""
        for _ in range(warm):
            fn(None)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nparts + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            fn(evs[i])
        torch.cuda.synchronize()
        return [_median([e[j].elapsed_time(e[j + 1]) for e in evs]) for j in range(nparts)]

    def prefill_inputs(w):
        ip = W.make_prefill(w)
        t = dict(q=dev_bf16(ip["q"]), k=dev_bf16(ip["k"]), v=dev_bf16(ip["v"]),
                 lam=torch.from_numpy(ip["lam"]).to(dev))
        t["out"] = torch.empty((w.B, w.T, w.P, w.d), dtype=torch.bfloat16, device=dev)
        return t

    def decode_inputs(w):
        idc = W.make_decode(w)
        t = dict(q=dev_bf16(idc["q"]), k=dev_bf16(idc["k"]), v=dev_bf16(idc["v"]),
                 lam=torch.from_numpy(idc["lam"]).to(dev))
        t["out"] = torch.empty((w.B, w.P, w.d), dtype=torch.bfloat16, device=dev)
        t["ws"] = bd.decode_workspace(w.B, w.T, w.Hq, w.Hkv, w.d, 0, dev)
        return t

    def run_prefill(t):
        bd.prefill(t["q"], t["k"], t["v"], t["lam"], out=t["out"])

    def run_decode(t, v1=False):
        bd.decode(t["q"], t["k"], t["v"], t["lam"], v1_rmsnorm=v1, eps=1e-5, workspace=t["ws"], out=t["out"])

    def prefill_entry(w, ms, kernel, traffic_key):
        f = w.prefill_flops()
        tf = f / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tf / PEAK_BF16_TFLOPS, "traffic": _traffic(traffic_key), "kernel": kernel,
                "ms_per_launch": ms, "algorithmic_flops_per_launch": f,
                "workload": f"{w.name}: B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} d={w.d} causal bf16"}

    def decode_entry(w, ms, traffic_key):
        b = w.decode_kv_bytes()
        gbs = b / (ms * 1e-3) / 1e9
        S = bd.diffattn_decode_num_splits(w.B, w.T, w.Hq, w.Hkv, w.d)
        kernel = "decode_split_kernel<128, 128>" + ("" if S == 1 else " + decode_combine_kernel<128>")
        return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "traffic": _traffic(traffic_key), "kernel": kernel, "splits": S, "ms_per_launch": ms,
                "algorithmic_bytes_per_launch": b,
                "workload": f"{w.name}: B={w.B} L={w.T} Hq={w.Hq} Hkv={w.Hkv} d={w.d} bf16"}

    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded normals from the host generator; no dataset)"}
    w3, w5 = W.PREFILL_T32768, W.DECODE_B8_L131072
    w2, w4 = W.PREFILL_T4096, W.DECODE_B64_L8192

    # ---- main step: T=32768 prefill + B=8, L=131072 decode ------------------------
    if do["main"]:
        P3, D5 = prefill_inputs(w3), decode_inputs(w5)

        def step(ev):
            if ev: ev[0].record(stream)
            run_prefill(P3)
            if ev: ev[1].record(stream)
            run_decode(D5)
            if ev: ev[2].record(stream)

        settle(lambda: step(None), args.settle_ms)
        for _ in range(args.warmup):
            step(None)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(args.steps):
            step(evs[i])
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_total = t_start.elapsed_time(t_end)
        ms_pre = _median([e[0].elapsed_time(e[1]) for e in evs])
        ms_dec = _median([e[1].elapsed_time(e[2]) for e in evs])
        roof = prefill_entry(w3, ms_pre, "prefill_kernel<128, 0, true> (persistent, per-XCD work queues)", "prefill_long")
        res.update(value=roof["achieved"], unit="TFLOP/s", ms_per_step=ms_total / args.steps)
        res["roofline"] = roof
        res["roofline_decode"] = decode_entry(w5, ms_dec, "decode_long")
        (ms_v1,) = time_parts(lambda ev: (ev and ev[0].record(stream), run_decode(D5, v1=True),
                                          ev and ev[1].record(stream)), 1, args.steps, 3)
        res["decode_v1_mode"] = dict(decode_entry(w5, ms_v1, "decode_long"),
                                     workload=f"{w5.name}, V1 reference mode (RMSNorm after the difference, "
                                              "eps 1e-5)")
        del P3, D5
        torch.cuda.empty_cache()

    if do["main"]:
        progress("main")
    # ---- T=4096 prefill and B=64, L=8192 decode -------------------------------------
    if do["short"]:
        P2, D4 = prefill_inputs(w2), decode_inputs(w4)

        def sstep(ev):
            if ev: ev[0].record(stream)
            run_prefill(P2)
            if ev: ev[1].record(stream)
            run_decode(D4)
            if ev: ev[2].record(stream)

        settle(lambda: sstep(None), min(args.settle_ms, 100.0))
        ms_p2, ms_d4 = time_parts(sstep, 2, args.steps, max(3, args.warmup))
        res["short_configs"] = {"prefill": prefill_entry(w2, ms_p2, "prefill_kernel<128, 0, false>", "prefill"),
                                "decode": decode_entry(w4, ms_d4, "decode")}
        del P2, D4
        torch.cuda.empty_cache()

    if do["short"]:
        progress("short")
    # ---- training forward + backward on the T=4096 prefill ---------------------------
    if do["backward"]:
        P2 = prefill_inputs(w2)
        pq, pk, pv, plam = P2["q"], P2["k"], P2["v"], P2["lam"]
        bdout = dev_bf16(W.make_dout(w2))
        tout, to2, tlse = bd.prefill_train(pq, pk, pv, plam)
        bws = torch.empty(bd.diffattn_prefill_bwd_workspace_bytes(w2.B, w2.T, w2.Hq, w2.Hkv, w2.d),
                          dtype=torch.uint8, device=dev)
        grads = (torch.empty_like(pq), torch.empty_like(pk), torch.empty_like(pv), torch.empty_like(plam))

        def bstep(ev):
            if ev: ev[0].record(stream)
            bd.prefill_train(pq, pk, pv, plam, out=(tout, to2, tlse))
            if ev: ev[1].record(stream)
            bd.prefill_backward(pq, pk, pv, plam, tout, to2, tlse, bdout, workspace=bws, grads=grads)
            if ev: ev[2].record(stream)

        settle(lambda: bstep(None), min(args.settle_ms, 100.0))
        ms_tf, ms_bw = time_parts(bstep, 2, args.steps, max(3, args.warmup // 5))
        bw_tf = w2.prefill_bwd_flops() / (ms_bw * 1e-3) / 1e12
        res["backward"] = {
            "value": bw_tf, "unit": "TFLOP/s", "frac": bw_tf / PEAK_BF16_TFLOPS, "ms_per_launch": ms_bw,
            "algorithmic_flops_per_launch": w2.prefill_bwd_flops(),
            "flop_count": "8*d per visible (query, key, head): dP, dV, dQ, dK products, no recompute",
            "kernels": BACKWARD_KERNELS, "traffic": _traffic("backward"),
            "train_forward_ms": ms_tf, "train_forward_tflops": w2.prefill_flops() / (ms_tf * 1e-3) / 1e12,
            "workload": f"{w2.name} causal bf16, dout ~ N(0,1)"}
        del P2, bdout, tout, to2, tlse, bws, grads
        torch.cuda.empty_cache()

    if do["backward"]:
        progress("backward")
    # ---- serving variants -------------------------------------------------------------
    if do["serving"]:
        # the T=4096 prefill with a 1024-key causal window, and the B=64, L=8192 decode
        # over caches with lengths uniform in [1, 8192]
        SWA = 1024
        P2, D4 = prefill_inputs(w2), decode_inputs(w4)
        lens_np = W.ragged_lengths(w4.B, w4.T)
        lens = torch.from_numpy(lens_np).to(dev)
        vws = torch.empty(bd.diffattn_decode_varlen_workspace_bytes(w4.B, w4.T, w4.Hq, w4.Hkv, w4.d, 0),
                          dtype=torch.uint8, device=dev)

        def vstep(ev):
            if ev: ev[0].record(stream)
            bd.prefill_window(P2["q"], P2["k"], P2["v"], P2["lam"], SWA, out=P2["out"])
            if ev: ev[1].record(stream)
            bd.decode_varlen(D4["q"], D4["k"], D4["v"], D4["lam"], seq_lens=lens, workspace=vws, out=D4["out"])
            if ev: ev[2].record(stream)

        settle(lambda: vstep(None), min(args.settle_ms, 100.0))
        ms_sw, ms_vl = time_parts(vstep, 2, args.steps, max(3, args.warmup // 2))
        vl_bytes = 2.0 * float(lens_np.sum()) * w4.Hkv * w4.d * 2
        fw = w2.prefill_flops(SWA)
        res["serving"] = {
            "prefill_window": {"value": fw / (ms_sw * 1e-3) / 1e12, "unit": "TFLOP/s",
                               "ms_per_launch": ms_sw, "window": SWA, "algorithmic_flops_per_launch": fw,
                               "kernel": "prefill_kernel<128, 1, false>", "traffic": _traffic("prefill_window"),
                               "frac": fw / (ms_sw * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                               "workload": f"{w2.name} causal, window {SWA}"},
            "decode_varlen": {"value": vl_bytes / (ms_vl * 1e-3) / 1e9, "unit": "GB/s", "ms_per_launch": ms_vl,
                              "traffic": _traffic("decode_varlen"), "algorithmic_bytes_per_launch": vl_bytes,
                              "frac": vl_bytes / (ms_vl * 1e-3) / 1e9 / PEAK_HBM_GBS,
                              "workload": f"{w4.name} with lengths uniform in [1, {w4.T}] (mean "
                                          f"{float(lens_np.mean()):.0f})"}}
        del P2, D4, lens, vws
        torch.cuda.empty_cache()

    if do["serving"]:
        progress("serving")
    # ---- decode layouts: standard transformer, DIFF V1, V2 ---------------------------
    if do["layouts"]:
        # the pages' decode-speed claim on the B=64, L=8192 cache geometry (Hkv=8,
        # d=128): a standard transformer with H=32 heads, DIFF V1 with the same 32
        # heads (q, k halves per branch, V read once per branch) and V2 (64 query
        # heads = 32 pairs)
        H = w4.P
        ic = W.make_compare_decode(w4.B, w4.T, H, w4.Hkv, w4.d, seed=9300)
        cq, ck, cv = dev_bf16(ic["q"]), dev_bf16(ic["k"]), dev_bf16(ic["v"])
        clam = torch.from_numpy(ic["lam"]).to(dev)
        del ic
        D4 = decode_inputs(w4)
        cws = torch.empty(bd.diffattn_decode_compare_workspace_bytes(w4.B, w4.T, H, w4.Hkv, w4.d, 0),
                          dtype=torch.uint8, device=dev)
        cout = torch.empty((w4.B, H, w4.d), dtype=torch.bfloat16, device=dev)
        runs = {"standard": lambda: bd.decode_standard(cq, ck, cv, workspace=cws, out=cout),
                "v1_layout": lambda: bd.decode_v1_layout(cq, ck, cv, clam, workspace=cws, out=cout),
                "v2": lambda: run_decode(D4)}
        cache = w4.B * w4.T * w4.Hkv * w4.d * 2
        bytes_read = {"standard": 2.0 * cache, "v1_layout": 3.0 * cache, "v2": 2.0 * cache}
        layouts = {}
        for name, fn in runs.items():
            settle(fn, min(args.settle_ms, 100.0))
            (ms,) = time_parts(lambda ev, fn=fn: (ev and ev[0].record(stream), fn(), ev and ev[1].record(stream)),
                               1, args.steps, max(3, args.warmup // 2))
            layouts[name] = {"ms_per_launch": ms, "cache_bytes_read": bytes_read[name],
                             "GB_per_s": bytes_read[name] / (ms * 1e-3) / 1e9}
        for name in ("v1_layout", "v2"):
            layouts[name]["time_vs_standard"] = layouts[name]["ms_per_launch"] / layouts["standard"]["ms_per_launch"]
        layouts["workload"] = (f"B={w4.B} L={w4.T} Hkv={w4.Hkv} d={w4.d} bf16 cache; standard and V1: {H} heads; "
                               f"V2: {w4.Hq} query heads ({w4.P} pairs)")
        res["decode_layouts"] = layouts
        del cq, ck, cv, clam, D4, cws, cout
        torch.cuda.empty_cache()

    if do["layouts"]:
        progress("layouts")
    # ---- projections either side of the core ------------------------------------------
    if do["projections"]:
        # lambda for 4096 tokens x 32 pairs from d_model = 4096, and O_W from P*d = 4096
        # back to d_model = 4096: this library's kernel and rocBLAS on the same operands
        rows, dm, kin = w2.B * w2.T, w2.P * w2.d, w2.P * w2.d
        ij = W.make_projections(rows, dm, w2.P, kin, dm)
        jx, jw = dev_bf16(ij["x"]), dev_bf16(ij["w_lambda"])
        ja, jo = dev_bf16(ij["attn"]), dev_bf16(ij["w_o"])
        del ij
        jl = torch.empty((rows, w2.P), dtype=torch.float32, device=dev)
        jy = torch.empty((rows, dm), dtype=torch.bfloat16, device=dev)
        jruns = {"lambda_proj": lambda: bd.lambda_proj(jx, jw, out=jl),
                 "output_proj": lambda: bd.output_proj(ja, jo, out=jy)}
        # the same product by torch's library GEMM (hipBLASLt), as a baseline
        jy2 = torch.empty_like(jy)
        jruns["output_proj_library"] = lambda: torch.matmul(ja, jo, out=jy2)
        jt = {}
        for name, fn in jruns.items():
            settle(fn, min(args.settle_ms, 100.0))
            (jt[name],) = time_parts(lambda ev, fn=fn: (ev and ev[0].record(stream), fn(),
                                                        ev and ev[1].record(stream)),
                                     1, args.steps, max(3, args.warmup // 2))
        lp_bytes = rows * dm * 2.0 + w2.P * dm * 2.0 + rows * w2.P * 4.0
        op_flops = 2.0 * rows * kin * dm
        proj = {"lambda_proj": {"value": lp_bytes / (jt["lambda_proj"] * 1e-3) / 1e9, "unit": "GB/s",
                                "ms_per_launch": jt["lambda_proj"], "algorithmic_bytes_per_launch": lp_bytes,
                                "frac": lp_bytes / (jt["lambda_proj"] * 1e-3) / 1e9 / PEAK_HBM_GBS, "bound": "hbm",
                                "workload": f"x [{rows}, {dm}] bf16, w [{w2.P}, {dm}] -> lambda [{rows}, {w2.P}] fp32"}}
        for name in ("output_proj", "output_proj_library"):
            if name in jt:
                tf = op_flops / (jt[name] * 1e-3) / 1e12
                proj[name] = {"value": tf, "unit": "TFLOP/s", "ms_per_launch": jt[name],
                              "algorithmic_flops_per_launch": op_flops, "frac": tf / PEAK_BF16_TFLOPS,
                              "bound": "mfma", "engine": OUTPUT_PROJ_ENGINES[name],
                              "workload": f"[{rows}, {kin}] x [{kin}, {dm}] bf16"}
        res["projections"] = proj
        del jx, jw, ja, jo, jl, jy, jy2
        torch.cuda.empty_cache()

    if do["projections"]:
        progress("projections")
    # ---- signal-plus-noise SNR from the device's outputs --------------------------------
    if do["snr"]:
        res["snr"] = snr_section(W, bd, torch, np, dev, dev_bf16)

    res["config"] = {"workload": f"{w3.name}: B={w3.B} T={w3.T} Hq={w3.Hq} Hkv={w3.Hkv} d={w3.d} causal bf16",
                     "decode_workload": f"{w5.name}: B={w5.B} L={w5.T} Hq={w5.Hq} Hkv={w5.Hkv} d={w5.d} bf16",
                     "global_batch": w3.B, "seq_len": w3.T, "parallelism": "none (1 GPU)",
                     "timing": f"median of {args.steps} HIP-event-bracketed launches per kernel"}
    if "value" not in res:
        # a partial run (--only): report the first timed section as the value
        for key in ("short_configs", "backward", "serving", "projections"):
            if key in res:
                first = res[key]["prefill"] if key == "short_configs" else (
                    res[key] if key == "backward" else next(iter(res[key].values())))
                res.update(value=first["achieved"] if "achieved" in first else first["value"],
                           unit=first["unit"])
                break
        res.setdefault("ms_per_step", None)
    if do["snr"]:
        progress("snr")
    if not args.no_cpu_baseline and do["main"]:
        res["cpu_baseline"] = cpu_baseline()
    order = ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
             "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "roofline_decode", "decode_v1_mode",
             "short_configs", "backward", "serving", "decode_layouts", "projections", "snr", "cpu_baseline"]
    print(json.dumps({k: res[k] for k in order if k in res}), flush=True)
    return 0


def snr_section(W, bd, torch, np, dev, dev_bf16) -> dict:
    """The signal-plus-noise variant of the T=32768 prefill (differential-attention
    lesson, 建立它 / 步骤4): 16 keys per probe row set to 4 q/|q|, the rest N(0, 1).
    With value columns that are 0/1 indicators of each probe's planted keys plus an
    all-ones column, the prefill's output holds each probe's planted mass and row
    sum; run once with the workload's lambda (A1 - lambda A2) and once with lambda = 0
    (A1).  SNR = mean weight on the planted keys / signed mean weight on the other
    visible keys; gain = differential SNR / standard SNR."""
    w = W.PREFILL_T32768
    n_sig = 16
    inp = W.plant_signal(w, W.make_prefill(w), n_signal=n_sig)
    plan = inp["plan"]
    v_ind, col = W.signal_indicator_v(w, plan)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(v_ind)
    lam = torch.from_numpy(inp["lam"]).to(dev)
    out_d = bd.prefill(q, k, v, lam).float().cpu().numpy()
    out_s = bd.prefill(q, k, v, torch.zeros_like(lam)).float().cpu().numpy()
    ones = col["ones"]
    rows = []
    for b, p, i, _ in plan:
        c, n = col[(b, p, i)], i + 1
        lam_i = float(inp["lam"][b, i, p])
        sd, rd = float(out_d[b, i, p, c]), float(out_d[b, i, p, ones])
        ss, rs = float(out_s[b, i, p, c]), float(out_s[b, i, p, ones])
        snr_s = (ss / n_sig) / ((rs - ss) / (n - n_sig))
        snr_d = (sd / n_sig) / ((rd - sd) / (n - n_sig))
        rows.append((lam_i, snr_s, snr_d, rd - (1.0 - lam_i), ss))
    a = np.array(rows)
    gain = a[:, 2] / a[:, 1]
    bins = []
    for lo, hi in ((0.0, 0.3), (0.3, 0.5), (0.5, 0.67), (0.67, 0.8), (0.8, 0.9), (0.9, 1.0)):
        m = (a[:, 0] >= lo) & (a[:, 0] < hi)
        if m.any():
            bins.append({"lambda": [lo, hi], "probes": int(m.sum()), "gain_median": float(np.median(gain[m])),
                         "gain_min": float(gain[m].min()), "gain_max": float(gain[m].max()),
                         "inv_one_minus_lambda_median": float(np.median(1.0 / (1.0 - a[m, 0])))})
    band = (a[:, 0] >= 0.67) & (a[:, 0] <= 0.9)
    return {"workload": f"{w.name} signal-plus-noise: {len(plan)} probe rows (8 per pair, 16 planted keys each "
                        "at 4 q/|q| of the pair's first head), other keys N(0,1)",
            "probes": len(plan), "planted_mass_median": float(np.median(a[:, 4])),
            "standard_snr_median": float(np.median(a[:, 1])), "differential_snr_median": float(np.median(a[:, 2])),
            "gain_median": float(np.median(gain)), "gain_by_lambda": bins,
            "lambda_0.67_0.9": {"probes": int(band.sum()),
                                "in_3x_to_10x": int(((gain >= 3) & (gain <= 10) & band).sum()),
                                "gain_min": float(gain[band].min()) if band.any() else None,
                                "gain_max": float(gain[band].max()) if band.any() else None},
            "row_sum_max_dev_from_1_minus_lambda": float(np.abs(a[:, 3]).max()),
            "source": "device outputs only (indicator values); the GPU test checks them against the oracle"}


if __name__ == "__main__":
    sys.exit(main())
