"""Summarise rocprofv3 CSV output into short text reports and HBM-traffic records.

    # kernel-trace statistics (from rocprofv3 --kernel-trace --stats --output-format csv)
    python -m differential_attention_v2_amd.rocprof_summary stats DIR/run_kernel_stats.csv \
        --cmd "<the rocprofv3 command>" --title "..." --out profiles/NAME.txt

    # MFMA utilisation and effective shader clock from one counter run of
    # GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA
    python -m differential_attention_v2_amd.rocprof_summary util DIR/run_counter_collection.csv \
        --cmd "..." --title "..." --out profiles/NAME.txt

    # HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE runs, scaled by what the
    # same counters read for a plain device copy of known size
    python -m differential_attention_v2_amd.rocprof_summary traffic \
        --fetch DIR/run_counter_collection.csv --write DIR/run_counter_collection.csv \
        --copy-fetch DIR/... --copy-write DIR/... --copy-bytes N \
        --kernel prefill=prefill_kernel<128>:prefill_bf16.hip,dev_common.h:ALGO_BYTES \
        --cmd "..." --out profiles/NAME.txt --json profiles/traffic.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "differential_attention_v2_amd", "csrc")


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = name.replace("diffattn::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "")


def cmd_stats(a) -> None:
    rows = list(csv.DictReader(open(a.csv)))
    lines = [f"# {a.title}", "", "command:", f"  {a.cmd}", "",
             f"{'kernel':48s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share%':>7s}"]
    for r in rows:
        lines.append(f"{_short(r['Name'])[:48]:48s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} "
                     f"{float(r['MinNs'])/1e3:10.2f} {float(r['MaxNs'])/1e3:10.2f} {float(r['Percentage']):7.2f}")
    if a.trace:
        # the last N dispatches of each kernel: the steps that bench.py times
        per = {}
        for r in csv.DictReader(open(a.trace)):
            per.setdefault(_short(r["Kernel_Name"]), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        lines += ["", f"last {a.last} dispatches of each kernel (the timed steps):",
                  f"{'kernel':48s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
        for k, v in per.items():
            if len(v) < a.last:
                continue
            d = [x[1] / 1e3 for x in sorted(v)[-a.last:]]
            lines.append(f"{k[:48]:48s} {len(d):6d} {statistics.mean(d):10.2f} {min(d):10.2f} {max(d):10.2f}")
    if a.note:
        lines += ["", a.note]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_kernel(path: str) -> dict:
    vals = {}
    for r in csv.DictReader(open(path)):
        vals.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return vals


def cmd_traffic(a) -> None:
    n = a.copy_bytes / 1024.0   # KiB moved each way by one copy dispatch
    cf = _per_kernel(a.copy_fetch)
    cw = _per_kernel(a.copy_write)
    copy_name = [k for k in cf if "copyBuffer" in k or "copy" in k.lower()][0]
    f_fetch = n / statistics.median(cf[copy_name])
    f_write = n / statistics.median(cw[copy_name])
    fe, wr = _per_kernel(a.fetch), _per_kernel(a.write)
    lines = [f"# {a.title}", "", "commands:"] + [f"  {c}" for c in a.cmd] + [
        "", f"calibration: copy of {a.copy_bytes} B per dispatch: FETCH_SIZE reads "
            f"{statistics.median(cf[copy_name]):.1f} KiB (factor {f_fetch:.4f}), WRITE_SIZE reads "
            f"{statistics.median(cw[copy_name]):.1f} KiB (factor {f_write:.4f})", "",
        f"{'kernel':40s} {'FETCH KiB':>12s} {'WRITE KiB':>12s} {'read MB':>10s} {'write MB':>10s} {'algo MB':>10s}"]
    out = json.load(open(a.json)) if (a.json and os.path.exists(a.json)) else {}
    for spec in a.kernel:
        key, rest = spec.split("=", 1)
        names, srcs, algo = rest.split(":")
        total_r = total_w = 0.0
        for kname in names.split("+"):
            match = [k for k in fe if k.startswith(kname)]
            if not match:
                raise SystemExit(f"kernel {kname} not in counter data: {list(fe)}")
            k = match[0]
            fk, wk = statistics.median(fe[k]), statistics.median(wr[k])
            rb, wb = fk * f_fetch * 1024, wk * f_write * 1024
            total_r += rb
            total_w += wb
            lines.append(f"{kname[:40]:40s} {fk:12.1f} {wk:12.1f} {rb/1e6:10.2f} {wb/1e6:10.2f} {'':>10s}")
        lines.append(f"{'  = ' + key + ' per launch':40s} {'':12s} {'':12s} {total_r/1e6:10.2f} {total_w/1e6:10.2f} "
                     f"{float(algo)/1e6:10.2f}")
        src_list = srcs.split(",")
        out[key] = {"kernels": names.split("+"), "sources": src_list, "source_hash": source_hash(src_list),
                    "read_bytes_per_launch": total_r, "write_bytes_per_launch": total_w,
                    "bytes_per_launch": total_r + total_w, "algorithmic_bytes": float(algo),
                    "fetch_factor": f_fetch, "write_factor": f_write}
    open(a.out, "w").write("\n".join(lines) + "\n")
    if a.json:
        json.dump(out, open(a.json, "w"), indent=1)
    print("\n".join(lines))


XCDS = 8      # MI355X: GRBM_GUI_ACTIVE is summed over the 8 XCDs
SIMDS = 1024  # 256 CUs x 4 SIMDs


def cmd_util(a) -> None:
    """Per kernel (medians over dispatches): duration, effective shader clock
    (GRBM_GUI_ACTIVE per XCD / duration) and MFMA busy share of all SIMD cycles."""
    per = {}
    for r in csv.DictReader(open(a.csv)):
        d = per.setdefault(_short(r["Kernel_Name"]), {})
        key = (r["Dispatch_Id"])
        rec = d.setdefault(key, {"dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
        rec[r["Counter_Name"]] = float(r["Counter_Value"])
    lines = [f"# {a.title}", "", "command:", f"  {a.cmd}", "",
             f"{'kernel':44s} {'dispatches':>10s} {'dur_us':>9s} {'sclk_GHz':>9s} {'mfma_busy%':>10s} "
             f"{'mfma_insts':>12s}"]
    for k, recs in per.items():
        if any(k.startswith(pre) for pre in a.skip):
            continue
        ok = [x for x in recs.values() if "GRBM_GUI_ACTIVE" in x and x["dur"] > 0]
        if not ok:
            continue
        dur = statistics.median(x["dur"] for x in ok)
        clk = statistics.median(x["GRBM_GUI_ACTIVE"] / XCDS / x["dur"] for x in ok) / 1e9
        busy = [x["SQ_VALU_MFMA_BUSY_CYCLES"] / (x["GRBM_GUI_ACTIVE"] / XCDS * SIMDS) * 100
                for x in ok if "SQ_VALU_MFMA_BUSY_CYCLES" in x]
        insts = [x["SQ_INSTS_MFMA"] for x in ok if "SQ_INSTS_MFMA" in x]
        lines.append(f"{k[:44]:44s} {len(ok):10d} {dur * 1e6:9.1f} {clk:9.3f} "
                     f"{(statistics.median(busy) if busy else float('nan')):10.1f} "
                     f"{(statistics.median(insts) if insts else float('nan')):12.0f}")
    if a.note:
        lines += ["", a.note]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--trace", default=None, help="run_kernel_trace.csv, for the mean of the last dispatches")
    s.add_argument("--last", type=int, default=20)
    s.add_argument("--out", required=True)
    u = sub.add_parser("util")
    u.add_argument("csv")
    u.add_argument("--cmd", required=True)
    u.add_argument("--title", required=True)
    u.add_argument("--note", default="")
    u.add_argument("--out", required=True)
    u.add_argument("--skip", action="append", default=[], help="kernel-name prefix to leave out (repeatable)")
    t = sub.add_parser("traffic")
    for n in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + n.replace("_", "-"), dest=n, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", action="append", required=True,
                   help="key=name[+name]:src[,src]:algorithmic_bytes")
    t.add_argument("--cmd", action="append", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--json", default=None)
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "util": cmd_util}[a.what](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
