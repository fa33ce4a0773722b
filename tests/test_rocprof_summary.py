"""Host logic of the rocprofv3 summariser: kernel statistics, HBM traffic scaling and
MFMA utilisation, on small synthetic CSV files."""
import csv
import json

import pytest

from differential_attention_v2_amd import rocprof_summary as rs

KN = "void diffattn::(anonymous namespace)::prefill_kernel<128>(diffattn::(anonymous namespace)::Args)"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def _counters(path, recs):
    """recs: (dispatch, kernel, counter, value, start_ns, end_ns)"""
    return _write(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                         "End_Timestamp"], recs)


def test_short_names():
    assert rs._short(KN) == "prefill_kernel<128>"
    assert rs._short("void foo(int)") == "foo"


def test_stats_last_dispatches(tmp_path):
    stats = _write(tmp_path / "s.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
                   [[KN, 3, 2000, 1000, 3000, 100.0]])
    trace = _write(tmp_path / "t.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
                   [[KN, 0, 1000], [KN, 5000, 8000], [KN, 10000, 12000]])
    out = tmp_path / "o.txt"
    rs.main(["stats", stats, "--trace", trace, "--last", "2", "--cmd", "c", "--title", "t", "--out", str(out)])
    text = out.read_text()
    # mean of the last two dispatches by start time: (3000 + 2000) / 2 ns = 2.5 us
    line = [ln for ln in text.splitlines() if ln.startswith("prefill_kernel<128>") and ln.split()[1] == "2"][0]
    assert float(line.split()[2]) == pytest.approx(2.5)


def test_traffic_scaled_by_copy_calibration(tmp_path):
    # a 1 MiB copy reads FETCH 512 KiB (factor 2) and WRITE 1024 KiB (factor 1)
    cf = _counters(tmp_path / "cf.csv", [(1, "void copyBuffer(x)", "FETCH_SIZE", 512.0, 0, 1)])
    cw = _counters(tmp_path / "cw.csv", [(1, "void copyBuffer(x)", "WRITE_SIZE", 1024.0, 0, 1)])
    fe = _counters(tmp_path / "fe.csv", [(1, KN, "FETCH_SIZE", 100.0, 0, 1), (2, KN, "FETCH_SIZE", 300.0, 0, 1),
                                          (3, KN, "FETCH_SIZE", 200.0, 0, 1)])
    wr = _counters(tmp_path / "wr.csv", [(1, KN, "WRITE_SIZE", 50.0, 0, 1)])
    js = tmp_path / "traffic.json"
    rs.main(["traffic", "--fetch", fe, "--write", wr, "--copy-fetch", cf, "--copy-write", cw,
             "--copy-bytes", str(1 << 20), "--kernel", "prefill=prefill_kernel<128>:prefill_bf16.hip:1000",
             "--cmd", "c", "--title", "t", "--out", str(tmp_path / "o.txt"), "--json", str(js)])
    rec = json.loads(js.read_text())["prefill"]
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    assert rec["read_bytes_per_launch"] == pytest.approx(200.0 * 2.0 * 1024)   # median FETCH x factor
    assert rec["write_bytes_per_launch"] == pytest.approx(50.0 * 1024)
    assert rec["source_hash"] == rs.source_hash(["prefill_bf16.hip"])


def test_util_clock_and_mfma_share(tmp_path):
    # 100 us at 2.0 GHz on every XCD -> GRBM_GUI_ACTIVE = 8 x 200000; a quarter of the
    # SIMD cycles busy -> MFMA busy = 0.25 x 200000 x 1024
    recs = []
    for d in (1, 2, 3):
        recs += [(d, KN, "GRBM_GUI_ACTIVE", 8 * 200000.0, 0, 100000),
                 (d, KN, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 200000 * 1024, 0, 100000),
                 (d, KN, "SQ_INSTS_MFMA", 1600000.0, 0, 100000),
                 (d, "void at::native::k(x)", "GRBM_GUI_ACTIVE", 8.0, 0, 10)]
    c = _counters(tmp_path / "u.csv", recs)
    out = tmp_path / "u.txt"
    rs.main(["util", c, "--skip", "at::", "--cmd", "c", "--title", "t", "--out", str(out)])
    rows = [ln.split() for ln in out.read_text().splitlines() if ln.startswith("prefill_kernel")]
    assert len(rows) == 1 and not any(ln.startswith("at::") for ln in out.read_text().splitlines())
    _, n, dur, clk, busy, insts = rows[0]
    assert int(n) == 3
    assert float(dur) == pytest.approx(100.0)
    assert float(clk) == pytest.approx(2.0)
    assert float(busy) == pytest.approx(25.0)
    assert float(insts) == pytest.approx(1600000)
