"""The decode entry point that allocates nothing (needs an MI355X).

diffattn_decode_fwd_noalloc keeps the key-range records in a fixed device array
inside the library instead of a caller workspace.  Called through the C ABI, its
output must equal the workspace entry point's (same kernels, same split plan) on
two calls in a row, the second with a smaller problem, and it must match the fp64
oracle.  Sizes beyond the array are refused on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from differential_attention_v2_amd import binding as bd
from differential_attention_v2_amd import workloads as W

from _helpers import assert_parity, from_device, to_device

pytestmark = pytest.mark.gpu


def _inputs(w, dev):
    inp = W.make_decode(w)
    t = {n: to_device(inp[n], "bf16", dev) for n in ("q", "k", "v")}
    t["lam"] = torch.from_numpy(inp["lam"]).to(dev)
    return inp, t


def _noalloc(w, t, out, splits, v1=False):
    torch.cuda.synchronize()
    st = bd.diffattn_decode_fwd_noalloc(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                        t["lam"].data_ptr(), out.data_ptr(), w.B, w.T, w.Hq, w.Hkv, w.d,
                                        bd.DIFFATTN_BF16, bd.DIFFATTN_FLAG_V1_RMSNORM if v1 else 0, 1e-5, splits,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == bd.DIFFATTN_OK, bd.status_string(st)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("v1", [False, True])
def test_noalloc_decode_matches_workspace_decode(gpu_device, v1):
    dev = gpu_device
    # first call: 16 key ranges per (b, KV head), so every record goes through the
    # fixed array and the combine kernel; second call: a smaller problem with
    # another head count and head dim, whose records cover only part of the array
    big = W.Workload("na_big", "decode", "bf16", B=4, T=20000, Hq=64, Hkv=8, d=128, seed=8101)
    small = W.Workload("na_small", "decode", "bf16", B=2, T=3000, Hq=16, Hkv=2, d=64, seed=8102)
    for w, splits in ((big, 0), (small, 5)):
        inp, t = _inputs(w, dev)
        S = bd.diffattn_decode_num_splits(w.B, w.T, w.Hq, w.Hkv, w.d) if splits == 0 else splits
        assert S > 1
        ref_dev = bd.decode(t["q"], t["k"], t["v"], t["lam"], v1_rmsnorm=v1, eps=1e-5, num_splits=splits)
        got = _noalloc(w, t, torch.empty_like(ref_dev), splits, v1)
        assert torch.equal(got, ref_dev), f"{w.name}: differs from the workspace entry point"
        ref = oracle.diffattn_decode(*(W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")), inp["lam"],
                                     v1_rmsnorm=v1, eps=1e-5)
        if v1:
            # unit-RMS outputs: compared at the scale of the difference (as in the prefill V1 test)
            x = oracle.diffattn_decode(*(W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")), inp["lam"])
            r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-5)
            assert_parity(from_device(got) * r, x, f"no-alloc decode {w.name} V1 at the scale of x")
        else:
            assert_parity(from_device(got), ref, f"no-alloc decode {w.name}")


def test_noalloc_decode_refuses_records_beyond_the_array(gpu_device):
    # B * Hq * splits * (d + 4) * 4 bytes > 32 MiB: refused before anything is enqueued
    P = 0x7F0000000000
    assert bd.diffattn_decode_fwd_noalloc(P, P, P, P, P, 64, 8192, 64, 8, 128, bd.DIFFATTN_BF16, 0, 1e-5, 64,
                                          None) == bd.DIFFATTN_ERR_WORKSPACE
