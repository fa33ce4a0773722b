"""Decode in the layouts V2 is compared against, through the C ABI vs the fp64
oracle (needs an MI355X): a standard transformer (one softmax per head) and
DIFF V1 (q and k halves per branch, the full V read once per branch).  Bar:
max-abs <= 2e-2, mean-abs <= 2e-3; V1 with its per-head RMSNorm (unit-RMS
output) is checked by relative L2 <= 1e-2."""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_v2_amd import binding as bd
from differential_attention_v2_amd import workloads as W

from _helpers import assert_parity, from_device, to_device

pytestmark = pytest.mark.gpu


def _inputs(B, L, H, Hkv, d, seed, dev):
    inp = W.make_compare_decode(B, L, H, Hkv, d, seed)
    t = [to_device(inp[n], "bf16", dev) for n in ("q", "k", "v")]
    f = [W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")]
    return inp, t + [torch.from_numpy(inp["lam"]).to(dev)], f


@pytest.mark.parametrize("shape", [(4, 1000, 32, 8, 128), (3, 777, 8, 2, 64), (2, 300, 16, 1, 128)])
def test_standard_decode(gpu_device, shape):
    B, L, H, Hkv, d = shape
    inp, (q, k, v, lam), f = _inputs(B, L, H, Hkv, d, 9000 + L, gpu_device)
    for splits in (0, 1, 7):
        got = from_device(bd.decode_standard(q, k, v, num_splits=splits))
        assert_parity(got, oracle.standard_decode(*f), f"standard B{B} L{L} H{H} Hkv{Hkv} d{d} splits={splits}")


@pytest.mark.parametrize("shape", [(4, 1000, 32, 8, 128), (3, 777, 8, 2, 64)])
def test_v1_layout_decode(gpu_device, shape):
    B, L, H, Hkv, d = shape
    inp, (q, k, v, lam), f = _inputs(B, L, H, Hkv, d, 9100 + L, gpu_device)
    got = from_device(bd.decode_v1_layout(q, k, v, lam, v1_rmsnorm=False))
    assert_parity(got, oracle.v1_layout_decode(*f, inp["lam"], v1_rmsnorm=False), f"V1 layout no norm d{d}")
    got = from_device(bd.decode_v1_layout(q, k, v, lam, v1_rmsnorm=True, num_splits=5))
    ref = oracle.v1_layout_decode(*f, inp["lam"], v1_rmsnorm=True)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"[parity] V1 layout with RMSNorm d{d}: rel_l2={rel:.3e}", flush=True)
    assert np.isfinite(got).all() and rel <= 1e-2


def test_compare_B64_L8192_cache_shape(gpu_device):
    """B=64, L=8192, Hkv=8, d=128 caches with H=32 heads (the V2 workload's 32 pairs), 4 sequences checked."""
    inp, (q, k, v, lam), f = _inputs(64, 8192, 32, 8, 128, 9200, gpu_device)
    sel = np.array([0, 21, 42, 63])
    got = from_device(bd.decode_standard(q, k, v))[sel]
    assert_parity(got, oracle.standard_decode(*f, batches=sel), "standard, B=64 L=8192 cache")
    got = from_device(bd.decode_v1_layout(q, k, v, lam, v1_rmsnorm=False))[sel]
    assert_parity(got, oracle.v1_layout_decode(*f, inp["lam"], v1_rmsnorm=False, batches=sel), "V1 layout, B=64 L=8192 cache")
