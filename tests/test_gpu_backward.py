"""Training forward and backward pass: HIP path vs the fp64 oracle (needs an MI355X).

Every call goes through libdiffattn's C ABI.  The training forward's `out` must
equal the plain prefill's bit for bit; `o2` meets the forward bar and `lse` an
absolute 4e-3 (its denominator sums bf16-rounded weights: relative error up to
2^-9).  Gradients are compared relative to their own scale, since they are not
O(1): max |got - ref| <= 2e-2 * max(max|ref|, 1) and
mean |got - ref| <= 1e-2 * max(mean|ref|, 0.1) (P and dS enter the MFMA products
as bf16; D = dout . O_r is formed from the saved bf16 out and o2, so even an
exactly zero gradient, as dq of a one-token sequence, carries rounding of the
order of 2^-9 |dout| |v|; the floors are the scale of a gradient of an O(1) loss).
"""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_v2_amd import binding as bd
from differential_attention_v2_amd import workloads as W

from _helpers import assert_parity, errors, from_device, to_device

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 2e-2, 1e-2


def _case(B, T, Hq, Hkv, d, causal=True, seed=7001, scale=1.0 / np.sqrt(2.0)):
    return W.Workload(f"bwd_B{B}_T{T}_Hq{Hq}_Hkv{Hkv}_d{d}", "prefill", "bf16", B=B, T=T, Hq=Hq, Hkv=Hkv, d=d,
                      qkv_scale=scale, causal=causal, seed=seed)


def _run(w, dev):
    inp = W.make_prefill(w)
    dout_np = W.make_dout(w)
    q, k, v = (to_device(inp[n], "bf16", dev) for n in ("q", "k", "v"))
    lam = torch.from_numpy(inp["lam"]).to(dev)
    dout = to_device(dout_np, "bf16", dev)
    out, o2, lse = bd.prefill_train(q, k, v, lam, causal=w.causal)
    grads = bd.prefill_backward(q, k, v, lam, out, o2, lse, dout, causal=w.causal)
    torch.cuda.synchronize()
    f64 = {n: W.to_f64(inp[n], "bf16") for n in ("q", "k", "v")}
    return inp, dout_np, f64, (q, k, v, lam, dout), (out, o2, lse), grads


def _assert_rel(got, ref, what):
    e = errors(got, ref)
    scale_max = float(np.max(np.abs(ref)))
    scale_mean = float(np.mean(np.abs(ref)))
    print(f"[parity] {what}: max_abs={e['max_abs']:.3e} (ref max {scale_max:.3e}) mean_abs={e['mean_abs']:.3e} "
          f"(ref mean {scale_mean:.3e}) rel_l2={e['rel_l2']:.3e}", flush=True)
    assert e["nonfinite"] == 0, (what, e)
    assert e["max_abs"] <= REL_MAX * max(scale_max, 1.0), (what, e)
    assert e["mean_abs"] <= REL_MEAN * max(scale_mean, 0.1), (what, e)


def _check_grads(w, dev, groups=None):
    inp, dout_np, f, dev_in, saved, grads = _run(w, dev)
    dq, dk, dv, dlam = (from_device(t) for t in grads)
    rq, rk, rv, rl = oracle.diffattn_prefill_bwd(f["q"], f["k"], f["v"], inp["lam"], W.to_f64(dout_np, "bf16"),
                                                 causal=w.causal, groups=groups)
    if groups is not None:   # compare the heads, KV heads and pairs of the sampled groups only
        hq = np.concatenate([np.arange(2 * w.G * g, 2 * w.G * (g + 1)) for g in groups])
        pp = np.concatenate([np.arange(w.G * g, w.G * (g + 1)) for g in groups])
        dq, rq = dq[:, :, hq], rq[:, :, hq]
        dk, rk, dv, rv = dk[:, :, groups], rk[:, :, groups], dv[:, :, groups], rv[:, :, groups]
        dlam, rl = dlam[:, :, pp], rl[:, :, pp]
    _assert_rel(dq, rq, f"{w.name} dq")
    _assert_rel(dk, rk, f"{w.name} dk")
    _assert_rel(dv, rv, f"{w.name} dv")
    _assert_rel(dlam, rl, f"{w.name} dlambda")
    return dev_in, saved, grads


def test_training_forward_matches_prefill_and_oracle(gpu_device):
    w = _case(2, 300, 16, 2, 128)
    inp, dout_np, f, (q, k, v, lam, dout), (out, o2, lse), _ = _run(w, gpu_device)
    plain = bd.prefill(q, k, v, lam, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16)), "training forward changed out"
    r_out, r_o2, r_lse = oracle.prefill_saved(f["q"], f["k"], f["v"], inp["lam"], causal=True)
    assert_parity(from_device(out), r_out, "train fwd out")
    assert_parity(from_device(o2), r_o2, "train fwd o2")
    assert_parity(from_device(lse), r_lse, "train fwd lse", max_abs=4e-3, mean_abs=1e-3)


@pytest.mark.parametrize("shape", [
    (1, 96, 8, 2, 128, True),      # one partial key block, 3 query tiles
    (2, 300, 16, 2, 64, True),     # ragged T, G = 4, d = 64
    (1, 200, 8, 1, 128, False),    # non-causal
    (1, 1100, 4, 2, 128, True),    # G = 1, several key blocks and query chunks
    (1, 64, 16, 1, 64, True),      # G = 8
    (1, 1, 8, 2, 128, True),       # a single token
    (1, 33, 8, 2, 64, False),      # one row past a tile
    (1, 1300, 16, 2, 64, False),   # non-causal over several query chunks, d = 64
    (2, 700, 24, 4, 128, True),    # G = 3 (a partial pair chunk), two batches
])
def test_backward_small(gpu_device, shape):
    B, T, Hq, Hkv, d, causal = shape
    _check_grads(_case(B, T, Hq, Hkv, d, causal, seed=7000 + T), gpu_device)


def test_backward_T4096_sampled_groups(gpu_device):
    """The bench shape (B=1, T=4096, Hq=64, Hkv=8, d=128, causal), two KV groups checked in full."""
    w = W.PREFILL_T4096
    _check_grads(w, gpu_device, groups=[0, 5])


def test_backward_lambda_zero_and_determinism(gpu_device):
    w = _case(1, 160, 8, 2, 128, seed=7100)
    inp = W.make_prefill(w)
    q, k, v = (to_device(inp[n], "bf16", gpu_device) for n in ("q", "k", "v"))
    lam = torch.zeros((w.B, w.T, w.P), dtype=torch.float32, device=gpu_device)
    dout = to_device(W.make_dout(w), "bf16", gpu_device)
    out, o2, lse = bd.prefill_train(q, k, v, lam)
    g1 = bd.prefill_backward(q, k, v, lam, out, o2, lse, dout)
    g2 = bd.prefill_backward(q, k, v, lam, out, o2, lse, dout)
    torch.cuda.synchronize()
    assert torch.all(g1[0][:, :, 1::2] == 0), "lambda = 0: the subtracted heads get no gradient"
    assert torch.equal(g1[0].view(torch.int16), g2[0].view(torch.int16)), "dq must be deterministic"
    assert torch.equal(g1[3], g2[3]), "dlambda must be deterministic"
    for a, b in ((g1[1], g2[1]), (g1[2], g2[2])):   # dk, dv: fp32 atomics, order may vary
        assert torch.allclose(a.float(), b.float(), rtol=1e-2, atol=1e-3)


def test_backward_rejects(gpu_device):
    w = _case(1, 64, 8, 2, 128)
    inp = W.make_prefill(w)
    q, k, v = (to_device(inp[n], "bf16", gpu_device) for n in ("q", "k", "v"))
    lam = torch.from_numpy(inp["lam"]).to(gpu_device)
    out, o2, lse = bd.prefill_train(q, k, v, lam)
    dout = torch.zeros_like(out)
    small = torch.empty(16, dtype=torch.uint8, device=gpu_device)
    with pytest.raises(bd.DiffAttnError) as e:
        bd.prefill_backward(q, k, v, lam, out, o2, lse, dout, workspace=small)
    assert e.value.status == bd.DIFFATTN_ERR_WORKSPACE
