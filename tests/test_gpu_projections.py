"""The projections on either side of the attention core through the C ABI vs the
fp64 oracle (needs an MI355X).  lambda: fp32 accumulation of exact bf16
products, so max-abs <= 1e-4; O_W: bf16 output of unit-variance values, the
usual bar (max-abs <= 2e-2, mean-abs <= 2e-3, rel-L2 <= 1e-2)."""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_v2_amd import binding as bd
from differential_attention_v2_amd import workloads as W

from _helpers import assert_parity, from_device, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,dm,P", [(4096, 4096, 32), (100, 512, 16), (37, 1024, 64), (50, 1536, 48), (16, 8192, 32)])
def test_lambda_projection(gpu_device, rows, dm, P):
    inp = W.make_projections(rows, dm, P, 512, 512, seed=6100 + rows)
    x, w = to_device(inp["x"], "bf16", gpu_device), to_device(inp["w_lambda"], "bf16", gpu_device)
    got = from_device(bd.lambda_proj(x, w))
    ref = oracle.lambda_projection(W.to_f64(inp["x"], "bf16"), W.to_f64(inp["w_lambda"], "bf16"))
    assert_parity(got, ref, f"lambda projection rows={rows} d_model={dm} P={P}", max_abs=1e-4, mean_abs=1e-5)


@pytest.mark.parametrize("rows,kin,nout", [(4096, 4096, 4096), (77, 512, 384), (300, 1024, 264), (5, 32, 8),
                                          (257, 64, 520), (1000, 8192, 1024), (1, 96, 4096)])
def test_output_projection(gpu_device, rows, kin, nout):
    """The library's own GEMM (256 x 256 tiles, 32-wide k steps): full and ragged
    row and column tiles, one, two and many k steps."""
    inp = W.make_projections(rows, 512, 16, kin, nout, seed=6200 + rows)
    a, wo = to_device(inp["attn"], "bf16", gpu_device), to_device(inp["w_o"], "bf16", gpu_device)
    got = from_device(bd.output_proj(a, wo))
    sel = np.unique(np.concatenate([np.arange(min(rows, 16)), np.arange(max(0, rows - 16), rows),
                                    np.random.default_rng(3).choice(rows, min(rows, 32), replace=False)]))
    ref = oracle.output_projection(W.to_f64(inp["attn"], "bf16")[sel], W.to_f64(inp["w_o"], "bf16"))
    assert_parity(got[sel], ref, f"O_W rows={rows} in={kin} out={nout} ({sel.size} rows)")


def test_lambda_feeds_prefill(gpu_device):
    """End to end: lambda from the producer drives the prefill; parity against the oracle chain."""
    w = W.Workload("proj_chain", "prefill", "bf16", B=1, T=128, Hq=32, Hkv=2, d=128, qkv_scale=0.7, seed=6300)
    pre = W.make_prefill(w)
    inp = W.make_projections(w.T, 512, w.P, 512, 512, seed=6301)
    lam = bd.lambda_proj(to_device(inp["x"], "bf16", gpu_device),
                         to_device(inp["w_lambda"], "bf16", gpu_device)).view(1, w.T, w.P)
    q, k, v = (to_device(pre[n], "bf16", gpu_device) for n in ("q", "k", "v"))
    got = from_device(bd.prefill(q, k, v, lam))
    lam_ref = oracle.lambda_projection(W.to_f64(inp["x"], "bf16"), W.to_f64(inp["w_lambda"], "bf16"))
    ref = oracle.diffattn_prefill(*(W.to_f64(pre[n], "bf16") for n in ("q", "k", "v")), lam_ref[None])
    assert_parity(got, ref, "lambda producer -> prefill")


def test_output_projection_matches_library_gemm(gpu_device):
    """Every element of the 4096 x 4096 x 4096 product against torch's bf16 matmul
    (hipBLASLt, fp32 accumulation): both round an fp32 sum to bf16, so they may
    differ by accumulation order only."""
    inp = W.make_projections(4096, 512, 16, 4096, 4096, seed=6250)
    a, wo = to_device(inp["attn"], "bf16", gpu_device), to_device(inp["w_o"], "bf16", gpu_device)
    got = bd.output_proj(a, wo).float()
    ref = torch.matmul(a, wo).float()
    err = (got - ref).abs()
    print(f"[parity] O_W vs torch.matmul: max_abs={err.max().item():.3e} mean_abs={err.mean().item():.3e}", flush=True)
    # one bf16 rounding step apart at most: 2^-8 of the value, 2^-7 at a binade's low end
    assert bool((err <= ref.abs() * 2.0 ** -7 + 1e-4).all())
