"""Pins of the fp64 backward oracle to facts other than itself.

- central finite differences of L = sum(dout * out), computed through the
  forward oracle, on tiny shapes (V2 and V1 mode, causal and not): a dropped
  term, a wrong sign or a transposed operand in any of the four gradients fails;
- an independent torch fp64 autograd implementation of the forward (written here
  with torch ops, differentiated by torch) on a medium shape;
- special cases: lambda = 0 (the subtracted head gets no gradient; dK, dV equal
  torch's SDPA backward of the positive heads alone); Q2 = Q1 with lambda = 1
  (the output is 0 for any K, V, so dK = dV = 0 and dQ1 = -dQ2);
- identities: shifting every key by one vector leaves every output unchanged, so
  sum_j dK_j = 0 per (b, KV head); sum_j dV_j = sum over the group's pairs and
  rows of (1 - lam) dout (each softmax row sums to one).
"""
import math

import numpy as np
import pytest
import torch

from oracle import diffattn_prefill, diffattn_prefill_bwd, prefill_saved


def _rand(rng, B=1, T=6, Hq=4, Hkv=1, d=8):
    q = rng.standard_normal((B, T, Hq, d))
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    lam = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hq // 2))))
    dout = rng.standard_normal((B, T, Hq // 2, d))
    return q, k, v, lam, dout


def _loss(q, k, v, lam, dout, causal, v1):
    return float(np.sum(dout * diffattn_prefill(q, k, v, lam, causal=causal, v1_rmsnorm=v1)))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("v1", [False, True])
def test_finite_differences(causal, v1):
    rng = np.random.default_rng(11 + causal + 2 * v1)
    q, k, v, lam, dout = _rand(rng, B=1, T=5, Hq=4, Hkv=1, d=6)
    if v1:
        lam = lam - 0.3 * rng.standard_normal(lam.shape)   # V1 lambda may be any real
    dq, dk, dv, dlam = diffattn_prefill_bwd(q, k, v, lam, dout, causal=causal, v1_rmsnorm=v1)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv), (lam, dlam)):
        num = np.empty_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + h
            lp = _loss(q, k, v, lam, dout, causal, v1)
            x[i] = old - h
            lm = _loss(q, k, v, lam, dout, causal, v1)
            x[i] = old
            num[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def _torch_forward(q, k, v, lam, causal):
    """The forward map in torch ops (own code, not the oracle's): [B,T,Hq,d] etc."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // (2 * Hkv)
    kk = k.repeat_interleave(2 * G, dim=2)        # query head h reads KV head h // (2G)
    vv = v.repeat_interleave(2 * G, dim=2)
    s = torch.einsum("bihc,bjhc->bhij", q, kk) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    o = torch.einsum("bhij,bjhc->bihc", torch.softmax(s, dim=-1), vv)
    return o[:, :, 0::2] - lam[..., None] * o[:, :, 1::2]


@pytest.mark.parametrize("causal", [True, False])
def test_matches_independent_torch_autograd(causal):
    rng = np.random.default_rng(5)
    q, k, v, lam, dout = _rand(rng, B=2, T=40, Hq=8, Hkv=2, d=16)
    ts = [torch.tensor(x, requires_grad=True) for x in (q, k, v, lam)]
    out = _torch_forward(*ts, causal)
    out.backward(torch.tensor(dout))
    ref = [t.grad.numpy() for t in ts]
    got = diffattn_prefill_bwd(q, k, v, lam, dout, causal=causal)
    for r, g in zip(ref, got):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


def test_lambda_zero_reduces_to_sdpa_backward():
    rng = np.random.default_rng(6)
    q, k, v, lam, dout = _rand(rng, B=1, T=24, Hq=4, Hkv=1, d=8)
    lam[:] = 0.0
    dq, dk, dv, dlam = diffattn_prefill_bwd(q, k, v, lam, dout, causal=True)
    assert np.all(dq[:, :, 1::2] == 0.0)
    # torch SDPA (fp64) backward of the positive heads 0 and 2, both on KV head 0
    tq = torch.tensor(q[:, :, 0::2].transpose(0, 2, 1, 3).copy(), requires_grad=True)   # [B, 2, T, d]
    tk = torch.tensor(np.repeat(k.transpose(0, 2, 1, 3), 2, axis=1).copy(), requires_grad=True)
    tv = torch.tensor(np.repeat(v.transpose(0, 2, 1, 3), 2, axis=1).copy(), requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    o.backward(torch.tensor(dout.transpose(0, 2, 1, 3).copy()))
    np.testing.assert_allclose(dq[:, :, 0::2], tq.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk[:, :, 0], tk.grad.numpy().sum(axis=1), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv[:, :, 0], tv.grad.numpy().sum(axis=1), rtol=1e-10, atol=1e-12)
    out, o2, _ = prefill_saved(q, k, v, lam, causal=True)
    np.testing.assert_allclose(dlam, -np.sum(dout * o2, axis=-1), rtol=1e-12, atol=1e-14)


def test_identical_branches_with_lambda_one_cancel():
    rng = np.random.default_rng(7)
    q, k, v, lam, dout = _rand(rng, B=1, T=20, Hq=4, Hkv=1, d=8)
    q[:, :, 1::2] = q[:, :, 0::2]
    lam[:] = 1.0
    dq, dk, dv, dlam = diffattn_prefill_bwd(q, k, v, lam, dout, causal=True)
    assert np.max(np.abs(dk)) < 1e-12 and np.max(np.abs(dv)) < 1e-12
    np.testing.assert_allclose(dq[:, :, 0::2], -dq[:, :, 1::2], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_shift_invariance_and_row_sums(causal):
    rng = np.random.default_rng(8)
    q, k, v, lam, dout = _rand(rng, B=2, T=33, Hq=8, Hkv=2, d=8)
    dq, dk, dv, dlam = diffattn_prefill_bwd(q, k, v, lam, dout, causal=causal)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-11)
    G = 2
    for g in range(2):
        pairs = slice(g * G, (g + 1) * G)
        want = ((1.0 - lam[:, :, pairs])[..., None] * dout[:, :, pairs]).sum(axis=(1, 2))
        np.testing.assert_allclose(dv[:, :, g].sum(axis=1), want, rtol=1e-10, atol=1e-11)


def test_saved_values():
    """o2 is the subtracted branch alone, lse its row normaliser: checked against torch fp64."""
    rng = np.random.default_rng(9)
    q, k, v, lam, dout = _rand(rng, B=1, T=30, Hq=4, Hkv=1, d=8)
    out, o2, lse = prefill_saved(q, k, v, lam, causal=True)
    np.testing.assert_allclose(out, diffattn_prefill(q, k, v, lam, causal=True), rtol=1e-12, atol=1e-13)
    s = torch.einsum("bihc,bjc->bhij", torch.tensor(q), torch.tensor(k[:, :, 0])) / math.sqrt(8)
    s = s.masked_fill(torch.triu(torch.ones(30, 30, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy().transpose(0, 2, 1), rtol=1e-12)
    o = torch.einsum("bhij,bjc->bihc", torch.softmax(s, -1), torch.tensor(v[:, :, 0])).numpy()
    np.testing.assert_allclose(o2, o[:, :, 1::2], rtol=1e-12, atol=1e-13)
