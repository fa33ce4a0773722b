"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a library
routine in a special case (torch's CPU scaled-dot-product attention in fp64), a
closed form, an invariant, or brute force written as plain Python loops.  A
plausible slip in the oracle (wrong scale, swapped branch, wrong pair->KV-head
map, off-by-one in the causal mask, lambda indexed by the wrong axis, RMSNorm
applied before the difference) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (attention_weights, diffattn_decode, diffattn_prefill, rmsnorm,
                    snr, softmax_rows, v1_lambda)


def _rand(rng, B=2, T=37, Hq=8, Hkv=2, d=16):
    q = rng.standard_normal((B, T, Hq, d))
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    lam = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hq // 2))))
    return q, k, v, lam


def _sdpa(q, k, v, causal):
    """torch fp64 CPU SDPA of one head: q [B,T,d], k/v [B,N,d] -> [B,T,d]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[:, None]  # noqa: E731
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    return o[:, 0].numpy()


# --------------------------------------------------------------------------
# library routine in special cases
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
def test_lambda_zero_is_standard_gqa_attention(causal):
    """lambda = 0 leaves the pure first softmax (lesson exercise 4): head 2p over KV head p//G."""
    rng = np.random.default_rng(1)
    q, k, v, lam = _rand(rng)
    G = q.shape[2] // (2 * k.shape[2])
    out = diffattn_prefill(q, k, v, np.zeros_like(lam), causal=causal)
    for p in range(q.shape[2] // 2):
        ref = _sdpa(q[:, :, 2 * p], k[:, :, p // G], v[:, :, p // G], causal)
        np.testing.assert_allclose(out[:, :, p], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_full_formula_against_sdpa_branches(causal):
    """out = SDPA(head 2p) - lambda[b,i,p] * SDPA(head 2p+1): branch order and lambda axis."""
    rng = np.random.default_rng(2)
    q, k, v, lam = _rand(rng, B=2, T=29, Hq=12, Hkv=3, d=8)
    G = 2
    out = diffattn_prefill(q, k, v, lam, causal=causal)
    for p in range(6):
        g = p // G
        o1 = _sdpa(q[:, :, 2 * p], k[:, :, g], v[:, :, g], causal)
        o2 = _sdpa(q[:, :, 2 * p + 1], k[:, :, g], v[:, :, g], causal)
        np.testing.assert_allclose(out[:, :, p], o1 - lam[:, :, p, None] * o2, rtol=1e-11, atol=1e-12)


def test_decode_matches_sdpa_last_row():
    rng = np.random.default_rng(3)
    B, L, Hq, Hkv, d = 3, 50, 8, 1, 16
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, L, Hkv, d))
    v = rng.standard_normal((B, L, Hkv, d))
    lam = rng.uniform(0, 1, (B, Hq // 2))
    out = diffattn_decode(q, k, v, lam)
    for p in range(Hq // 2):
        o1 = _sdpa(q[:, None, 2 * p], k[:, :, 0], v[:, :, 0], False)[:, 0]
        o2 = _sdpa(q[:, None, 2 * p + 1], k[:, :, 0], v[:, :, 0], False)[:, 0]
        np.testing.assert_allclose(out[:, p], o1 - lam[:, p, None] * o2, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms and invariants
# --------------------------------------------------------------------------
def test_identical_branches_cancel_exactly():
    """Q2 := Q1 and lambda = 1: the shared map cancels to exactly zero (lesson, differential idea)."""
    rng = np.random.default_rng(4)
    q, k, v, lam = _rand(rng)
    q[:, :, 1::2] = q[:, :, 0::2]
    out = diffattn_prefill(q, k, v, np.ones_like(lam))
    assert np.all(out == 0.0)
    # general lambda: (1 - lambda) * SDPA(Q1)
    out = diffattn_prefill(q, k, v, lam)
    for p in range(4):
        ref = _sdpa(q[:, :, 2 * p], k[:, :, p // 2], v[:, :, p // 2], True)
        np.testing.assert_allclose(out[:, :, p], (1 - lam[:, :, p, None]) * ref, rtol=1e-11, atol=1e-12)


def test_row_sums_one_minus_lambda():
    """Each row of A1 - lambda*A2 sums to 1 - lambda, so constant V gives (1 - lambda) * c."""
    rng = np.random.default_rng(5)
    q, k, v, lam = _rand(rng, d=8)
    c = rng.standard_normal(8)
    v[:] = c
    out = diffattn_prefill(q, k, v, lam)
    np.testing.assert_allclose(out, (1 - lam)[..., None] * c, rtol=1e-12, atol=1e-13)
    # and the weights themselves
    a1 = attention_weights(q[0, :, 0], k[0, :, 0], np.arange(q.shape[1]), True)
    a2 = attention_weights(q[0, :, 1], k[0, :, 0], np.arange(q.shape[1]), True)
    np.testing.assert_allclose((a1 - lam[0, :, 0, None] * a2).sum(-1), 1 - lam[0, :, 0], rtol=1e-13)


def test_pair_to_kv_group_map():
    """V constant per KV head g: pair p reads KV head p // G (adjacent pairs share a group)."""
    rng = np.random.default_rng(6)
    B, T, Hq, Hkv, d = 1, 21, 16, 2, 4
    q, k, v, lam = _rand(rng, B, T, Hq, Hkv, d)
    cg = np.array([[1.0, 2.0, 3.0, 4.0], [-5.0, 6.0, -7.0, 8.0]])
    v[:, :, 0] = cg[0]
    v[:, :, 1] = cg[1]
    out = diffattn_prefill(q, k, v, lam)
    G = Hq // (2 * Hkv)
    for p in range(Hq // 2):
        np.testing.assert_allclose(out[:, :, p], (1 - lam[:, :, p, None]) * cg[p // G], rtol=1e-12)


def test_causal_first_row_sees_only_itself():
    rng = np.random.default_rng(7)
    q, k, v, lam = _rand(rng)
    out = diffattn_prefill(q, k, v, lam)
    for p in range(4):
        np.testing.assert_allclose(out[:, 0, p], (1 - lam[:, 0, p, None]) * v[:, 0, p // 2], rtol=1e-12)


def test_causal_ignores_future_keys():
    rng = np.random.default_rng(8)
    q, k, v, lam = _rand(rng)
    i = 17
    out = diffattn_prefill(q, k, v, lam)
    k2, v2 = k.copy(), v.copy()
    k2[:, i + 1:] = rng.standard_normal(k2[:, i + 1:].shape) * 10
    v2[:, i + 1:] = rng.standard_normal(v2[:, i + 1:].shape) * 10
    out2 = diffattn_prefill(q, k2, v2, lam)
    np.testing.assert_array_equal(out[:, : i + 1], out2[:, : i + 1])
    assert not np.allclose(out[:, i + 1:], out2[:, i + 1:])


def test_zero_query_gives_prefix_mean():
    """q = 0 makes every visible key equally likely: weight 1/(i+1), the noise-floor picture."""
    rng = np.random.default_rng(9)
    q, k, v, lam = _rand(rng)
    q[:] = 0
    out = diffattn_prefill(q, k, v, lam)
    T = q.shape[1]
    prefix = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None, None]
    for p in range(4):
        np.testing.assert_allclose(out[:, :, p], (1 - lam[:, :, p, None]) * prefix[:, :, p // 2], rtol=1e-12, atol=1e-13)


def test_two_key_closed_form_pins_scale():
    """Row 1 of a causal length-2 sequence: weight on key 0 = 1/(1 + exp((s1 - s0))) with s = q.k/sqrt(d)."""
    d = 9
    q = np.zeros((1, 2, 2, d))
    k = np.zeros((1, 2, 1, d))
    v = np.zeros((1, 2, 1, d))
    q[0, 1, 0, 0] = 3.0
    q[0, 1, 1, 1] = -2.0
    k[0, 0, 0, :2] = [1.0, 0.5]
    k[0, 1, 0, :2] = [-0.5, 1.5]
    v[0, 0, 0, 0] = 1.0
    v[0, 1, 0, 1] = 1.0
    lam = np.full((1, 2, 1), 0.3)
    out = diffattn_prefill(q, k, v, lam)
    s = lambda a, b: a @ b / 3.0  # noqa: E731  sqrt(9) = 3
    w1 = 1 / (1 + math.exp(s(q[0, 1, 0], k[0, 1, 0]) - s(q[0, 1, 0], k[0, 0, 0])))
    w2 = 1 / (1 + math.exp(s(q[0, 1, 1], k[0, 1, 0]) - s(q[0, 1, 1], k[0, 0, 0])))
    np.testing.assert_allclose(out[0, 1, 0, :2], [w1 - 0.3 * w2, (1 - w1) - 0.3 * (1 - w2)], rtol=1e-14)


def test_sampled_rows_equal_full_rows():
    rng = np.random.default_rng(10)
    q, k, v, lam = _rand(rng, T=70)
    full = diffattn_prefill(q, k, v, lam, row_block=16)
    rows = np.array([0, 5, 33, 34, 69])
    part = diffattn_prefill(q, k, v, lam, rows=rows)
    np.testing.assert_allclose(part, full[:, rows], rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# brute force on tiny inputs: plain Python, unnormalised exponentials
# --------------------------------------------------------------------------
def _brute(q, k, v, lam, causal):
    B, T, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    G = Hq // (2 * Hkv)
    out = [[[[0.0] * d for _ in range(Hq // 2)] for _ in range(T)] for _ in range(B)]
    for b in range(B):
        for i in range(T):
            for p in range(Hq // 2):
                g = p // G
                mix = [0.0] * d
                for branch, coef in ((2 * p, 1.0), (2 * p + 1, -lam[b][i][p])):
                    keys = range(i + 1) if causal else range(T)
                    e = [math.exp(sum(q[b][i][branch][c] * k[b][j][g][c] for c in range(d)) / math.sqrt(d))
                         for j in keys]
                    z = sum(e)
                    for w, j in zip(e, keys):
                        for c in range(d):
                            mix[c] += coef * (w / z) * v[b][j][g][c]
                out[b][i][p] = mix
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_tiny(causal):
    rng = np.random.default_rng(11)
    q, k, v, lam = _rand(rng, B=2, T=6, Hq=4, Hkv=1, d=3)
    ref = np.array(_brute(q.tolist(), k.tolist(), v.tolist(), lam.tolist(), causal))
    np.testing.assert_allclose(diffattn_prefill(q, k, v, lam, causal=causal), ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# decode vs prefill, V1 mode
# --------------------------------------------------------------------------
def test_decode_equals_prefill_last_row():
    rng = np.random.default_rng(12)
    q, k, v, lam = _rand(rng, B=2, T=33)
    L = 33
    pre = diffattn_prefill(q, k, v, lam, rows=[L - 1])[:, 0]
    dec = diffattn_decode(q[:, L - 1], k, v, lam[:, L - 1])
    np.testing.assert_allclose(dec, pre, rtol=1e-13, atol=1e-14)
    pre1 = diffattn_prefill(q, k, v, lam, rows=[L - 1], v1_rmsnorm=True)[:, 0]
    dec1 = diffattn_decode(q[:, L - 1], k, v, lam[:, L - 1], v1_rmsnorm=True)
    np.testing.assert_allclose(dec1, pre1, rtol=1e-13, atol=1e-14)


def test_v1_lambda_closed_forms():
    z = np.zeros((3, 5))
    np.testing.assert_allclose(v1_lambda(z, z, z, z, 0.8), [0.8] * 3, rtol=0, atol=1e-15)
    lq1 = np.array([[1.0, 0.0]]); lk1 = np.array([[2.0, 7.0]])
    lq2 = np.array([[0.5, 0.5]]); lk2 = np.array([[1.0, 1.0]])
    np.testing.assert_allclose(v1_lambda(lq1, lk1, lq2, lk2, 0.8), [math.e ** 2 - math.e + 0.8], rtol=1e-15)
    # may be negative (key terms: lambda can be negative)
    assert v1_lambda(lq2, lk2, lq1, lk1, 0.8)[0] < 0


def test_rmsnorm_after_difference():
    """V1 mode normalises x = o1 - lambda*o2 (not each branch): mean(y^2) = m/(m+eps)."""
    rng = np.random.default_rng(13)
    q, k, v, lam = _rand(rng)
    eps = 1e-3
    x = diffattn_prefill(q, k, v, lam)
    y = diffattn_prefill(q, k, v, lam, v1_rmsnorm=True, eps=eps)
    m = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), m / (m + eps), rtol=1e-12)
    np.testing.assert_allclose(y * np.sqrt(m + eps)[..., None], x, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(rmsnorm(np.array([[3.0, 4.0]]), 0.0), [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]])


def test_softmax_rows_masked_entries_are_zero():
    s = np.array([[0.0, -np.inf, 1.0], [5.0, 5.0, -np.inf]])
    a = softmax_rows(s)
    assert a[0, 1] == 0.0 and a[1, 2] == 0.0
    np.testing.assert_allclose(a[1, :2], [0.5, 0.5], rtol=1e-15)
    np.testing.assert_allclose(a[0, [0, 2]], [1 / (1 + math.e), math.e / (1 + math.e)], rtol=1e-15)


# --------------------------------------------------------------------------
# the signal-plus-noise toy
# --------------------------------------------------------------------------
def _toy_row(rng, N, d, lam):
    q1 = rng.standard_normal(d) / math.sqrt(2)
    q2 = rng.standard_normal(d) / math.sqrt(2)
    k = rng.standard_normal((N, d))
    pos = rng.choice(N, 16, replace=False)
    k[pos] = 4 * q1 / np.linalg.norm(q1)
    a1 = attention_weights(q1[None], k, np.array([N - 1]), False)[0]
    a2 = attention_weights(q2[None], k, np.array([N - 1]), False)[0]
    return a1, a2, pos


def test_snr_absolute_values_worked_by_hand():
    """Rows worked out by hand (SNR = mean weight on the signal positions over the
    signed mean weight on the other visible positions)."""
    # signal {0, 2}: mean 0.3; others {1, 3, 4}: mean 0.4/3; the sixth entry is not visible
    w = np.array([0.4, 0.1, 0.2, 0.1, 0.2, 0.9])
    assert snr(w, [0, 2], 5) == pytest.approx(0.3 / (0.4 / 3), rel=1e-15)      # 2.25
    # a differential row whose unrelated weights average below zero: the SNR is negative
    w = np.array([0.2, -0.1, 0.05, 0.02])
    assert snr(w, [0], 4) == pytest.approx(0.2 / (-0.03 / 3), rel=1e-12)         # -20
    # uniform weights carry no signal: SNR 1
    assert snr(np.full(10, 0.1), [3, 7], 10) == pytest.approx(1.0, rel=1e-15)


@pytest.mark.parametrize("N", [1024, 32768])
def test_snr_identity_from_row_sums(N):
    """SNR_diff/SNR_std = ((s1 - lam s2)/s1) (1 - s1) / ((1 - s1) - lam (1 - s2)) with s_r = signal mass."""
    rng = np.random.default_rng(14)
    for lam in (0.3, 0.6, 0.85):
        a1, a2, pos = _toy_row(rng, N, 64, lam)
        s1, s2 = a1[pos].sum(), a2[pos].sum()
        ratio = snr(a1 - lam * a2, pos, N) / snr(a1, pos, N)
        expect = ((s1 - lam * s2) / s1) * (1 - s1) / ((1 - s1) - lam * (1 - s2))
        np.testing.assert_allclose(ratio, expect, rtol=1e-9)


def test_snr_gain_three_to_ten_fold():
    """The lesson's toy claim: differential attention gives 3x-10x the SNR of softmax attention.

    Holds in the long-context, small-signal regime (N = 32768, d = 128, 16
    planted keys at 4 q/|q|) for lambda in [0.7, 0.9], where the gain tracks
    1/(1 - lambda).  At N = 1024 the planted mass is ~17% and the regime breaks.
    """
    rng = np.random.default_rng(15)
    gains = {}
    for lam in (0.7, 0.8, 0.9):
        g = []
        for _ in range(3):
            a1, a2, pos = _toy_row(rng, 32768, 128, lam)
            g.append(snr(a1 - lam * a2, pos, 32768) / snr(a1, pos, 32768))
        gains[lam] = float(np.median(g))
        assert 2.9 <= min(g) and max(g) <= 10.6, (lam, g)
        assert abs(gains[lam] * (1 - lam) - 1) < 0.1
    assert gains[0.7] < gains[0.8] < gains[0.9]


# --------------------------------------------------------------------------
# sliding window and per-sequence cache lengths
# --------------------------------------------------------------------------
def _sdpa_mask(q, k, v, mask):
    """torch fp64 SDPA of one head with an explicit boolean mask (True = visible)."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[:, None]  # noqa: E731
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(mask))
    return o[:, 0].numpy()


@pytest.mark.parametrize("window", [1, 5, 16, 40])
def test_sliding_window_matches_masked_sdpa(window):
    rng = np.random.default_rng(31 + window)
    q, k, v, lam = _rand(rng, B=2, T=37, Hq=8, Hkv=2, d=16)
    out = diffattn_prefill(q, k, v, lam, causal=True, window=window)
    i = np.arange(37)[:, None]
    j = np.arange(37)[None, :]
    mask = (j <= i) & (j > i - window)          # the lesson's swa_mask, written as a predicate
    G = 2
    for p in range(4):
        g = p // G
        o1 = _sdpa_mask(q[:, :, 2 * p], k[:, :, g], v[:, :, g], mask)
        o2 = _sdpa_mask(q[:, :, 2 * p + 1], k[:, :, g], v[:, :, g], mask)
        np.testing.assert_allclose(out[:, :, p], o1 - lam[:, :, p][..., None] * o2, rtol=1e-12, atol=1e-12)


def test_window_extremes():
    rng = np.random.default_rng(41)
    q, k, v, lam = _rand(rng, B=1, T=20, Hq=4, Hkv=1, d=8)
    np.testing.assert_array_equal(diffattn_prefill(q, k, v, lam, window=20), diffattn_prefill(q, k, v, lam))
    np.testing.assert_array_equal(diffattn_prefill(q, k, v, lam, window=1000), diffattn_prefill(q, k, v, lam))
    # window 1: each token attends to itself only, so out = (1 - lambda) v_i
    out = diffattn_prefill(q, k, v, lam, window=1)
    np.testing.assert_allclose(out, (1.0 - lam)[..., None] * v[:, :, [0, 0]], rtol=1e-13, atol=1e-14)


def test_decode_lengths_and_window_match_masked_sdpa():
    rng = np.random.default_rng(43)
    B, L, Hq, Hkv, d = 3, 50, 8, 2, 16
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, L, Hkv, d))
    v = rng.standard_normal((B, L, Hkv, d))
    lam = rng.uniform(0.2, 0.9, (B, Hq // 2))
    lens = np.array([1, 17, 50])
    for window in (0, 1, 8, 64):
        out = diffattn_decode(q, k, v, lam, seq_lens=lens, window=window)
        for b in range(B):
            j = np.arange(L)
            vis = (j < lens[b]) & ((j >= lens[b] - window) if window > 0 else True)
            for p in range(Hq // 2):
                g = p // 2
                qq = q[b:b + 1, [2 * p, 2 * p + 1]].transpose(1, 0, 2)       # [2, 1, d]
                kk = np.repeat(k[b:b + 1, :, g], 2, axis=0)
                vv = np.repeat(v[b:b + 1, :, g], 2, axis=0)
                o = _sdpa_mask(qq, kk, vv, vis[None, :])
                np.testing.assert_allclose(out[b, p], o[0, 0] - lam[b, p] * o[1, 0], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# decode layouts compared: standard transformer and DIFF V1
# --------------------------------------------------------------------------
from oracle import standard_decode, v1_layout_decode  # noqa: E402


def test_standard_decode_matches_sdpa():
    rng = np.random.default_rng(51)
    B, L, H, Hkv, d = 2, 40, 8, 2, 16
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, L, Hkv, d))
    v = rng.standard_normal((B, L, Hkv, d))
    out = standard_decode(q, k, v)
    for h in range(H):
        g = h // (H // Hkv)
        ref = _sdpa(q[:, None, h], k[:, :, g], v[:, :, g], causal=False)[:, 0]
        np.testing.assert_allclose(out[:, h], ref, rtol=1e-12, atol=1e-13)


def test_v1_layout_decode_pins():
    rng = np.random.default_rng(52)
    B, L, H, Hkv, d = 2, 30, 4, 2, 16
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, L, Hkv, d))
    v = rng.standard_normal((B, L, Hkv, d))
    lam = rng.uniform(-0.3, 0.9, (B, H))
    # lambda = 0, no norm: plain attention of the first halves (scale 1/sqrt(d/2)) over the full V
    out0 = v1_layout_decode(q, k, v, np.zeros((B, H)), v1_rmsnorm=False)
    for h in range(H):
        g = h // 2
        ref = _sdpa(q[:, None, h, :8], k[:, :, g, :8], v[:, :, g], causal=False)[:, 0]
        np.testing.assert_allclose(out0[:, h], ref, rtol=1e-12, atol=1e-13)
    # identical halves and lambda = 1 cancel exactly
    qs = np.concatenate([q[..., :8], q[..., :8]], axis=-1)
    ks = np.concatenate([k[..., :8], k[..., :8]], axis=-1)
    assert np.max(np.abs(v1_layout_decode(qs, ks, v, np.ones((B, H)), v1_rmsnorm=False))) < 1e-13
    # with the norm: rms of every head = sqrt(m / (m + eps)), direction of the raw difference kept
    raw = v1_layout_decode(q, k, v, lam, v1_rmsnorm=False)
    nrm = v1_layout_decode(q, k, v, lam, v1_rmsnorm=True, eps=1e-5)
    m = np.mean(raw * raw, axis=-1, keepdims=True)
    np.testing.assert_allclose(nrm, raw / np.sqrt(m + 1e-5), rtol=1e-12)
