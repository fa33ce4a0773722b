"""The pages' own printed values, reproduced through the oracle (fixtures in tests/golden/)."""
import json
import math
import os

import numpy as np

from differential_attention_v2_amd.workloads import Workload
from oracle import attention_weights, diffattn_decode, snr, v1_lambda

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def test_noise_floor_thirteen_percent():
    """128k context, every unmatched token at 1e-6 weight: they hold ~13% of the attention mass."""
    g = GOLD["noise_floor"]
    N, per = g["context_tokens"], g["per_token_weight"]
    # d = 1; the matched key's score is chosen so each of the N-1 others gets weight `per` exactly
    s_match = math.log(1.0 / per - (N - 1))
    q = np.array([[[1.0], [1.0]]])                      # [B=1, Hq=2, d=1]
    k = np.zeros((1, N, 1, 1)); k[0, 0, 0, 0] = s_match
    v = np.ones((1, N, 1, 1)); v[0, 0, 0, 0] = 0.0      # indicator of the unmatched tokens
    mass = diffattn_decode(q, k, v, np.zeros((1, 1)))[0, 0, 0]
    assert abs(mass - g["unrelated_tokens"] * per) < 1e-12
    assert round(100 * mass) == g["unrelated_mass_percent_rounded"]


def test_v1_lambda_init_only():
    z = np.zeros((4, 128))
    assert np.allclose(v1_lambda(z, z, z, z, GOLD["v1_lambda_init"]["lambda_init"]), 0.8, atol=1e-15)


def test_v2_kv_cache_equals_baseline_gqa():
    """Doubling query heads at fixed KV heads leaves the decode KV bytes unchanged."""
    g = GOLD["gqa_kv_cache"]
    base = Workload("base", "decode", "bf16", B=1, T=4096, Hq=g["query_heads"] // 2 * 2, Hkv=g["kv_heads"], d=128)
    v2 = base.with_(Hq=2 * g["query_heads"])
    assert v2.decode_kv_bytes() == base.decode_kv_bytes() == 2 * 4096 * 8 * 128 * 2


def test_toy_gain_range_through_the_oracle():
    """The printed 3x-10x SNR gain of differential over softmax attention, reproduced
    through the oracle on the toy's rows (16 keys at 4 q/|q| among N(0, 1) keys, the
    branches' queries independent) in the long-context regime, for lambda from 0.7 to
    0.85, where the gain (about 1/(1 - lambda)) spans the printed range."""
    t = GOLD["toy_snr_gain"]
    rng = np.random.default_rng(2024)
    N, d = 32768, 128
    gains = []
    for lam in (0.7, 0.75, 0.8, 0.85):
        q1, q2 = rng.standard_normal(d) / math.sqrt(2), rng.standard_normal(d) / math.sqrt(2)
        k = rng.standard_normal((N, d))
        pos = rng.choice(N, 16, replace=False)
        k[pos] = 4 * q1 / np.linalg.norm(q1)
        a1 = attention_weights(q1[None], k, np.array([N - 1]), False)[0]
        a2 = attention_weights(q2[None], k, np.array([N - 1]), False)[0]
        gains.append(snr(a1 - lam * a2, pos, N) / snr(a1, pos, N))
    assert all(t["low"] <= g <= t["high"] for g in gains), gains
    assert gains == sorted(gains)
