"""The seeded generator: determinism, bf16 rounding, shapes, signal planting."""
import numpy as np
import torch

from differential_attention_v2_amd import workloads as W


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0039062, 1.0117188, -2.5e-39, 65504.0, 3.3895314e38], np.float32)])
    ours = W.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_chunk_stable(monkeypatch):
    w = W.TINY_PREFILL_FP32
    a = W.make_prefill(w)
    b = W.make_prefill(w)
    for key in ("q", "k", "v", "lam"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["q"].shape == (1, 128, 2, 64) and a["q"].dtype == np.float32
    assert a["lam"].shape == (1, 128, 1) and np.all((a["lam"] > 0) & (a["lam"] < 1))
    # thread count does not change bytes
    monkeypatch.setattr(W, "_threads", lambda: 1)
    w2 = w.with_(dtype="bf16", T=40000, Hq=8, Hkv=4, d=64)
    x1 = W.make_prefill(w2)["k"]
    monkeypatch.setattr(W, "_threads", lambda: 7)
    x2 = W.make_prefill(w2)["k"]
    np.testing.assert_array_equal(x1, x2)


def test_distribution_scale():
    w = W.PREFILL_T4096.with_(T=512)
    x = W.bf16_to_f32(W.make_prefill(w)["q"])
    assert abs(x.std() - 1 / np.sqrt(2)) < 0.01 and abs(x.mean()) < 0.01


def test_signal_planting():
    w = W.PREFILL_T32768.with_(T=2048, Hkv=2, Hq=16)
    inp = W.plant_signal(w, W.make_prefill(w))
    plan = inp["plan"]
    assert len(plan) == w.B * w.Hkv * w.G * 8
    seen = {}
    for b, p, i, pos in plan:
        g = p // w.G
        assert w.T // 2 <= i < w.T and pos.max() <= i and len(set(pos.tolist())) == 16
        for j in pos:
            assert (b, g, int(j)) not in seen
            seen[(b, g, int(j))] = True
        qi = W.bf16_to_f32(inp["q"][b, i, 2 * p])
        kj = W.bf16_to_f32(inp["k"][b, pos, g])
        np.testing.assert_allclose(kj, np.broadcast_to(4 * qi / np.linalg.norm(qi), kj.shape), rtol=1e-2, atol=4e-3)
    k = W.bf16_to_f32(inp["k"])
    planted = np.zeros(k.shape[:3], dtype=bool)
    for (b, g, j) in seen:
        planted[b, j, g] = True
    assert abs(k[~planted].std() - 1.0) < 0.02   # non-planted rows are N(0, 1)
