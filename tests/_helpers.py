"""Shared test plumbing: moving generator bytes onto the device and comparing
device results with the fp64 oracle."""
from __future__ import annotations

import numpy as np

# Parity bar for bf16 inputs with fp32 accumulation (also applied to fp32 inputs).
TOL_MAX_ABS = 2e-2
TOL_MEAN_ABS = 2e-3
# Relative L2 error over the compared elements.  Long rows average many values,
# so outputs shrink like 1/sqrt(keys) and the absolute bounds above loosen there;
# a scale-free bound keeps the check meaningful (bf16 P and output rounding give
# about 2e-3).
TOL_REL_L2 = 1e-2


def to_device(x: np.ndarray, dtype: str, device):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def from_device(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    e = np.abs(got - ref)
    return dict(max_abs=float(e.max()), mean_abs=float(e.mean()),
                rel_l2=float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)),
                nonfinite=int((~np.isfinite(got)).sum()))


def assert_parity(got, ref, what: str, max_abs: float = TOL_MAX_ABS, mean_abs: float = TOL_MEAN_ABS,
                  rel_l2: float = TOL_REL_L2) -> dict:
    err = errors(got, ref)
    print(f"[parity] {what}: max_abs={err['max_abs']:.3e} mean_abs={err['mean_abs']:.3e} "
          f"rel_l2={err['rel_l2']:.3e}", flush=True)
    assert err["nonfinite"] == 0, (what, err)
    assert err["max_abs"] <= max_abs and err["mean_abs"] <= mean_abs, (what, err)
    assert err["rel_l2"] <= rel_l2, (what, err)
    return err
