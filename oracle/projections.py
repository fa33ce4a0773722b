"""fp64 CPU oracle for the projections on either side of the V2 attention core.

TEST INFRASTRUCTURE ONLY (imported by tests/ and bench.py's CPU-baseline leg,
never by the product path).

* lambda producer: V2 projects, for every token and every head (here: every
  differential pair), a sigmoid-bounded lambda from the token's hidden state --
  dailytechsnack.ch article "Differential Transformer V2 soll KI-Training
  stabiler machen", section "Weniger Ausreisser und Gradientenspitzen".
  Reading: a linear projection without bias, lambda[r, p] = sigmoid(x[r] . w[p]),
  with one projection vector per pair (w stored [P, d_model]).
* output projection: after the subtraction the extra dimension is projected back
  to the baseline width by O_W -- differential-attention lesson "差异性注意力 (V2)",
  section "V1 vs V2".  y[r] = attn[r] @ W_O, attn [rows, P*d], W_O [P*d, d_model].
Both are plain definitions written out; parity pins in tests/test_projection_oracle.py.
"""
from __future__ import annotations

import numpy as np

__all__ = ["lambda_projection", "output_projection"]


def lambda_projection(x, w) -> np.ndarray:
    """lambda [rows, P] = 1 / (1 + exp(-(x @ w^T))) in fp64; x [rows, d_model], w [P, d_model]."""
    z = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    return 1.0 / (1.0 + np.exp(-z))


def output_projection(attn, w_o) -> np.ndarray:
    """y [rows, d_model] = attn [rows, P*d] @ w_o [P*d, d_model] in fp64."""
    return np.asarray(attn, np.float64) @ np.asarray(w_o, np.float64)
