"""Pins of the projection oracle: special cases with closed forms and a library
routine (scipy's expit), and brute force in plain loops on tiny shapes."""
import numpy as np
from scipy.special import expit

from oracle import lambda_projection, output_projection


def test_lambda_projection_closed_forms():
    rng = np.random.default_rng(61)
    x = rng.standard_normal((7, 32))
    # zero weights: sigmoid(0) = 1/2 exactly
    assert np.all(lambda_projection(x, np.zeros((4, 32))) == 0.5)
    # unit vectors pick one input feature: lambda = expit(x[:, c])
    w = np.zeros((3, 32))
    w[0, 5] = w[1, 0] = w[2, 31] = 1.0
    np.testing.assert_allclose(lambda_projection(x, w), expit(x[:, [5, 0, 31]]), rtol=1e-15)
    # opposite projections are complementary: sigmoid(z) + sigmoid(-z) = 1
    w = rng.standard_normal((5, 32))
    np.testing.assert_allclose(lambda_projection(x, w) + lambda_projection(x, -w), 1.0, rtol=1e-14)
    lam = lambda_projection(100 * x, w)
    assert np.all((lam >= 0) & (lam <= 1))


def test_projections_brute_force():
    rng = np.random.default_rng(62)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((2, 5))
    lam = lambda_projection(x, w)
    for r in range(3):
        for p in range(2):
            z = sum(x[r, c] * w[p, c] for c in range(5))
            assert abs(lam[r, p] - 1.0 / (1.0 + np.exp(-z))) < 1e-15
    a = rng.standard_normal((3, 4))
    wo = rng.standard_normal((4, 6))
    y = output_projection(a, wo)
    for r in range(3):
        for j in range(6):
            assert abs(y[r, j] - sum(a[r, i] * wo[i, j] for i in range(4))) < 1e-13
