"""Pins of the oracle's input projection (a plain matrix product)."""
import numpy as np

import oracle


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    y = oracle.linear(x, w)
    assert y.shape == (3, 4)
    for t in range(3):
        for f in range(4):
            s = 0.0
            for k in range(5):
                s += x[t, k] * w[f, k]
            assert abs(y[t, f] - s) < 1e-12


def test_identity_rows_copy_the_input():
    rng = np.random.default_rng(1)
    d = 6
    x = rng.standard_normal((4, d))
    w = np.concatenate([np.eye(d), 2.0 * np.eye(d), -np.eye(d)[:3]])
    y = oracle.linear(x, w)
    np.testing.assert_array_equal(y[:, :d], x)
    np.testing.assert_array_equal(y[:, d:2 * d], 2.0 * x)
    np.testing.assert_array_equal(y[:, 2 * d:], -x[:, :3])


def test_rows_of_w_are_output_features():
    """A one-hot weight row f picks input feature k(f); stacking rows stacks output columns."""
    x = np.arange(12.0).reshape(3, 4)
    w = np.zeros((2, 4))
    w[0, 3] = 1.0
    w[1, 0] = 0.5
    np.testing.assert_array_equal(oracle.linear(x, w), np.stack([x[:, 3], 0.5 * x[:, 0]], axis=1))
