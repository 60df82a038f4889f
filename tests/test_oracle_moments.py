"""Pins of the variance and moment-of-inertia oracle against exact rational
arithmetic, closed forms, the parallel-axis theorem, invariances and numpy."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from online_softmax_attention_cascaded_amd import inputs


def _exact_inertia(xs, ws):
    xs = [Fraction(float(v)) for v in xs]
    ws = [Fraction(float(v)) for v in ws]
    total = sum(ws)
    c = sum(w * x for w, x in zip(ws, xs)) / total
    return c, sum(w * (x - c) ** 2 for w, x in zip(ws, xs))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_rational_small_rows(seed):
    """fp32 inputs are exact rationals: the float64 oracle must agree with the
    exact centre and inertia (and mean and variance) to float64 rounding."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, 9)) * [[1.0], [0.01], [30.0]] + [[0.0], [1000.0], [-7.0]]).astype(np.float32)
    w = rng.random((3, 9), dtype=np.float32)
    c, inertia = oracle.row_inertia(x, w)
    mean, var = oracle.row_variance(x)
    for i in range(3):
        ce, ie = _exact_inertia(x[i], w[i])
        assert abs(c[i] - float(ce)) <= 1e-15 * max(1.0, abs(float(ce)))
        assert abs(inertia[i] - float(ie)) <= 1e-9 * float(ie)
        me, m2 = _exact_inertia(x[i], np.ones(9))
        assert abs(mean[i] - float(me)) <= 1e-15 * max(1.0, abs(float(me)))
        assert abs(var[i] - float(m2 / 9)) <= 1e-9 * float(m2 / 9)


def test_closed_forms():
    n = 101
    mean, var = oracle.row_variance(np.arange(n, dtype=np.float64)[None])
    assert mean[0] == 50.0 and abs(var[0] - (n * n - 1) / 12) <= 1e-12 * var[0]
    # Two equal masses m at -d and +d, plus a massless point far away.
    c, inertia = oracle.row_inertia(np.array([[-3.0, 3.0, 1e6]]), np.array([[2.5, 2.5, 0.0]]))
    assert c[0] == 0.0 and inertia[0] == 2 * 2.5 * 9.0
    # A single massive point: centre at it, no inertia.
    c, inertia = oracle.row_inertia(np.array([[4.0, -1.0]]), np.array([[0.0, 7.0]]))
    assert c[0] == -1.0 and inertia[0] == 0.0
    # No mass at all: no centre.
    c, inertia = oracle.row_inertia(np.array([[1.0, 2.0]]), np.zeros((1, 2)))
    assert np.isnan(c[0]) and inertia[0] == 0.0


def test_parallel_axis_and_invariances():
    x, w = inputs.moment_inputs(4, 8, 300)
    x = x.numpy().astype(np.float64)
    w = w.numpy().astype(np.float64)
    x = x - x.mean(axis=1, keepdims=True) * 0.9          # keep the first moments moderate
    c, inertia = oracle.row_inertia(x, w)
    W = w.sum(axis=1)
    assert np.allclose((w * x * x).sum(axis=1), inertia + W * c * c, rtol=1e-12, atol=0)
    c2, i2 = oracle.row_inertia(x + 12.5, w)
    assert np.allclose(c2, c + 12.5, rtol=1e-12, atol=1e-12) and np.allclose(i2, inertia, rtol=1e-9)
    c3, i3 = oracle.row_inertia(-3.0 * x, w)
    assert np.allclose(c3, -3.0 * c, rtol=1e-12) and np.allclose(i3, 9.0 * inertia, rtol=1e-12)
    c4, i4 = oracle.row_inertia(x, 5.0 * w)
    assert np.allclose(c4, c, rtol=1e-12) and np.allclose(i4, 5.0 * inertia, rtol=1e-12)


def test_unit_masses_match_numpy_var():
    x, _ = inputs.moment_inputs(5, 12, 1000)
    x = x.numpy()
    mean, var = oracle.row_variance(x)
    xd = x.astype(np.float64)
    assert np.allclose(mean, xd.mean(axis=1), rtol=1e-14, atol=0)
    assert np.allclose(var, xd.var(axis=1), rtol=1e-10, atol=0)
    c, inertia = oracle.row_inertia(x, np.ones_like(x))
    assert np.allclose(inertia, 1000 * var, rtol=1e-10, atol=0)
