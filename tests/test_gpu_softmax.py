"""GPU parity of rf_softmax (through the C ABI) at every fusion level against
the fp64 oracle (the three-stage safe softmax).

Bar, from the fp32 arithmetic: y_ij = exp2((x_ij - m) * log2 e) / l. The
rounded difference, the rounded product and the rounded constant each perturb
the exponent by at most |x_ij - m| * log2(e) * 2^-24, so that step alone gives
a relative error of up to 3 * 2^-24 * |x_ij - m| (about 1.8e-7 |x_ij - m|);
the exponential itself, the sum l (at most 32 sequential terms per thread, then
a tree), the reciprocal and the product add a few ulp more. The test takes
relative error <= 5e-6 + 2.5e-7 |x_ij - m| for every weight above 1e-30, and
every row of the output summing to 1 within 1e-5. That is the flat fp32 bar
of 1e-5 for every weight within 20 of its row's max (checked separately
below); only weights below e^-20 (2e-9) of the row's largest one get the wider
bar, which grows because x_ij - m itself carries a rounding error of up to
2^-24 |x_ij - m| in fp32."""

import numpy as np
import pytest
import torch

import oracle
import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import DEV, needs_gpu, print_case

pytestmark = [pytest.mark.gpu, needs_gpu]

SOFTMAX_REL = 1e-5
LEVELS = [rf.RF_FUSE_NONE, rf.RF_FUSE_THREAD, rf.RF_FUSE_WAVE, rf.RF_FUSE_BLOCK]


def _tol(x):
    x = np.asarray(x, np.float64)
    return 5e-6 + 2.5e-7 * (x.max(axis=1, keepdims=True) - x)


def _compare(y, x, ref):
    """Weights above 1e-30 within the relative bar, the rest within 1e-30."""
    big = ref > 1e-30
    err = np.abs(y - ref)
    rel = np.where(big, err / np.where(big, ref, 1.0), 0.0)
    excess = rel - _tol(x)
    assert excess.max() <= 0, (rel.max(), np.unravel_index(excess.argmax(), excess.shape))
    near = np.asarray(x, np.float64).max(axis=1, keepdims=True) - np.asarray(x, np.float64) <= 20
    assert rel[near & big].max(initial=0.0) <= SOFTMAX_REL
    assert err[~big].max(initial=0.0) <= 1e-30


def _check(x, level, rows=None):
    y = rf.softmax(x.to(DEV), level).cpu().numpy().astype(np.float64)
    assert np.abs(y.sum(axis=1) - 1.0).max() <= SOFTMAX_REL
    xs = x.numpy() if rows is None else x.numpy()[rows]
    ys = y if rows is None else y[rows]
    _compare(ys, xs, oracle.softmax_rows(xs))


@pytest.mark.parametrize("level", LEVELS)
@pytest.mark.parametrize("E", [4, 12, 100, 256, 1020, 1024, 1028, 2048, 3000, 4096, 6004, 8192])
def test_softmax_shapes(level, E):
    """37 rows (ramped rows among them) per size: single and several chunks per
    thread, ragged tails inside a wave and inside a workgroup tile."""
    print_case(test="softmax_shapes", level=level, E=E)
    _check(inputs.softmax_inputs(11, 37, E), level)


@pytest.mark.parametrize("level", LEVELS)
@pytest.mark.parametrize("E", [1024, 2048, 4096, 8192])
def test_softmax_config_sampled(level, E):
    """The measured workload (2^26 values in rows of E): row sums everywhere,
    elementwise against the oracle on 257 sampled rows."""
    print_case(test="softmax_config", level=level, E=E)
    T = (1 << 26) // E
    x = inputs.softmax_inputs(5, T, E)
    rows = np.unique(np.concatenate([np.random.default_rng(E).choice(T, 256, replace=False), [T - 1]]))
    _check(x, level, rows)


@pytest.mark.parametrize("level", LEVELS)
def test_softmax_degenerate_rows(level):
    """Constant rows (uniform output), rows offset by +-1000 (a softmax without
    the max subtraction overflows or underflows), one dominant value, -inf
    entries beside finite ones, and values far apart in magnitude."""
    print_case(test="softmax_degenerate", level=level)
    E = 2052
    x = inputs.softmax_inputs(12, 8, E).numpy().copy()
    x[0] = 3.0
    x[1] += 1000.0
    x[2] -= 1000.0
    x[3, 1500] = 200.0
    x[4, ::3] = -np.inf
    x[5] = np.linspace(-1e4, 1e4, E, dtype=np.float32)
    x[6, :2048] = -np.inf   # the only finite values sit in the last ragged chunk
    x = torch.from_numpy(x)
    y = rf.softmax(x.to(DEV), level).cpu().numpy().astype(np.float64)
    _compare(y, x.numpy(), oracle.softmax_rows(x.numpy()))
    assert np.abs(y.sum(axis=1) - 1.0).max() <= SOFTMAX_REL
    assert np.all(y[4, ::3] == 0.0) and np.all(y[6, :2048] == 0.0)
    assert np.allclose(y[0], 1.0 / E, rtol=1e-6, atol=0)


def test_softmax_empty():
    x = torch.empty((0, 1024), device=DEV)
    for level in LEVELS:
        assert rf.softmax(x, level).shape == (0, 1024)
