"""GPU parity of rf_row_variance and rf_row_inertia (through the C ABI) at
every fusion level against the fp64 oracle (the textbook two-pass cascade).

Bar, from the fp32 arithmetic. The second moment is a sum of non-negative
terms w (y - c)^2, each with a relative error of a few units of 2^-24, summed
in trees of depth at most 18 (32 values per lane, 64 lanes, 4 waves) plus
non-negative shift corrections; positions enter relative to the row's first
value, so the centre's own rounding moves the moment only to second order.
That gives a relative error of order 25 * 2^-24 = 1.5e-6; the test takes
1e-5 (zero only where the oracle's value is zero). The centre (or mean) is
x_0 + c: one rounding of the result (2^-24 |centre|) plus sums of shifted
positions with an absolute error of order 20 * 2^-24 times their spread; the
test takes 2^-22 |centre| + 2e-5 * spread (spread = sqrt(I / W))."""

import numpy as np
import pytest
import torch

import oracle
import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import DEV, needs_gpu, print_case

pytestmark = [pytest.mark.gpu, needs_gpu]

MOMENT_REL = 1e-5
LEVELS = [rf.RF_FUSE_NONE, rf.RF_FUSE_THREAD, rf.RF_FUSE_WAVE, rf.RF_FUSE_BLOCK]


def _compare(c, i, c_ref, i_ref, total, what):
    c = np.asarray(c, np.float64)
    i = np.asarray(i, np.float64)
    nan = np.isnan(c_ref)
    assert np.array_equal(np.isnan(c), nan), f"{what}: NaN centres differ"
    assert np.all(i[nan] == 0.0), f"{what}: massless rows must have zero inertia"
    ok = ~nan
    err_i = np.abs(i[ok] - i_ref[ok])
    assert np.all(err_i <= MOMENT_REL * i_ref[ok]), (what, (err_i / np.maximum(i_ref[ok], 1e-300)).max())
    spread = np.sqrt(i_ref[ok] / total[ok])
    err_c = np.abs(c[ok] - c_ref[ok])
    bound = 2.0 ** -22 * np.abs(c_ref[ok]) + 2e-5 * spread
    print(f"{what}: max relative moment error {(err_i / np.maximum(i_ref[ok], 1e-300)).max():.2e}, "
          f"max centre error / bound {(err_c / bound).max():.3f}", flush=True)
    assert np.all(err_c <= bound), (what, (err_c - bound).max())


def _check_variance(x, level, what):
    mean, var = rf.row_variance(x.to(DEV), level)
    m_ref, v_ref = oracle.row_variance(x.numpy())
    E = x.shape[1]
    _compare(mean.cpu().numpy(), var.cpu().numpy() * E, m_ref, v_ref * E, np.full(len(m_ref), float(E)),
             what + " variance")


def _check_inertia(x, w, level, what):
    c, i = rf.row_inertia(x.to(DEV), w.to(DEV), level)
    c_ref, i_ref = oracle.row_inertia(x.numpy(), w.numpy())
    _compare(c.cpu().numpy(), i.cpu().numpy(), c_ref, i_ref, w.numpy().astype(np.float64).sum(axis=1),
             what + " inertia")


@pytest.mark.parametrize("level", LEVELS)
@pytest.mark.parametrize("E", [4, 12, 100, 256, 1020, 1024, 1028, 2048, 3000, 4096, 6004, 8192])
def test_moments_shapes(level, E):
    """37 rows (the four offset/scale classes, a partial group of four rows for
    the wave-per-row forms): one and several chunks per lane, ragged tails."""
    print_case(test="moments_shapes", level=level, E=E)
    x, w = inputs.moment_inputs(21, 37, E)
    _check_variance(x, level, f"E={E} level={level}")
    _check_inertia(x, w, level, f"E={E} level={level}")


@pytest.mark.parametrize("E", [1024, 2048, 4096, 8192])
def test_moments_config(E):
    """The measured workload (2^26 values in rows of E), every row, every level."""
    T = (1 << 26) // E
    x, w = inputs.moment_inputs(7, T, E)
    m_ref, v_ref = oracle.row_variance(x.numpy())
    c_ref, i_ref = oracle.row_inertia(x.numpy(), w.numpy())
    total = w.numpy().astype(np.float64).sum(axis=1)
    xd, wd = x.to(DEV), w.to(DEV)
    for level in LEVELS:
        print_case(test="moments_config", level=level, E=E)
        mean, var = rf.row_variance(xd, level)
        _compare(mean.cpu().numpy(), var.cpu().numpy() * E, m_ref, v_ref * E, np.full(T, float(E)), "variance")
        c, i = rf.row_inertia(xd, wd, level)
        _compare(c.cpu().numpy(), i.cpu().numpy(), c_ref, i_ref, total, "inertia")


@pytest.mark.parametrize("level", LEVELS)
def test_moments_degenerate_rows(level):
    """Constant rows (zero variance, exactly), an offset of 1e4 with spread
    1e-2, no mass at all (centre NaN), one massive point, mass only in the
    last ragged chunk, and two clusters far apart."""
    print_case(test="moments_degenerate", level=level)
    E = 2052
    x, w = inputs.moment_inputs(22, 8, E)
    x, w = x.numpy().copy(), w.numpy().copy()
    x[0] = 3.5
    x[1] = (1e4 + 1e-2 * np.random.default_rng(1).standard_normal(E)).astype(np.float32)
    w[2] = 0.0
    x[3] = 5.0 + np.random.default_rng(2).random(E, dtype=np.float32)   # within a factor 2: exact shifts
    w[3] = 0.0
    w[3, 777] = 2.0
    w[4, :2048] = 0.0
    x[5, : E // 2] -= 500.0
    x[5, E // 2:] += 500.0
    x, w = torch.from_numpy(x), torch.from_numpy(w)
    mean, var = rf.row_variance(x.to(DEV), level)
    assert var[0].item() == 0.0 and mean[0].item() == 3.5
    _check_variance(x, level, "degenerate")
    _check_inertia(x, w, level, "degenerate")
    c, i = rf.row_inertia(x.to(DEV), w.to(DEV), level)
    assert c[3].item() == x[3, 777].item() and i[3].item() == 0.0


def test_moments_empty():
    x = torch.empty((0, 1024), device=DEV)
    for level in LEVELS:
        assert rf.row_variance(x, level)[1].shape == (0,)
        assert rf.row_inertia(x, x, level)[1].shape == (0,)
