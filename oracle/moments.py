"""Oracle for the variance and moment-of-inertia cascades.

Test infrastructure only (see the package docstring).

"RedFuser episode transcript", cue 47, names variance and moment of inertia as
further cascaded reductions the method was run on, without stating them. The
plainest reading of each, taken here:

* variance of a row x_1..x_n: the mean mu = (1/n) sum x_i (first reduction),
  then the centred second moment (1/n) sum (x_i - mu)^2 (second reduction,
  which needs the first one's result); the population variance, dividing by n;
* moment of inertia of point masses w_i >= 0 at positions x_i on a line, about
  their centre of mass: c = sum w_i x_i / sum w_i (first reduction), then
  I = sum w_i (x_i - c)^2 (second reduction). With unit masses I = n * variance.
  A row whose masses sum to 0 has no centre: c = NaN and I = 0.

Both are written as the textbook two-pass cascade, in float64, and one is not
computed through the other.

Parity: pinned by exact rational arithmetic (fractions.Fraction) on small rows
of fp32 values, closed forms (0..n-1 has variance (n^2 - 1) / 12; equal masses
at -d and +d have centre 0 and I = 2 m d^2), the parallel-axis theorem
(sum w x^2 = I + W c^2, a different formula), invariance under a shift of the
positions and the scalings I(a x) = a^2 I(x), I(k w) = k I(w), and numpy.var
for unit masses.
"""

import numpy as np


def row_variance(x):
    """x: [T, E] values. Returns (mean [T], variance [T]) in float64."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    mean = x.sum(axis=-1) / n                                  # reduction 1
    var = ((x - mean[..., None]) ** 2).sum(axis=-1) / n        # reduction 2
    return mean, var


def row_inertia(x, w):
    """x, w: [T, E] positions and masses. Returns (centre [T], inertia [T])
    in float64; centre NaN and inertia 0 where the masses sum to 0."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    total = w.sum(axis=-1)
    moment = (w * x).sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        centre = np.where(total > 0, moment / np.where(total > 0, total, 1.0), np.nan)  # reduction 1
    dev = x - np.where(total > 0, centre, 0.0)[..., None]
    inertia = (w * dev * dev).sum(axis=-1)                     # reduction 2
    return centre, np.where(total > 0, inertia, 0.0)
