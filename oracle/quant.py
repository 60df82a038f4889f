"""Oracle for the FP8 cascade: per-token abs-max, scale, e4m3 cast, then GEMM.

Test infrastructure only (see the package docstring).

"RedFuser episode transcript", cue 33. In formulas: for row i of A,
a_i = max_k |A_ik| and s_i = a_i / 448; then C_ij = s_i t_j sum_k Aq_ik Bq_jk,
where Aq_ik is A_ik / s_i cast to e4m3 and t_j, Bq_j are the same for row j of
the K x N operand stored by columns. Since s_i is a single factor outside the
sum, a one-pass loop can carry a running s_i and, whenever it increases from
s_old to s_new, multiply the partial sum by s_old / s_new. The cue (and cue 61)
treats these as exact real numbers and does not fix the FP8 rounding. Readings
taken (each a plain choice the rest supports):

* scale s_i = fp32(absmax_i / 448), division correctly rounded in float32;
* code q_ik = e4m3(fp32(A_ik / s_i)), float32 division correctly rounded, then
  the saturating round-to-nearest-even e4m3 encoding of ``oracle.codec``;
* a row whose abs-max is 0 gets s_i = 0 and all codes 0x00;
* the gated path quantises with the row's *final* scale (the unfused cascade:
  abs-max first, then quantise, then GEMM). ``quant_gemm_running_scale`` is the
  pages' one-pass loop with a running scale, kept as a separate form.

``quant_gemm``: C_ij = s_i * t_j * sum_k dec(Aq_ik) * dec(Bq_jk) in float64.
Every e4m3 value is an integer multiple of 2^-9 of magnitude at most 448, so
each product is an integer multiple of 2^-18 below 2^18, i.e. an integer below
2^36 in units of 2^-18; a sum of fewer than 2^13 such products stays below
2^49 units, inside float64's 53-bit significand: the float64 matmul sum is
exact in any order.
Parity: pinned by that closed form (checked against Python integer arithmetic
on sampled entries), by the codec's pins, by the invariant that a row's
abs-max element encodes to +-448, and (for the running form) by the identity
that with quantisation switched off it equals the plain product to rounding.
"""

import numpy as np

from .codec import e4m3_decode, e4m3_encode

FP8_MAX = 448.0


def absmax_quant(x):
    """Per-row quantisation of x [rows, cols] (float32 values; bf16 inputs upcast exactly).

    Returns (codes uint8 [rows, cols], scale float32 [rows]).
    """
    xf = np.asarray(x, dtype=np.float32)
    a = np.abs(xf).max(axis=1)                                 # reduction 1: abs-max
    s = (a / np.float32(FP8_MAX)).astype(np.float32)          # correctly rounded fp32
    codes = np.zeros(xf.shape, dtype=np.uint8)
    nz = s > 0
    if np.any(nz):
        y = (xf[nz] / s[nz][:, None]).astype(np.float32)      # correctly rounded fp32
        codes[nz] = e4m3_encode(y.astype(np.float64))
    return codes, s


def quant_gemm(aq, a_scale, bq, b_scale):
    """C [M, N] float64 from codes aq [M, K], bq [N, K] and scales a_scale [M], b_scale [N]."""
    a = e4m3_decode(aq)
    b = e4m3_decode(bq)
    acc = a @ b.T                                              # exact (see docstring)
    return np.asarray(a_scale, np.float64)[:, None] * np.asarray(b_scale, np.float64)[None, :] * acc


def quant_gemm_running_scale(x, bq, b_scale, k_tile, quantize=True):
    """One-pass form with a running per-row abs-max over K tiles of ``k_tile`` columns.

    For each K tile: raise the running abs-max with the tile's values; if it
    grew, multiply the accumulator row by old scale / new scale; quantise the
    tile with the current scale (or, with ``quantize=False``, use the exact
    value x / scale); add its product with B. At the end multiply by the final
    scale and the column scales. A running abs-max of 0 means nothing has been
    added yet, so the correction factor is 1 (the identity).
    Returns C [M, N] float64.
    """
    xf = np.asarray(x, dtype=np.float32)
    M, K = xf.shape
    b = e4m3_decode(bq)
    acc = np.zeros((M, b.shape[0]))
    a_run = np.zeros(M, dtype=np.float32)
    s_run = np.zeros(M, dtype=np.float32)
    for t0 in range(0, K, k_tile):
        t1 = min(t0 + k_tile, K)
        tile = xf[:, t0:t1]
        a_new = np.maximum(a_run, np.abs(tile).max(axis=1))
        s_new = (a_new / np.float32(FP8_MAX)).astype(np.float32)
        grew = (a_new > a_run) & (a_run > 0)
        factor = np.where(grew, s_run.astype(np.float64) / np.where(s_new > 0, s_new, 1), 1.0)
        acc *= factor[:, None]
        a_run, s_run = a_new, s_new
        safe_s = np.where(s_run > 0, s_run, np.float32(1))
        if quantize:
            y = (tile / safe_s[:, None]).astype(np.float32)
            vals = e4m3_decode(e4m3_encode(y.astype(np.float64)))
        else:
            vals = tile.astype(np.float64) / safe_s.astype(np.float64)[:, None]
        vals = np.where((s_run > 0)[:, None], vals, 0.0)
        acc += vals @ b[:, t0:t1].T
    return s_run.astype(np.float64)[:, None] * np.asarray(b_scale, np.float64)[None, :] * acc
