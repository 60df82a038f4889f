"""Pins of the e4m3 codec and the abs-max -> quantise -> GEMM oracle (no GPU)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.codec import e4m3_decode, e4m3_encode, e4m3_table
from online_softmax_attention_cascaded_amd import inputs


# ---------------------------------------------------------------- codec


def test_table_landmarks_from_the_format_definition():
    t = e4m3_table()
    assert len(t) == 127 and np.all(np.diff(t) > 0)
    assert t[0] == 0 and t[1] == 2.0 ** -9 and t[7] == 7 * 2.0 ** -9
    assert t[8] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0             # exponent field 7 = bias
    assert t[0x7E] == 448.0           # largest finite
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert len(codes) == 254
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


@pytest.mark.parametrize(
    "x,expect",
    [
        (17.0, 16.0),             # tie between 16 (even) and 18
        (19.0, 20.0),             # tie between 18 and 20 (even)
        (2.0 ** -10, 0.0),        # tie between 0 (even) and 2^-9
        (1.5 * 2.0 ** -9, 2.0 ** -8),  # tie between 2^-9 and 2^-8 (even)
        (7.5 * 2.0 ** -9, 2.0 ** -6),  # subnormal/normal boundary tie goes to the even code
        (464.0, 448.0),           # tie with the (absent) 480 rounds down
        (470.0, 448.0),           # saturation
        (1e6, 448.0),
        (-1e6, -448.0),
        (0.3, 0.3125),            # nearest of 0.28125 and 0.3125
    ],
)
def test_rounding_cases(x, expect):
    assert e4m3_decode(e4m3_encode(np.array([x])))[0] == expect


def test_matches_torch_cpu_cast_inside_range():
    """Library pin: torch's float8_e4m3fn cast (round to nearest even) where it is
    defined without saturation (|x| < 464)."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000) * 40,
        rng.uniform(-2 ** -5, 2 ** -5, 100_000),
        (e4m3_table()[:-1] + e4m3_table()[1:]) / 2,       # every midpoint
        -(e4m3_table()[:-1] + e4m3_table()[1:]) / 2,
    ]).astype(np.float32)
    x = x[np.abs(x) < 464]
    ours = e4m3_encode(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


# ---------------------------------------------------------------- quantiser


def test_quantiser_scale_and_absmax_element():
    a, _ = inputs.quant_inputs(1, 16, 4, 300)
    x = a.float().numpy()
    codes, s = oracle.absmax_quant(x)
    amax = np.abs(x).max(axis=1)
    assert s.dtype == np.float32
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    j = np.abs(x).argmax(axis=1)
    c = codes[np.arange(16), j]
    assert np.all((c == 0x7E) | (c == 0xFE))
    assert np.all(np.sign(e4m3_decode(c)) == np.sign(x[np.arange(16), j]))


def test_quantiser_error_bound():
    """Dequantised values are within half a step of the input: relative 2^-4 in the
    normal range, absolute 2^-10 * s below it."""
    a, _ = inputs.quant_inputs(2, 32, 4, 512)
    x = a.float().numpy().astype(np.float64)
    codes, s = oracle.absmax_quant(x.astype(np.float32))
    deq = e4m3_decode(codes) * s[:, None]
    y = np.abs(x / s[:, None])
    err = np.abs(deq - x)
    normal = y >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= (2.0 ** -10 * np.broadcast_to(s[:, None], x.shape)[~normal]) * (1 + 1e-6))


def test_zero_row():
    x = np.zeros((3, 10), np.float32)
    x[1] = np.linspace(-1, 1, 10)
    x[2, 4] = -0.0
    codes, s = oracle.absmax_quant(x)
    assert s[0] == 0 and s[2] == 0 and s[1] > 0
    assert np.all(codes[0] == 0) and np.all(codes[2] == 0)


# ---------------------------------------------------------------- GEMM


def test_gemm_is_exact_against_integer_arithmetic():
    a, b = inputs.quant_inputs(3, 24, 20, 1000)
    aq, sa = oracle.absmax_quant(a.float().numpy())
    bq, sb = oracle.absmax_quant(b.float().numpy())
    c = oracle.quant_gemm(aq, sa, bq, sb)
    ai = np.rint(e4m3_decode(aq) * 512).astype(np.int64)
    bi = np.rint(e4m3_decode(bq) * 512).astype(np.int64)
    assert np.array_equal(ai / 512, e4m3_decode(aq))
    rng = np.random.default_rng(0)
    for _ in range(40):
        i, j = int(rng.integers(24)), int(rng.integers(20))
        exact = sum(int(p) * int(r) for p, r in zip(ai[i], bi[j]))
        ref = Fraction(exact, 2 ** 18) * Fraction(float(sa[i])) * Fraction(float(sb[j]))
        assert abs(Fraction(c[i, j]) - ref) <= abs(ref) * Fraction(1, 2 ** 51)


def test_gemm_transposition_pin():
    """C_ij uses row i of A and row j of the [N, K] B operand (not its transpose)."""
    aq = np.zeros((2, 3), np.uint8)
    bq = np.zeros((2, 3), np.uint8)
    aq[0, 0] = e4m3_encode(np.array([2.0]))[0]
    bq[1, 0] = e4m3_encode(np.array([3.0]))[0]
    c = oracle.quant_gemm(aq, np.array([1.0, 1.0]), bq, np.array([1.0, 0.5]))
    assert c.tolist() == [[0.0, 3.0], [0.0, 0.0]]


def test_running_scale_without_quantisation_is_the_plain_product():
    """Transcript cue 33 in real arithmetic: rescaling the accumulator by old/new
    abs-max whenever it grows gives exactly the unfused product."""
    a, b = inputs.quant_inputs(5, 8, 6, 700)
    x = a.float().numpy()
    bq, sb = oracle.absmax_quant(b.float().numpy())
    ref = x.astype(np.float64) @ (e4m3_decode(bq) * sb[:, None].astype(np.float64)).T
    for kt in (64, 100, 700):
        c = oracle.quant_gemm_running_scale(x, bq, sb, kt, quantize=False)
        assert np.allclose(c, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_running_scale_single_tile_is_the_final_scale_path():
    a, b = inputs.quant_inputs(6, 8, 6, 640)
    x = a.float().numpy()
    bq, sb = oracle.absmax_quant(b.float().numpy())
    aq, sa = oracle.absmax_quant(x)
    c1 = oracle.quant_gemm(aq, sa, bq, sb)
    c2 = oracle.quant_gemm_running_scale(x, bq, sb, 640, quantize=True)
    assert np.allclose(c1, c2, rtol=1e-15, atol=0)


def test_running_scale_growth_worked_case():
    """Transcript cue 33 with a scale that grows between two K tiles, by hand:
    tile 1 = [1, 0.5] (abs-max 1), tile 2 = [4, -2] (abs-max 4), B = ones with
    column scale 1. Tile 1 is quantised with s1 = 1/448 (codes 448, 224), the
    accumulator (672) is multiplied by s1/s2 = 1/4 when tile 2 raises the scale
    to s2 = 4/448, tile 2 adds 448 - 224; the final scale gives
    s2 * (168 + 224) = 3.5 = 1 + 0.5 + 4 - 2. (B's codes decode to 448 with
    column scale 1/448.) A wrong rescale direction gives s2 * (2688 + 224), a
    missing rescale s2 * 896."""
    x = np.array([[1.0, 0.5, 4.0, -2.0]], np.float32)
    bq, sb = oracle.absmax_quant(np.ones((1, 4), np.float32))
    assert sb[0] == np.float32(1.0 / 448.0) and np.all(e4m3_decode(bq) == 448.0)
    c = oracle.quant_gemm_running_scale(x, bq, sb, 2)
    assert abs(c[0, 0] - 3.5) <= 1e-6


def test_outlier_generator():
    a, _ = inputs.quant_inputs(7, 100, 2, 1000)
    x = a.float().numpy()
    assert (np.abs(x) > 20).sum() >= 50   # about 100 entries scaled by 50


# ---------------------------------------------------------------- the quotient x / s, exactly


def _rn32(fr):
    """Nearest fp32 to a positive Fraction (ties to even), normal range only,
    computed from the binary definition with integer arithmetic."""
    assert fr > 0
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    assert -126 <= e <= 127
    ulp = Fraction(2) ** (e - 23)
    n = fr / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * ulp


def _e4m3_nearest(fr):
    """Code of the nearest E4M3 value to a Fraction in [0, 448] (ties to the even
    code), from the format definition: m 2^-9 for exponent field 0, else
    (1 + m/8) 2^(e-7), the all-ones code excluded."""
    best = None
    for code, val in enumerate(_E4M3_VALUES):
        d = abs(val - fr)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


_E4M3_VALUES = [Fraction(c & 7, 512) if c >> 3 == 0 else (1 + Fraction(c & 7, 8)) * Fraction(2) ** ((c >> 3) - 7)
                for c in range(127)]


def _quotient_cases():
    """fp32 values x near s * (an E4M3 midpoint), for several row maxima: the
    exact quotient x / s sits within a few fp32 ulps of a rounding boundary of
    the E4M3 grid, where fp32 rounding of the quotient decides the code."""
    mids = [Fraction(17), Fraction(19), Fraction(3, 2) * Fraction(1, 512), Fraction(9, 8) + Fraction(1, 16),
            Fraction(100), Fraction(208), Fraction(5, 64) + Fraction(1, 256)]
    cases = []
    for amax in (1.0, 3.7, 0.3, 123.456, 7.0e-3, 5.5e4, 0.91):
        a32 = np.float32(amax)
        s = _rn32(Fraction(float(a32)) / 448)
        s32 = np.float32(float(s))
        assert Fraction(float(s32)) == s
        for m in mids:
            centre = np.float32(float(m * s))
            xs = [centre]
            lo = hi = centre
            for _ in range(48):
                lo = np.nextafter(lo, np.float32(0))
                hi = np.nextafter(hi, np.float32(np.inf))
                xs += [lo, hi]
            for x in xs:
                if 0 < x <= a32:
                    cases.append((a32, s32, np.float32(x)))
    return cases


def test_quantiser_quotient_is_the_correctly_rounded_fp32_division():
    """The code of x is the nearest E4M3 value to the fp32 value nearest to the
    exact quotient x / s (exact rational arithmetic; reading of the FP8
    rounding that transcript cues 33 and 61 leave open). Cases sit next to the
    E4M3 rounding boundaries, where a reciprocal-multiply quotient
    fp32(x * fp32(1/s)) and an unrounded float64 quotient choose other codes
    for some of them; the test checks that both would fail."""
    cases = _quotient_cases()
    assert len(cases) > 1000
    recip_differs = f64_differs = 0
    by_row = {}
    for a32, s32, x in cases:
        by_row.setdefault(float(a32), []).append((s32, x))
    for amax, items in by_row.items():
        row = np.array([amax] + [x for _, x in items], np.float32)[None, :]
        codes, s = oracle.absmax_quant(row)
        s32 = items[0][0]
        assert s[0] == s32
        sf = Fraction(float(s32))
        for col, (_, x) in enumerate(items, start=1):
            q = Fraction(float(x)) / sf
            want = _e4m3_nearest(_rn32(q))
            assert int(codes[0, col]) == want, (amax, float(x))
            rinv = _rn32(1 / sf)
            recip_differs += _e4m3_nearest(_rn32(Fraction(float(x)) * rinv)) != want
            f64_differs += _e4m3_nearest(Fraction(float(x) / float(s32))) != want
    assert recip_differs > 0 and f64_differs > 0, (recip_differs, f64_differs)
