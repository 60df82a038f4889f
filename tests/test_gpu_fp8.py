"""GPU parity of the FP8 cascade (rf_absmax_quant_fp8, rf_absmax_quant_gemm_fp8,
and the one-pass running-scale form) through the C ABI: quantised codes and
scales bit-exact against the oracle, the GEMM within 3e-2 relative Frobenius
error of the oracle's fp64 result for the same quantised operands, and every
entry of C within the fp32-accumulation bound of assert_fp8_entries."""

import numpy as np
import pytest
import torch

import oracle
import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import DEV, FP8_REL_FRO, assert_fp8_entries, needs_gpu, np32, print_case, rel_fro

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.mark.parametrize("rows,cols", [(4, 8), (37, 520), (64, 7168), (3, 8192)])
def test_quantiser_bit_exact(rows, cols):
    print_case(test="quant", rows=rows, cols=cols)
    a, _ = inputs.quant_inputs(10, rows, 2, cols)
    x = a.clone()
    x[0] = 0                                   # zero row
    if rows > 2:
        x[2, ::3] = -0.0                       # signed zeros
    q, s = rf.absmax_quant_fp8(x.to(DEV))
    q_ref, s_ref = oracle.absmax_quant(x.float().numpy())
    assert np.array_equal(s.cpu().numpy(), s_ref)
    got = q.cpu().numpy()
    bad = np.argwhere(got != q_ref)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}"


def test_quantiser_rounding_edges():
    """Values placed on e4m3 midpoints after scaling by 448 / absmax = 1."""
    t = oracle.e4m3_table()
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    row = np.concatenate([[448.0], mids, -mids])
    row = np.concatenate([row, np.zeros((-len(row)) % 8)]).astype(np.float32)
    x = torch.from_numpy(np.stack([row, row * 0.5])).to(torch.bfloat16)
    q, s = rf.absmax_quant_fp8(x.to(DEV))
    q_ref, s_ref = oracle.absmax_quant(x.float().numpy())
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _all_bf16_rows(amax_values, seed):
    """Rows holding every positive bf16 pattern up to each abs-max value A (random
    signs), A itself first in every row, zero-padded to 8192 columns."""
    rng = np.random.default_rng(seed)
    rows = []
    for a in amax_values:
        abits = int(torch.tensor([a], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        pats = np.arange(1, abits, dtype=np.uint32)
        vals = (pats << 16).view(np.float32) * rng.choice([-1.0, 1.0], size=len(pats)).astype(np.float32)
        top = np.float32((np.uint32(abits) << 16).view(np.float32))
        for i in range(0, len(vals), 8191):
            row = np.zeros(8192, np.float32)
            row[0] = top
            part = vals[i:i + 8191]
            row[1:1 + len(part)] = part
            rows.append(row)
    return torch.from_numpy(np.stack(rows)).to(torch.bfloat16)


def test_quantiser_every_bf16_pattern():
    """The division x / s and the e4m3 rounding on every input bit pattern a row can
    hold, for 16 row maxima: one so small that 1/s overflows fp32, two whose scale
    is an fp32 subnormal with a finite reciprocal (there x - s q underflows and one
    correction step of x * (1/s) is not always the correctly rounded quotient),
    and two around 448 * 2^-90, the smallest scale the fast path takes."""
    x = _all_bf16_rows([448.0, 1.0, 3.5, 0.0078125, 1e-3, 17.25, 6.0e4, 2.0 ** -100, 123.456, 0.3,
                        1e30, 5e-38, 2e-36, 4e-36, 1e-25, 1e-24], seed=13)
    print_case(test="quant_all_bf16", rows=x.shape[0])
    q, s = rf.absmax_quant_fp8(x.to(DEV))
    q_ref, s_ref = oracle.absmax_quant(x.float().numpy())
    assert np.array_equal(s.cpu().numpy(), s_ref)
    got = q.cpu().numpy()
    bad = np.argwhere(got != q_ref)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(64, 64, 256), (300, 200, 512), (256, 512, 1024), (1, 3, 128),
                                   (40, 260, 8192),    # largest supported K, ragged M and N
                                   (520, 264, 256), (72, 776, 384)])   # N % 8 == 0, partial tiles
def test_gemm_small(M, N, K):
    print_case(test="gemm_small", M=M, N=N, K=K)
    a, bsrc = inputs.quant_inputs(11, M, N, K)
    bq, bs = rf.absmax_quant_fp8(bsrc.to(DEV))
    c, aq, sa = rf.absmax_quant_gemm_fp8(a.to(DEV), bq, bs)
    aq_ref, sa_ref = oracle.absmax_quant(a.float().numpy())
    assert np.array_equal(aq.cpu().numpy(), aq_ref) and np.array_equal(sa.cpu().numpy(), sa_ref)
    c_ref = oracle.quant_gemm(aq_ref, sa_ref, bq.cpu().numpy(), bs.cpu().numpy())
    assert rel_fro(np32(c), c_ref) <= FP8_REL_FRO
    # Much tighter in fact: fp32 accumulation + one bf16 rounding, entry by entry.
    assert rel_fro(np32(c), c_ref) <= 5e-3
    assert_fp8_entries(np32(c), c_ref, two_pass_magnitude(aq_ref, sa_ref, bq.cpu().numpy(), bs.cpu().numpy()),
                       K + 4, f"gemm {M}x{N}x{K}")


def two_pass_magnitude(aq, sa, bq, bs):
    """s_i t_j sum_k |a_ik b_jk| over the e4m3 codes (exact in fp64)."""
    ma, mb = np.abs(oracle.e4m3_decode(aq)), np.abs(oracle.e4m3_decode(bq))
    return sa.astype(np.float64)[:, None] * bs.astype(np.float64)[None, :] * (ma @ mb.T)


def running_magnitude(x, bq, bs):
    """The one-pass sum over absolute values: the running-scale oracle on |A|
    and |B| (the codes of |x| are the magnitudes of the codes of x, and the
    scales, running ones included, are the same)."""
    return oracle.quant_gemm_running_scale(np.abs(x), bq & 0x7F, bs, K_TILE)


def running_units(K):
    """K additions, at most K / 64 rescales of three roundings each, scales."""
    return K + 3 * K // K_TILE + 4


# ---- one-pass form with a running per-row scale (K tiles of 64 columns)

K_TILE = 64


def _running_case(a, bsrc):
    bq, bs = rf.absmax_quant_fp8(bsrc.to(DEV))
    c, sa = rf.absmax_quant_gemm_fp8_running(a.to(DEV), bq, bs)
    x = a.float().numpy()
    c_ref = oracle.quant_gemm_running_scale(x, bq.cpu().numpy(), bs.cpu().numpy(), K_TILE)
    _, sa_ref = oracle.absmax_quant(x)
    return np32(c), c_ref, sa.cpu().numpy(), sa_ref, bq, bs


@pytest.mark.parametrize("M,N,K", [(64, 64, 256), (300, 200, 512), (256, 512, 1024), (1, 3, 128),
                                   (513, 260, 7168), (129, 517, 256)])
def test_running_scale_gemm_small(M, N, K):
    print_case(test="gemm_running", M=M, N=N, K=K)
    a, bsrc = inputs.quant_inputs(12, M, N, K)
    c, c_ref, sa, sa_ref, bq, bs = _running_case(a, bsrc)
    assert np.array_equal(sa, sa_ref)          # the final running scale is the row's scale
    assert rel_fro(c, c_ref) <= 5e-3
    assert_fp8_entries(c, c_ref, running_magnitude(a.float().numpy(), bq.cpu().numpy(), bs.cpu().numpy()),
                       running_units(K), f"running {M}x{N}x{K}")


def test_running_scale_tiny_scales():
    """Rows with tiny scales: fp32 subnormal scales whose reciprocal overflows and
    ones whose reciprocal is finite, normal scales below 2^-90, a row that grows
    from tiny to normal size and one that shrinks. The divisions of those rows do
    not take the one-correction path, and the result still matches the
    oracle."""
    M, N, K = 64, 128, 1024
    a, bsrc = inputs.quant_inputs(14, M, N, K)
    a = a.clone()
    a[0:8] *= 1e-37      # abs-max ~4e-37: s ~1e-39, 1/s overflows
    a[8:16] *= 1e-36     # abs-max ~4e-36: s ~1e-38 (subnormal), 1/s finite
    a[16:24] *= 1e-26    # s ~1e-28: normal, below 2^-90
    a[24, :512] *= 1e-36
    a[25, 512:] *= 1e-36
    print_case(test="gemm_running_tiny")
    c, c_ref, sa, sa_ref, bq, bs = _running_case(a, bsrc)
    assert np.array_equal(sa, sa_ref)
    for r in range(M):
        assert rel_fro(c[r], c_ref[r]) <= 5e-3, r
    assert_fp8_entries(c, c_ref, running_magnitude(a.float().numpy(), bq.cpu().numpy(), bs.cpu().numpy()),
                       running_units(K), "running, tiny scales")


def test_running_scale_growth_and_zero_rows():
    """Rows whose abs-max grows late (an outlier in the last K tile), rows that
    start with zero tiles, and an all-zero row."""
    M, N, K = 96, 128, 1024
    a, bsrc = inputs.quant_inputs(13, M, N, K)
    a = a.clone()
    a[1, :] = 0
    a[2, : K // 2] = 0
    a[3, -1] = 1000.0
    a[4, 5 * K_TILE + 3] = -300.0
    print_case(test="gemm_running_growth")
    c, c_ref, sa, sa_ref, bq, bs = _running_case(a, bsrc)
    assert np.array_equal(sa, sa_ref)
    assert np.all(c[1] == 0)
    assert rel_fro(c, c_ref) <= 5e-3
    for r in (2, 3, 4):
        assert rel_fro(c[r], c_ref[r]) <= 5e-3
    assert_fp8_entries(c, c_ref, running_magnitude(a.float().numpy(), bq.cpu().numpy(), bs.cpu().numpy()),
                       running_units(K), "running, growth and zero rows")
