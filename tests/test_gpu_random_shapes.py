"""Seeded random shapes for every entry point of the path, compared with the
fp64 oracle at the bars the per-kernel tests use. The per-kernel tests pick
their shapes by hand (one tile, ragged tails, empty segments, the configs);
these draw the sizes at random within what each entry point accepts (GQA
groups 1-16, head sizes 64 and 128, 1-69 segments, rows of any multiple of 4
or 8 values up to the limits, GEMM sides of any length and K any multiple of
128), so that combinations nobody picked meet the kernels too. The draws are
fixed by the seed below, so every run tests the same cases."""

import math

import numpy as np
import pytest
import torch

import oracle
import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import (DEV, FP32_REL, assert_bf16_attention, assert_fp8_entries, needs_gpu, normwise,
                      np32, print_case, rel_fro)
from test_gpu_decode import _check_partials
from test_gpu_fp8 import running_magnitude, running_units, two_pass_magnitude
from test_gpu_moments import _compare as _compare_moments
from test_gpu_softmax import _compare as _compare_softmax

pytestmark = [pytest.mark.gpu, needs_gpu]

_rng = np.random.default_rng(20261202)


def _draw(n, fn):
    return [fn(_rng) for _ in range(n)]


def _attn_case(r):
    d = int(r.choice([64, 128]))
    Hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 4, 8]))
    causal = bool(r.integers(0, 2))
    Lk = int(r.integers(1, 400))
    Lq = Lk if causal else int(r.integers(1, 400))
    return (int(r.integers(1, 3)), Hkv * G, Hkv, Lq, Lk, d, causal)


def _decode_case(r):
    d = int(r.choice([64, 128]))
    Hkv = int(r.integers(1, 4))
    G = int(r.integers(1, 17))
    Lk = int(r.integers(1, 3000))
    S = int(r.integers(1, 70))
    return (int(r.integers(1, 3)), Hkv * G, Hkv, Lk, d, S)


ATTN_BF16 = _draw(30, _attn_case)
ATTN_F32 = _draw(12, _attn_case)
DECODE_BF16 = _draw(30, _decode_case)
DECODE_F32 = _draw(20, _decode_case)
ROUTING = _draw(30, lambda r: (int(r.integers(1, 200)), int(4 * r.integers(1, 257)), int(r.integers(1, 33)),
                               bool(r.integers(0, 2))))
QUANT = _draw(20, lambda r: (int(r.integers(1, 40)), int(8 * r.integers(1, 1025))))
GEMM = _draw(20, lambda r: (int(r.integers(1, 300)), int(r.integers(1, 300)), int(128 * r.integers(1, 17))))
MLA = _draw(12, lambda r: (int(r.integers(1, 4)), int(r.choice([16, 32])), int(r.integers(1, 1500)),
                          int(r.integers(1, 13)), bool(r.integers(0, 2))))
ROWS = _draw(30, lambda r: (int(r.integers(1, 40)), int(4 * r.integers(1, 2049)), int(r.integers(0, 4))))


@pytest.mark.parametrize("case", ATTN_BF16, ids=str)
def test_random_attention_bf16(case):
    B, Hq, Hkv, Lq, Lk, d, causal = case
    print_case(test="random_attn_bf16", shape=case)
    q, k, v = inputs.attention_inputs(31, B, Hq, Hkv, Lq, Lk, d)
    scale = 1 / math.sqrt(d)
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal=causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
    assert_bf16_attention(np32(o), o_ref, np32(lse), lse_ref, what=str(case))


@pytest.mark.parametrize("case", ATTN_F32, ids=str)
def test_random_attention_fp32(case):
    B, Hq, Hkv, Lq, Lk, d, causal = case
    print_case(test="random_attn_fp32", shape=case)
    q, k, v = inputs.attention_inputs(32, B, Hq, Hkv, Lq, Lk, d, dtype=torch.float32)
    scale = 1 / math.sqrt(d)
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal=causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
    assert normwise(np32(o), o_ref) <= FP32_REL
    assert np.abs(np32(lse) - lse_ref).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


def _decode(case, dtype, seed, acc_bar, out_bar):
    B, Hq, Hkv, Lk, d, S = case
    q, k, v = inputs.decode_inputs(seed, B, Hq, Hkv, Lk, d, dtype=dtype)
    scale = 1 / math.sqrt(d)
    o, lse, (m, l, acc) = rf.attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, S, out_dtype=torch.float32)
    _check_partials(m, l, acc, *oracle.decode_partials(q, k, v, scale, S), acc_bar=acc_bar)
    o_ref, lse_ref = oracle.attention(q[:, :, None], k, v, scale)
    assert normwise(np32(o), o_ref[:, :, 0]) <= out_bar
    assert np.abs(np32(lse) - lse_ref[:, :, 0]).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


@pytest.mark.parametrize("case", DECODE_BF16, ids=str)
def test_random_decode_bf16(case):
    print_case(test="random_decode_bf16", shape=case)
    _decode(case, torch.bfloat16, 33, 1e-4, 1e-4)


@pytest.mark.parametrize("case", DECODE_F32, ids=str)
def test_random_decode_fp32(case):
    print_case(test="random_decode_fp32", shape=case)
    _decode(case, torch.float32, 34, FP32_REL, FP32_REL)


@pytest.mark.parametrize("case", ROUTING, ids=str)
def test_random_routing(case):
    T, E, k, renorm = case
    k = min(k, E)
    print_case(test="random_routing", T=T, E=E, k=k, renormalize=renorm)
    x = inputs.routing_inputs(35, T, E)
    w, idx = rf.softmax_topk(x.to(DEV), k, renorm)
    w_ref, idx_ref = oracle.softmax_topk(x.numpy(), k, renorm)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert (np.abs(np32(w) - w_ref) / w_ref).max() <= 1e-5


@pytest.mark.parametrize("case", QUANT, ids=str)
def test_random_quantiser(case):
    rows, cols = case
    print_case(test="random_quant", rows=rows, cols=cols)
    x, _ = inputs.quant_inputs(36, rows, 1, cols)
    q, s = rf.absmax_quant_fp8(x.to(DEV))
    q_ref, s_ref = oracle.absmax_quant(x.float().numpy())
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("case", GEMM, ids=str)
def test_random_fp8_gemms(case):
    """The two-pass cascade (codes, scales and C) and the one-pass running-scale
    form (final scales and C) on the same operands."""
    M, N, K = case
    print_case(test="random_fp8", M=M, N=N, K=K)
    a, bsrc = inputs.quant_inputs(37, M, N, K)
    bq, bs = rf.absmax_quant_fp8(bsrc.to(DEV))
    c, aq, sa = rf.absmax_quant_gemm_fp8(a.to(DEV), bq, bs)
    aq_ref, sa_ref = oracle.absmax_quant(a.float().numpy())
    assert np.array_equal(sa.cpu().numpy(), sa_ref)
    assert np.array_equal(aq.cpu().numpy(), aq_ref)
    bqh, bsh = bq.cpu().numpy(), bs.cpu().numpy()
    c_ref = oracle.quant_gemm(aq_ref, sa_ref, bqh, bsh)
    assert rel_fro(np32(c), c_ref) <= 5e-3
    assert_fp8_entries(np32(c), c_ref, two_pass_magnitude(aq_ref, sa_ref, bqh, bsh), K + 4, "two-pass")
    c2, sa2 = rf.absmax_quant_gemm_fp8_running(a.to(DEV), bq, bs)
    x = a.float().numpy()
    c2_ref = oracle.quant_gemm_running_scale(x, bqh, bsh, 64)
    assert np.array_equal(sa2.cpu().numpy(), sa_ref)
    assert rel_fro(np32(c2), c2_ref) <= 5e-3
    assert_fp8_entries(np32(c2), c2_ref, running_magnitude(x, bqh, bsh), running_units(K), "running")


@pytest.mark.parametrize("case", MLA, ids=str)
def test_random_mla(case):
    B, H, Lk, S, fused = case
    print_case(test="random_mla", B=B, H=H, Lk=Lk, S=S, fused=fused)
    q, kv = inputs.mla_inputs(38, B, H, Lk)
    scale = 1 / math.sqrt(576)
    o, lse, _ = rf.mla_decode(q.to(DEV), kv.to(DEV), scale, S, out_dtype=torch.float32, fused=fused)
    lat = kv[:, None]
    o_ref, lse_ref = oracle.attention(q[:, :, None], lat, lat[..., :512], scale)
    o_ref, lse_ref = o_ref[:, :, 0], lse_ref[:, :, 0]
    assert (np.abs(np32(o) - o_ref).max(-1) / np.abs(o_ref).max(-1)).max() <= 1e-4
    assert np.abs(np32(lse) - lse_ref).max() <= 1e-5 * np.abs(lse_ref).max()


@pytest.mark.parametrize("case", ROWS, ids=str)
def test_random_row_cascades(case):
    """Softmax, variance and inertia of the same row sizes at one fusion level."""
    T, E, level = case
    print_case(test="random_rows", T=T, E=E, level=level)
    x = inputs.softmax_inputs(39, T, E)
    y = rf.softmax(x.to(DEV), level).cpu().numpy().astype(np.float64)
    _compare_softmax(y, x.numpy(), oracle.softmax_rows(x.numpy()))
    xm, w = inputs.moment_inputs(40, T, E)
    mean, var = rf.row_variance(xm.to(DEV), level)
    m_ref, v_ref = oracle.row_variance(xm.numpy())
    _compare_moments(mean.cpu().numpy(), var.cpu().numpy() * E, m_ref, v_ref * E, np.full(T, float(E)),
                     f"{case} variance")
    centre, inertia = rf.row_inertia(xm.to(DEV), w.to(DEV), level)
    c_ref, i_ref = oracle.row_inertia(xm.numpy(), w.numpy())
    _compare_moments(centre.cpu().numpy(), inertia.cpu().numpy(), c_ref, i_ref, w.numpy().astype(np.float64).sum(1),
                     f"{case} inertia")


# ---- large logits: scores of standard deviation sigma^2 (one-hot softmax rows,
# the reference of every row moving many times along the key axis)

@pytest.mark.parametrize("sigma", [4.0, 8.0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_large_logits_attention(sigma, causal, dtype):
    B, Hq, Hkv, L, d = 1, 4, 2, 333, 128
    print_case(test="large_logits_attn", sigma=sigma, causal=causal, dtype=dtype)
    q, k, v = inputs.attention_inputs(41, B, Hq, Hkv, L, L, d, dtype=dtype)
    q = (q.float() * sigma).to(dtype)
    k = (k.float() * sigma).to(dtype)
    scale = 1 / math.sqrt(d)
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal=causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
    if dtype == torch.bfloat16:
        assert_bf16_attention(np32(o), o_ref, np32(lse), lse_ref, what=f"sigma={sigma}")
    else:
        # fp32: the probabilities' relative error grows with the score
        # magnitude (see the decode test below)
        grow = 4 * 2.0 ** -24 * np.abs(lse_ref).max()
        assert normwise(np32(o), o_ref) <= FP32_REL + grow
        assert np.abs(np32(lse) - lse_ref).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


@pytest.mark.parametrize("sigma", [4.0, 8.0])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_large_logits_decode(sigma, dtype):
    B, Hq, Hkv, Lk, d, S = 2, 8, 2, 2500, 128, 7
    print_case(test="large_logits_decode", sigma=sigma, dtype=dtype)
    q, k, v = inputs.decode_inputs(42, B, Hq, Hkv, Lk, d, dtype=dtype)
    q = (q.float() * sigma).to(dtype)
    k = (k.float() * sigma).to(dtype)
    scale = 1 / math.sqrt(d)
    o, lse, (m, l, acc) = rf.attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, S, out_dtype=torch.float32)
    bar = 1e-4 if dtype == torch.bfloat16 else FP32_REL
    m_ref, l_ref, acc_ref = oracle.decode_partials(q, k, v, scale, S)
    m, l, acc = (np.asarray(np32(t), np.float64) for t in (m, l, acc))
    assert np.array_equal(np.isinf(m), np.isinf(m_ref))
    fin = ~np.isinf(m_ref)
    assert np.abs(m[fin] - m_ref[fin]).max() <= 1e-5 * np.abs(m_ref[fin]).max()
    # (m, l, acc) stands for sum e^s = l e^m: compare l and acc moved to the
    # oracle's max. Each probability is exp2 of an fp32 fma on scores and a
    # max of magnitude |m| log2(e), so its relative error grows like
    # 4 * 2^-24 * |m| (on top of the 1e-5 of the small-logit tests).
    shift = np.exp(m[fin] - m_ref[fin])
    grow = 4 * 2.0 ** -24 * np.abs(m_ref[fin]).max()
    assert normwise(l[fin] * shift, l_ref[fin]) <= 1e-5 + grow
    assert normwise(acc[fin] * shift[:, None], acc_ref[fin]) <= bar + grow
    o_ref, lse_ref = oracle.attention(q[:, :, None], k, v, scale)
    assert normwise(np32(o), o_ref[:, :, 0]) <= bar
    assert np.abs(np32(lse) - lse_ref[:, :, 0]).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


@pytest.mark.parametrize("fused", [False, True])
def test_large_logits_mla(fused):
    """Latent rows and queries scaled by 4: scores of standard deviation about 16."""
    B, H, Lk, S = 2, 16, 1100, 5
    print_case(test="large_logits_mla", fused=fused)
    q, kv = inputs.mla_inputs(43, B, H, Lk)
    q = (q.float() * 4).to(torch.bfloat16)
    kv = (kv.float() * 4).to(torch.bfloat16)
    scale = 1 / math.sqrt(576)
    o, lse, _ = rf.mla_decode(q.to(DEV), kv.to(DEV), scale, S, out_dtype=torch.float32, fused=fused)
    lat = kv[:, None]
    o_ref, lse_ref = oracle.attention(q[:, :, None], lat, lat[..., :512], scale)
    o_ref, lse_ref = o_ref[:, :, 0], lse_ref[:, :, 0]
    grow = 4 * 2.0 ** -24 * np.abs(lse_ref).max()
    assert (np.abs(np32(o) - o_ref).max(-1) / np.abs(o_ref).max(-1)).max() <= 1e-4 + grow
    assert np.abs(np32(lse) - lse_ref).max() <= 1e-5 * np.abs(lse_ref).max()


@pytest.mark.parametrize("spread", [100.0, 1e4])
@pytest.mark.parametrize("renormalize", [True, False])
def test_wide_logits_routing(spread, renormalize):
    """Logits of standard deviation 100 and 10^4: all but a few probabilities
    of each row underflow."""
    print_case(test="wide_routing", spread=spread, renormalize=renormalize)
    x = (inputs.routing_inputs(44, 300, 256).double() * spread).float()
    w, idx = rf.softmax_topk(x.to(DEV), 8, renormalize)
    w_ref, idx_ref = oracle.softmax_topk(x.numpy(), 8, renormalize)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    big = w_ref > 1e-30
    w = np32(w)
    assert (np.abs(w[big] - w_ref[big]) / w_ref[big]).max() <= 1e-5
    assert np.abs(w[~big] - w_ref[~big]).max(initial=0.0) <= 1e-30


@pytest.mark.parametrize("scale", [0.0, -0.0, -0.125, -2.0])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_zero_and_negative_scale(scale, dtype):
    """Scale 0 (every unmasked key weighted equally: O is the mean of V, lse =
    ln of the key count) and negative scales, for prefill in both modes (a
    ragged last key tile and the causal diagonal are masked) and for decode."""
    B, Hq, Hkv, L, d = 1, 4, 2, 200, 128
    print_case(test="odd_scale", scale=scale, dtype=dtype)
    q, k, v = inputs.attention_inputs(45, B, Hq, Hkv, L, L, d, dtype=dtype)
    for causal in (False, True):
        o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal=causal)
        o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
        if dtype == torch.bfloat16:
            assert_bf16_attention(np32(o), o_ref, np32(lse), lse_ref, what=f"scale={scale} causal={causal}")
        else:
            grow = 4 * 2.0 ** -24 * np.abs(lse_ref).max()
            assert normwise(np32(o), o_ref) <= FP32_REL + grow
            assert np.abs(np32(lse) - lse_ref).max() <= 1e-5 * max(1, np.abs(lse_ref).max())
        if scale == 0.0:
            n_keys = np.arange(1, L + 1) if causal else np.full(L, L)
            assert np.abs(np32(lse) - np.log(n_keys)).max() <= 1e-5 * math.log(L)
    qd = q[:, :, 0].contiguous()
    o, lse, _ = rf.attn_decode(qd.to(DEV), k.to(DEV), v.to(DEV), scale, 3, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.attention(qd[:, :, None], k, v, scale)
    bar = 1e-4 if dtype == torch.bfloat16 else FP32_REL
    assert normwise(np32(o), o_ref[:, :, 0]) <= bar
    assert np.abs(np32(lse) - lse_ref[:, :, 0]).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


@pytest.mark.parametrize("scale", [0.0, -0.05])
@pytest.mark.parametrize("fused", [False, True])
def test_zero_and_negative_scale_mla(scale, fused):
    B, H, Lk, S = 2, 16, 700, 3
    print_case(test="odd_scale_mla", scale=scale, fused=fused)
    q, kv = inputs.mla_inputs(46, B, H, Lk)
    o, lse, _ = rf.mla_decode(q.to(DEV), kv.to(DEV), scale, S, out_dtype=torch.float32, fused=fused)
    lat = kv[:, None]
    o_ref, lse_ref = oracle.attention(q[:, :, None], lat, lat[..., :512], scale)
    o_ref, lse_ref = o_ref[:, :, 0], lse_ref[:, :, 0]
    assert (np.abs(np32(o) - o_ref).max(-1) / np.abs(o_ref).max(-1)).max() <= 1e-4
    assert np.abs(np32(lse) - lse_ref).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


@pytest.mark.parametrize("d", [4, 100, 128, 260, 512, 1024])
@pytest.mark.parametrize("S", [1, 2, 9, 33])
def test_merge_widths(d, S):
    """The merge at every supported width class (one 128-column block or
    several, a partial block) and segment counts, with empty states mixed in;
    bf16 and fp32 outputs."""
    print_case(test="merge_widths", d=d, S=S)
    rng = np.random.default_rng(100 + d + S)
    rows = 19
    m = (rng.standard_normal((rows, S)) * 4).astype(np.float32)
    l = rng.uniform(0.5, 50, (rows, S)).astype(np.float32)
    acc = rng.standard_normal((rows, S, d)).astype(np.float32)
    m[rng.random((rows, S)) < 0.3] = -np.inf
    m[3] = -np.inf
    l[np.isinf(m)] = 0
    acc[np.isinf(m)] = 0
    o_ref, lse_ref = oracle.merge_states(m, l, acc)
    args = [torch.from_numpy(x).to(DEV) for x in (m, l, acc)]
    o, lse = rf.merge_states(*args, out_dtype=torch.float32)
    assert normwise(np32(o), o_ref) <= FP32_REL
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(np32(lse)), fin)
    assert np.abs(np32(lse)[fin] - lse_ref[fin]).max() <= 1e-5 * max(1, np.abs(lse_ref[fin]).max())
    o16, _ = rf.merge_states(*args, out_dtype=torch.bfloat16)
    assert np.abs(np32(o16) - o_ref).max() <= 2 ** -8 * max(1e-30, np.abs(o_ref).max())


@pytest.mark.parametrize("Lk,S", [(1, 1), (3, 8), (31, 4), (33, 2), (97, 12)])
@pytest.mark.parametrize("fused", [False, True])
def test_mla_short_caches(Lk, S, fused):
    """Latent caches shorter than a step or than the segment count (empty
    segments), in both launch forms."""
    B, H = 2, 16
    print_case(test="mla_short", Lk=Lk, S=S, fused=fused)
    q, kv = inputs.mla_inputs(47, B, H, Lk)
    scale = 1 / math.sqrt(576)
    o, lse, _ = rf.mla_decode(q.to(DEV), kv.to(DEV), scale, S, out_dtype=torch.float32, fused=fused)
    lat = kv[:, None]
    o_ref, lse_ref = oracle.attention(q[:, :, None], lat, lat[..., :512], scale)
    o_ref, lse_ref = o_ref[:, :, 0], lse_ref[:, :, 0]
    assert (np.abs(np32(o) - o_ref).max(-1) / np.abs(o_ref).max(-1)).max() <= 1e-4
    assert np.abs(np32(lse) - lse_ref).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


@pytest.mark.parametrize("renormalize", [True, False])
@pytest.mark.parametrize("E,k", [(256, 8), (64, 4), (1024, 16)])
def test_routing_masked_experts(renormalize, E, k):
    """Experts masked with -inf logits (a common way to disable experts): every
    row keeps at least k finite logits, so the masked ones are never chosen
    and weigh nothing in the denominator."""
    print_case(test="routing_masked", E=E, k=k, renormalize=renormalize)
    rng = np.random.default_rng(48 + E)
    x = inputs.routing_inputs(49, 101, E).numpy().copy()
    for r in range(x.shape[0]):
        n_masked = int(rng.integers(0, E - k + 1))
        x[r, rng.choice(E, size=n_masked, replace=False)] = -np.inf
    x = torch.from_numpy(x)
    w, idx = rf.softmax_topk(x.to(DEV), k, renormalize)
    w_ref, idx_ref = oracle.softmax_topk(x.numpy(), k, renormalize)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.all(np.isfinite(x.numpy()[np.arange(x.shape[0])[:, None], idx.cpu().numpy()]))
    assert (np.abs(np32(w) - w_ref) / w_ref).max() <= 1e-5
