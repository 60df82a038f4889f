"""Repeatability and NaN locality of the kernels, through the C ABI.

Repeatability: the same call on the same inputs gives bit-identical outputs
(no atomics race on a float sum, no order that depends on scheduling).

NaN locality: a NaN planted in one input row reaches only the outputs that
read it; every other output is bit-identical to the run without the NaN.
"""

import math

import numpy as np
import pytest
import torch

import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import DEV, needs_gpu, print_case

pytestmark = [pytest.mark.gpu, needs_gpu]

NAN = float("nan")


def same(a, b):
    """Bitwise equality (NaN patterns included)."""
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def nan_where(t):
    return torch.isnan(t.float())


# ------------------------------------------------------------- repeatability


def test_decode_repeatable():
    print_case(test="decode_repeat")
    q, k, v = (t.to(DEV) for t in inputs.decode_inputs(31, 2, 16, 4, 5000, 128))
    a = rf.attn_decode(q, k, v, 0.08, 16)
    b = rf.attn_decode(q, k, v, 0.08, 16)
    assert same(a[0], b[0]) and same(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        assert same(x, y)


def test_decode_fp32_repeatable():
    print_case(test="decode_fp32_repeat")
    q, k, v = (t.to(DEV) for t in inputs.decode_inputs(32, 2, 8, 2, 3000, 64, dtype=torch.float32))
    a = rf.attn_decode(q, k, v, 0.1, 4, out_dtype=torch.float32)
    b = rf.attn_decode(q, k, v, 0.1, 4, out_dtype=torch.float32)
    assert same(a[0], b[0]) and same(a[1], b[1])


def test_merge_repeatable():
    print_case(test="merge_repeat")
    g = torch.Generator().manual_seed(33)
    m = (torch.randn(64, 9, generator=g) * 4).to(DEV)
    l = (torch.rand(64, 9, generator=g) * 50 + 0.5).to(DEV)
    acc = torch.randn(64, 9, 128, generator=g).to(DEV)
    for dt in (torch.float32, torch.bfloat16):
        a = rf.merge_states(m, l, acc, out_dtype=dt)
        b = rf.merge_states(m, l, acc, out_dtype=dt)
        assert same(a[0], b[0]) and same(a[1], b[1])


def test_mla_fused_repeatable():
    print_case(test="mla_fused_repeat")
    q, kv = (t.to(DEV) for t in inputs.mla_inputs(34, 3, 32, 1500))
    a = rf.mla_decode(q, kv, 0.05, 7, fused=True)
    b = rf.mla_decode(q, kv, 0.05, 7, fused=True)
    assert same(a[0], b[0]) and same(a[1], b[1])


def test_routing_repeatable():
    print_case(test="routing_repeat")
    x = inputs.routing_inputs(35, 4096, 256).to(DEV)
    for renorm in (True, False):
        a = rf.softmax_topk(x, 8, renorm)
        b = rf.softmax_topk(x, 8, renorm)
        assert same(a[0], b[0]) and same(a[1], b[1])


def test_gemms_repeatable():
    print_case(test="gemm_repeat")
    a, bsrc = inputs.quant_inputs(36, 520, 776, 1024)
    a = a.to(DEV)
    bq, bs = rf.absmax_quant_fp8(bsrc.to(DEV))
    c1 = rf.absmax_quant_gemm_fp8(a, bq, bs)
    c2 = rf.absmax_quant_gemm_fp8(a, bq, bs)
    for x, y in zip(c1, c2):
        assert same(x, y)
    r1 = rf.absmax_quant_gemm_fp8_running(a, bq, bs)
    r2 = rf.absmax_quant_gemm_fp8_running(a, bq, bs)
    assert same(r1[0], r2[0]) and same(r1[1], r2[1])


# ---------------------------------------------------------------- NaN locality


@pytest.mark.parametrize("causal", [False, True])
def test_attention_nan_in_a_query_row(causal):
    print_case(test="attn_nan_q", causal=causal)
    q, k, v = (t.to(DEV) for t in inputs.attention_inputs(37, 2, 4, 2, 300, 300, 128))
    o0, l0 = rf.attn_fwd(q, k, v, 0.1, causal=causal)
    q2 = q.clone()
    q2[1, 2, 70, 5] = NAN
    o1, l1 = rf.attn_fwd(q2, k, v, 0.1, causal=causal)
    hit = torch.zeros(o0.shape[:3], dtype=torch.bool, device=DEV)
    hit[1, 2, 70] = True
    assert nan_where(o1[hit]).all() and nan_where(l1[hit]).all()
    assert same(o1[~hit], o0[~hit]) and same(l1[~hit], l0[~hit])


def test_attention_nan_in_a_key_row_causal():
    """Causal: query rows before the key never see it (their score is masked
    before it is used); rows from the key on, in the heads that read that
    key/value head, are NaN; other heads are untouched."""
    print_case(test="attn_nan_k")
    q, k, v = (t.to(DEV) for t in inputs.attention_inputs(38, 2, 4, 2, 300, 300, 64))
    o0, l0 = rf.attn_fwd(q, k, v, 0.1, causal=True)
    k2 = k.clone()
    k2[0, 1, 100, 3] = NAN
    o1, l1 = rf.attn_fwd(q, k2, v, 0.1, causal=True)
    hit = torch.zeros(o0.shape[:3], dtype=torch.bool, device=DEV)
    hit[0, 2:4, 100:] = True                    # query heads 2, 3 read key/value head 1
    assert nan_where(o1[hit]).all() and nan_where(l1[hit]).all()
    assert same(o1[~hit], o0[~hit]) and same(l1[~hit], l0[~hit])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_nan_locality(dtype):
    """A NaN in one query row spoils that head only; a NaN in one key row
    spoils the segment holding it, for the heads reading that key/value head,
    and the merged outputs of those heads."""
    print_case(test="decode_nan", dtype=dtype)
    B, Hq, Hkv, Lk, d, S = 2, 8, 2, 1000, 128, 4
    q, k, v = (t.to(DEV) for t in inputs.decode_inputs(39, B, Hq, Hkv, Lk, d, dtype=dtype))
    o0, l0, (m0, s0, a0) = rf.attn_decode(q, k, v, 0.1, S, out_dtype=torch.float32)

    q2 = q.clone()
    q2[1, 5, 17] = NAN
    o1, l1, (m1, s1, a1) = rf.attn_decode(q2, k, v, 0.1, S, out_dtype=torch.float32)
    row = torch.zeros((B, Hq), dtype=torch.bool, device=DEV)
    row[1, 5] = True
    assert nan_where(o1[row]).all() and nan_where(l1[row]).all() and nan_where(s1[row]).all()
    assert same(o1[~row], o0[~row]) and same(l1[~row], l0[~row])
    assert same(m1[~row], m0[~row]) and same(s1[~row], s0[~row]) and same(a1[~row], a0[~row])

    k2 = k.clone()
    k2[0, 1, 600, 9] = NAN                      # segment 600 // 250 = 2 of key/value head 1
    o2, l2, (m2, s2, a2) = rf.attn_decode(q, k2, v, 0.1, S, out_dtype=torch.float32)
    seg = torch.zeros((B, Hq, S), dtype=torch.bool, device=DEV)
    seg[0, 4:8, 2] = True
    assert nan_where(s2[seg]).all() and nan_where(a2[seg]).all()
    assert same(s2[~seg], s0[~seg]) and same(a2[~seg], a0[~seg])
    heads = seg.any(-1)
    assert nan_where(o2[heads]).all() and nan_where(l2[heads]).all()
    assert same(o2[~heads], o0[~heads]) and same(l2[~heads], l0[~heads])


def test_merge_nan_locality():
    print_case(test="merge_nan")
    g = torch.Generator().manual_seed(40)
    m = (torch.randn(16, 5, generator=g) * 4).to(DEV)
    l = (torch.rand(16, 5, generator=g) * 50 + 0.5).to(DEV)
    acc = torch.randn(16, 5, 128, generator=g).to(DEV)
    o0, l0 = rf.merge_states(m, l, acc, out_dtype=torch.float32)
    acc2 = acc.clone()
    acc2[6, 3, 40] = NAN
    o1, l1 = rf.merge_states(m, l, acc2, out_dtype=torch.float32)
    assert torch.isnan(o1[6, 40]) and same(l1, l0)
    keep = torch.ones(16, dtype=torch.bool, device=DEV)
    keep[6] = False
    assert same(o1[keep], o0[keep])
    assert same(o1[6, :40], o0[6, :40]) and same(o1[6, 41:], o0[6, 41:])


@pytest.mark.parametrize("E,k", [(256, 8), (128, 4), (1024, 8)])
def test_routing_nan_locality(E, k):
    """A NaN logit in one token's row leaves every other token's weights and
    expert indices bit-identical."""
    print_case(test="routing_nan", E=E, k=k)
    T = 1000
    x = inputs.routing_inputs(41, T, E).to(DEV)
    w0, i0 = rf.softmax_topk(x, k, True)
    x2 = x.clone()
    x2[7, 3] = NAN
    x2[600, E - 1] = NAN
    w1, i1 = rf.softmax_topk(x2, k, True)
    keep = torch.ones(T, dtype=torch.bool, device=DEV)
    keep[[7, 600]] = False
    assert same(w1[keep], w0[keep]) and same(i1[keep], i0[keep])
    assert ((i1[~keep] >= 0) & (i1[~keep] < E)).all()       # indices still name experts


@pytest.mark.parametrize("fused", [False, True])
def test_mla_nan_locality(fused):
    """A NaN in one query head spoils that head only, in both launch forms; a
    NaN in one latent row spoils the sequence's heads and no other sequence."""
    print_case(test="mla_nan", fused=fused)
    B, H, Lk, S = 3, 32, 700, 5
    q, kv = (t.to(DEV) for t in inputs.mla_inputs(42, B, H, Lk))
    o0, l0, _ = rf.mla_decode(q, kv, 0.05, S, out_dtype=torch.float32, fused=fused)
    q2 = q.clone()
    q2[1, 20, 300] = NAN
    o1, l1, _ = rf.mla_decode(q2, kv, 0.05, S, out_dtype=torch.float32, fused=fused)
    row = torch.zeros((B, H), dtype=torch.bool, device=DEV)
    row[1, 20] = True
    assert nan_where(o1[row]).all() and nan_where(l1[row]).all()
    assert same(o1[~row], o0[~row]) and same(l1[~row], l0[~row])
    kv2 = kv.clone()
    kv2[2, 450, 7] = NAN
    o2, l2, _ = rf.mla_decode(q, kv2, 0.05, S, out_dtype=torch.float32, fused=fused)
    seq = torch.zeros((B, H), dtype=torch.bool, device=DEV)
    seq[2] = True
    assert nan_where(o2[seq]).all() and nan_where(l2[seq]).all()
    assert same(o2[~seq], o0[~seq]) and same(l2[~seq], l0[~seq])


def test_merge_all_nan_state_row():
    """A row whose only non-empty state has l = NaN (what a segment of all-NaN
    scores leaves: max -inf, l NaN) merges to NaN, not to an empty row."""
    print_case(test="merge_nan_state")
    m = torch.full((2, 3), float("-inf"), device=DEV)
    l = torch.zeros((2, 3), device=DEV)
    acc = torch.zeros((2, 3, 128), device=DEV)
    l[0, 1] = NAN
    acc[0, 1] = NAN
    o, lse = rf.merge_states(m, l, acc, out_dtype=torch.float32)
    assert torch.isnan(o[0]).all() and torch.isnan(lse[0])
    assert (o[1] == 0).all() and lse[1] == float("-inf")
