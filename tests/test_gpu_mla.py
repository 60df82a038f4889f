"""GPU parity of split-KV decode over a shared latent cache
(rf_mla_decode_split + rf_merge_states, through the C ABI) against the fp64
oracle: the partial states against oracle.decode_partials with the values
taken as the first 512 columns of the latent rows, the merged output against
oracle.attention. Bars as for split-KV decode: P enters the value product as
a bf16 hi + lo pair (about 16-bit weights), everything else is fp32."""

import math

import numpy as np
import pytest
import torch

import oracle
import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import DEV, needs_gpu, normwise, np32, print_case

pytestmark = [pytest.mark.gpu, needs_gpu]

DQK, DV = 576, 512


def _check(B, H, Lk, S, scale, seed=5, partials=True, fused=False):
    q, kv = inputs.mla_inputs(seed, B, H, Lk)
    o, lse, (m, l, acc) = rf.mla_decode(q.to(DEV), kv.to(DEV), scale, S, out_dtype=torch.float32, fused=fused)
    lat = kv[:, None]                      # [B, 1, Lk, 576]: one shared latent head
    if partials:
        m_ref, l_ref, acc_ref = oracle.decode_partials(q, lat, lat[..., :DV], scale, S)
        m, l, acc = np32(m), np32(l), np32(acc)
        empty = np.isinf(m_ref)
        assert np.array_equal(np.isinf(m), empty)
        assert np.all(l[empty] == 0) and np.all(acc[empty] == 0)
        fin = ~empty
        assert np.abs(m[fin] - m_ref[fin]).max() <= 1e-5 * max(1, np.abs(m_ref[fin]).max())
        assert normwise(l[fin], l_ref[fin]) <= 1e-5
        assert normwise(acc[fin], acc_ref[fin]) <= 1e-4
    o_ref, lse_ref = oracle.attention(q[:, :, None], lat, lat[..., :DV], scale)
    assert normwise(np32(o), o_ref[:, :, 0]) <= 1e-4
    assert np.abs(np32(lse) - lse_ref[:, :, 0]).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


@pytest.mark.parametrize(
    "B,H,Lk,S",
    [
        (1, 16, 1000, 1),
        (1, 16, 1000, 4),
        (2, 16, 777, 16),     # ragged last segment and ragged steps
        (1, 16, 5, 4),        # segment lengths 2, 2, 1, 0: an empty segment
        (1, 16, 100, 64),     # segment length 2: many trailing empty segments
        (2, 32, 513, 3),      # two groups of 16 heads
        (1, 128, 300, 2),     # eight head groups
        (1, 16, 31, 1),       # fewer keys than a step
        (1, 16, 32, 1),
        (1, 16, 33, 2),
        (20, 16, 777, 16),    # 320 workgroups, more than the CUs: two-stage ring
    ],
)
def test_mla_partials_and_merge_small(B, H, Lk, S):
    print_case(test="mla_small", B=B, H=H, Lk=Lk, S=S)
    _check(B, H, Lk, S, 1 / math.sqrt(DQK))


@pytest.mark.parametrize(
    "B,H,Lk,S",
    [
        (1, 16, 1000, 1),     # one workgroup per group: it merges its own state
        (2, 16, 777, 16),
        (1, 16, 5, 4),        # an empty segment still counts itself in
        (1, 16, 100, 64),     # many empty segments
        (3, 32, 513, 3),      # two head groups per sequence, three sequences
        (1, 128, 300, 2),
        (20, 16, 777, 16),    # two-stage ring (more workgroups than CUs)
    ],
)
def test_mla_fused_merge(B, H, Lk, S):
    """rf_mla_decode: split and merge in one launch, against the oracle."""
    print_case(test="mla_fused", B=B, H=H, Lk=Lk, S=S)
    _check(B, H, Lk, S, 1 / math.sqrt(DQK), fused=True)


def test_mla_fused_counters_return_to_zero():
    """Two calls in a row on one counters array (bf16 output): the counters are
    0 after each, and both calls give the same output as the two-launch path
    merged by rf_merge_states (equal up to the merge order's rounding)."""
    print_case(test="mla_fused_repeat")
    B, H, Lk, S = 4, 32, 1200, 8
    scale = 1 / math.sqrt(DQK)
    q, kv = (t.to(DEV) for t in inputs.mla_inputs(9, B, H, Lk))
    pm = torch.empty((B, H, S), device=DEV)
    pl = torch.empty_like(pm)
    pa = torch.empty((B, H, S, DV), device=DEV)
    counters = torch.zeros(B * H // 16, dtype=torch.int32, device=DEV)
    o_ref, lse_ref, _ = rf.mla_decode(q, kv, scale, S, out_dtype=torch.float32)
    for _ in range(2):
        o = torch.full((B, H, DV), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((B, H), float("nan"), device=DEV)
        rf.rf_mla_decode(q, kv, pm, pl, pa, counters, o, lse, scale)
        torch.cuda.synchronize()
        assert int(counters.abs().sum()) == 0
        assert normwise(np32(o), np32(o_ref)) <= 8e-3          # bf16 output rounding
        assert np.abs(np32(lse) - np32(lse_ref)).max() <= 1e-5 * max(1, np.abs(np32(lse_ref)).max())


def test_mla_large_scores():
    """scale 1 with N(0,1) rows: scores with a spread of about 24, so the
    reference max moves often within a segment."""
    print_case(test="mla_large_scores")
    _check(2, 16, 2000, 3, 1.0)


def test_mla_deterministic():
    q, kv = (t.to(DEV) for t in inputs.mla_inputs(3, 2, 32, 1500))
    a = rf.mla_decode(q, kv, 0.05, 5)
    b = rf.mla_decode(q, kv, 0.05, 5)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
