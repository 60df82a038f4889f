"""GPU parity of split-KV decode (rf_attn_decode_split + rf_merge_states) and of
the merge alone, through the C ABI, against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import (DEV, FP32_REL, assert_bf16_attention, needs_gpu, normwise, np32,
                      print_case)

pytestmark = [pytest.mark.gpu, needs_gpu]


def test_worked_example_through_the_kernels():
    """Scores 1, 3 | 5 (transcript cue 15) as a 3-key decode split into
    ceil(3/2) = 2 segments: the partial states are tile A and tile B of the
    worked example, and the merge gives the from-scratch result."""
    print_case(test="worked_example")
    q, k, v = inputs.worked_example_decode(d=128)
    m, l, acc = rf.attn_decode_partials(q.to(DEV), k.to(DEV), v.to(DEV), 1.0, 2)
    m, l, acc = np32(m)[0, 0], np32(l)[0, 0], np32(acc)[0, 0]
    assert abs(m[0] - 3.0) <= 1e-6 and abs(m[1] - 5.0) <= 1e-6
    assert abs(l[0] - (math.exp(-2) + 1)) <= 1e-6 * l[0]
    assert abs(l[1] - 1.0) <= 1e-6
    assert abs(acc[0, 0] - (2 * math.exp(-2) - 1)) <= 1e-5
    assert abs(acc[1, 0] - 4.0) <= 1e-5
    assert np.all(acc[:, 1:] == 0)
    o, lse = rf.merge_states(*(torch.from_numpy(x[None, None]).to(DEV) for x in (m, l, acc)),
                             out_dtype=torch.float32)
    den = math.exp(-4) + math.exp(-2) + 1
    assert abs(np32(lse)[0, 0] - (5 + math.log(den))) <= 1e-5
    assert abs(np32(o)[0, 0, 0] - (2 * math.exp(-4) - math.exp(-2) + 4) / den) <= 1e-5


@pytest.mark.parametrize(
    "B,Hq,Hkv,Lk,S",
    [
        (1, 4, 1, 1000, 1),
        (1, 4, 1, 1000, 4),
        (2, 8, 2, 777, 16),       # ragged last segment and ragged steps
        (1, 4, 1, 5, 4),          # lengths 2, 2, 1, 0: an empty segment
        (1, 4, 4, 100, 64),       # seg length 2: 14 trailing empty segments, G = 1
        (1, 16, 1, 513, 3),       # G = 16
        (2, 6, 2, 96, 2),         # G = 3
    ],
)
def test_partials_and_merge_small(B, Hq, Hkv, Lk, S):
    print_case(test="decode_small", B=B, Hq=Hq, Hkv=Hkv, Lk=Lk, S=S)
    q, k, v = inputs.decode_inputs(5, B, Hq, Hkv, Lk, 128)
    scale = 1 / math.sqrt(128)
    o, lse, (m, l, acc) = rf.attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, S,
                                         out_dtype=torch.float32)
    m_ref, l_ref, acc_ref = oracle.decode_partials(q, k, v, scale, S)
    m, l, acc = np32(m), np32(l), np32(acc)
    empty = np.isinf(m_ref)
    assert np.array_equal(np.isinf(m), empty)
    assert np.all(l[empty] == 0) and np.all(acc[empty] == 0)
    fin = ~empty
    assert np.abs(m[fin] - m_ref[fin]).max() <= 1e-5 * max(1, np.abs(m_ref[fin]).max())
    assert normwise(l[fin], l_ref[fin]) <= 1e-5
    assert normwise(acc[fin], acc_ref[fin]) <= 1e-4
    o_ref, lse_ref = oracle.attention(q[:, :, None], k, v, scale)
    assert normwise(np32(o), o_ref[:, :, 0]) <= 1e-4
    assert np.abs(np32(lse) - lse_ref[:, :, 0]).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


@pytest.fixture(scope="module")
def decode_config():
    """The decode workload: B=8, Hq=32, Hkv=8 (GQA 4:1), Lk=32768, d=128, bf16."""
    q, k, v = inputs.decode_inputs(2, 8, 32, 8, 32768, 128)
    return q, k, v, q.to(DEV), k.to(DEV), v.to(DEV)


@pytest.mark.parametrize("S", [1, 4, 8, 16, 64])
def test_decode_config_sampled(decode_config, S):
    q, k, v, qd, kd, vd = decode_config
    print_case(test="decode_full", S=S)
    scale = 1 / math.sqrt(128)
    o, lse, (m, l, acc) = rf.attn_decode(qd, kd, vd, scale, S)
    o, lse, m, l, acc = np32(o), np32(lse), np32(m), np32(l), np32(acc)
    assert np.isfinite(o).all()
    for b, h in [(0, 0), (3, 13), (7, 31)]:
        hk = h // 4
        qs, ks, vs = q[b:b + 1, h:h + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1]
        m_ref, l_ref, acc_ref = oracle.decode_partials(qs, ks, vs, scale, S)
        assert np.abs(m[b, h] - m_ref[0, 0]).max() <= 1e-5 * np.abs(m_ref).max()
        assert normwise(l[b, h], l_ref[0, 0]) <= 1e-5
        assert normwise(acc[b, h], acc_ref[0, 0]) <= 1e-4
        o_ref, lse_ref = oracle.attention(qs[:, :, None], ks, vs, scale)
        assert_bf16_attention(o[b, h], o_ref[0, 0, 0], lse[b, h], lse_ref[0, 0, 0], what=f"b={b} h={h}")


def test_cross_segment_consistency(decode_config):
    """Different segment counts merge to the same answer (fp32 output)."""
    q, k, v, qd, kd, vd = decode_config
    outs = [np32(rf.attn_decode(qd[:2], kd[:2], vd[:2], 0.1, S, out_dtype=torch.float32)[0])
            for S in (1, 4, 16, 64)]
    for o in outs[1:]:
        assert normwise(o, outs[0]) <= 1e-4


# ---------------------------------------------------------------- merge alone


def test_merge_random_states_with_identities():
    rng = np.random.default_rng(8)
    rows, S, d = 37, 9, 128
    m = (rng.standard_normal((rows, S)) * 4).astype(np.float32)
    l = rng.uniform(0.5, 50, (rows, S)).astype(np.float32)
    acc = rng.standard_normal((rows, S, d)).astype(np.float32)
    m[rng.random((rows, S)) < 0.3] = -np.inf
    m[5] = -np.inf                          # a row with nothing in it
    l[np.isinf(m)] = 0
    acc[np.isinf(m)] = 0
    args = [torch.from_numpy(x).to(DEV) for x in (m, l, acc)]
    o, lse = rf.merge_states(*args, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.merge_states(m, l, acc)
    o, lse = np32(o), np32(lse)
    assert np.all(o[5] == 0) and lse[5] == -np.inf
    keep = np.arange(rows) != 5
    assert normwise(o[keep], o_ref[keep]) <= FP32_REL
    assert normwise(lse[keep], lse_ref[keep]) <= FP32_REL
    ob, _ = rf.merge_states(*args, out_dtype=torch.bfloat16)
    assert np.abs(np32(ob)[keep] - o_ref[keep]).max() <= 2 ** -8 * np.abs(o_ref).max()
