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


def _check_partials(m, l, acc, m_ref, l_ref, acc_ref, acc_bar):
    m, l, acc = np32(m), np32(l), np32(acc)
    empty = np.isinf(m_ref)
    assert np.array_equal(np.isinf(m), empty)
    assert np.all(l[empty] == 0) and np.all(acc[empty] == 0)
    fin = ~empty
    assert np.abs(m[fin] - m_ref[fin]).max() <= 1e-5 * max(1, np.abs(m_ref[fin]).max())
    assert normwise(l[fin], l_ref[fin]) <= 1e-5
    assert normwise(acc[fin], acc_ref[fin]) <= acc_bar


@pytest.mark.parametrize(
    "B,Hq,Hkv,Lk,S",
    [
        (1, 4, 1, 3000, 1),
        (2, 8, 2, 3000, 4),
        (2, 8, 2, 777, 64),       # segments of 13 keys, ragged
        (1, 4, 1, 5, 4),          # an empty segment
        (1, 16, 1, 513, 3),       # G = 16
        (2, 6, 2, 96, 2),         # G = 3
    ],
)
def test_head64_partials_and_merge(B, Hq, Hkv, Lk, S):
    """Head size 64 on the bf16 MFMA path."""
    print_case(test="decode_head64", B=B, Hq=Hq, Hkv=Hkv, Lk=Lk, S=S)
    d = 64
    q, k, v = inputs.decode_inputs(15, B, Hq, Hkv, Lk, d)
    scale = 1 / math.sqrt(d)
    o, lse, (m, l, acc) = rf.attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, S,
                                         out_dtype=torch.float32)
    _check_partials(m, l, acc, *oracle.decode_partials(q, k, v, scale, S), acc_bar=1e-4)
    o_ref, lse_ref = oracle.attention(q[:, :, None], k, v, scale)
    assert normwise(np32(o), o_ref[:, :, 0]) <= 1e-4
    assert np.abs(np32(lse) - lse_ref[:, :, 0]).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


@pytest.mark.parametrize(
    "B,Hq,Hkv,Lk,d,S",
    [
        (1, 4, 1, 3000, 128, 1),
        (2, 8, 2, 777, 128, 4),   # ragged last segment and chunk
        (1, 4, 1, 5, 128, 4),     # an empty segment
        (1, 4, 4, 100, 64, 64),   # many trailing empty segments, G = 1
        (1, 16, 1, 513, 64, 3),   # G = 16
        (2, 6, 2, 96, 64, 2),     # G = 3
        (2, 8, 2, 4096, 64, 16),
    ],
)
def test_fp32_partials_and_merge(B, Hq, Hkv, Lk, d, S):
    """fp32 K/V: every step in fp32, bar 1e-5 normwise for the states and the
    merged output."""
    print_case(test="decode_fp32", B=B, Hq=Hq, Hkv=Hkv, Lk=Lk, d=d, S=S)
    q, k, v = inputs.decode_inputs(16, B, Hq, Hkv, Lk, d, dtype=torch.float32)
    scale = 1 / math.sqrt(d)
    o, lse, (m, l, acc) = rf.attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, S,
                                         out_dtype=torch.float32)
    _check_partials(m, l, acc, *oracle.decode_partials(q, k, v, scale, S), acc_bar=FP32_REL)
    o_ref, lse_ref = oracle.attention(q[:, :, None], k, v, scale)
    assert normwise(np32(o), o_ref[:, :, 0]) <= FP32_REL
    assert np.abs(np32(lse) - lse_ref[:, :, 0]).max() <= 1e-5 * max(1, np.abs(lse_ref).max())


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
