"""GPU parity of rf_attn_fwd (through the C ABI) against the fp64 oracle."""

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


# ---------------------------------------------------------------- fp32 (the tiny configuration)


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_tiny_config(causal):
    """B=1, H=1, Lq=64, Lk=256, d=64, fp32, scale 1/8 (causal needs Lq == Lk, so the
    causal variant uses Lq = Lk = 256)."""
    Lq = 256 if causal else 64
    print_case(test="fp32_tiny", causal=causal)
    q, k, v = inputs.attention_inputs(0, 1, 1, 1, Lq, 256, 64, dtype=torch.float32)
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 1 / 8, causal=causal)
    o_ref, lse_ref = oracle.attention(q, k, v, 1 / 8, causal=causal)
    assert normwise(np32(o), o_ref) <= FP32_REL
    assert normwise(np32(lse), lse_ref) <= FP32_REL


@pytest.mark.parametrize("shape", [(2, 4, 2, 50, 77, 128), (1, 3, 3, 1, 1, 64), (1, 2, 1, 33, 300, 64)])
def test_fp32_ragged_gqa(shape):
    B, Hq, Hkv, Lq, Lk, d = shape
    print_case(test="fp32_ragged", shape=shape)
    q, k, v = inputs.attention_inputs(1, B, Hq, Hkv, Lq, Lk, d, dtype=torch.float32)
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 0.3)
    o_ref, lse_ref = oracle.attention(q, k, v, 0.3)
    assert normwise(np32(o), o_ref) <= FP32_REL
    assert normwise(np32(lse), lse_ref) <= FP32_REL


# ---------------------------------------------------------------- bf16 MFMA path


@pytest.mark.parametrize(
    "shape,causal",
    [
        ((1, 2, 2, 128, 128, 128), False),     # one query block, two key tiles
        ((1, 2, 2, 300, 300, 128), False),     # several blocks and a ragged tail
        ((1, 2, 2, 300, 300, 128), True),
        ((2, 4, 2, 257, 257, 128), True),      # GQA 2:1, tail of one row
        ((1, 2, 2, 512, 512, 128), True),      # four query blocks: pairs (3, 0) and (2, 1)
        ((1, 1, 1, 640, 640, 128), True),      # five blocks: pairs and a lone middle block
        ((1, 4, 1, 130, 200, 128), False),     # Lq != Lk, GQA 4:1
        ((1, 1, 1, 5, 3, 128), False),         # fewer keys than a tile
        ((1, 1, 1, 1, 1, 128), True),
    ],
)
def test_bf16_small(shape, causal):
    B, Hq, Hkv, Lq, Lk, d = shape
    print_case(test="bf16_small", shape=shape, causal=causal)
    q, k, v = inputs.attention_inputs(2, B, Hq, Hkv, Lq, Lk, d)
    scale = 1 / math.sqrt(d)
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal=causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
    assert_bf16_attention(np32(o), o_ref, np32(lse), lse_ref, what=f"{shape} causal={causal}")


@pytest.mark.parametrize(
    "shape,causal",
    [
        ((1, 2, 2, 128, 128, 64), False),
        ((1, 2, 2, 300, 300, 64), False),      # ragged tail
        ((1, 2, 2, 300, 300, 64), True),
        ((2, 4, 2, 257, 257, 64), True),       # GQA 2:1, tail of one row
        ((1, 1, 1, 640, 640, 64), True),       # five blocks: pairs and a lone middle block
        ((1, 4, 1, 130, 200, 64), False),      # Lq != Lk, GQA 4:1
        ((1, 1, 1, 5, 3, 64), False),          # fewer keys than a tile
        ((1, 1, 1, 1, 1, 64), True),
        ((2, 8, 8, 1024, 1024, 64), True),
    ],
)
def test_bf16_head64(shape, causal):
    """Head size 64 on the MFMA path (K rows of 128 bytes: two rows per
    1024-byte load group, the other LDS swizzle)."""
    B, Hq, Hkv, Lq, Lk, d = shape
    print_case(test="bf16_head64", shape=shape, causal=causal)
    q, k, v = inputs.attention_inputs(21, B, Hq, Hkv, Lq, Lk, d)
    scale = 1 / math.sqrt(d)
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal=causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
    assert_bf16_attention(np32(o), o_ref, np32(lse), lse_ref, what=f"{shape} causal={causal}")


def test_bf16_head64_large_scores():
    q, k, v = inputs.attention_inputs(22, 1, 2, 2, 384, 384, 64)
    q = (q.float() * 3).to(torch.bfloat16)
    print_case(test="bf16_head64_large_scores")
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 1.0, causal=True)
    o_ref, lse_ref = oracle.attention(q, k, v, 1.0, causal=True)
    assert np.abs(np32(o) - o_ref).max() <= 2e-2
    assert np.abs(np32(lse) - lse_ref).max() <= 1e-2 * max(1.0, np.abs(lse_ref).max() / 100)


def test_bf16_large_scores():
    """Scores far from 0 (scale 1, inputs x3): the running max changes often and
    exp(m_old - m_new) is far from 1."""
    q, k, v = inputs.attention_inputs(3, 1, 2, 2, 256, 256, 128)
    q = (q.float() * 3).to(torch.bfloat16)
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 1.0, causal=True)
    o_ref, lse_ref = oracle.attention(q, k, v, 1.0, causal=True)
    err = np.abs(np32(o) - o_ref).max()
    assert err <= 2e-2
    assert np.abs(np32(lse) - lse_ref).max() <= 1e-2 * max(1.0, np.abs(lse_ref).max() / 100)


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_reference_moves(causal):
    """Scores set tile by tile (scale ln 2, so scores are in exp2 units): tile 0
    at 0, tile 1 at 7 (every probability 2^7: each lane's sum passes 2^8 but no
    score passes the reference by more than 8, so nothing may move), tile 2 at
    20 and tile 3 at 27.5 (the reference must move and the tile be recomputed),
    then back down, with a ragged last tile. Rows scale the scores by 1 + r/64."""
    print_case(test="bf16_reference_moves", causal=causal)
    d, Lk = 128, 6 * 64 + 17
    Lq = Lk if causal else 70
    levels = [0.0, 7.0, 20.0, 27.5, 10.0, 26.0, 3.0]
    kk = np.zeros((1, 1, Lk, d), np.float32)
    for j in range(Lk):
        kk[0, 0, j, 0] = levels[j // 64]
    kk[0, 0, :, 1] = np.random.default_rng(5).standard_normal(Lk) * 0.25
    qq = np.zeros((1, 1, Lq, d), np.float32)
    qq[0, 0, :, 0] = 1.0 + np.arange(Lq) / 64.0
    qq[0, 0, :, 1] = 1.0
    vv = np.random.default_rng(6).standard_normal((1, 1, Lk, d)).astype(np.float32)
    q, k, v = inputs.as_bf16(qq), inputs.as_bf16(kk), inputs.as_bf16(vv)
    scale = math.log(2.0)
    o, lse = rf.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal=causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
    assert_bf16_attention(np32(o), o_ref, np32(lse), lse_ref, what=f"reference moves causal={causal}")


def test_bf16_deterministic():
    q, k, v = (t.to(DEV) for t in inputs.attention_inputs(4, 1, 4, 4, 512, 512, 128))
    o1, l1 = rf.attn_fwd(q, k, v, 0.1, causal=True)
    o2, l2 = rf.attn_fwd(q, k, v, 0.1, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
