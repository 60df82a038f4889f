"""The Python binding on the host (no GPU): every C-named wrapper checks each
buffer's shape and dtype against the sizes it passes to the C ABI, and raises
ValueError naming the entry point and the buffer before any launch. Host
tensors of the right shape pass those checks and are then refused as host
memory, so no call reaches the library's kernels."""

import pytest
import torch

from online_softmax_attention_cascaded_amd import binding as bd

F32, BF16, U8, I32 = torch.float32, torch.bfloat16, torch.uint8, torch.int32


def z(*shape, dtype=F32):
    return torch.zeros(*shape, dtype=dtype)


def refused(fn, match, *args):
    with pytest.raises(ValueError, match=match):
        fn(*args)


HOST = "device tensors"


# ------------------------------------------------------------------ attention


def attn_args(dt=BF16, B=1, Hq=4, Hkv=2, Lq=8, Lk=16, d=64, lse=True):
    return [z(B, Hq, Lq, d, dtype=dt), z(B, Hkv, Lk, d, dtype=dt), z(B, Hkv, Lk, d, dtype=dt),
            z(B, Hq, Lq, d, dtype=dt), z(B, Hq, Lq) if lse else None, 0.1, False]


def test_attn_fwd_checks():
    f = bd.rf_attn_fwd
    refused(f, HOST, *attn_args())
    refused(f, HOST, *attn_args(dt=F32, lse=False))
    a = attn_args(); a[0] = z(1, 4, 8, 64)                  # q fp32, k bf16
    refused(f, r"rf_attn_fwd: k has dtype", *a)
    a = attn_args(); a[1] = z(1, 2, 15, 64, dtype=BF16)     # v longer than k
    refused(f, r"rf_attn_fwd: v has shape", *a)
    a = attn_args(); a[3] = z(1, 4, 8, 32, dtype=BF16)
    refused(f, r"rf_attn_fwd: o has shape", *a)
    a = attn_args(); a[4] = z(1, 4, 9)
    refused(f, r"rf_attn_fwd: lse has shape", *a)
    a = attn_args(); a[4] = z(1, 4, 8, dtype=BF16)
    refused(f, r"rf_attn_fwd: lse has dtype", *a)
    a = attn_args(); a[0] = z(4, 8, 64, dtype=BF16)
    refused(f, r"rf_attn_fwd: q must have 4 dimensions", *a)
    a = attn_args(dt=torch.float16)
    refused(f, r"rf_attn_fwd: q has dtype", *a)


def decode_args(dt=BF16, B=2, Hq=8, Hkv=2, Lk=40, d=64, S=4):
    return [z(B, Hq, d, dtype=dt), z(B, Hkv, Lk, d, dtype=dt), z(B, Hkv, Lk, d, dtype=dt),
            z(B, Hq, S), z(B, Hq, S), z(B, Hq, S, d), 0.1]


def test_attn_decode_split_checks():
    f = bd.rf_attn_decode_split
    refused(f, HOST, *decode_args())
    refused(f, HOST, *decode_args(dt=F32, d=128))
    a = decode_args(); a[0] = z(2, 8, 128, dtype=BF16)
    refused(f, r"rf_attn_decode_split: q has shape", *a)
    a = decode_args(); a[2] = z(2, 2, 40, 64)
    refused(f, r"rf_attn_decode_split: v has dtype", *a)
    a = decode_args(); a[4] = z(2, 8, 5)
    refused(f, r"rf_attn_decode_split: part_l has shape", *a)
    a = decode_args(); a[5] = z(2, 8, 4, 64, dtype=BF16)
    refused(f, r"rf_attn_decode_split: part_acc has dtype", *a)
    a = decode_args(); a[3] = z(2, 8)
    refused(f, r"rf_attn_decode_split: part_m must have 3 dimensions", *a)


def mla_args(B=2, H=16, Lk=30, S=3):
    return [z(B, H, 576, dtype=BF16), z(B, Lk, 576, dtype=BF16), z(B, H, S), z(B, H, S),
            z(B, H, S, 512)]


def test_mla_checks():
    f = bd.rf_mla_decode_split
    refused(f, HOST, *mla_args(), 0.1)
    a = mla_args(); a[1] = z(2, 30, 576)
    refused(f, r"rf_mla_decode_split: kv has dtype", *a, 0.1)
    a = mla_args(); a[2] = z(2, 16, 4)
    refused(f, r"rf_mla_decode_split: part_m has shape", *a, 0.1)
    g = bd.rf_mla_decode
    refused(g, HOST, *mla_args(), z(2, dtype=I32), z(2, 16, 512, dtype=BF16), z(2, 16), 0.1)
    refused(g, r"rf_mla_decode: counters has shape", *mla_args(), z(3, dtype=I32),
            z(2, 16, 512, dtype=BF16), None, 0.1)
    refused(g, r"rf_mla_decode: counters has dtype", *mla_args(), z(2),
            z(2, 16, 512, dtype=BF16), None, 0.1)
    refused(g, r"rf_mla_decode: o has shape", *mla_args(), z(2, dtype=I32),
            z(2, 16, 576, dtype=BF16), None, 0.1)
    refused(g, r"rf_mla_decode: lse has shape", *mla_args(), z(2, dtype=I32),
            z(2, 16, 512), z(2, 17), 0.1)


def test_merge_states_checks():
    f = bd.rf_merge_states
    refused(f, HOST, z(3, 5, 4), z(3, 5, 4), z(3, 5, 4, 128), z(3, 5, 128, dtype=BF16), z(3, 5))
    refused(f, r"rf_merge_states: part_m has shape", z(3, 5, 3), z(3, 5, 4), z(3, 5, 4, 128),
            z(3, 5, 128), None)
    refused(f, r"rf_merge_states: o has shape", z(3, 5, 4), z(3, 5, 4), z(3, 5, 4, 128),
            z(3, 5, 64), None)
    refused(f, r"rf_merge_states: part_acc has dtype", z(3, 5, 4), z(3, 5, 4),
            z(3, 5, 4, 128, dtype=BF16), z(3, 5, 128), None)
    refused(f, r"rf_merge_states: lse has shape", z(3, 5, 4), z(3, 5, 4), z(3, 5, 4, 128),
            z(3, 5, 128), z(15))


# ------------------------------------------------------------ row reductions


def test_softmax_topk_checks():
    f = bd.rf_softmax_topk
    refused(f, HOST, z(10, 256), 8, True, z(10, 8), z(10, 8, dtype=I32))
    refused(f, r"rf_softmax_topk: logits has dtype", z(10, 256, dtype=BF16), 8, True, z(10, 8),
            z(10, 8, dtype=I32))
    refused(f, r"rf_softmax_topk: weights has shape", z(10, 256), 8, True, z(10, 4),
            z(10, 8, dtype=I32))
    refused(f, r"rf_softmax_topk: indices has dtype", z(10, 256), 8, True, z(10, 8),
            z(10, 8, dtype=torch.int64))
    refused(f, r"rf_softmax_topk: logits must have 2 dimensions", z(256), 8, True, z(1, 8),
            z(1, 8, dtype=I32))


def test_softmax_checks():
    f = bd.rf_softmax
    refused(f, HOST, z(10, 1024), 3, None, z(10, 1024))
    refused(f, HOST, z(10, 1024), 0, z(20), z(10, 1024))
    refused(f, r"rf_softmax: y has shape", z(10, 1024), 3, None, z(10, 1020))
    refused(f, r"rf_softmax: work has shape", z(10, 1024), 0, z(10), z(10, 1024))
    refused(f, r"rf_softmax: x has dtype", z(10, 1024, dtype=BF16), 3, None, z(10, 1024))


def test_moment_checks():
    refused(bd.rf_row_variance, HOST, z(10, 1024), 2, z(10), z(10))
    refused(bd.rf_row_variance, r"rf_row_variance: var has shape", z(10, 1024), 2, z(10), z(11))
    refused(bd.rf_row_variance, r"rf_row_variance: mean has dtype", z(10, 1024), 2,
            z(10, dtype=BF16), z(10))
    refused(bd.rf_row_inertia, HOST, z(10, 1024), z(10, 1024), 2, z(10), z(10))
    refused(bd.rf_row_inertia, r"rf_row_inertia: w has shape", z(10, 1024), z(10, 512), 2, z(10),
            z(10))
    refused(bd.rf_row_inertia, r"rf_row_inertia: inertia has shape", z(10, 1024), z(10, 1024), 2,
            z(10), z(9))


# ----------------------------------------------------------------------- FP8


def test_quant_checks():
    f = bd.rf_absmax_quant_fp8
    refused(f, HOST, z(4, 256, dtype=BF16), z(4, 256, dtype=U8), z(4))
    refused(f, r"rf_absmax_quant_fp8: x has dtype", z(4, 256), z(4, 256, dtype=U8), z(4))
    refused(f, r"rf_absmax_quant_fp8: q has dtype", z(4, 256, dtype=BF16), z(4, 256), z(4))
    refused(f, r"rf_absmax_quant_fp8: scale has shape", z(4, 256, dtype=BF16),
            z(4, 256, dtype=U8), z(8))


def gemm_args(M=32, N=48, K=256):
    return [z(M, K, dtype=BF16), z(N, K, dtype=U8), z(N), z(M), z(M, N, dtype=BF16)]


def test_gemm_checks():
    f = bd.rf_absmax_quant_gemm_fp8
    a, bq, bs, as_, c = gemm_args()
    refused(f, HOST, a, bq, bs, z(32, 256, dtype=U8), as_, c)
    refused(f, r"rf_absmax_quant_gemm_fp8: a_q has shape", a, bq, bs, z(32, 128, dtype=U8), as_, c)
    refused(f, r"rf_absmax_quant_gemm_fp8: b_q has shape", a, z(48, 128, dtype=U8), bs,
            z(32, 256, dtype=U8), as_, c)
    refused(f, r"rf_absmax_quant_gemm_fp8: c has shape", a, bq, bs, z(32, 256, dtype=U8), as_,
            z(48, 32, dtype=BF16))
    refused(f, r"rf_absmax_quant_gemm_fp8: b_scale has shape", a, bq, z(32),
            z(32, 256, dtype=U8), as_, c)
    g = bd.rf_absmax_quant_gemm_fp8_running
    refused(g, HOST, a, bq, bs, as_, c)
    refused(g, r"rf_absmax_quant_gemm_fp8_running: a_scale has shape", a, bq, bs, z(48), c)
    refused(g, r"rf_absmax_quant_gemm_fp8_running: c has dtype", a, bq, bs, as_, z(32, 48))


def test_gemm_noalloc_checks():
    f = bd.rf_absmax_quant_gemm_fp8_noalloc
    a, bq, bs, as_, c = gemm_args()
    refused(f, HOST, a, bq, bs, as_, c)
    refused(f, r"rf_absmax_quant_gemm_fp8_noalloc: a_scale has shape", a, bq, bs, z(48), c)
    refused(f, r"rf_absmax_quant_gemm_fp8_noalloc: b_q has dtype", a, z(48, 256), bs, as_, c)
