"""Shared helpers of the GPU parity tests (comparisons and the device handle)."""

import math

import numpy as np
import pytest
import torch

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
DEV = "cuda:0"

# Tolerances (written out here so every test states the bar it checks):
FP32_REL = 1e-5          # fp32 paths: max |diff| / max |ref| (normwise)
BF16_ABS = 2e-2          # bf16 attention outputs: max absolute error
BF16_REL_FRO = 1e-2      # bf16 diagnostic: relative Frobenius error
LSE_ABS = 1e-3           # log-sum-exp of bf16 paths: max absolute error
FP8_REL_FRO = 3e-2       # FP8 GEMM: relative Frobenius error vs the fp64 oracle


def np32(t):
    return t.detach().float().cpu().numpy()


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    return np.abs(got - ref).max() / (scale if scale > 0 else 1.0)


def rel_fro(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)


def assert_bf16_attention(o, o_ref, lse=None, lse_ref=None, what=""):
    err = np.abs(np.asarray(o, np.float64) - o_ref).max()
    assert err <= BF16_ABS, f"{what}: max abs error {err}"
    fro = rel_fro(o, o_ref)
    assert fro <= BF16_REL_FRO, f"{what}: relative Frobenius error {fro}"
    if lse is not None:
        lerr = np.abs(np.asarray(lse, np.float64) - lse_ref).max()
        assert lerr <= LSE_ABS, f"{what}: lse max abs error {lerr}"


def assert_fp8_entries(c, c_ref, mag, units, what=""):
    """Every entry of an FP8 GEMM result against the fp64 oracle:
    |c - c_ref| <= 2^-8 |c_ref| + units * 2^-23 * mag, where mag is
    s_i t_j sum_k |a_ik b_jk| (the sum the fp32 accumulation rounds along) and
    units counts the fp32 roundings (K additions, the scale products and, for
    the running scale, the accumulator rescales); 2^-8 is the bf16 output
    rounding."""
    c = np.asarray(c, np.float64)
    tol = 2.0 ** -8 * np.abs(c_ref) + units * 2.0 ** -23 * mag
    bad = np.argwhere(np.abs(c - c_ref) > tol)
    assert len(bad) == 0, f"{what}: {len(bad)} entries outside the bound, first {bad[:3].tolist()}"


def print_case(**kw):
    print("case " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def sqrt_scale(d):
    return 1.0 / math.sqrt(d)
