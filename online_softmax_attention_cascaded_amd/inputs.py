"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and rounds them once to the storage dtype; it
holds none of the method's arithmetic. Both the oracle and the HIP path are fed
the very same arrays. Draws use numpy's PCG64 generator
(``numpy.random.default_rng(seed)``), ``standard_normal(dtype=float32)`` in C
order; rounding to bf16 uses torch's CPU cast (round to nearest even).

Workload shapes (synthetic stand-ins for the model workloads the pages
measure -- attention, MoE routing and FP8 quantise-then-GEMM -- whose shapes the
pages do not print):

* tiny fp32 attention: B=1, H=1, Lq=64, Lk=256, d=64;
* prefill: B=4, H=32, Lq=Lk=2048, d=128, bf16;
* decode: B=8, Hq=32, Hkv=8, Lk=32768, d=128, bf16 KV cache;
* multi-latent decode: B=32 sequences, 16 query heads (one tensor-parallel
  shard), Lk=8192 latent rows of 576 bf16 values (512 latent + 64 positional),
  values = the first 512 columns;
* routing: 16384 tokens x 256 experts fp32 logits, 1 % of rows with +6 on one
  random expert;
* safe softmax: rows of 1024 .. 8192 fp32 values, 2^26 values in all;
* variance / moment of inertia: rows of 1024 .. 8192 fp32 positions and
  masses, 2^26 values in all;
* FP8: A 4096 x 7168 bf16 with 0.1 % of entries scaled by 50, B source
  4096 x 7168 bf16 (quantised per row of B, i.e. per output column).
"""

import numpy as np
import torch


def normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def as_bf16(x):
    """float32 numpy array -> bf16 torch CPU tensor (one round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def attention_inputs(seed, B, Hq, Hkv, Lq, Lk, d, dtype=torch.bfloat16):
    """q [B,Hq,Lq,d], k, v [B,Hkv,Lk,d] ~ N(0,1), as torch CPU tensors of ``dtype``."""
    rng = np.random.default_rng(seed)
    q = normal(rng, (B, Hq, Lq, d))
    k = normal(rng, (B, Hkv, Lk, d))
    v = normal(rng, (B, Hkv, Lk, d))
    if dtype == torch.float32:
        return torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    return as_bf16(q), as_bf16(k), as_bf16(v)


def decode_inputs(seed, B, Hq, Hkv, Lk, d, dtype=torch.bfloat16):
    """q [B,Hq,d], k, v [B,Hkv,Lk,d] ~ N(0,1), torch CPU tensors of ``dtype``."""
    rng = np.random.default_rng(seed)
    q = normal(rng, (B, Hq, d))
    k = normal(rng, (B, Hkv, Lk, d))
    v = normal(rng, (B, Hkv, Lk, d))
    if dtype == torch.float32:
        return torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    return as_bf16(q), as_bf16(k), as_bf16(v)


def mla_inputs(seed, B, H, Lk, dqk=576):
    """q [B,H,dqk] and latent rows [B,Lk,dqk] ~ N(0,1), bf16 torch CPU tensors."""
    rng = np.random.default_rng(seed)
    q = as_bf16(normal(rng, (B, H, dqk)))
    kv = as_bf16(normal(rng, (B, Lk, dqk)))
    return q, kv


def worked_example_decode(d=128):
    """Three keys whose scores against the single query are 1, 3 and 5 (scale 1),
    with value rows whose first component is 2, -1 and 4; every other component
    is 0. With two segments of ceil(3/2) = 2 keys the tiles are {1, 3} and {5}.
    Returns bf16 torch CPU tensors q [1,1,d], k, v [1,1,3,d]."""
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, 3, d), np.float32)
    k[0, 0, :, 0] = [1.0, 3.0, 5.0]
    v = np.zeros((1, 1, 3, d), np.float32)
    v[0, 0, :, 0] = [2.0, -1.0, 4.0]
    return as_bf16(q), as_bf16(k), as_bf16(v)


def routing_inputs(seed, T, E, spike_frac=0.01, spike=6.0):
    """fp32 logits [T, E] ~ N(0,1); round(spike_frac*T) rows, drawn without
    replacement, get +spike on one uniformly drawn expert."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (T, E))
    n = int(round(spike_frac * T))
    rows = rng.choice(T, size=n, replace=False)
    cols = rng.integers(0, E, size=n)
    x[rows, cols] += np.float32(spike)
    return torch.from_numpy(x)


def softmax_inputs(seed, T, E, sigma=4.0, ramp=8.0):
    """fp32 rows [T, E] ~ sigma * N(0,1); row i with i % 4 == 1 also gets a
    ramp rising linearly from 0 to ``ramp`` along the row (its running max keeps
    growing, so every tile rescales the state), and i % 4 == 2 the same ramp
    falling (the max is met early)."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (T, E)) * np.float32(sigma)
    r = np.linspace(0.0, ramp, E, dtype=np.float32)
    x[1::4] += r
    x[2::4] += r[::-1]
    return torch.from_numpy(x)


def moment_inputs(seed, T, E, offsets=(0.0, 1000.0, -50.0, 3.0), scales=(1.0, 0.01, 10.0, 1.0)):
    """Positions x [T, E] fp32: row i is offsets[i % 4] + scales[i % 4] * N(0,1)
    (mean-to-spread ratios up to 1e5, where the one-pass sum of squares minus
    the squared sum loses every digit in fp32); masses w [T, E] fp32 uniform on
    [0, 1)."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (T, E))
    off = np.asarray(offsets, np.float32)[np.arange(T) % len(offsets)][:, None]
    sc = np.asarray(scales, np.float32)[np.arange(T) % len(scales)][:, None]
    x = (x * sc + off).astype(np.float32)
    w = rng.random((T, E), dtype=np.float32)
    return torch.from_numpy(x), torch.from_numpy(w)


def tie_heavy_logits(seed, T, E, values=(-1.0, 0.0, 1.0, 2.0)):
    """fp32 logits drawn uniformly from a few values, so ties are everywhere."""
    rng = np.random.default_rng(seed)
    v = np.asarray(values, np.float32)
    return torch.from_numpy(v[rng.integers(0, len(v), size=(T, E))])


def quant_inputs(seed, M, N, K, outlier_frac=1e-3, outlier_scale=50.0):
    """A [M,K] bf16 ~ N(0,1) with round(outlier_frac*M*K) entries, drawn without
    replacement, scaled by outlier_scale before rounding; B source [N,K] bf16 ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    a = normal(rng, (M, K))
    n = int(round(outlier_frac * M * K))
    if n:
        pos = rng.choice(M * K, size=n, replace=False)
        a.reshape(-1)[pos] *= np.float32(outlier_scale)
    b = normal(rng, (N, K))
    return as_bf16(a), as_bf16(b)
