"""The largest inputs the entry points accept: one key/value head (or one
sequence's latent cache) just under the 2 GiB limit, where the byte offsets the
kernels compute in 32 bits come within 16 KB of 2^31. Every output is compared
with the oracle (few query rows, so the oracle stays cheap)."""

import math

import numpy as np
import pytest
import torch

import oracle
import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import DEV, BF16_ABS, LSE_ABS, needs_gpu, np32, print_case, rel_fro

pytestmark = [pytest.mark.gpu, needs_gpu]

D = 128
LK_MAX = (1 << 31) // (D * 2) - 64      # 8388544 keys: 2^31 - 16 KB of K per head


@pytest.fixture(scope="module")
def big_kv():
    """q [1, 4, 16, d] (prefill rows) and qd [1, 4, d] (decode rows) as bf16, k, v
    [1, 1, LK_MAX, d] as their exact float64 values for the oracle, and the
    device copies (bf16) of all four."""
    q, k, v = inputs.attention_inputs(61, 1, 4, 1, 16, LK_MAX, D)
    qd = q[:, :, 0].contiguous()
    dev = (q.to(DEV), qd.to(DEV), k.to(DEV), v.to(DEV))
    k64, v64 = k.to(torch.float64).numpy(), v.to(torch.float64).numpy()   # exact, once
    return dict(q=q, qd=qd, k=k64, v=v64, dev=dev)


def test_decode_at_the_size_limit(big_kv):
    print_case(test="decode_limit", Lk=LK_MAX, S=64)
    _, qd_d, k_d, v_d = big_kv["dev"]
    scale = 1 / math.sqrt(D)
    S = 64
    o, lse, (m, l, acc) = rf.attn_decode(qd_d, k_d, v_d, scale, S, out_dtype=torch.float32)
    m_ref, l_ref, acc_ref = oracle.decode_partials(big_kv["qd"], big_kv["k"], big_kv["v"], scale, S)
    m, l, acc = np32(m), np32(l), np32(acc)
    assert np.abs(m - m_ref).max() <= 1e-5 * np.abs(m_ref).max()
    assert (np.abs(l - l_ref) / l_ref).max() <= 1e-5
    rows = np.abs(acc - acc_ref).max(-1) / np.abs(acc_ref).max(-1)
    assert rows.max() <= 1e-4
    o_ref, lse_ref = oracle.merge_states(m_ref, l_ref, acc_ref)
    assert (np.abs(np32(o) - o_ref).max(-1) / np.abs(o_ref).max(-1)).max() <= 1e-4
    assert np.abs(np32(lse) - lse_ref).max() <= 1e-5 * np.abs(lse_ref).max()


def test_prefill_at_the_size_limit(big_kv):
    """16 query rows against 8.4 M keys (the last key tile starts 16 KB below
    2^31 bytes into the head)."""
    print_case(test="prefill_limit", Lk=LK_MAX)
    q_d, _, k_d, v_d = big_kv["dev"]
    scale = 1 / math.sqrt(D)
    o, lse = rf.attn_fwd(q_d, k_d, v_d, scale)
    o, lse = np32(o), np32(lse)
    for h in range(4):
        o_ref, lse_ref = oracle.attention(big_kv["q"][:, h:h + 1], big_kv["k"], big_kv["v"], scale)
        assert np.abs(o[0, h] - o_ref[0, 0]).max() <= BF16_ABS
        assert rel_fro(o[0, h], o_ref[0, 0]) <= 2e-2
        assert np.abs(lse[0, h] - lse_ref[0, 0]).max() <= LSE_ABS


def test_mla_at_the_size_limit():
    """One sequence whose latent cache (plus the 96 rows of step overhang the
    kernel may address) comes within 1.2 KB of 2 GiB."""
    Lk = (1 << 31) // (576 * 2) - 96 - 1
    print_case(test="mla_limit", Lk=Lk)
    q, kv = inputs.mla_inputs(62, 1, 16, Lk)
    scale = 1 / math.sqrt(576)
    S = 64
    for fused in (False, True):
        o, lse, _ = rf.mla_decode(q.to(DEV), kv.to(DEV), scale, S, out_dtype=torch.float32, fused=fused)
        lat = kv[:, None]
        o_ref, lse_ref = oracle.attention(q[:, :, None], lat, lat[..., :512], scale)
        o_ref, lse_ref = o_ref[:, :, 0], lse_ref[:, :, 0]
        assert (np.abs(np32(o) - o_ref).max(-1) / np.abs(o_ref).max(-1)).max() <= 1e-4
        assert np.abs(np32(lse) - lse_ref).max() <= 1e-5 * np.abs(lse_ref).max()
