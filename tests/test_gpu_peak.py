"""The MFMA measurement loop (rf_peak_mfma, not a step of the path) computes
what it claims: per wave, the sum of every accumulator element equals
iters * sum_j sum_k colsum(A_j)[k] * rowsum(B_j)[k], with A_j = operand j and
B_j = operand (j + 3) % 8 of each lane, k split over the two half-waves as the
MFMA operand layout places it. Checked in fp64 from the same bytes; the clock
record is positive and plausible."""

import numpy as np
import pytest
import torch

import online_softmax_attention_cascaded_amd as rf
from gpu_util import DEV, needs_gpu, print_case

pytestmark = [pytest.mark.gpu, needs_gpu]


def _operands(src, kind):
    """src uint8 [blocks*256, 256] -> fp64 operands [blocks, 4 waves, 64 lanes, 8, n]."""
    rows = src.shape[0]
    if kind == rf.RF_PEAK_BF16:
        raw = src.view(rows, 8, 32)[:, :, :16].contiguous().view(torch.bfloat16)   # [rows, 8, 8]
    else:
        raw = src.view(rows, 8, 32).contiguous().view(torch.float8_e4m3fn)        # [rows, 8, 32]
    v = raw.float().double().numpy()
    return v.reshape(rows // 256, 4, 64, 8, v.shape[-1])


def _expected(ops, iters):
    b, w, _, _, n = ops.shape
    halves = ops.reshape(b, w, 2, 32, 8, n).sum(axis=3)        # [b, w, half, j, n]: sums over a half-wave
    habs = np.abs(ops).reshape(b, w, 2, 32, 8, n).sum(axis=3)
    exp = np.zeros((b, w))
    mag = np.zeros((b, w))
    for j in range(8):
        jb = (j + 3) % 8
        exp += (halves[:, :, :, j, :] * halves[:, :, :, jb, :]).sum(axis=(2, 3))
        mag += (habs[:, :, :, j, :] * habs[:, :, :, jb, :]).sum(axis=(2, 3))
    return iters * exp, iters * mag


@pytest.mark.parametrize("kind", [0, 1])
def test_peak_checksum(kind):
    print_case(test="peak_mfma", kind=kind)
    blocks, iters = 3, 5
    g = torch.Generator().manual_seed(21 + kind)
    if kind == rf.RF_PEAK_BF16:
        vals = torch.randn((blocks * 256, 8, 8), generator=g).to(torch.bfloat16)
        src = torch.zeros((blocks * 256, 8, 32), dtype=torch.uint8)
        src[:, :, :16] = vals.view(torch.uint8).view(blocks * 256, 8, 16)
    else:
        vals = (torch.randn((blocks * 256, 8, 32), generator=g) * 8).to(torch.float8_e4m3fn)
        src = vals.view(torch.uint8)
    src = src.reshape(blocks * 256, 256).contiguous()
    out = torch.empty(blocks * 4, device=DEV)
    clock = torch.zeros((blocks, 2), dtype=torch.int64, device=DEV)
    rf.rf_peak_mfma(kind, src.to(DEV), iters, out, clock)
    torch.cuda.synchronize()
    exp, mag = _expected(_operands(src, kind), iters)
    got = out.cpu().double().numpy().reshape(blocks, 4)
    assert np.all(np.abs(got - exp) <= 1e-5 * mag + 1e-6), (got, exp)
    ck = clock.cpu().numpy()
    assert np.all(ck > 0)
    khz = rf.rf_wall_clock_khz()
    ghz = ck[:, 0] / ck[:, 1] * khz / 1e6
    assert khz > 0 and np.all((ghz > 0.3) & (ghz < 3.5)), (khz, ghz)


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096 * 16 + 48, 3), (3 << 20, 64), (40 << 20, 2048)])
def test_peak_read_xor(nbytes, blocks):
    """The read stream touches every 16-byte word exactly once: the XOR of the
    per-workgroup results equals the XOR of all 32-bit words of the buffer."""
    print_case(test="peak_read", nbytes=nbytes, blocks=blocks)
    g = torch.Generator().manual_seed(nbytes % 1000)
    x = torch.randint(-(2 ** 31), 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    out = torch.empty(blocks, dtype=torch.int32, device=DEV)
    rf.rf_peak_read(x.to(DEV), blocks, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    exp = np.bitwise_xor.reduce(x.numpy().view(np.uint32))
    assert got == exp
