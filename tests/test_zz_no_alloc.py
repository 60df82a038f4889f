"""rf_absmax_quant_gemm_fp8_noalloc (the FP8 cascade with library-owned
scratch) through the C ABI against rf_absmax_quant_gemm_fp8 with a caller
workspace: the same kernels, so C and the row scales must be bit-identical.
Two calls in a row share the scratch; the second is smaller, so it reads only
what it wrote itself."""

import pytest
import torch

import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import DEV, needs_gpu, print_case

pytestmark = [pytest.mark.gpu, needs_gpu]


def _noalloc(a, bq, bs):
    M, N = a.shape[0], bq.shape[0]
    sa = torch.full((M,), float("nan"), device=DEV)
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    rf.rf_absmax_quant_gemm_fp8_noalloc(a, bq, bs, sa, c)
    return c, sa


def test_noalloc_matches_workspace_entry_point():
    cases = [(4096, 1024, 7168, 50), (300, 520, 1024, 51)]    # the second call is smaller
    for M, N, K, seed in cases:
        print_case(test="noalloc", M=M, N=N, K=K)
        a, bsrc = inputs.quant_inputs(seed, M, N, K)
        a = a.to(DEV)
        bq, bs = rf.absmax_quant_fp8(bsrc.to(DEV))
        c_ref, _, sa_ref = rf.absmax_quant_gemm_fp8(a, bq, bs)
        c, sa = _noalloc(a, bq, bs)
        torch.cuda.synchronize()
        assert torch.equal(sa, sa_ref)
        assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))


def test_noalloc_rejects_oversize():
    a = torch.zeros((4097, 8192), dtype=torch.bfloat16, device=DEV)
    bq = torch.zeros((64, 8192), dtype=torch.uint8, device=DEV)
    bs = torch.ones(64, device=DEV)
    with pytest.raises(rf.RFError, match="scratch"):
        _noalloc(a, bq, bs)
