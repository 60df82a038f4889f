"""Cascaded reductions fused into one incremental loop, native on MI355X (gfx950).

The compute lives in ``librf.so`` (hand-written HIP kernels behind a C ABI,
``include/rf.h``); ``binding`` is the ctypes layer over it and ``inputs`` the
seeded synthetic input generator. Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""

from .binding import (  # noqa: F401
    RF_FUSE_BLOCK,
    RF_FUSE_NONE,
    RF_FUSE_THREAD,
    RF_FUSE_WAVE,
    RF_PEAK_BF16,
    RF_PEAK_FP8,
    RFError,
    attn_decode,
    attn_decode_partials,
    attn_fwd,
    absmax_quant_fp8,
    absmax_quant_gemm_fp8,
    absmax_quant_gemm_fp8_running,
    lib,
    merge_states,
    mla_decode,
    row_inertia,
    row_variance,
    rf_absmax_quant_fp8,
    rf_absmax_quant_gemm_fp8,
    rf_absmax_quant_gemm_fp8_noalloc,
    rf_absmax_quant_gemm_fp8_running,
    rf_attn_decode_split,
    rf_attn_fwd,
    rf_merge_states,
    rf_mla_decode,
    rf_mla_decode_split,
    rf_peak_mfma,
    rf_peak_read,
    rf_row_inertia,
    rf_row_variance,
    rf_softmax,
    rf_softmax_topk,
    rf_wall_clock_khz,
    softmax,
    softmax_topk,
)
