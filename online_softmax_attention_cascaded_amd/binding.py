"""ctypes binding of ``librf.so``: argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI declared in
``include/rf.h``; this module only checks tensor shapes/dtypes/devices, takes
raw device pointers and the current torch stream, and raises on a non-OK
status. The ``rf_*`` functions have the C names and take caller-allocated
output tensors; the short-named helpers allocate outputs with torch first.

There is no fallback: if ``librf.so`` is missing, every call raises.
"""

import ctypes
import os

import torch

from .build import LIB_PATH, source_digest

RF_OK, RF_ERR_INVALID_ARG, RF_ERR_UNSUPPORTED, RF_ERR_LAUNCH = 0, 1, 2, 3
RF_F32, RF_BF16 = 0, 1
RF_FUSE_NONE, RF_FUSE_THREAD, RF_FUSE_WAVE, RF_FUSE_BLOCK = 0, 1, 2, 3
RF_PEAK_BF16, RF_PEAK_FP8 = 0, 1

# Every entry point of the C ABI with its argument types.
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
SIGNATURES = {
    "rf_attn_fwd": [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P],
    "rf_attn_decode_split": [_I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P],
    "rf_merge_states": [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P],
    "rf_mla_decode_split": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P],
    "rf_mla_decode": [_P, _P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P],
    "rf_softmax_topk": [_P, _I, _I, _I, _I, _P, _P, _P],
    "rf_softmax": [_P, _I, _I, _I, _P, _P, _P],
    "rf_row_variance": [_P, _I, _I, _I, _P, _P, _P],
    "rf_row_inertia": [_P, _P, _I, _I, _I, _P, _P, _P],
    "rf_absmax_quant_fp8": [_P, _I, _I, _P, _P, _P],
    "rf_absmax_quant_gemm_fp8": [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P],
    "rf_absmax_quant_gemm_fp8_running": [_P, _P, _P, _I, _I, _I, _P, _P, _P],
    "rf_absmax_quant_gemm_fp8_noalloc": [_P, _P, _P, _I, _I, _I, _P, _P, _P],
    "rf_peak_mfma": [_I, _P, _I, _I, _P, _P, _P],
    "rf_peak_read": [_P, ctypes.c_longlong, _I, _P, _P],
    "rf_wall_clock_khz": [ctypes.POINTER(ctypes.c_int)],
    "rf_status_string": [_I],
    "rf_last_error": [],
    "rf_abi_version": [],
    "rf_build_id": [],
}
_RESTYPES = {"rf_status_string": ctypes.c_char_p, "rf_last_error": ctypes.c_char_p,
             "rf_build_id": ctypes.c_char_p}

_lib = None


class RFError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{_status_name(status)}: {detail}")


def _status_name(s):
    return {0: "RF_OK", 1: "RF_ERR_INVALID_ARG", 2: "RF_ERR_UNSUPPORTED", 3: "RF_ERR_LAUNCH"}.get(s, str(s))


def lib():
    """Load librf.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() or "
                "python -m online_softmax_attention_cascaded_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, ctypes.c_int)
        built, want = handle.rf_build_id().decode(), source_digest()
        if built != want:
            raise RuntimeError(
                f"{LIB_PATH} was built from other sources (build id {built}, sources {want}): "
                "rebuild it with __graft_entry__.build() or "
                "python -m online_softmax_attention_cascaded_amd.build")
        _lib = handle
    return _lib


def _check(status):
    if status != RF_OK:
        raise RFError(status, lib().rf_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("librf takes device tensors")
        if not t.is_contiguous():
            raise ValueError("librf takes contiguous tensors")


def _dtype_code(t):
    if t.dtype == torch.float32:
        return RF_F32
    if t.dtype == torch.bfloat16:
        return RF_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


_F32, _BF16, _U8, _I32 = torch.float32, torch.bfloat16, torch.uint8, torch.int32


def _expect(fn, name, t, shape, dtypes, optional=False):
    """The C ABI takes raw pointers and sizes: every buffer's shape and dtype
    must match the sizes passed beside it, or the kernels would read or write
    past it. Raises ValueError before anything is launched."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{fn}: {name} is required")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{fn}: {name} has dtype {t.dtype}, expected "
                         + " or ".join(str(d) for d in dtypes))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _ndim(fn, name, t, n):
    if t.dim() != n:
        raise ValueError(f"{fn}: {name} must have {n} dimensions, has shape {tuple(t.shape)}")


# ---------------------------------------------------------------- C-named calls


def rf_attn_fwd(q, k, v, o, lse, scale, causal):
    fn = "rf_attn_fwd"
    _ndim(fn, "q", q, 4)
    _ndim(fn, "k", k, 4)
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    _expect(fn, "q", q, (B, Hq, Lq, d), (_F32, _BF16))
    _expect(fn, "k", k, (B, Hkv, Lk, d), q.dtype)
    _expect(fn, "v", v, (B, Hkv, Lk, d), q.dtype)
    _expect(fn, "o", o, (B, Hq, Lq, d), q.dtype)
    _expect(fn, "lse", lse, (B, Hq, Lq), _F32, optional=True)
    _dev(q, k, v, o, lse)
    _check(lib().rf_attn_fwd(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             B, Hq, Hkv, Lq, Lk, d, float(scale), int(bool(causal)), _stream(q)))


def rf_attn_decode_split(q, k, v, part_m, part_l, part_acc, scale):
    fn = "rf_attn_decode_split"
    _ndim(fn, "k", k, 4)
    _ndim(fn, "part_m", part_m, 3)
    B, Hkv, Lk, d = k.shape
    Hq, S = part_m.shape[1], part_m.shape[2]
    _expect(fn, "k", k, (B, Hkv, Lk, d), (_F32, _BF16))
    _expect(fn, "q", q, (B, Hq, d), k.dtype)
    _expect(fn, "v", v, (B, Hkv, Lk, d), k.dtype)
    _expect(fn, "part_m", part_m, (B, Hq, S), _F32)
    _expect(fn, "part_l", part_l, (B, Hq, S), _F32)
    _expect(fn, "part_acc", part_acc, (B, Hq, S, d), _F32)
    _dev(q, k, v, part_m, part_l, part_acc)
    _check(lib().rf_attn_decode_split(_dtype_code(k), _ptr(q), _ptr(k), _ptr(v), _ptr(part_m),
                                      _ptr(part_l), _ptr(part_acc), B, Hq, Hkv, Lk, d, S,
                                      float(scale), _stream(k)))


def _mla_shapes(fn, q, kv, part_m, part_l, part_acc):
    _ndim(fn, "q", q, 3)
    _ndim(fn, "kv", kv, 3)
    _ndim(fn, "part_acc", part_acc, 4)
    B, H, Dqk = q.shape
    Lk = kv.shape[1]
    S, Dv = part_acc.shape[2], part_acc.shape[3]
    _expect(fn, "q", q, (B, H, Dqk), _BF16)
    _expect(fn, "kv", kv, (B, Lk, Dqk), _BF16)
    _expect(fn, "part_m", part_m, (B, H, S), _F32)
    _expect(fn, "part_l", part_l, (B, H, S), _F32)
    _expect(fn, "part_acc", part_acc, (B, H, S, Dv), _F32)
    return B, H, Dqk, Lk, S, Dv


def rf_mla_decode_split(q, kv, part_m, part_l, part_acc, scale):
    fn = "rf_mla_decode_split"
    B, H, Dqk, Lk, S, Dv = _mla_shapes(fn, q, kv, part_m, part_l, part_acc)
    _dev(q, kv, part_m, part_l, part_acc)
    _check(lib().rf_mla_decode_split(_ptr(q), _ptr(kv), _ptr(part_m), _ptr(part_l), _ptr(part_acc),
                                     B, H, Lk, Dqk, Dv, S, float(scale), _stream(q)))


def rf_mla_decode(q, kv, part_m, part_l, part_acc, counters, o, lse, scale):
    """Split and merge in one launch; counters int32 [B * H / 16], zero on entry
    and left zero."""
    fn = "rf_mla_decode"
    B, H, Dqk, Lk, S, Dv = _mla_shapes(fn, q, kv, part_m, part_l, part_acc)
    _expect(fn, "counters", counters, (B * H // 16,), _I32)
    _expect(fn, "o", o, (B, H, Dv), (_F32, _BF16))
    _expect(fn, "lse", lse, (B, H), _F32, optional=True)
    _dev(q, kv, part_m, part_l, part_acc, counters, o, lse)
    _check(lib().rf_mla_decode(_ptr(q), _ptr(kv), _ptr(part_m), _ptr(part_l), _ptr(part_acc), _ptr(counters),
                               _dtype_code(o), _ptr(o), _ptr(lse), B, H, Lk, Dqk, Dv, S, float(scale), _stream(q)))


def rf_merge_states(part_m, part_l, part_acc, o, lse):
    fn = "rf_merge_states"
    if part_acc.dim() < 2:
        raise ValueError(f"{fn}: part_acc must be [..., S, d], has shape {tuple(part_acc.shape)}")
    lead, (S, d) = tuple(part_acc.shape[:-2]), tuple(part_acc.shape[-2:])
    rows = 1
    for x in lead:
        rows *= x
    _expect(fn, "part_acc", part_acc, lead + (S, d), _F32)
    _expect(fn, "part_m", part_m, lead + (S,), _F32)
    _expect(fn, "part_l", part_l, lead + (S,), _F32)
    _expect(fn, "o", o, lead + (d,), (_F32, _BF16))
    _expect(fn, "lse", lse, lead, _F32, optional=True)
    _dev(part_m, part_l, part_acc, o, lse)
    _check(lib().rf_merge_states(_ptr(part_m), _ptr(part_l), _ptr(part_acc), rows, S, d,
                                 _dtype_code(o), _ptr(o), _ptr(lse), _stream(part_m)))


def rf_softmax_topk(logits, k, renormalize, weights, indices):
    fn = "rf_softmax_topk"
    _ndim(fn, "logits", logits, 2)
    T, E = logits.shape
    k = int(k)
    _expect(fn, "logits", logits, (T, E), _F32)
    _expect(fn, "weights", weights, (T, k), _F32)
    _expect(fn, "indices", indices, (T, k), _I32)
    _dev(logits, weights, indices)
    _check(lib().rf_softmax_topk(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(weights),
                                 _ptr(indices), _stream(logits)))


def rf_softmax(x, level, work, y):
    fn = "rf_softmax"
    _ndim(fn, "x", x, 2)
    T, E = x.shape
    _expect(fn, "x", x, (T, E), _F32)
    _expect(fn, "y", y, (T, E), _F32)
    _expect(fn, "work", work, (2 * T,), _F32, optional=True)
    _dev(x, work, y)
    _check(lib().rf_softmax(_ptr(x), T, E, int(level), _ptr(work), _ptr(y), _stream(x)))


def rf_row_variance(x, level, mean, var):
    fn = "rf_row_variance"
    _ndim(fn, "x", x, 2)
    T, E = x.shape
    _expect(fn, "x", x, (T, E), _F32)
    _expect(fn, "mean", mean, (T,), _F32)
    _expect(fn, "var", var, (T,), _F32)
    _dev(x, mean, var)
    _check(lib().rf_row_variance(_ptr(x), T, E, int(level), _ptr(mean), _ptr(var), _stream(x)))


def rf_row_inertia(x, w, level, centre, inertia):
    fn = "rf_row_inertia"
    _ndim(fn, "x", x, 2)
    T, E = x.shape
    _expect(fn, "x", x, (T, E), _F32)
    _expect(fn, "w", w, (T, E), _F32)
    _expect(fn, "centre", centre, (T,), _F32)
    _expect(fn, "inertia", inertia, (T,), _F32)
    _dev(x, w, centre, inertia)
    _check(lib().rf_row_inertia(_ptr(x), _ptr(w), T, E, int(level), _ptr(centre), _ptr(inertia),
                                _stream(x)))


def rf_absmax_quant_fp8(x, q, scale):
    fn = "rf_absmax_quant_fp8"
    _ndim(fn, "x", x, 2)
    rows, cols = x.shape
    _expect(fn, "x", x, (rows, cols), _BF16)
    _expect(fn, "q", q, (rows, cols), _U8)
    _expect(fn, "scale", scale, (rows,), _F32)
    _dev(x, q, scale)
    _check(lib().rf_absmax_quant_fp8(_ptr(x), rows, cols, _ptr(q), _ptr(scale), _stream(x)))


def _gemm_shapes(fn, a, b_q, b_scale, a_scale, c):
    _ndim(fn, "a", a, 2)
    _ndim(fn, "b_q", b_q, 2)
    M, K = a.shape
    N = b_q.shape[0]
    _expect(fn, "a", a, (M, K), _BF16)
    _expect(fn, "b_q", b_q, (N, K), _U8)
    _expect(fn, "b_scale", b_scale, (N,), _F32)
    _expect(fn, "a_scale", a_scale, (M,), _F32)
    _expect(fn, "c", c, (M, N), _BF16)
    return M, N, K


def rf_absmax_quant_gemm_fp8(a, b_q, b_scale, a_q, a_scale, c):
    fn = "rf_absmax_quant_gemm_fp8"
    M, N, K = _gemm_shapes(fn, a, b_q, b_scale, a_scale, c)
    _expect(fn, "a_q", a_q, (M, K), _U8)
    _dev(a, b_q, b_scale, a_q, a_scale, c)
    _check(lib().rf_absmax_quant_gemm_fp8(_ptr(a), _ptr(b_q), _ptr(b_scale), M, N, K, _ptr(a_q),
                                          _ptr(a_scale), _ptr(c), _stream(a)))


def rf_absmax_quant_gemm_fp8_noalloc(a, b_q, b_scale, a_scale, c):
    """The FP8 cascade with the quantised A in the library's own device scratch
    (no workspace argument, nothing allocated)."""
    fn = "rf_absmax_quant_gemm_fp8_noalloc"
    M, N, K = _gemm_shapes(fn, a, b_q, b_scale, a_scale, c)
    _dev(a, b_q, b_scale, a_scale, c)
    _check(lib().rf_absmax_quant_gemm_fp8_noalloc(_ptr(a), _ptr(b_q), _ptr(b_scale), M, N, K,
                                                  _ptr(a_scale), _ptr(c), _stream(a)))


def rf_absmax_quant_gemm_fp8_running(a, b_q, b_scale, a_scale, c):
    fn = "rf_absmax_quant_gemm_fp8_running"
    M, N, K = _gemm_shapes(fn, a, b_q, b_scale, a_scale, c)
    _dev(a, b_q, b_scale, a_scale, c)
    _check(lib().rf_absmax_quant_gemm_fp8_running(_ptr(a), _ptr(b_q), _ptr(b_scale), M, N, K,
                                                  _ptr(a_scale), _ptr(c), _stream(a)))


def rf_peak_mfma(kind, src, iters, out, clock=None):
    """Measurement loop (not a step of the path): src is a uint8 tensor
    [blocks * 256, 256]; out fp32 [blocks * 4]; clock int64 [blocks, 2] or None."""
    _dev(src, out, clock)
    if src.dtype != torch.uint8 or src.dim() != 2 or src.shape[1] != 256 or src.shape[0] % 256:
        raise ValueError("src must be uint8 [blocks * 256, 256]")
    blocks = src.shape[0] // 256
    if out.dtype != torch.float32 or out.numel() != 4 * blocks:
        raise ValueError("out must be fp32 with 4 values per workgroup")
    if clock is not None and (clock.dtype != torch.int64 or clock.numel() != 2 * blocks):
        raise ValueError("clock must be int64 [blocks, 2]")
    _check(lib().rf_peak_mfma(int(kind), _ptr(src), blocks, int(iters), _ptr(out), _ptr(clock),
                              _stream(src)))


def rf_peak_read(src, blocks, out):
    """HBM read stream (not a step of the path): src any contiguous device
    tensor (16-byte multiple); out int32 [blocks] gets per-workgroup XORs."""
    _dev(src, out)
    nbytes = src.numel() * src.element_size()
    if out.dtype != torch.int32 or out.numel() != blocks:
        raise ValueError("out must be int32 [blocks]")
    _check(lib().rf_peak_read(_ptr(src), nbytes, int(blocks), _ptr(out), _stream(src)))


def rf_wall_clock_khz():
    khz = ctypes.c_int(0)
    _check(lib().rf_wall_clock_khz(ctypes.byref(khz)))
    return khz.value


# ---------------------------------------------------------------- allocating helpers


def attn_fwd(q, k, v, scale, causal=False, with_lse=True):
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if with_lse else None
    rf_attn_fwd(q, k, v, o, lse, scale, causal)
    return o, lse


def attn_decode_partials(q, k, v, scale, S):
    B, Hq, d = q.shape
    part_m = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    part_l = torch.empty_like(part_m)
    part_acc = torch.empty((B, Hq, S, d), dtype=torch.float32, device=q.device)
    rf_attn_decode_split(q, k, v, part_m, part_l, part_acc, scale)
    return part_m, part_l, part_acc


def merge_states(part_m, part_l, part_acc, out_dtype=torch.bfloat16):
    o = torch.empty(part_acc.shape[:-2] + part_acc.shape[-1:], dtype=out_dtype, device=part_acc.device)
    lse = torch.empty(part_m.shape[:-1], dtype=torch.float32, device=part_m.device)
    rf_merge_states(part_m, part_l, part_acc, o, lse)
    return o, lse


def attn_decode(q, k, v, scale, S, out_dtype=torch.bfloat16):
    """Split-KV decode: partial states over S segments, then their merge."""
    parts = attn_decode_partials(q, k, v, scale, S)
    o, lse = merge_states(*parts, out_dtype=out_dtype)
    return o, lse, parts


def mla_decode(q, kv, scale, S, dv=512, out_dtype=torch.bfloat16, fused=False):
    """Split-KV decode over a shared latent cache, then the merge of the
    partials: two launches, or one (rf_mla_decode) with fused=True."""
    B, H, _ = q.shape
    part_m = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    part_l = torch.empty_like(part_m)
    part_acc = torch.empty((B, H, S, dv), dtype=torch.float32, device=q.device)
    if fused:
        counters = torch.zeros(B * H // 16, dtype=torch.int32, device=q.device)
        o = torch.empty((B, H, dv), dtype=out_dtype, device=q.device)
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
        rf_mla_decode(q, kv, part_m, part_l, part_acc, counters, o, lse, scale)
        return o, lse, (part_m, part_l, part_acc)
    rf_mla_decode_split(q, kv, part_m, part_l, part_acc, scale)
    o, lse = merge_states(part_m, part_l, part_acc, out_dtype=out_dtype)
    return o, lse, (part_m, part_l, part_acc)


def softmax_topk(logits, k, renormalize=True):
    T = logits.shape[0]
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    rf_softmax_topk(logits, k, renormalize, w, idx)
    return w, idx


def softmax(x, level=RF_FUSE_BLOCK):
    """Row softmax of fp32 x [T, E] with the cascade fused at ``level``."""
    y = torch.empty_like(x)
    work = torch.empty(2 * x.shape[0], dtype=torch.float32, device=x.device) if level == RF_FUSE_NONE else None
    rf_softmax(x, level, work, y)
    return y


def row_variance(x, level=RF_FUSE_WAVE):
    """Per-row mean and population variance of fp32 x [T, E]."""
    mean = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    var = torch.empty_like(mean)
    rf_row_variance(x, level, mean, var)
    return mean, var


def row_inertia(x, w, level=RF_FUSE_WAVE):
    """Per-row centre of mass and moment of inertia about it."""
    centre = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    inertia = torch.empty_like(centre)
    rf_row_inertia(x, w, level, centre, inertia)
    return centre, inertia


def absmax_quant_fp8(x):
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    rf_absmax_quant_fp8(x, q, s)
    return q, s


def absmax_quant_gemm_fp8(a, b_q, b_scale):
    M, K = a.shape
    N = b_q.shape[0]
    a_q = torch.empty((M, K), dtype=torch.uint8, device=a.device)
    a_scale = torch.empty(M, dtype=torch.float32, device=a.device)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    rf_absmax_quant_gemm_fp8(a, b_q, b_scale, a_q, a_scale, c)
    return c, a_q, a_scale


def absmax_quant_gemm_fp8_running(a, b_q, b_scale):
    """One-pass FP8 GEMM with a running per-row scale; returns (c, a_scale)."""
    M, K = a.shape
    N = b_q.shape[0]
    a_scale = torch.empty(M, dtype=torch.float32, device=a.device)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    rf_absmax_quant_gemm_fp8_running(a, b_q, b_scale, a_scale, c)
    return c, a_scale
