"""The C ABI on the host (no GPU): the library loads, exports every entry point
that include/rf.h declares, and rejects bad arguments before launching anything.
Only argument combinations that fail validation are passed here, so no call
reaches the HIP runtime."""

import ctypes
import os
import re

import pytest

from online_softmax_attention_cascaded_amd import binding
from online_softmax_attention_cascaded_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rf.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
F32, BF16 = 0, 1
FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10004)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        from online_softmax_attention_cascaded_amd import build

        build.build()
    return binding.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(rf_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = _declared()
    assert names == sorted(binding.SIGNATURES), names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_argument_counts_match_header():
    text = open(HEADER).read()
    for name, args in binding.SIGNATURES.items():
        m = re.search(r"\b" + name + r"\s*\(([^;]*?)\)\s*;", text, flags=re.S)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(args), (name, len(params), len(args))


def test_status_helpers(lib):
    assert lib.rf_abi_version() == 8
    assert lib.rf_status_string(OK) == b"RF_OK"
    assert lib.rf_status_string(INVALID) == b"RF_ERR_INVALID_ARG"
    assert lib.rf_status_string(UNSUPPORTED) == b"RF_ERR_UNSUPPORTED"
    assert lib.rf_status_string(3) == b"RF_ERR_LAUNCH"


def attn(lib, dt=BF16, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=4, Hkv=2, Lq=64, Lk=64,
         d=128, scale=0.1, causal=0):
    return lib.rf_attn_fwd(dt, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, scale, causal, None)


@pytest.mark.parametrize(
    "kw,expect",
    [
        (dict(dt=7), INVALID),
        (dict(B=-1), INVALID),
        (dict(Hkv=3), INVALID),
        (dict(Hkv=0), INVALID),
        (dict(Lk=0), INVALID),
        (dict(causal=1, Lk=32), INVALID),
        (dict(q=None), INVALID),
        (dict(o=MISALIGNED), INVALID),
        (dict(scale=float("nan")), INVALID),
        (dict(scale=float("inf")), INVALID),
        (dict(scale=float("-inf")), INVALID),
        (dict(d=96), UNSUPPORTED),
        (dict(dt=F32, d=96), UNSUPPORTED),
        (dict(d=32), UNSUPPORTED),
        (dict(Lk=1 << 23), UNSUPPORTED),     # one head's K/V reaches 2 GiB
        (dict(d=64, Lk=1 << 24), UNSUPPORTED),
    ],
)
def test_attn_validation(lib, kw, expect):
    assert attn(lib, **kw) == expect
    assert lib.rf_last_error().startswith(b"rf_attn_fwd")


def test_attn_empty_is_ok_without_pointers(lib):
    assert attn(lib, q=None, k=None, v=None, o=None, B=0) == OK
    assert attn(lib, q=None, k=None, v=None, o=None, Lq=0) == OK
    assert lib.rf_last_error() == b""


def decode(lib, dt=BF16, q=FAKE, k=FAKE, v=FAKE, m=FAKE, l=FAKE, acc=FAKE, B=1, Hq=8, Hkv=2,
           Lk=100, d=128, S=4, scale=0.1):
    return lib.rf_attn_decode_split(dt, q, k, v, m, l, acc, B, Hq, Hkv, Lk, d, S, scale, None)


@pytest.mark.parametrize(
    "kw,expect",
    [
        (dict(S=0), INVALID),
        (dict(Hkv=3), INVALID),
        (dict(Lk=0), INVALID),
        (dict(acc=None), INVALID),
        (dict(k=MISALIGNED), INVALID),
        (dict(dt=7), INVALID),
        (dict(scale=float("nan")), INVALID),
        (dict(scale=float("inf")), INVALID),
        (dict(scale=float("-inf")), INVALID),
        (dict(d=96), UNSUPPORTED),
        (dict(dt=F32, d=32), UNSUPPORTED),
        (dict(Hq=34, Hkv=2), UNSUPPORTED),
        (dict(dt=F32, Hq=34, Hkv=2), UNSUPPORTED),
        (dict(Lk=1 << 23), UNSUPPORTED),     # one head's K/V reaches 2 GiB
        (dict(dt=F32, Lk=1 << 22), UNSUPPORTED),
        (dict(dt=F32, d=64, Lk=1 << 23), UNSUPPORTED),
    ],
)
def test_decode_validation(lib, kw, expect):
    assert decode(lib, **kw) == expect
    assert lib.rf_last_error().startswith(b"rf_attn_decode_split")


def test_decode_empty_is_ok_without_pointers(lib):
    for dt in (F32, BF16):
        assert decode(lib, dt=dt, q=None, k=None, v=None, m=None, l=None, acc=None, B=0) == OK


def mla(lib, q=FAKE, kv=FAKE, m=FAKE, l=FAKE, acc=FAKE, B=2, H=16, Lk=100, Dqk=576, Dv=512, S=4,
        scale=0.1):
    return lib.rf_mla_decode_split(q, kv, m, l, acc, B, H, Lk, Dqk, Dv, S, scale, None)


@pytest.mark.parametrize(
    "kw,expect",
    [
        (dict(S=0), INVALID),
        (dict(Lk=0), INVALID),
        (dict(B=-1), INVALID),
        (dict(Dv=600), INVALID),
        (dict(acc=None), INVALID),
        (dict(kv=MISALIGNED), INVALID),
        (dict(scale=float("nan")), INVALID),
        (dict(scale=float("inf")), INVALID),
        (dict(scale=float("-inf")), INVALID),
        (dict(Dqk=192, Dv=128), UNSUPPORTED),
        (dict(Dv=256), UNSUPPORTED),
        (dict(H=8), UNSUPPORTED),
        (dict(H=144), UNSUPPORTED),
        (dict(Lk=1 << 21), UNSUPPORTED),   # one sequence's cache reaches 2 GiB
    ],
)
def test_mla_validation(lib, kw, expect):
    assert mla(lib, **kw) == expect
    assert lib.rf_last_error().startswith(b"rf_mla_decode_split")


def test_mla_empty_is_ok_without_pointers(lib):
    assert mla(lib, q=None, kv=None, m=None, l=None, acc=None, B=0) == OK


def mla_fused(lib, q=FAKE, kv=FAKE, m=FAKE, l=FAKE, acc=FAKE, cnt=FAKE, dt=BF16, o=FAKE, lse=None, B=2, H=16,
              Lk=100, Dqk=576, Dv=512, S=4, scale=0.1):
    return lib.rf_mla_decode(q, kv, m, l, acc, cnt, dt, o, lse, B, H, Lk, Dqk, Dv, S, scale, None)


@pytest.mark.parametrize(
    "kw,expect",
    [
        (dict(S=0), INVALID),
        (dict(Lk=0), INVALID),
        (dict(acc=None), INVALID),
        (dict(kv=MISALIGNED), INVALID),
        (dict(Dv=256), UNSUPPORTED),
        (dict(H=8), UNSUPPORTED),
        (dict(cnt=None), INVALID),
        (dict(cnt=ctypes.c_void_p(0x10002)), INVALID),
        (dict(o=None), INVALID),
        (dict(o=MISALIGNED), INVALID),
        (dict(lse=ctypes.c_void_p(0x10002)), INVALID),
        (dict(dt=5), INVALID),
    ],
)
def test_mla_fused_validation(lib, kw, expect):
    assert mla_fused(lib, **kw) == expect
    assert lib.rf_last_error().startswith(b"rf_mla_decode")


def test_mla_fused_empty_is_ok_without_pointers(lib):
    assert mla_fused(lib, q=None, kv=None, m=None, l=None, acc=None, cnt=None, o=None, B=0) == OK


def test_merge_validation(lib):
    f = lib.rf_merge_states
    assert f(FAKE, FAKE, FAKE, 4, 0, 128, BF16, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, FAKE, -1, 2, 128, BF16, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 4, 2, 130, BF16, FAKE, None, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, 4, 2, 2048, BF16, FAKE, None, None) == UNSUPPORTED
    assert f(FAKE, FAKE, None, 4, 2, 128, BF16, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 4, 2, 128, 5, FAKE, None, None) == INVALID
    assert f(None, None, None, 0, 2, 128, BF16, None, None, None) == OK


def test_topk_validation(lib):
    f = lib.rf_softmax_topk
    assert f(FAKE, 10, 256, 0, 1, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 10, 8, 9, 1, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 10, 2048, 8, 1, FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, 10, 254, 8, 1, FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, 10, 256, 40, 1, FAKE, FAKE, None) == UNSUPPORTED
    assert f(MISALIGNED, 10, 256, 8, 1, FAKE, FAKE, None) == INVALID
    assert f(None, 0, 256, 8, 1, None, None, None) == OK


def test_softmax_validation(lib):
    f = lib.rf_softmax
    assert f(FAKE, 10, 1024, 4, None, FAKE, None) == INVALID      # unknown level
    assert f(FAKE, -1, 1024, 3, None, FAKE, None) == INVALID
    assert f(FAKE, 10, 1022, 3, None, FAKE, None) == INVALID      # E % 4
    assert f(FAKE, 10, 0, 3, None, FAKE, None) == INVALID
    assert f(FAKE, 10, 8196, 3, None, FAKE, None) == UNSUPPORTED
    assert f(FAKE, 10, 1024, 0, None, FAKE, None) == INVALID      # unfused needs work
    assert f(MISALIGNED, 10, 1024, 2, None, FAKE, None) == INVALID
    assert f(FAKE, 10, 1024, 1, None, None, None) == INVALID
    assert f(None, 0, 1024, 0, None, None, None) == OK
    assert lib.rf_last_error() == b""


@pytest.mark.parametrize("name", ["rf_row_variance", "rf_row_inertia"])
def test_moments_validation(lib, name):
    weighted = name == "rf_row_inertia"

    def call(x=FAKE, w=FAKE, T=10, E=1024, level=2, c=FAKE, i=FAKE):
        args = [x] + ([w] if weighted else []) + [T, E, level, c, i, None]
        return getattr(lib, name)(*args)

    assert call(level=4) == INVALID
    assert call(level=-1) == INVALID
    assert call(T=-1) == INVALID
    assert call(E=1022) == INVALID
    assert call(E=0) == INVALID
    assert call(E=8196) == UNSUPPORTED
    assert call(x=None) == INVALID
    assert call(i=None) == INVALID
    assert call(x=MISALIGNED) == INVALID
    if weighted:
        assert call(w=None) == INVALID
        assert call(w=MISALIGNED) == INVALID
    assert lib.rf_last_error().startswith(name.encode())
    assert call(x=None, w=None, T=0, c=None, i=None) == OK


def test_quant_validation(lib):
    f = lib.rf_absmax_quant_fp8
    assert f(FAKE, 4, 12, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 4, 16384, FAKE, FAKE, None) == UNSUPPORTED
    assert f(None, 4, 64, FAKE, FAKE, None) == INVALID
    assert f(None, 0, 64, None, None, None) == OK
    g = lib.rf_absmax_quant_gemm_fp8
    assert g(FAKE, FAKE, FAKE, 64, 64, 100, FAKE, FAKE, FAKE, None) == INVALID
    assert g(FAKE, FAKE, FAKE, 64, 64, 16384, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert g(FAKE, FAKE, FAKE, 64, 64, 256, None, FAKE, FAKE, None) == INVALID
    assert g(None, None, None, 0, 64, 256, None, None, None, None) == OK
    n = lib.rf_absmax_quant_gemm_fp8_noalloc
    assert n(FAKE, FAKE, FAKE, 64, 64, 100, FAKE, FAKE, None) == INVALID
    assert n(FAKE, FAKE, FAKE, 64, 64, 16384, FAKE, FAKE, None) == UNSUPPORTED
    assert n(FAKE, FAKE, FAKE, 64, 64, 256, None, FAKE, None) == INVALID
    assert n(MISALIGNED, FAKE, FAKE, 64, 64, 256, FAKE, FAKE, None) == INVALID
    # the quantised A must fit the 32 MiB scratch: 4097 x 8192 bytes does not
    assert n(FAKE, FAKE, FAKE, 4097, 64, 8192, FAKE, FAKE, None) == UNSUPPORTED
    assert b"scratch" in lib.rf_last_error()
    assert n(None, None, None, 0, 64, 256, None, None, None) == OK


def test_binding_refuses_host_tensors():
    import torch

    x = torch.zeros(4, 256)
    with pytest.raises(ValueError):
        binding.softmax_topk(x, 8)


def test_peak_validation(lib):
    f = lib.rf_peak_mfma
    assert f(2, FAKE, 4, 8, FAKE, None, None) == INVALID          # unknown kind
    assert f(0, FAKE, 0, 8, FAKE, None, None) == INVALID
    assert f(0, FAKE, 65537, 8, FAKE, None, None) == INVALID
    assert f(1, FAKE, 4, 0, FAKE, None, None) == INVALID
    assert f(1, FAKE, 4, (1 << 20) + 1, FAKE, None, None) == INVALID
    assert f(0, None, 4, 8, FAKE, None, None) == INVALID
    assert f(0, FAKE, 4, 8, None, None, None) == INVALID
    assert f(0, ctypes.c_void_p(0x10010), 4, 8, FAKE, None, None) == INVALID   # src not 32-byte aligned
    assert f(0, FAKE, 4, 8, FAKE, MISALIGNED, None) == INVALID
    assert lib.rf_last_error().startswith(b"rf_peak_mfma")
    assert lib.rf_wall_clock_khz(None) == INVALID
    g = lib.rf_peak_read
    assert g(FAKE, 100, 4, FAKE, None) == INVALID                 # bytes % 16
    assert g(FAKE, -16, 4, FAKE, None) == INVALID
    assert g(FAKE, 1024, 0, FAKE, None) == INVALID
    assert g(FAKE, 1024, 4, None, None) == INVALID
    assert g(MISALIGNED, 1024, 4, FAKE, None) == INVALID


def test_build_id_matches_the_sources(lib):
    from online_softmax_attention_cascaded_amd.build import source_digest

    assert lib.rf_build_id().decode() == source_digest()


def test_binding_refuses_a_library_from_other_sources(monkeypatch):
    """A librf.so whose build id differs from the digest of the sources next to
    it (a stale build) is refused when it is loaded."""
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "source_digest", lambda: "0000000000000000")
    with pytest.raises(RuntimeError, match="built from other sources"):
        binding.lib()
