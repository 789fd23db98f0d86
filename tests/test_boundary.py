"""The C-ABI library: it loads, exports every function include/attn.h
declares, and rejects invalid arguments on the host (before any HIP call, so
these run without a GPU)."""

import ctypes
import math
import os
import re

import pytest

import exact_attention_tile_amd as eat
from exact_attention_tile_amd import build as eat_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(eat.lib_path()):
        eat_build.build()
    return eat.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(names) == {"attn_fwd", "attn_fwd_fp8", "attn_fwd_gqa", "attn_fwd_varlen",
                          "attn_fwd_fp8_gqa", "attn_fwd_fp8_varlen", "attn_bwd", "attn_fp8_quantize",
                          "attn_fwd_fp8_2pass", "attn_bwd_noalloc",
                          "attn_status_string", "attn_version"}


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings(lib):
    assert eat.attn_status_string(eat.ATTN_OK) == "ATTN_OK"
    assert eat.attn_status_string(eat.ATTN_ERR_INVALID_ARG) == "ATTN_ERR_INVALID_ARG"
    assert eat.attn_status_string(eat.ATTN_ERR_UNSUPPORTED) == "ATTN_ERR_UNSUPPORTED"
    assert eat.attn_status_string(eat.ATTN_ERR_HIP) == "ATTN_ERR_HIP"
    assert eat.attn_status_string(42) == "ATTN_ERR_UNKNOWN"
    assert "gfx950" in eat.attn_version()


# Fake, 16-byte-aligned, never-dereferenced "device" addresses: every case
# below must be rejected by host-side validation before anything touches
# them.
P = 0x10000
GOOD = dict(q=P, k=P + 0x1000, v=P + 0x2000, o=P + 0x3000, lse=P + 0x4000,
            B=1, H=2, N=128, d=64, causal=0, scale=0.125)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return eat.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                        a["causal"], a["scale"], None, check=False)


def call8(**kw):
    a = dict(GOOD, dq=P + 0x5000, dk=P + 0x5100, dv=P + 0x5200)
    a.update(kw)
    return eat.attn_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dq"], a["dk"], a["dv"],
                            a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], None,
                            check=False)


def call_gqa(**kw):
    a = dict(GOOD, Hkv=1)
    a.update(kw)
    return eat.attn_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                            a["N"], a["d"], a["causal"], a["scale"], None, check=False)


def call8_gqa(**kw):
    a = dict(GOOD, Hkv=1, dq=P + 0x5000, dk=P + 0x5100, dv=P + 0x5200)
    a.update(kw)
    return eat.attn_fwd_fp8_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dq"], a["dk"],
                                a["dv"], a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["causal"],
                                a["scale"], None, check=False)


# variable-length calls: B sequences packed into N (= total) tokens
def call_var(**kw):
    a = dict(GOOD, Hkv=2, cu=P + 0x6000, maxlen=64)
    a.update(kw)
    return eat.attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["B"], a["N"],
                               a["maxlen"], a["H"], a["Hkv"], a["d"], a["causal"], a["scale"],
                               None, check=False)


def call8_var(**kw):
    a = dict(GOOD, Hkv=2, cu=P + 0x6000, maxlen=64, dq=P + 0x5000, dk=P + 0x5100, dv=P + 0x5200)
    a.update(kw)
    return eat.attn_fwd_fp8_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dq"], a["dk"],
                                   a["dv"], a["cu"], a["B"], a["N"], a["maxlen"], a["H"], a["Hkv"],
                                   a["d"], a["causal"], a["scale"], None, check=False)


def call_bwd(**kw):
    a = dict(GOOD, do=P + 0x7000, dq=P + 0x8000, dk=P + 0x9000, dv=P + 0xA000, delta=P + 0xB000)
    a.update(kw)
    return eat.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                        a["dv"], a["delta"], a["B"], a["H"], a["N"], a["d"], a["causal"],
                        a["scale"], None, check=False)


def call8_2p(**kw):
    a = dict(GOOD, Hkv=1, dq=P + 0x5000, dk=P + 0x5100, dv=P + 0x5200)
    a.update(kw)
    return eat.attn_fwd_fp8_2pass(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dq"], a["dk"],
                                  a["dv"], a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["causal"],
                                  a["scale"], None, check=False)


ALL_CALLS = [call, call8, call_gqa, call8_gqa, call_var, call8_var, call_bwd, call8_2p]


@pytest.mark.parametrize("fn", ALL_CALLS)
@pytest.mark.parametrize("kw,status", [
    (dict(q=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(k=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(v=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(o=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(lse=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(B=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(H=-1), eat.ATTN_ERR_INVALID_ARG),
    (dict(N=-1), eat.ATTN_ERR_INVALID_ARG),
    (dict(causal=2), eat.ATTN_ERR_INVALID_ARG),
    (dict(causal=-1), eat.ATTN_ERR_INVALID_ARG),
    (dict(scale=math.inf), eat.ATTN_ERR_INVALID_ARG),
    (dict(scale=math.nan), eat.ATTN_ERR_INVALID_ARG),
    (dict(d=96), eat.ATTN_ERR_UNSUPPORTED),
    (dict(d=256), eat.ATTN_ERR_UNSUPPORTED),
    (dict(d=0), eat.ATTN_ERR_UNSUPPORTED),
    (dict(q=P + 8), eat.ATTN_ERR_UNSUPPORTED),
    (dict(o=P + 0x3002), eat.ATTN_ERR_UNSUPPORTED),
    (dict(lse=P + 0x4002), eat.ATTN_ERR_UNSUPPORTED),
    (dict(H=1 << 18, d=128, Hkv=1), eat.ATTN_ERR_UNSUPPORTED),  # H*d beyond 2^24
])
def test_invalid_arguments_rejected_on_host(lib, fn, kw, status):
    assert fn(**kw) == status


@pytest.mark.parametrize("fn", [call, call8, call_bwd, call8_2p])
@pytest.mark.parametrize("kw,status", [
    (dict(N=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(B=1 << 30, N=1 << 30, H=1 << 30), eat.ATTN_ERR_INVALID_ARG),
    (dict(B=65535, H=65535, N=1 << 20), eat.ATTN_ERR_UNSUPPORTED),   # grid beyond 2^31 blocks
])
def test_fixed_length_sizes(lib, fn, kw, status):
    assert fn(**kw) == status


@pytest.mark.parametrize("fn", [call_gqa, call8_gqa, call_var, call8_var, call8_2p])
@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=-2), eat.ATTN_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4), eat.ATTN_ERR_INVALID_ARG),    # H not a multiple of H_kv
    (dict(H=2, Hkv=4), eat.ATTN_ERR_INVALID_ARG),
])
def test_kv_heads_checked(lib, fn, kw, status):
    assert fn(**kw) == status


@pytest.mark.parametrize("fn", [call_var, call8_var])
@pytest.mark.parametrize("kw,status", [
    (dict(cu=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(cu=P + 0x6002), eat.ATTN_ERR_UNSUPPORTED),
    (dict(B=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(N=-5), eat.ATTN_ERR_INVALID_ARG),           # total < 0
    (dict(maxlen=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(maxlen=129), eat.ATTN_ERR_INVALID_ARG),     # longer than total (128)
    (dict(N=1 << 30, maxlen=1 << 30, B=1 << 20, H=64, Hkv=64), eat.ATTN_ERR_UNSUPPORTED),  # grid
    (dict(N=0, q=0, k=0, v=0, o=0, lse=0), eat.ATTN_OK),   # empty batch: nothing launched
    (dict(N=0, H=3, Hkv=2), eat.ATTN_ERR_INVALID_ARG),
    (dict(N=0, d=80), eat.ATTN_ERR_UNSUPPORTED),
])
def test_varlen_sizes(lib, fn, kw, status):
    assert fn(**kw) == status


@pytest.mark.parametrize("fn", [call8, call8_gqa, call8_var, call8_2p])
@pytest.mark.parametrize("kw", [dict(dq=0), dict(dk=0), dict(dv=0)])
def test_fp8_requires_descales(lib, fn, kw):
    assert fn(**kw) == eat.ATTN_ERR_INVALID_ARG


def test_binding_raises_with_status_name(lib):
    with pytest.raises(eat.AttnError, match="ATTN_ERR_UNSUPPORTED"):
        eat.attn_fwd(P, P, P, P, P, 1, 1, 16, 80, 0, 1.0)


@pytest.mark.parametrize("kw,status", [
    (dict(do=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(dq=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(dk=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(dv=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(delta=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(dq=P + 0x8008), eat.ATTN_ERR_UNSUPPORTED),
    (dict(delta=P + 0xB002), eat.ATTN_ERR_UNSUPPORTED),
])
def test_backward_buffers_checked(lib, kw, status):
    assert call_bwd(**kw) == status


def call_quant(**kw):
    a = dict(x=P, codes=P + 0x1000, descale=P + 0x2000, signs=P + 0x3000, B=2, N=128, H=4, d=128)
    a.update(kw)
    return eat.attn_fp8_quantize(a["x"], a["codes"], a["descale"], a["signs"], a["B"], a["N"],
                                 a["H"], a["d"], None, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(codes=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(descale=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(B=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(N=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(H=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(H=-3), eat.ATTN_ERR_INVALID_ARG),
    (dict(B=1 << 30, N=1 << 30, H=1 << 30), eat.ATTN_ERR_INVALID_ARG),
    (dict(d=96), eat.ATTN_ERR_UNSUPPORTED),
    (dict(d=32), eat.ATTN_ERR_UNSUPPORTED),
    (dict(x=P + 8), eat.ATTN_ERR_UNSUPPORTED),
    (dict(codes=P + 0x1004), eat.ATTN_ERR_UNSUPPORTED),
    (dict(descale=P + 0x2002), eat.ATTN_ERR_UNSUPPORTED),
    (dict(signs=P + 0x3001), eat.ATTN_ERR_UNSUPPORTED),
    (dict(B=65535, H=65535, N=1 << 20), eat.ATTN_ERR_UNSUPPORTED),   # grid beyond 2^31 blocks
])
def test_quantize_arguments_rejected_on_host(lib, kw, status):
    assert call_quant(**kw) == status


def call_bwd_na(**kw):
    a = dict(GOOD, do=P + 0x7000, dq=P + 0x8000, dk=P + 0x9000, dv=P + 0xA000)
    a.update(kw)
    return eat.attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["causal"],
                                a["scale"], None, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), eat.ATTN_ERR_INVALID_ARG), (dict(lse=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(do=0), eat.ATTN_ERR_INVALID_ARG), (dict(dv=0), eat.ATTN_ERR_INVALID_ARG),
    (dict(B=0), eat.ATTN_ERR_INVALID_ARG), (dict(H=-1), eat.ATTN_ERR_INVALID_ARG),
    (dict(N=0), eat.ATTN_ERR_INVALID_ARG),
    # the static workspace holds ATTN_BWD_NOALLOC_MAX_ROWS rows of B * H * N
    (dict(B=1, H=1, N=eat.ATTN_BWD_NOALLOC_MAX_ROWS + 1), eat.ATTN_ERR_UNSUPPORTED),
    (dict(B=2, H=64, N=32769), eat.ATTN_ERR_UNSUPPORTED),
])
def test_bwd_noalloc_rejects_before_any_hip_call(lib, kw, status):
    assert call_bwd_na(**kw) == status


def test_bwd_noalloc_limit_matches_header():
    text = open(HEADER).read()
    assert "#define ATTN_BWD_NOALLOC_MAX_ROWS (1 << 22)" in text
    assert eat.ATTN_BWD_NOALLOC_MAX_ROWS == 1 << 22
