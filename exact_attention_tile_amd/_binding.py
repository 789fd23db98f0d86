"""ctypes marshalling for libattn.so (C ABI in include/attn.h).

Pointer arguments accept a plain integer device address or any object with a
``data_ptr()`` method (a torch tensor); ``stream`` accepts an integer HIP
stream handle, ``None``/0 (the null stream) or an object with a
``cuda_stream`` attribute (a torch stream).
"""

import ctypes
import os

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_HIP = 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path():
    """The in-tree libattn.so, or the library named by EXACT_ATTN_LIB (the
    tests use this to run the host-side checks against the sanitizer build,
    libattn_hostcheck.so)."""
    return os.environ.get("EXACT_ATTN_LIB") or os.path.join(_HERE, "libattn.so")


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s returned %d (%s)" % (where, status, attn_status_string(status)))


def load_library():
    """Loads the in-tree libattn.so once; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    try:
        # share torch's HIP runtime (same SONAME) so its streams and device
        # pointers are valid in the library's calls
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError("libattn.so is not built (%s); run "
                           "`python -m exact_attention_tile_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.attn_fwd_fp8.restype = i
    lib.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_gqa.restype = i
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_varlen.restype = i
    lib.attn_fwd_fp8_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_fp8_gqa.restype = i
    lib.attn_fwd_fp8_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                        f, vp]
    lib.attn_fwd_fp8_varlen.restype = i
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.attn_bwd_noalloc.restype = i
    lib.attn_fwd_fp8_2pass.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_fp8_2pass.restype = i
    lib.attn_fp8_quantize.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    lib.attn_fp8_quantize.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s or None
    return s.cuda_stream or None


def attn_status_string(status):
    return load_library().attn_status_string(int(status)).decode()


def attn_version():
    return load_library().attn_version().decode()


def attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None, check=True):
    """bf16 forward; see attn_fwd in include/attn.h.  Returns the status;
    raises AttnError on a non-zero status when ``check``."""
    st = load_library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                 int(N), int(d), int(causal), float(scale), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd")
    return st


def attn_fwd_fp8(q, k, v, o, lse, descale_q, descale_k, descale_v, B, H, N, d, causal, scale,
                 stream=None, check=True):
    """OCP e4m3 forward; see attn_fwd_fp8 in include/attn.h."""
    st = load_library().attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     _ptr(descale_q), _ptr(descale_k), _ptr(descale_v), int(B),
                                     int(H), int(N), int(d), int(causal), float(scale),
                                     _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd_fp8")
    return st


def attn_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, stream=None, check=True):
    """bf16 grouped-query forward; see attn_fwd_gqa in include/attn.h."""
    st = load_library().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B),
                                     int(H), int(H_kv), int(N), int(d), int(causal), float(scale),
                                     _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd_gqa")
    return st


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, total, max_seqlen, H, H_kv, d, causal, scale,
                    stream=None, check=True):
    """bf16 variable-length forward; see attn_fwd_varlen in include/attn.h
    (``cu_seqlens`` is a device int32 array of B+1 offsets)."""
    st = load_library().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                        _ptr(cu_seqlens), int(B), int(total), int(max_seqlen),
                                        int(H), int(H_kv), int(d), int(causal), float(scale),
                                        _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd_varlen")
    return st


def attn_fwd_fp8_gqa(q, k, v, o, lse, descale_q, descale_k, descale_v, B, H, H_kv, N, d, causal,
                     scale, stream=None, check=True):
    """OCP e4m3 grouped-query forward; see attn_fwd_fp8_gqa in include/attn.h."""
    st = load_library().attn_fwd_fp8_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                         _ptr(descale_q), _ptr(descale_k), _ptr(descale_v),
                                         int(B), int(H), int(H_kv), int(N), int(d), int(causal),
                                         float(scale), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd_fp8_gqa")
    return st


def attn_fwd_fp8_varlen(q, k, v, o, lse, descale_q, descale_k, descale_v, cu_seqlens, B, total,
                        max_seqlen, H, H_kv, d, causal, scale, stream=None, check=True):
    """OCP e4m3 variable-length forward; see attn_fwd_fp8_varlen in include/attn.h."""
    st = load_library().attn_fwd_fp8_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                            _ptr(descale_q), _ptr(descale_k), _ptr(descale_v),
                                            _ptr(cu_seqlens), int(B), int(total), int(max_seqlen),
                                            int(H), int(H_kv), int(d), int(causal), float(scale),
                                            _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd_fp8_varlen")
    return st


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, causal, scale, stream=None,
             check=True):
    """bf16 backward; see attn_bwd in include/attn.h (``delta`` is a device
    fp32 [B][H][N] workspace)."""
    st = load_library().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta), int(B), int(H),
                                 int(N), int(d), int(causal), float(scale), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return st


ATTN_BWD_NOALLOC_MAX_ROWS = 1 << 22


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, causal, scale, stream=None,
                     check=True):
    """bf16 backward with the library's static workspace (no allocation);
    see attn_bwd_noalloc in include/attn.h (B * H * N <=
    ATTN_BWD_NOALLOC_MAX_ROWS; calls on one GPU must not overlap)."""
    st = load_library().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                         _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), int(B), int(H),
                                         int(N), int(d), int(causal), float(scale),
                                         _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_bwd_noalloc")
    return st


def attn_fp8_quantize(x, codes, descale, sign_bits, B, N, H, d, stream=None, check=True):
    """bf16 -> E4M3 codes + per-(batch, head) descale, optionally rotated;
    see attn_fp8_quantize in include/attn.h (``sign_bits`` None: no
    rotation)."""
    st = load_library().attn_fp8_quantize(_ptr(x), _ptr(codes), _ptr(descale), _ptr(sign_bits),
                                          int(B), int(N), int(H), int(d), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fp8_quantize")
    return st


def attn_fwd_fp8_2pass(q, k, v, o, lse, descale_q, descale_k, descale_v, B, H, H_kv, N, d, causal,
                       scale, stream=None, check=True):
    """Two-pass OCP e4m3 forward (exact row maximum first); see
    attn_fwd_fp8_2pass in include/attn.h."""
    st = load_library().attn_fwd_fp8_2pass(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                           _ptr(descale_q), _ptr(descale_k), _ptr(descale_v),
                                           int(B), int(H), int(H_kv), int(N), int(d),
                                           int(causal), float(scale), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd_fp8_2pass")
    return st
