"""MI355X (gfx950) tiled exact attention forward.

A thin ctypes binding over the C ABI declared in ``include/attn.h``
(``libattn.so``, built in-tree by ``exact_attention_tile_amd.build``).  Every
step of the attention runs in the library's HIP kernels; this module only
marshals arguments.  There is no CPU fallback: without the built library the
import of the binding raises.
"""

from ._binding import (ATTN_BWD_NOALLOC_MAX_ROWS, ATTN_ERR_HIP, ATTN_ERR_INVALID_ARG,
                       ATTN_ERR_UNSUPPORTED, ATTN_OK, AttnError, attn_bwd, attn_bwd_noalloc,
                       attn_fp8_quantize, attn_fwd, attn_fwd_fp8,
                       attn_fwd_fp8_2pass, attn_fwd_fp8_gqa, attn_fwd_fp8_varlen, attn_fwd_gqa, attn_fwd_varlen,
                       attn_status_string, attn_version, lib_path, load_library)

__all__ = [
    "ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_HIP", "AttnError",
    "attn_fwd", "attn_fwd_fp8", "attn_fwd_gqa", "attn_fwd_varlen", "attn_fwd_fp8_gqa",
    "attn_fwd_fp8_varlen", "attn_fwd_fp8_2pass", "attn_bwd", "attn_bwd_noalloc",
    "ATTN_BWD_NOALLOC_MAX_ROWS", "attn_fp8_quantize", "attn_status_string", "attn_version",
    "lib_path", "load_library",
]
