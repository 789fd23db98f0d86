"""Microbenchmarks of the gfx950 units the attention kernels are bound by
(vector ALU issue, transcendental rate, MFMA rate and its overlap with a
vector wave, LDS read bandwidth) and a one-instruction MFMA accuracy probe.

``build()`` compiles ``mb_kernels.hip`` into ``microbench/libattn_mb.so``
(in-tree, cross-compiled for gfx950); ``load()`` opens it with ctypes.
``python -m microbench.run`` runs the timings on the GPU and prints a
Markdown table.  Nothing here is part of the attention library.
"""

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libattn_mb.so")
SOURCE = os.path.join(HERE, "mb_kernels.hip")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

_LIB = None


def lib_path():
    return LIB


def build(verbose=False):
    hipcc = os.environ.get("HIPCC") or "/opt/rocm/bin/hipcc"
    tmp = LIB + ".tmp"
    cmd = [hipcc] + FLAGS + ["-o", tmp, SOURCE]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, out))
    os.replace(tmp, LIB)
    return LIB


def load():
    global _LIB
    if _LIB is not None:
        return _LIB
    try:
        import torch  # noqa: F401  (share torch's HIP runtime)
    except ImportError:
        pass
    if not os.path.exists(LIB):
        raise RuntimeError("libattn_mb.so is not built (%s); run microbench.build()" % LIB)
    lib = ctypes.CDLL(LIB)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.mb_valu_rate.argtypes = [i, i, i, i, vp, vp, vp]
    lib.mb_mfma_pair.argtypes = [i, i, i, i, i, vp, vp, vp]
    lib.mb_lds_read.argtypes = [i, i, i, i, vp, vp, vp]
    lib.mb_mfma_lds.argtypes = [i, i, i, i, vp, vp, vp]
    lib.mb_mfma_one.argtypes = [i, vp, vp, vp, vp, i, vp]
    lib.mb_mfma_inwave.argtypes = [i, i, i, i, i, vp, vp, vp]
    lib.mb_tile_loads.argtypes = [i, i, i, i, i, vp, ctypes.c_longlong, vp, vp, vp]
    lib.mb_mfma_chain.argtypes = [i, i, i, i, vp, vp, vp]
    lib.mb_lds_latency.argtypes = [i, i, i, vp, vp, vp]
    lib.mb_dq_atomics.argtypes = [i, i, i, vp, ctypes.c_float, vp]
    for f in (lib.mb_valu_rate, lib.mb_mfma_pair, lib.mb_lds_read, lib.mb_mfma_lds,
              lib.mb_mfma_one, lib.mb_mfma_inwave, lib.mb_tile_loads, lib.mb_mfma_chain,
              lib.mb_lds_latency, lib.mb_dq_atomics):
        f.restype = i
    _LIB = lib
    return lib


def mfma_one(dtype, a, b, c):
    """One MFMA per 32x32 problem on the GPU: D = A B^T + C.

    dtype "e4m3": a, b uint8 codes [n][32][64]; "bf16": a, b bf16 bit
    patterns (uint16) [n][32][16]; c float32 [n][32][32].  Returns D
    float32 [n][32][32] (numpy)."""
    import numpy as np
    import torch
    n = a.shape[0]
    if dtype == "e4m3":
        assert a.shape == (n, 32, 64) and b.shape == (n, 32, 64) and a.dtype == np.uint8
        ta = torch.from_numpy(np.ascontiguousarray(a)).cuda()
        tb = torch.from_numpy(np.ascontiguousarray(b)).cuda()
        code = 0
    else:
        assert a.shape == (n, 32, 16) and b.shape == (n, 32, 16) and a.dtype == np.uint16
        ta = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
        tb = torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).cuda()
        code = 1
    assert c.shape == (n, 32, 32)
    tc = torch.from_numpy(np.ascontiguousarray(c, dtype=np.float32)).cuda()
    td = torch.empty_like(tc)
    st = load().mb_mfma_one(code, ta.data_ptr(), tb.data_ptr(), tc.data_ptr(), td.data_ptr(), n,
                            torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise RuntimeError("mb_mfma_one failed: hipError %d" % st)
    torch.cuda.synchronize()
    return td.cpu().numpy()
