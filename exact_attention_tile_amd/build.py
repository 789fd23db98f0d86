"""Builds the HIP library ``libattn.so`` in-tree for gfx950.

    python -m exact_attention_tile_amd.build

compiles every source under ``csrc/`` with hipcc into
``exact_attention_tile_amd/libattn.so`` (cross-compiles; no GPU needed).
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")

SOURCES = ["attn_api.cpp", "attn_fwd_bf16.hip", "attn_fwd_fp8.hip", "attn_bwd_bf16.hip", "attn_quant.hip",
           "attn_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, out))
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


HOSTCHECK_LIB = os.path.join(PKG, "libattn_hostcheck.so")
HOSTCHECK_SOURCES = ["attn_api.cpp", "attn_noalloc.hip", "host_check_stubs.cpp"]


def build_host_check(verbose=False):
    """The C ABI's host code with the address and undefined-behaviour
    sanitizers (host side only; stub launchers, no kernels), for running the
    argument-validation tests on the CPU: libattn_hostcheck.so."""
    srcs = [os.path.join(CSRC, s) for s in HOSTCHECK_SOURCES]
    tmp = HOSTCHECK_LIB + ".tmp"
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
             "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    cmd = [hipcc()] + flags + ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, out))
    os.replace(tmp, HOSTCHECK_LIB)
    return HOSTCHECK_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
