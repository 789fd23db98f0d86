"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU
oracle on the same seeded inputs.

* every workload at its full size and in its launch configuration, each
  causal mode it lists; the oracle covers all rows when N <= 2048 and 512
  seeded rows per head (rows 0 and N-1 included) beyond that;
* ragged and degenerate shapes (N = 1, tails that leave partial K/V tiles
  and partial query tiles, grids that are not a multiple of 8) against the
  full oracle, both dtypes, both modes;
* negative and zero scale;
* a 65536-token causal context (both dtypes, 256 sampled rows per head);
* bitwise determinism of two identical calls, and untouched guard bands
  around O and LSE in every run.
Tolerances are in parity_common.py.
"""

import numpy as np
import pytest
import torch

from parity_common import (assert_bf16_ok, assert_fp8_ok, errors, fp8_lse_bound, reference,
                           require_gpu, run_bf16, run_fp8)
from workloads import WORKLOADS, Workload, make_inputs, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def _run(w, inp, causal, scale=None, shape=None):
    B, N, H, d = shape if shape is not None else (w.B, w.N, w.H, w.d)
    scale = w.scale if scale is None else scale
    print("case %s B=%d H=%d N=%d d=%d causal=%d scale=%g" % (w.name, B, H, N, d, causal, scale),
          flush=True)
    if w.dtype == "fp8":
        return run_fp8(inp, B, H, N, d, causal, scale)
    return run_bf16(inp, B, H, N, d, causal, scale)


def _check(w, inp, out, ro, rl, causal, scale, label, rows=None):
    assert out.guards_intact(), label + ": wrote outside O/LSE"
    if w.dtype == "fp8":
        bound = fp8_lse_bound(inp, causal, scale, rows)
        assert_fp8_ok(errors(out, ro, rl, rows, lse_bound=bound), label)
    else:
        assert_bf16_ok(errors(out, ro, rl, rows), label)


# ---------------------------------------------------------------------------
# ragged / degenerate shapes, full oracle
# ---------------------------------------------------------------------------

EDGE = [(1, 1, 1), (1, 1, 17), (2, 3, 130), (1, 2, 1000), (1, 5, 300), (3, 1, 257),
        # B*H = 8 with 3 query tiles: causal calls take the tile-major block order
        (2, 4, 700)]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", EDGE)
def test_edge_shapes(dtype, d, causal, B, H, N):
    w = Workload("edge_%s" % dtype, 50 + N % 17, B, H, N, d, dtype, (causal,))
    inp = make_inputs(w)
    out = _run(w, inp, causal)
    ro, rl = reference(inp, dtype, causal, w.scale)
    _check(w, inp, out, ro, rl, causal, w.scale, "edge %s d=%d causal=%d B=%d H=%d N=%d" %
           (dtype, d, causal, B, H, N))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.9])
@pytest.mark.parametrize("causal", [False, True])
def test_scale_sign_and_zero(dtype, scale, causal):
    w = Workload("scale_%s" % dtype, 60, 1, 2, 333, 128, dtype, (causal,))
    inp = make_inputs(w)
    out = _run(w, inp, causal, scale=scale)
    ro, rl = reference(inp, dtype, causal, scale)
    _check(w, inp, out, ro, rl, causal, scale, "scale %s %g causal=%d" % (dtype, scale, causal))


# ---------------------------------------------------------------------------
# the workloads, full size
# ---------------------------------------------------------------------------

CASES = [(name, c) for name in ("tiny", "mha2k", "long8k", "long8k64", "fp8_8k", "ctx32k")
         for c in WORKLOADS[name].modes]


@pytest.mark.parametrize("name,causal", CASES)
def test_workload(name, causal):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    out = _run(w, inp, causal)
    rows = None if w.N <= 2048 else sample_rows(w)
    ro, rl = reference(inp, w.dtype, causal, w.scale, rows=rows)
    _check(w, inp, out, ro, rl, causal, w.scale, "%s causal=%d" % (name, causal), rows)


# ---------------------------------------------------------------------------
# determinism
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_bitwise_deterministic(dtype):
    w = Workload("det_%s" % dtype, 70, 2, 4, 1531, 128, dtype, (True,))
    inp = make_inputs(w)
    a = _run(w, inp, True)
    b = _run(w, inp, True)
    assert torch.equal(a.o_raw, b.o_raw)
    assert torch.equal(a.l_raw, b.l_raw)


# ---------------------------------------------------------------------------
# a context longer than any benchmark workload (64-bit offsets, many tiles)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_long_context_64k(dtype):
    w = Workload("ctx64k", 92, 1, 2, 65536, 128, dtype, (True,), outliers=dtype == "fp8")
    inp = make_inputs(w)
    out = _run(w, inp, True)
    rows = sample_rows(w, count=256)
    ro, rl = reference(inp, dtype, True, w.scale, rows=rows)
    _check(w, inp, out, ro, rl, True, w.scale, "ctx64k %s" % dtype, rows=rows)
