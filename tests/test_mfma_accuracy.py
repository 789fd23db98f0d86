"""Accuracy of single gfx950 matrix-core instructions against the exact dot
products, on the attention kernels' own operand distributions.

Why: the fp8 forward's scores are sums of e4m3 products accumulated by
v_mfma_f32_32x32x64_f8f6f4 (64 products per instruction, d/64 instructions
chained through the fp32 accumulator), and the fp8 LSE tolerance in
parity_common.py is derived from this instruction's error model:

    |D - (sum_k a_k b_k + C)| <= EPS_E4M3_MFMA * 2^e + 2^-23 * (|C| + |D_exact|),
    e = floor(log2 max_k |a_k b_k|)

(the second term is ordinary binary32 rounding of the accumulator).  The
error is bounded by the largest product's binade, not by the sum of the
magnitudes: measured on 2M outputs of this instruction the ratio
|error| / sum_k |a_k b_k| kept growing with the sample (a heavy tail), while
|error| / 2^e stopped at 2^-11.04 with and without outliers and with a
nonzero accumulator -- the worst case of 64 products each placed on a grid
of 2^(e - 16) before an exact sum (64 half-steps = 2^(e - 11)).  The model's
constant EPS_E4M3_MFMA is the largest |error - fp32 terms| / 2^e seen,
rounded up to a power of two.  This test measures it on seeded e4m3 codes
drawn as the fp8 workloads draw them (N(0,1), per-block amax / 448
quantisation, with and without 0.1% x20 outliers), for one instruction with
a zero accumulator and for the d = 128 chain of two (bound: the sum of the
two instructions' terms), and fails if the hardware exceeds the model.  It
prints the measured ratios, and the ratio to sum_k |a_k b_k| for reference.

The bf16 instruction (v_mfma_f32_32x32x16_bf16) is measured against the
same kind of model for reference (its products are exact in binary32).

A layout check comes first: small-integer operands, whose products and
sums are exact in fp32, must give D exactly; that fixes which operand
element meets which, independently of any rounding.
"""

import numpy as np
import pytest

from oracle import bf16_bits_to_float64, e4m3fn_bits_to_float64
from parity_common import EPS_BF16_MFMA, EPS_E4M3_MFMA, require_gpu
from workloads import Workload, make_bf16, make_fp8

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -23


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def _mfma(dtype, a, b, c):
    import microbench
    return microbench.mfma_one(dtype, a, b, c).astype(np.float64)


def _e4m3_rows(wid, rows, outliers, d=64):
    """``rows`` e4m3 code rows of length d from the fp8 workload recipe:
    the q and k tensors of a [1][rows/4][4][d] workload."""
    w = Workload("mfma_acc", wid, 1, 4, rows // 4, d, "fp8", (False,), outliers=outliers)
    x = make_fp8(w)
    return x["q"].reshape(rows, d), x["k"].reshape(rows, d)


def _binade(x):
    """2^floor(log2 x) for x > 0 (1 where x is 0: no products, no error)."""
    return np.where(x > 0, 2.0 ** np.floor(np.log2(np.where(x > 0, x, 1.0))), 1.0)


def _check(label, d_gpu, exact, scale_ref, absprod, c, eps):
    """scale_ref: the model's per-output unit (2^e, or a sum of them for a
    chain)."""
    fp32_part = U32 * (np.abs(c) + np.abs(exact))
    excess = np.maximum(np.abs(d_gpu - exact) - fp32_part, 0.0)
    ratio = excess / scale_ref
    by_sum = np.abs(d_gpu - exact) / np.maximum(absprod, 1e-300)
    print("%s: max (|D - exact| - fp32 terms) / 2^e = %.3e (= 2^%.2f; 99.99th percentile "
          "%.3e) over %d outputs; model constant %.3e; for reference max |D - exact| / "
          "sum|a b| = %.3e"
          % (label, ratio.max(), np.log2(max(ratio.max(), 1e-30)), np.quantile(ratio, 0.9999),
             ratio.size, eps, by_sum.max()), flush=True)
    assert ratio.max() <= eps, label


def test_layout_exact_on_small_integers():
    rng = np.random.default_rng(11)
    n = 16
    # e4m3 codes of the integers -3..3 (exact), sums far below 2^24
    ints = np.array([-3, -2, -1, 0, 1, 2, 3])
    code_of = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44}
    ia = rng.choice(ints, size=(n, 32, 64))
    ib = rng.choice(ints, size=(n, 32, 64))

    def enc(v):
        c = np.vectorize(lambda t: code_of[abs(int(t))] | (0x80 if t < 0 else 0))(v)
        return c.astype(np.uint8)
    a, b = enc(ia), enc(ib)
    assert np.array_equal(e4m3fn_bits_to_float64(a), ia.astype(np.float64))
    c = rng.integers(-100, 100, size=(n, 32, 32)).astype(np.float32)
    d = _mfma("e4m3", a, b, c)
    exact = np.einsum("pmk,pnk->pmn", ia.astype(np.float64), ib.astype(np.float64)) + c
    assert np.array_equal(d, exact)
    # bf16: integers are exact too
    ia16 = rng.integers(-8, 8, size=(n, 32, 16))
    ib16 = rng.integers(-8, 8, size=(n, 32, 16))
    to_bits = lambda v: (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    d16 = _mfma("bf16", to_bits(ia16), to_bits(ib16), c)
    exact16 = np.einsum("pmk,pnk->pmn", ia16.astype(np.float64), ib16.astype(np.float64)) + c
    assert np.array_equal(d16, exact16)


@pytest.mark.parametrize("outliers", [False, True])
def test_e4m3_single_instruction(outliers):
    n = 1024
    qa, kb = _e4m3_rows(101 + outliers, n * 32, outliers)
    a, b = kb.reshape(n, 32, 64), qa.reshape(n, 32, 64)
    fa, fb = e4m3fn_bits_to_float64(a), e4m3fn_bits_to_float64(b)
    c = np.zeros((n, 32, 32), dtype=np.float32)
    d = _mfma("e4m3", a, b, c)
    exact = np.einsum("pmk,pnk->pmn", fa, fb)
    absprod = np.einsum("pmk,pnk->pmn", np.abs(fa), np.abs(fb))
    pmax = np.abs(fa[:, :, None, :] * fb[:, None, :, :]).max(-1)
    _check("e4m3 one MFMA, outliers=%d" % outliers, d, exact, _binade(pmax), absprod, c,
           EPS_E4M3_MFMA)


@pytest.mark.parametrize("outliers", [False, True])
def test_e4m3_d128_chain(outliers):
    # the d = 128 score: two instructions, the second accumulating onto the
    # first's fp32 result, as in the kernels' S^T = K Q^T
    n = 1024
    qa, kb = _e4m3_rows(103 + outliers, n * 32, outliers, d=128)
    a, b = kb.reshape(n, 32, 128), qa.reshape(n, 32, 128)
    fa, fb = e4m3fn_bits_to_float64(a), e4m3fn_bits_to_float64(b)
    zero = np.zeros((n, 32, 32), dtype=np.float32)
    d1 = _mfma("e4m3", np.ascontiguousarray(a[:, :, :64]), np.ascontiguousarray(b[:, :, :64]),
               zero)
    d2 = _mfma("e4m3", np.ascontiguousarray(a[:, :, 64:]), np.ascontiguousarray(b[:, :, 64:]),
               d1.astype(np.float32))
    exact = np.einsum("pmk,pnk->pmn", fa, fb)
    absprod = np.einsum("pmk,pnk->pmn", np.abs(fa), np.abs(fb))
    p1 = np.abs(fa[:, :, None, :64] * fb[:, None, :, :64]).max(-1)
    p2 = np.abs(fa[:, :, None, 64:] * fb[:, None, :, 64:]).max(-1)
    # the chain's fp32 terms: one rounding of d1 and one of d2
    _check("e4m3 d=128 chain, outliers=%d" % outliers, d2, exact, _binade(p1) + _binade(p2),
           absprod, np.abs(d1) + np.abs(d1), EPS_E4M3_MFMA)


def test_bf16_single_instruction():
    n = 256
    w = Workload("mfma_acc16", 105, 1, 4, n * 32 // 4, 16, "bf16", (False,))
    x = make_bf16(w)
    a, b = x["k"].reshape(n, 32, 16), x["q"].reshape(n, 32, 16)
    fa, fb = bf16_bits_to_float64(a), bf16_bits_to_float64(b)
    c = np.zeros((n, 32, 32), dtype=np.float32)
    d = _mfma("bf16", a, b, c)
    exact = np.einsum("pmk,pnk->pmn", fa, fb)
    absprod = np.einsum("pmk,pnk->pmn", np.abs(fa), np.abs(fb))
    pmax = np.abs(fa[:, :, None, :] * fb[:, None, :, :]).max(-1)
    _check("bf16 one MFMA", d, exact, _binade(pmax), absprod, c, EPS_BF16_MFMA)
