"""Accuracy of single gfx950 matrix-core instructions against the exact dot
products, on the attention kernels' own operand distributions.

Why: the fp8 forward's scores are sums of e4m3 products accumulated by
v_mfma_f32_32x32x64_f8f6f4 (64 products per instruction, d/64 instructions
chained through the fp32 accumulator), and the fp8 LSE tolerance in
parity_common.py is derived from this instruction's error model:

    |D - D_exact| <= EPS_E4M3_MFMA * sum_k |a_k b_k| + 2^-23 * (|C| + |D_exact|)

(the second term is ordinary binary32 rounding of the accumulator).  The
model's constant EPS_E4M3_MFMA is the largest ratio
|D - D_exact - (fp32 terms)| / sum_k |a_k b_k| seen on these operands,
rounded up to a power of two.  This test measures it on seeded e4m3 codes
drawn as the fp8 workloads draw them (N(0,1), per-block amax / 448
quantisation, with and without 0.1% x20 outliers), for one instruction with
a zero accumulator and for the d = 128 chain of two, and fails if the
model's constant does not cover what the hardware does.  It prints the
measured ratios.

The bf16 instruction (v_mfma_f32_32x32x16_bf16) is measured the same way
for reference (its products are exact in binary32).

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


def _check(label, d_gpu, exact, absprod, c, eps):
    fp32_part = U32 * (np.abs(c) + np.abs(exact))
    excess = np.maximum(np.abs(d_gpu - exact) - fp32_part, 0.0)
    ratio = excess / np.maximum(absprod, 1e-300)
    raw = np.abs(d_gpu - exact) / np.maximum(absprod, 1e-300)
    print("%s: max |D - exact| / sum|a b| = %.3e (after the fp32 terms %.3e, = 2^%.2f); "
          "model constant %.3e" % (label, raw.max(), ratio.max(), np.log2(max(ratio.max(), 1e-30)),
                                   eps), flush=True)
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
    n = 256
    qa, kb = _e4m3_rows(101 + outliers, n * 32, outliers)
    a, b = kb.reshape(n, 32, 64), qa.reshape(n, 32, 64)
    fa, fb = e4m3fn_bits_to_float64(a), e4m3fn_bits_to_float64(b)
    c = np.zeros((n, 32, 32), dtype=np.float32)
    d = _mfma("e4m3", a, b, c)
    exact = np.einsum("pmk,pnk->pmn", fa, fb)
    absprod = np.einsum("pmk,pnk->pmn", np.abs(fa), np.abs(fb))
    _check("e4m3 one MFMA, outliers=%d" % outliers, d, exact, absprod, c, EPS_E4M3_MFMA)


@pytest.mark.parametrize("outliers", [False, True])
def test_e4m3_d128_chain(outliers):
    # the d = 128 score: two instructions, the second accumulating onto the
    # first's fp32 result, as in the kernels' S^T = K Q^T
    n = 256
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
    # the chain's fp32 terms: one rounding of d1 and one of d2
    _check("e4m3 d=128 chain, outliers=%d" % outliers, d2, exact, absprod,
           np.abs(d1) + np.abs(d1), EPS_E4M3_MFMA)


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
    _check("bf16 one MFMA", d, exact, absprod, c, EPS_BF16_MFMA)
