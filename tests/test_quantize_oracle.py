"""Pins of the E4M3 quantisation oracle (oracle/quantize.py): the encoder
against the format's own decoder and torch's conversion, the Hadamard
transform against its closed form, the rotation's invariance of the scores,
the unrotated quantiser against the input generator's (torch) one, and, on
real (non-integer) bf16 inputs, the binary32 butterfly and the codes against
the exact fp64 rotation within the derived rounding bound."""

import math

import numpy as np
import pytest
import torch

from oracle import (e4m3fn_bits_to_float64, e4m3fn_encode, fwht32, hadamard, quantize_e4m3)
from workloads import Workload, make_fp8


def test_encoder_round_trips_every_finite_code():
    c = np.arange(256, dtype=np.uint8)
    v = e4m3fn_bits_to_float64(c)
    ok = ~np.isnan(v)
    assert np.array_equal(e4m3fn_encode(v[ok]), c[ok])


def test_encoder_matches_torch_on_a_sweep_and_on_every_tie():
    x = np.linspace(-448.0, 448.0, 400001).astype(np.float32)
    grid = np.sort(e4m3fn_bits_to_float64(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)     # exact ties (binary32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3fn_encode(x.astype(np.float64)), ref)


def test_encoder_saturates_and_maps_nan():
    assert e4m3fn_encode(np.array([1e6]))[0] == 0x7E
    assert e4m3fn_encode(np.array([-500.0]))[0] == 0xFE
    assert e4m3fn_encode(np.array([np.nan]))[0] == 0x7F


def test_hadamard_closed_form_and_orthogonality():
    for d in (2, 8, 64, 128):
        h = hadamard(d)
        assert np.array_equal(h @ h.T, d * np.eye(d))
        assert np.array_equal(h, h.T)
        assert h[0].tolist() == [1.0] * d and h[:, 0].tolist() == [1.0] * d


def test_fast_transform_equals_matrix_product():
    # integer inputs keep every butterfly exact in binary32
    rng = np.random.default_rng(3)
    x = rng.integers(-50, 50, size=(7, 128)).astype(np.float32)
    assert np.array_equal(fwht32(x).astype(np.float64), x.astype(np.float64) @ hadamard(128))


def test_rotation_leaves_scores_unchanged():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((9, 64)), rng.standard_normal((11, 64))
    s = np.where(rng.integers(0, 2, 64) == 1, -1.0, 1.0)
    m = np.diag(s) @ hadamard(64) / math.sqrt(64)
    assert np.allclose((q @ m) @ (k @ m).T, q @ k.T, atol=1e-12)


def test_unrotated_quantiser_matches_the_input_generator():
    # the generator quantises binary32 N(0,1) (with x20 outliers) with torch;
    # the oracle, given the same binary32 values, must produce the same codes
    w = Workload("q", 91, 2, 3, 50, 64, "fp8", (False,), outliers=True)
    gen = make_fp8(w)
    from workloads import _randn, _perm_prefix, seed_for
    x = _randn((2, 50, 3, 64), seed_for(w.wid, 0))
    idx = _perm_prefix(x.numel(), int(round(0.001 * x.numel())), seed_for(w.wid, 4))
    x.view(-1)[idx] *= 20.0
    codes, ds = quantize_e4m3(x.numpy().astype(np.float64))
    assert np.array_equal(codes, gen["q"])
    assert np.allclose(ds, gen["dq"], rtol=0, atol=0)


def test_rotated_quantisation_reconstructs_the_rotated_rows():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 40, 2, 128)).astype(np.float32).astype(np.float64)
    s = np.where(rng.integers(0, 2, 128) == 1, -1.0, 1.0)
    codes, ds = quantize_e4m3(x, s)
    m = np.diag(s) @ hadamard(128) / math.sqrt(128)
    for h in range(2):
        rot = x[0, :, h, :] @ m
        deq = e4m3fn_bits_to_float64(codes[0, :, h, :]) * float(ds[0, h])
        step = np.abs(rot).max() * 2.0 ** -4 * 1.01          # half an E4M3 step at the top
        assert np.abs(deq - rot).max() <= step


# ---------------------------------------------------------------------------
# the binary32 butterfly and the codes against the exact rotation
# ---------------------------------------------------------------------------
#
# On bf16 inputs the exact y = x diag(s) H_d is exact in fp64 (sums of d
# values with 8-bit significands over a bounded exponent range), so it is the
# reference.  The butterfly has m = log2(d) stages, each output the rounded
# sum or difference of two values of the previous stage.  With u = 2^-24 and
# the stages' absolute-value matrices multiplying to the all-ones matrix,
# rounding errors add up to at most
#     |fwht32(x s)_j - y_j| <= m u (1 + u)^m sum_i |x_i|        (every j).
# The codes may then differ from the e4m3 rounding of the exact y / (amax /
# 448) only where that exact value lies within the propagated bound of a
# rounding boundary (a midpoint of the e4m3 grid), and by one grid step.

U = 2.0 ** -24


def _real_inputs(d, rows, wid):
    from workloads import make_bf16
    from oracle import bf16_bits_to_float64
    w = Workload("qpin", wid, 1, rows // 4, 4, d, "bf16", (False,), outliers=True)
    x = bf16_bits_to_float64(make_bf16(w)["q"])          # [1][4][rows/4][d] as [B][N][H][d]
    return x


def _signs(d, seed):
    rng = np.random.default_rng(seed)
    return np.where(rng.integers(0, 2, d) == 1, -1.0, 1.0)


def _butterfly_bound(x):
    m = int(round(math.log2(x.shape[-1])))
    return m * U * (1.0 + U) ** m * np.abs(x).sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("d", [64, 128])
def test_butterfly_within_rounding_bound_of_exact_rotation(d):
    x = _real_inputs(d, 512, 93 + d)
    assert not np.array_equal(x, np.round(x))           # real, non-integer values
    s = _signs(d, 7 + d)
    exact = (x * s) @ hadamard(d)
    got = fwht32((x * s).astype(np.float32)).astype(np.float64)
    err = np.abs(got - exact)
    bound = _butterfly_bound(x)
    assert (err <= bound).all()
    # the rounding is real: a transform without it would not be tested
    assert err.max() > 0


@pytest.mark.parametrize("d", [64, 128])
def test_butterfly_bound_catches_a_mis_rounded_stage(d):
    # a butterfly whose middle stage rounds to bf16 instead of binary32 (a
    # plausible slip) breaks the bound on these inputs
    x = _real_inputs(d, 512, 95 + d)
    s = _signs(d, 9 + d)
    y = (x * s).astype(np.float32)
    h, stage = 1, 0
    while h < d:
        z = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = z[..., 0, :], z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(y.shape)
        if stage == 2:
            y = torch.from_numpy(y).to(torch.bfloat16).to(torch.float32).numpy()
        h, stage = 2 * h, stage + 1
    err = np.abs(y.astype(np.float64) - (x * s) @ hadamard(d))
    assert (err > _butterfly_bound(x)).any()


def _e4m3_grid():
    g = e4m3fn_bits_to_float64(np.arange(0, 0x7F, dtype=np.uint8))
    return np.sort(np.concatenate([-g[1:], g]))          # every finite value, ascending


@pytest.mark.parametrize("rot", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_codes_follow_the_exact_rotation(d, rot):
    x = _real_inputs(d, 1024, 97 + d)                    # [1][N][H][d]
    s = _signs(d, 11 + d) if rot else None
    codes, ds = quantize_e4m3(x, s)
    grid = _e4m3_grid()
    H = x.shape[2]
    for h in range(H):
        xh = x[0, :, h, :]
        y = (xh * s) @ hadamard(d) if rot else xh.copy()
        beta = _butterfly_bound(xh) if rot else np.zeros((xh.shape[0], 1))
        amax = np.abs(y).max()
        ds_exact = amax / 448.0
        # descale: fl(fl(amax32) / 448) (rotated: times fl(1/sqrt(d)), rounded)
        rho = beta.max() / amax + 2 * U
        want = ds_exact / math.sqrt(d) if rot else ds_exact
        assert abs(float(ds[0, h]) - want) <= want * (rho + (3 * U if rot else 0.0))
        v = y / ds_exact
        dv = beta / ds_exact * (1 + 2 * rho) + np.abs(v) * (rho + U) * (1 + 2 * rho)
        c = codes[0, :, h, :]
        got = e4m3fn_bits_to_float64(c)
        ref = e4m3fn_bits_to_float64(e4m3fn_encode(np.clip(v, -448.0, 448.0)))
        diff = got != ref
        # the rounding bound is far below an e4m3 step: codes of the exact
        # rotation and the oracle's binary32 ones almost always coincide
        # (none differ on these inputs)
        assert diff.mean() < 1e-3
        for i, j in zip(*np.nonzero(diff)):
            gi = np.searchsorted(grid, got[i, j])
            ri = np.searchsorted(grid, ref[i, j])
            assert abs(gi - ri) == 1                    # one grid step apart
            mid = 0.5 * (got[i, j] + ref[i, j])
            assert abs(v[i, j] - mid) <= dv[i, j]       # the exact value sits at the boundary
