"""Pins of the E4M3 quantisation oracle (oracle/quantize.py): the encoder
against the format's own decoder and torch's conversion, the Hadamard
transform against its closed form, the rotation's invariance of the scores,
and the unrotated quantiser against the input generator's (torch) one."""

import math

import numpy as np
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
