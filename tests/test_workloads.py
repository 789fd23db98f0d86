"""The seeded input generator: reproducible, right shapes and structure."""

import numpy as np
import torch

from oracle import bf16_bits_to_float64, dequantize_e4m3
from workloads import WORKLOADS, Workload, make_bf16, make_fp8, sample_rows, make_inputs


def test_bf16_inputs_are_seeded_and_shaped():
    w = WORKLOADS["tiny"]
    a = make_bf16(w)
    b = make_bf16(w)
    for name in "qkv":
        assert a[name].dtype == np.uint16
        assert a[name].shape == (w.B, w.N, w.H, w.d)
        np.testing.assert_array_equal(a[name], b[name])
    assert not np.array_equal(a["q"], a["k"])
    x = bf16_bits_to_float64(a["q"])
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05


def test_peaked_rows_are_one_percent_times_eight():
    w = Workload("peak", 99, 1, 2, 1000, 16, "bf16", (True,), peaked_k=True)
    base = Workload("plain", 99, 1, 2, 1000, 16, "bf16", (True,))
    kp = bf16_bits_to_float64(make_bf16(w)["k"])
    k0 = bf16_bits_to_float64(make_bf16(base)["k"])
    for h in range(2):
        ratio = np.abs(kp[0, :, h, :]).sum(1) / np.abs(k0[0, :, h, :]).sum(1)
        peaked = np.isclose(ratio, 8.0, rtol=1e-2)
        assert peaked.sum() == 10
        assert np.allclose(ratio[~peaked], 1.0)


def test_fp8_inputs_use_range_and_outliers():
    w = Workload("f8", 98, 1, 2, 512, 32, "fp8", (False,), outliers=True)
    a = make_fp8(w)
    b = make_fp8(w)
    for name in "qkv":
        assert a[name].dtype == np.uint8 and a[name].shape == (1, 512, 2, 32)
        assert a["d" + name].shape == (1, 2) and a["d" + name].dtype == np.float32
        np.testing.assert_array_equal(a[name], b[name])
        codes = torch.from_numpy(a[name]).view(torch.float8_e4m3fn).float()
        assert not torch.isnan(codes).any()
        # the per-(b,h) amax maps to (close to) the top of the e4m3 range
        for h in range(2):
            assert codes[0, :, h, :].abs().max().item() >= 416.0
        x = dequantize_e4m3(a[name], a["d" + name])
        # about 0.1% outliers of ~20 sigma
        assert (np.abs(x) > 8.0).sum() >= 0.0005 * x.size


def test_row_sample_includes_ends_and_is_distinct():
    w = WORKLOADS["long8k"]
    r = sample_rows(w)
    assert r.shape == (w.B, w.H, 512)
    for b in range(w.B):
        for h in range(w.H):
            assert r[b, h, 0] == 0 and r[b, h, 1] == w.N - 1
            assert len(np.unique(r[b, h])) == 512
            assert r[b, h].min() >= 0 and r[b, h].max() < w.N
    np.testing.assert_array_equal(r, sample_rows(w))
    small = sample_rows(WORKLOADS["tiny"])
    assert small.shape == (1, 2, 128)


def test_grouped_query_shapes():
    w = Workload("g", 95, 2, 8, 40, 64, "bf16", (True,), Hkv=2)
    x = make_inputs(w)
    assert x["q"].shape == (2, 40, 8, 64)
    assert x["k"].shape == x["v"].shape == (2, 40, 2, 64)
    w8 = Workload("g8", 96, 2, 8, 40, 64, "fp8", (False,), Hkv=4, outliers=True)
    x8 = make_inputs(w8)
    assert x8["dq"].shape == (2, 8) and x8["dk"].shape == (2, 4) and x8["dv"].shape == (2, 4)


def test_varlen_layout_and_offsets():
    w = WORKLOADS["varlen"]
    assert w.lengths[0] == 8192 and w.lengths[1] == 1 and len(w.lengths) == w.B
    assert all(1 <= n <= 8192 for n in w.lengths) and w.N == max(w.lengths)
    assert w.flops(True) == sum(2.0 * w.H * n * n * w.d for n in w.lengths)
    small = Workload("v", 97, 3, 4, 9, 64, "fp8", (False,), Hkv=2, lengths=(9, 0, 4),
                     outliers=True)
    x = make_inputs(small)
    assert list(x["cu"]) == [0, 9, 9, 13]
    assert x["q"].shape == (1, 13, 4, 64) and x["k"].shape == (1, 13, 2, 64)
    assert x["dq"].shape == (3, 4) and x["dk"].shape == (3, 2)
    # per-sequence descale: every sequence's largest code magnitude is the
    # e4m3 maximum (448 = code 0x7e with the sign bit cleared)
    for b, (s0, s1) in enumerate([(0, 9), (9, 9), (9, 13)]):
        if s1 > s0:
            for h in range(4):
                assert (x["q"][0, s0:s1, h] & 0x7F).max() == 0x7E


def test_rotation_signs_and_bits_agree():
    from workloads import rotation_signs
    w = WORKLOADS["fp8_8k"]
    s, words = rotation_signs(w)
    assert s.shape == (w.d,) and words.shape == (w.d // 32,) and words.dtype == np.uint32
    bits = np.array([(int(words[i // 32]) >> (i % 32)) & 1 for i in range(w.d)])
    assert np.array_equal(bits == 1, s < 0)
    assert 0.3 < np.mean(s < 0) < 0.7
    s2, words2 = rotation_signs(w)
    assert np.array_equal(s, s2) and np.array_equal(words, words2)


def test_bf16_source_of_outlier_workload_has_the_outliers():
    # the bf16 input of an outlier workload carries the x20 outliers at the
    # same positions as the fp8 workload's float32 draws
    from workloads import make_bf16
    w = Workload("o", 98, 1, 2, 500, 64, "fp8", (False,), outliers=True)
    plain = Workload("p", 98, 1, 2, 500, 64, "bf16", (False,))
    a = bf16_to_f32(make_bf16(w)["k"])
    b = bf16_to_f32(make_bf16(plain)["k"])
    changed = a != b
    assert changed.sum() == round(0.001 * a.size)
    assert np.allclose(a[changed], 20 * b[changed], rtol=1e-2)


def bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)
