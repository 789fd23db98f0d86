"""Pins for the CPU oracle: each test checks it against something other than
itself (closed forms, a textbook special case, brute force, invariants of
the definition, the tiled recurrence, library decoders, page-given counts).

The definition being pinned is softmax(Q K^T * scale) V with a per-row
natural-log log-sum-exp, on [B][N][H][d] tensors ("FlashAttention-4 no
Blackwell B200 ...", section "Por que o Blackwell exige mais do que
multiplicações rápidas"; layout from the usage example of "FlashAttention-3:
Pipeline Assíncrono ...", section "Implementando FlashAttention-3 em
produção").
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attention_backward, attention_brute, attention_delta, attention_forward,
                    attention_forward_gqa,
                    attention_forward_varlen, attention_head_rows,
                    bf16_bits_to_float64, dequantize_e4m3, e4m3fn_bits_to_float64,
                    simulator_counts, tiled_online_softmax_head)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_mean_of_visible_values(causal):
    """Q = 0: every visible score is 0, so o_i is the plain mean of the
    visible v_j and lse_i = ln(number of visible keys)."""
    B, N, H, d = 2, 37, 3, 8
    q = np.zeros((B, N, H, d))
    k = _rand((B, N, H, d), 1)
    v = _rand((B, N, H, d), 2)
    o, lse = attention_forward(q, k, v, 0.3, causal)
    for i in range(N):
        n_vis = i + 1 if causal else N
        np.testing.assert_allclose(o[:, i], v[:, :n_vis].mean(axis=1), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], math.log(n_vis), rtol=0, atol=1e-13)


def test_equal_key_rows_give_mean_and_shifted_lse():
    """All K rows equal: row i's scores all equal s_i = scale*q_i.k, so
    o_i = mean of V over keys and lse_i = s_i + ln N."""
    B, N, H, d = 1, 29, 2, 16
    q = _rand((B, N, H, d), 3)
    krow = _rand((B, 1, H, d), 4)
    k = np.repeat(krow, N, axis=1)
    v = _rand((B, N, H, d), 5)
    scale = 0.25
    o, lse = attention_forward(q, k, v, scale, False)
    for b in range(B):
        for h in range(H):
            s = scale * q[b, :, h, :] @ krow[b, 0, h, :]
            np.testing.assert_allclose(lse[b, h], s + math.log(N), rtol=0, atol=1e-12)
            np.testing.assert_allclose(o[b, :, h, :], np.broadcast_to(v[b, :, h, :].mean(0), (N, d)),
                                       rtol=0, atol=1e-13)


def test_single_dominant_key_returns_its_value_row():
    """k_{j*} = lambda * q_i with lambda large: o_i -> v_{j*}; the error is at
    most (n-1) * exp(-margin) * 2 max|v| where margin is the score gap."""
    N, d = 64, 32
    rng = np.random.default_rng(6)
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d)) * 0.1
    v = rng.standard_normal((N, d))
    i, jstar = 17, 41
    k[jstar] = 12.0 * q[i]
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_head_rows(q, k, v, scale, False, rows=[i])
    s = scale * (k @ q[i])
    margin = s[jstar] - np.max(np.delete(s, jstar))
    assert margin > 30
    bound = (N - 1) * math.exp(-margin) * 2 * np.abs(v).max()
    assert np.abs(o[0] - v[jstar]).max() <= bound + 1e-15
    assert abs(lse[0] - s[jstar]) <= (N - 1) * math.exp(-margin) + 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    """With V = all ones, o_i = sum_j p_ij = 1; and sum_j exp(s_ij - lse_i) = 1
    over the visible keys (ties lse to the scores)."""
    B, N, H, d = 1, 50, 2, 8
    q = _rand((B, N, H, d), 7, 2.0)
    k = _rand((B, N, H, d), 8, 2.0)
    o, lse = attention_forward(q, k, np.ones((B, N, H, d)), 0.7, causal)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)
    for h in range(H):
        for i in range(N):
            js = range(i + 1) if causal else range(N)
            tot = math.fsum(math.exp(0.7 * float(q[0, i, h] @ k[0, j, h]) - lse[0, h, i]) for j in js)
            assert abs(tot - 1.0) < 1e-13


def test_causal_row_zero_is_first_value_row():
    """Causal: query 0 sees only key 0, so o_0 = v_0 exactly and
    lse_0 = scale * q_0 . k_0."""
    B, N, H, d = 2, 20, 3, 16
    q = _rand((B, N, H, d), 9)
    k = _rand((B, N, H, d), 10)
    v = _rand((B, N, H, d), 11)
    o, lse = attention_forward(q, k, v, 0.125, True)
    np.testing.assert_array_equal(o[:, 0], v[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.125 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]),
                               rtol=0, atol=1e-14)


def test_two_keys_logistic_weights():
    """N = 2, non-causal: the weights are logistic functions of the score
    difference, o_i = sigma(s_i0 - s_i1) v_0 + sigma(s_i1 - s_i0) v_1."""
    N, d = 2, 8
    q = _rand((N, d), 12, 3.0)
    k = _rand((N, d), 13, 3.0)
    v = _rand((N, d), 14)
    scale = 0.4
    o, lse = attention_head_rows(q, k, v, scale, False)
    for i in range(N):
        s0 = scale * q[i] @ k[0]
        s1 = scale * q[i] @ k[1]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        np.testing.assert_allclose(o[i], w0 * v[0] + w1 * v[1], rtol=0, atol=1e-14)
        assert abs(lse[i] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-14


def test_huge_scale_is_hard_argmax():
    """scale -> large: the softmax becomes a one-hot on each row's best key."""
    N, d = 40, 8
    q = _rand((N, d), 15)
    k = _rand((N, d), 16)
    v = _rand((N, d), 17)
    o, _ = attention_head_rows(q, k, v, 1e4, False)
    best = np.argmax(q @ k.T, axis=1)
    np.testing.assert_allclose(o, v[best], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 5, 2, 3), (2, 16, 2, 8), (1, 13, 3, 4)])
def test_brute_force_agrees(shape, causal):
    q = _rand(shape, 18, 1.5)
    k = _rand(shape, 19, 1.5)
    v = _rand(shape, 20)
    scale = 1.0 / math.sqrt(shape[3])
    o, lse = attention_forward(q, k, v, scale, causal)
    ob, lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_key_value_permutation_invariance():
    """Non-causal attention does not depend on the order of the key/value
    rows (permuting K and V together)."""
    B, N, H, d = 1, 33, 2, 8
    q, k, v = (_rand((B, N, H, d), s) for s in (21, 22, 23))
    perm = np.random.default_rng(24).permutation(N)
    o1, l1 = attention_forward(q, k, v, 0.5, False)
    o2, l2 = attention_forward(q, k[:, perm], v[:, perm], 0.5, False)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_linear_in_values(causal):
    B, N, H, d = 1, 24, 2, 8
    q, k, v1, v2 = (_rand((B, N, H, d), s) for s in (25, 26, 27, 28))
    o1, _ = attention_forward(q, k, v1, 0.5, causal)
    o2, _ = attention_forward(q, k, v2, 0.5, causal)
    o3, _ = attention_forward(q, k, 2.0 * v1 - 3.0 * v2, 0.5, causal)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_convexity_and_lse_bounds(causal):
    """Each o_i lies between the column-wise min and max of the visible v_j,
    and max_j s_ij <= lse_i <= max_j s_ij + ln(n_visible)."""
    B, N, H, d = 1, 40, 2, 8
    q, k, v = (_rand((B, N, H, d), s, 2.0) for s in (29, 30, 31))
    scale = 0.5
    o, lse = attention_forward(q, k, v, scale, causal)
    for h in range(H):
        s = scale * q[0, :, h] @ k[0, :, h].T
        for i in range(N):
            n = i + 1 if causal else N
            vis = v[0, :n, h]
            assert np.all(o[0, i, h] >= vis.min(0) - 1e-13)
            assert np.all(o[0, i, h] <= vis.max(0) + 1e-13)
            smax = s[i, :n].max()
            assert smax - 1e-13 <= lse[0, h, i] <= smax + math.log(n) + 1e-13


def test_row_shift_invariance():
    """Adding the same amount to every score of a row (k_j -> k_j + u) leaves
    o_i unchanged and shifts lse_i by scale * q_i . u."""
    B, N, H, d = 1, 30, 1, 8
    q, k, v = (_rand((B, N, H, d), s) for s in (32, 33, 34))
    u = _rand((d,), 35)
    scale = 0.6
    o1, l1 = attention_forward(q, k, v, scale, False)
    o2, l2 = attention_forward(q, k + u, v, scale, False)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, scale * (q[0, :, 0] @ u)[None, None, :], rtol=0, atol=1e-12)


def test_heads_and_batches_are_independent_in_bnhd_layout():
    """Swapping two heads (axis 2) and two batches (axis 0) of Q, K, V swaps
    the same slices of O and LSE; N is axis 1."""
    B, N, H, d = 2, 18, 3, 8
    q, k, v = (_rand((B, N, H, d), s) for s in (36, 37, 38))
    o, lse = attention_forward(q, k, v, 0.5, True)
    hp = [2, 0, 1]
    bp = [1, 0]
    o2, lse2 = attention_forward(q[bp][:, :, hp], k[bp][:, :, hp], v[bp][:, :, hp], 0.5, True)
    np.testing.assert_allclose(o2, o[bp][:, :, hp], rtol=0, atol=0)
    np.testing.assert_allclose(lse2, lse[bp][:, hp], rtol=0, atol=0)


def test_row_subset_matches_full():
    B, N, H, d = 1, 70, 2, 8
    q, k, v = (_rand((B, N, H, d), s) for s in (39, 40, 41))
    o, lse = attention_forward(q, k, v, 0.3, True)
    rows = np.array([[[0, 69, 5, 33], [12, 1, 68, 40]]])
    orow, lrow = attention_forward(q, k, v, 0.3, True, rows=rows)
    for h in range(H):
        np.testing.assert_allclose(orow[0, h], o[0, rows[0, h], h], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lrow[0, h], lse[0, h, rows[0, h]], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# tiled recurrence (exactness of the online softmax)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bk", [1, 7, 32, 64])
@pytest.mark.parametrize("tau", [0.0, 8.0 * math.log(2.0), math.inf])
def test_tiled_equals_untiled(causal, bk, tau):
    N, d = 150, 16
    q, k, v = (_rand((N, d), s, 1.5) for s in (42, 43, 44))
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_head_rows(q, k, v, scale, causal)
    ot, lt, _ = tiled_online_softmax_head(q, k, v, scale, causal, 32, bk, tau)
    np.testing.assert_allclose(ot, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lt, lse, rtol=0, atol=1e-12)


def test_threshold_reduces_rescales_on_peaked_keys():
    """Informative (the pages report ~10x fewer rescales for the adaptive
    rule); here only the direction is asserted: a positive threshold never
    rescales more often than the always-rescale rule."""
    N, d = 1024, 32
    rng = np.random.default_rng(45)
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    k[rng.choice(N, 10, replace=False)] *= 8.0
    v = rng.standard_normal((N, d))
    scale = 1.0 / math.sqrt(d)
    _, _, s0 = tiled_online_softmax_head(q, k, v, scale, True, 128, 64, 0.0)
    _, _, s8 = tiled_online_softmax_head(q, k, v, scale, True, 128, 64, 8.0 * math.log(2.0))
    assert s8["rescales"] <= s0["rescales"]
    assert s0["rescales"] > 0


def test_simulator_counts_match_page():
    with open(os.path.join(GOLDEN, "simulator_counts.json")) as f:
        g = json.load(f)
    got = simulator_counts(**g["inputs"])
    assert got == g["expected"]


# --------------------------------------------------------------------------
# input-format decoders
# --------------------------------------------------------------------------

def test_e4m3_decoder_matches_library_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_bits_to_float64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], lib[~nan])


def test_e4m3_decoder_known_values():
    vals = e4m3fn_bits_to_float64(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0xB8, 0x7E, 0xFE, 0x7F, 0x80],
                                           dtype=np.uint8))
    exp = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, -1.0, 448.0, -448.0]
    np.testing.assert_array_equal(vals[:8], exp)
    assert np.isnan(vals[8])
    assert vals[9] == 0.0 and math.copysign(1.0, vals[9]) == -1.0


def test_bf16_decoder_matches_library():
    bits = np.random.default_rng(46).integers(0, 1 << 16, 4096, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]           # drop inf/nan patterns
    ours = bf16_bits_to_float64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, lib)
    one = bf16_bits_to_float64(np.array([0x3F80, 0xC000, 0x0000], dtype=np.uint16))
    np.testing.assert_array_equal(one, [1.0, -2.0, 0.0])


def test_dequantize_uses_per_batch_head_descale():
    B, N, H, d = 2, 3, 2, 4
    codes = np.full((B, N, H, d), 0x38, dtype=np.uint8)     # 1.0
    ds = np.array([[0.5, 2.0], [3.0, 0.25]], dtype=np.float32)
    x = dequantize_e4m3(codes, ds)
    for b in range(B):
        for h in range(H):
            assert np.all(x[b, :, h, :] == ds[b, h])


# ---------------------------------------------------------------------------
# grouped-query and variable-length forms
# ---------------------------------------------------------------------------

def _rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_with_all_heads_is_plain_attention(causal):
    q, k, v = _rnd((2, 23, 4, 8), 1), _rnd((2, 23, 4, 8), 2), _rnd((2, 23, 4, 8), 3)
    o1, l1 = attention_forward_gqa(q, k, v, 0.4, causal)
    o2, l2 = attention_forward(q, k, v, 0.4, causal)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_mqa_head_is_an_independent_single_head_problem(causal):
    # one K/V head shared by every query head: head h alone, with that K/V,
    # is a one-head problem of the (separately pinned) plain definition
    q, k, v = _rnd((1, 19, 5, 8), 4), _rnd((1, 19, 1, 8), 5), _rnd((1, 19, 1, 8), 6)
    o, lse = attention_forward_gqa(q, k, v, 0.3, causal)
    for h in range(5):
        oh, lh = attention_forward(q[:, :, h:h + 1], k, v, 0.3, causal)
        assert np.allclose(o[:, :, h:h + 1], oh, rtol=0, atol=1e-15)
        assert np.allclose(lse[:, h:h + 1], lh, rtol=0, atol=1e-15)


def test_gqa_head_mapping_closed_form():
    # K/V head j carries the constant value j + 1: every query row of query
    # head h then averages constants, so it returns exactly the value of the
    # K/V head it reads, h // (H / Hkv) + 1 (a modular mapping h % Hkv, or a
    # swapped grouping, gives another number)
    H, Hkv = 8, 2
    q, k = _rnd((1, 9, H, 4), 7), _rnd((1, 9, Hkv, 4), 8)
    v = np.broadcast_to(np.arange(1, Hkv + 1, dtype=np.float64)[None, None, :, None],
                        (1, 9, Hkv, 4)).copy()
    o, _ = attention_forward_gqa(q, k, v, 0.7, True)
    for h in range(H):
        assert np.allclose(o[0, :, h, :], h // (H // Hkv) + 1, rtol=0, atol=1e-14)


def test_gqa_rejects_bad_head_counts():
    with pytest.raises(ValueError):
        attention_forward_gqa(_rnd((1, 4, 6, 4), 1), _rnd((1, 4, 4, 4), 2), _rnd((1, 4, 4, 4), 3),
                              1.0, False)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_of_equal_lengths_is_the_fixed_length_batch(causal):
    B, N, H, Hkv, d = 3, 11, 4, 2, 8
    q, k, v = _rnd((B, N, H, d), 9), _rnd((B, N, Hkv, d), 10), _rnd((B, N, Hkv, d), 11)
    cu = np.arange(B + 1) * N
    o, lse = attention_forward_varlen(q.reshape(B * N, H, d), k.reshape(B * N, Hkv, d),
                                      v.reshape(B * N, Hkv, d), cu, 0.5, causal)
    o2, l2 = attention_forward_gqa(q, k, v, 0.5, causal)
    assert np.allclose(o.reshape(B, N, H, d), o2, rtol=0, atol=1e-15)
    # lse [H][total] against [B][H][N]
    assert np.allclose(lse.reshape(H, B, N).transpose(1, 0, 2), l2, rtol=0, atol=1e-15)


def test_varlen_sequences_do_not_see_each_other():
    # a sequence's output is unchanged when the other sequences' keys and
    # values are replaced; each one equals its own one-sequence problem
    lengths = [5, 1, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, Hkv, d = cu[-1], 2, 1, 4
    q, k, v = _rnd((T, H, d), 12), _rnd((T, Hkv, d), 13), _rnd((T, Hkv, d), 14)
    o, lse = attention_forward_varlen(q, k, v, cu, 0.8, False)
    k2, v2 = k.copy(), v.copy()
    k2[cu[3]:], v2[cu[3]:] = 100.0, -100.0        # alter the last sequence only
    o2, l2 = attention_forward_varlen(q, k2, v2, cu, 0.8, False)
    assert np.array_equal(o[:cu[3]], o2[:cu[3]]) and np.array_equal(lse[:, :cu[3]], l2[:, :cu[3]])
    for b in range(len(lengths)):
        s0, s1 = cu[b], cu[b + 1]
        if s1 == s0:
            continue
        ob, lb = attention_forward_gqa(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], 0.8, False)
        assert np.allclose(o[s0:s1], ob[0], rtol=0, atol=1e-15)
        assert np.allclose(lse[:, s0:s1], lb[0], rtol=0, atol=1e-15)


def test_varlen_causal_first_token_of_each_sequence():
    # causal: the first query of every sequence sees only its own first key,
    # so its output is that key's value row and its lse the single score
    lengths = [3, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = cu[-1], 2, 4
    q, k, v = _rnd((T, H, d), 15), _rnd((T, H, d), 16), _rnd((T, H, d), 17)
    o, lse = attention_forward_varlen(q, k, v, cu, 0.6, True)
    for b in range(len(lengths)):
        t = cu[b]
        assert np.allclose(o[t], v[t], rtol=0, atol=1e-15)
        for h in range(H):
            assert math.isclose(lse[h, t], 0.6 * float(q[t, h] @ k[t, h]), abs_tol=1e-14)


def test_varlen_row_sample_matches_full():
    lengths = [7, 0, 12]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = cu[-1], 3, 4
    q, k, v = _rnd((T, H, d), 18), _rnd((T, 1, d), 19), _rnd((T, 1, d), 20)
    o, lse = attention_forward_varlen(q, k, v, cu, 0.5, True)
    rows = [np.tile(np.array([n - 1, 0][:min(n, 2)]), (H, 1)) for n in lengths]
    os_, ls_ = attention_forward_varlen(q, k, v, cu, 0.5, True, rows=rows)
    for b, n in enumerate(lengths):
        for h in range(H):
            for i, r in enumerate(rows[b][h]):
                assert np.array_equal(os_[b][h, i], o[cu[b] + r, h])
                assert ls_[b][h, i] == lse[h, cu[b] + r]


# ---------------------------------------------------------------------------
# gradients
# ---------------------------------------------------------------------------

def _loss(q, k, v, do, scale, causal):
    o, _ = attention_forward(q, k, v, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences_of_the_forward(causal):
    # L = sum(dO * O(q, k, v)): the analytic gradients against numerical
    # derivatives of the separately pinned forward definition
    B, N, H, d, scale = 1, 6, 2, 4, 0.7
    q, k, v, do = (_rnd((B, N, H, d), s) for s in (21, 22, 23, 24))
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)
    eps = 1e-6
    rng = np.random.default_rng(25)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num = (_loss(args_p["q"], args_p["k"], args_p["v"], do, scale, causal) -
                   _loss(args_m["q"], args_m["k"], args_m["v"], do, scale, causal)) / (2 * eps)
            assert math.isclose(g[idx], num, rel_tol=1e-6, abs_tol=1e-8), (name, idx, g[idx], num)


def test_zero_upstream_gradient_gives_zero_gradients():
    q, k, v = (_rnd((1, 5, 1, 4), s) for s in (26, 27, 28))
    for g in attention_backward(q, k, v, np.zeros_like(q), 0.5, True):
        assert np.array_equal(g, np.zeros_like(g))


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero_and_value_gradients_sum_to_dout(causal):
    # softmax is unchanged when every key of a head moves by one vector, so
    # the key gradients of a head sum to zero; each softmax row sums to 1,
    # so the value gradients of a head sum to the sum of the dO rows
    q, k, v, do = (_rnd((2, 9, 3, 5), s) for s in (29, 30, 31, 32))
    dq, dk, dv = attention_backward(q, k, v, do, 0.6, causal)
    assert np.allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    assert np.allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)


def test_causal_first_query_has_zero_gradient():
    q, k, v, do = (_rnd((1, 7, 2, 4), s) for s in (33, 34, 35, 36))
    dq, _, _ = attention_backward(q, k, v, do, 0.9, True)
    assert np.allclose(dq[:, 0], 0.0, atol=1e-15)


def test_delta_is_rowsum_of_p_times_dp():
    q, k, v, do = (_rnd((1, 8, 1, 4), s) for s in (37, 38, 39, 40))
    o, _ = attention_forward(q, k, v, 0.5, False)
    s = 0.5 * q[0, :, 0] @ k[0, :, 0].T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = do[0, :, 0] @ v[0, :, 0].T
    assert np.allclose(attention_delta(o, do)[0, 0], (p * dp).sum(axis=1), atol=1e-13)
