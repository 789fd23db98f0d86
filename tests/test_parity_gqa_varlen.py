"""GPU parity of the grouped-query and variable-length entry points against
the CPU oracle (oracle.attention_forward_gqa / attention_forward_varlen),
through the C ABI.

* grouped-query (and multi-query) shapes with ragged lengths, both dtypes,
  both masks, full oracle; the gqa8k workload at full size on sampled rows;
* variable-length batches with an empty and a length-1 sequence, both
  dtypes, both masks, full oracle; the varlen workload at full size on
  sampled rows (all rows of sequences up to 2048 tokens);
* malformed offsets: the sequences they describe are skipped (their rows of
  o and lse keep the sentinel) and the valid ones are still exact.
Tolerances are those of parity_common.py.
"""

import numpy as np
import pytest
import torch

import exact_attention_tile_amd as eat
from oracle import (attention_forward_gqa, attention_forward_varlen, bf16_bits_to_float64,
                    dequantize_e4m3)
from parity_common import (SENTINEL_BF16, SENTINEL_F32, Guarded, assert_bf16_ok, assert_fp8_ok,
                           dev_u16, dev_u8, error_figures, errors, lse_bound_rows, require_gpu)
from workloads import WORKLOADS, Workload, make_inputs, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def _dev(inp, dtype):
    if dtype == "fp8":
        return dev_u8(inp["q"]), dev_u8(inp["k"]), dev_u8(inp["v"])
    return dev_u16(inp["q"]), dev_u16(inp["k"]), dev_u16(inp["v"])


def _descales(inp):
    return tuple(torch.from_numpy(inp[n]).reshape(-1).cuda() for n in ("dq", "dk", "dv"))


def _decode(inp, dtype, cu=None):
    """float64 q, k, v exactly as the GPU sees them (fp8: dequantised per
    (batch, head), or per (sequence, head) when packed)."""
    if dtype != "fp8":
        return tuple(bf16_bits_to_float64(inp[n]) for n in ("q", "k", "v"))
    out = []
    for n in ("q", "k", "v"):
        codes, ds = inp[n], inp["d" + n]
        if cu is None:
            out.append(dequantize_e4m3(codes, ds))
        else:
            x = np.zeros(codes.shape, dtype=np.float64)
            for b in range(len(cu) - 1):
                if cu[b + 1] > cu[b]:
                    x[:, cu[b]:cu[b + 1]] = dequantize_e4m3(codes[:, cu[b]:cu[b + 1]], ds[b:b + 1])
            out.append(x)
    return tuple(out)


# ---------------------------------------------------------------------------
# grouped-query
# ---------------------------------------------------------------------------

def _run_gqa(w, inp, causal):
    B, N, H, Hkv, d = w.B, w.N, w.H, w.kv_heads, w.d
    print("case %s B=%d H=%d Hkv=%d N=%d d=%d causal=%d" % (w.name, B, H, Hkv, N, d, causal),
          flush=True)
    q, k, v = _dev(inp, w.dtype)
    out = Guarded(B, N, H, d)
    s = torch.cuda.current_stream()
    if w.dtype == "fp8":
        dq, dk, dv = _descales(inp)
        eat.attn_fwd_fp8_gqa(q, k, v, out.o_ptr, out.l_ptr, dq, dk, dv, B, H, Hkv, N, d,
                             int(causal), w.scale, s)
    else:
        eat.attn_fwd_gqa(q, k, v, out.o_ptr, out.l_ptr, B, H, Hkv, N, d, int(causal), w.scale, s)
    torch.cuda.synchronize()
    return out


def _check_gqa(w, inp, out, causal, rows=None):
    assert out.guards_intact()
    q, k, v = _decode(inp, w.dtype)
    ro, rl = attention_forward_gqa(q, k, v, w.scale, causal, rows=rows)
    label = "%s causal=%d" % (w.name, causal)
    if w.dtype == "fp8":
        g = w.H // w.kv_heads
        R = w.N if rows is None else rows.shape[2]
        bound = np.empty((w.B, w.H, R))
        for b in range(w.B):
            for h in range(w.H):
                r = np.arange(w.N) if rows is None else rows[b, h]
                bound[b, h] = lse_bound_rows(q[b, :, h], k[b, :, h // g], w.scale, causal, r)
        assert_fp8_ok(errors(out, ro, rl, rows, lse_bound=bound), label)
    else:
        assert_bf16_ok(errors(out, ro, rl, rows), label)


GQA_EDGE = [("bf16", 2, 8, 2, 300, 128), ("bf16", 1, 4, 1, 257, 64), ("bf16", 1, 6, 3, 1000, 128),
            ("fp8", 1, 8, 2, 300, 128), ("fp8", 2, 4, 1, 129, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,B,H,Hkv,N,d", GQA_EDGE)
def test_gqa_edge_shapes(dtype, B, H, Hkv, N, d, causal):
    w = Workload("gqa_%s" % dtype, 40 + N % 11, B, H, N, d, dtype, (causal,), Hkv=Hkv,
                 outliers=(dtype == "fp8"))
    inp = make_inputs(w)
    _check_gqa(w, inp, _run_gqa(w, inp, causal), causal)


def test_gqa_workload_full_size():
    w = WORKLOADS["gqa8k"]
    inp = make_inputs(w)
    out = _run_gqa(w, inp, True)
    _check_gqa(w, inp, out, True, rows=sample_rows(w))


# ---------------------------------------------------------------------------
# variable-length
# ---------------------------------------------------------------------------

def _run_varlen(w, inp, causal, cu=None, maxlen=None):
    T, H, Hkv, d = w.total, w.H, w.kv_heads, w.d
    cu = inp["cu"] if cu is None else np.asarray(cu, dtype=np.int32)
    B = cu.shape[0] - 1
    maxlen = w.N if maxlen is None else maxlen
    print("case %s B=%d total=%d max=%d H=%d Hkv=%d d=%d causal=%d" %
          (w.name, B, T, maxlen, H, Hkv, d, causal), flush=True)
    q, k, v = _dev(inp, w.dtype)
    cu_d = torch.from_numpy(cu).cuda()
    out = Guarded(1, T, H, d)
    s = torch.cuda.current_stream()
    if w.dtype == "fp8":
        dq, dk, dv = _descales(inp)
        eat.attn_fwd_fp8_varlen(q, k, v, out.o_ptr, out.l_ptr, dq, dk, dv, cu_d, B, T, maxlen, H,
                                Hkv, d, int(causal), w.scale, s)
    else:
        eat.attn_fwd_varlen(q, k, v, out.o_ptr, out.l_ptr, cu_d, B, T, maxlen, H, Hkv, d,
                            int(causal), w.scale, s)
    torch.cuda.synchronize()
    return out


def _varlen_rows(w, limit=2048):
    """Rows checked per sequence: all of a sequence up to ``limit`` tokens,
    else its first and last rows plus seeded distinct rows (512 in all)."""
    rows = []
    for b, n in enumerate(w.lengths):
        if n <= limit:
            r = np.arange(n)
        else:
            g = np.random.default_rng(1000 * w.wid + 50 + b)
            r = np.concatenate([[0, n - 1], np.sort(g.choice(np.arange(1, n - 1), 510, replace=False))])
        rows.append(np.tile(r, (w.H, 1)))
    return rows


def _check_varlen(w, inp, out, causal, rows, skip=()):
    cu = inp["cu"]
    q, k, v = _decode(inp, w.dtype, cu)
    ro, rl = attention_forward_varlen(q[0], k[0], v[0], cu, w.scale, causal, rows=rows)
    o = out.o().float().cpu().numpy().astype(np.float64)[0]      # [T][H][d]
    lse = out.lse().cpu().numpy().astype(np.float64)[0]          # [H][T]
    go, gr, gl, grl, bnd = [], [], [], [], []
    g = w.H // w.kv_heads
    for b, r in enumerate(rows):
        if b in skip or r.shape[1] == 0:
            continue
        s0 = cu[b]
        for h in range(w.H):
            go.append(o[s0 + r[h], h])
            gr.append(ro[b][h])
            gl.append(lse[h, s0 + r[h]])
            grl.append(rl[b][h])
            if w.dtype == "fp8":
                bnd.append(lse_bound_rows(q[0, s0:cu[b + 1], h], k[0, s0:cu[b + 1], h // g], w.scale,
                                      causal, r[h]))
    go, gr = np.concatenate(go), np.concatenate(gr)
    gl, grl = np.concatenate(gl), np.concatenate(grl)
    label = "%s causal=%d" % (w.name, causal)
    if w.dtype == "fp8":
        assert_fp8_ok(error_figures(go, gr, gl, grl, np.concatenate(bnd)), label)
    else:
        assert_bf16_ok(error_figures(go, gr, gl, grl), label)


# H a multiple of 8 with B <= 128 takes the rank-ordered mapping (sequences
# ranked by length on the device, longest first, ties by index; B > 64 needs
# the second candidate round); other shapes take the head-major or
# tile-major mappings.  Short-sequence batches hold zero lengths and ties.
_SHORT100 = tuple((7 * i) % 45 for i in range(100))
_SHORT128 = tuple((11 * i + 3) % 37 for i in range(128))
_SHORT129 = tuple((5 * i + 1) % 29 for i in range(129))
VARLEN_EDGE = [("bf16", (300, 1, 0, 129, 64), 4, 2, 64), ("bf16", (1000, 17, 256, 1), 6, 3, 128),
               ("fp8", (200, 1, 77), 4, 4, 128), ("fp8", (65, 0, 300), 4, 2, 64),
               ("bf16", (300, 1, 0, 129, 64, 700), 8, 2, 128), ("fp8", (513, 33, 1, 250, 0), 16, 4, 64),
               ("fp8", (200, 77, 1000), 8, 8, 128), ("bf16", _SHORT100, 8, 4, 64),
               ("fp8", _SHORT128, 16, 2, 128), ("bf16", _SHORT129, 8, 8, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,lengths,H,Hkv,d", VARLEN_EDGE,
                         ids=["%s-B%d-H%d-Hkv%d-d%d" % (c[0], len(c[1]), c[2], c[3], c[4]) for c in VARLEN_EDGE])
def test_varlen_edge_batches(dtype, lengths, H, Hkv, d, causal):
    w = Workload("varlen_%s" % dtype, 30 + len(lengths), len(lengths), H, max(lengths), d, dtype,
                 (causal,), Hkv=Hkv, lengths=lengths, outliers=(dtype == "fp8"))
    inp = make_inputs(w)
    out = _run_varlen(w, inp, causal)
    assert out.guards_intact()
    _check_varlen(w, inp, out, causal, _varlen_rows(w))


def test_varlen_workload_full_size():
    w = WORKLOADS["varlen"]
    inp = make_inputs(w)
    out = _run_varlen(w, inp, True)
    assert out.guards_intact()
    _check_varlen(w, inp, out, True, _varlen_rows(w))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_varlen_malformed_offsets_are_skipped(dtype):
    # 40 tokens; offsets [0, 10, 50, 20, 40] with max_seqlen 20: sequence 0
    # (rows 0..9) and sequence 3 (rows 20..39) are valid; sequence 1 runs
    # past the end and sequence 2 has a decreasing offset: both are skipped,
    # so rows 10..19 are never written
    cu = np.array([0, 10, 50, 20, 40], dtype=np.int32)
    w = Workload("bad_cu_%s" % dtype, 61, 4, 4, 20, 128, dtype, (True,), Hkv=2,
                 lengths=(10, 10, 10, 10), outliers=(dtype == "fp8"))
    inp = make_inputs(w)
    inp["cu"] = cu
    if dtype == "fp8":   # descales of the skipped sequences are never read
        pass
    out = _run_varlen(w, inp, True, cu=cu, maxlen=20)
    assert out.guards_intact()
    o = out.o_raw[4096:4096 + out.no].view(w.total, w.H, w.d).cpu()
    lse = out.l_raw[4096:4096 + out.nl].view(w.H, w.total).cpu()
    assert bool((o[10:20] == SENTINEL_BF16).all())
    assert bool((lse[:, 10:20] == SENTINEL_F32).all())
    rows = [np.tile(np.arange(10), (w.H, 1)), np.zeros((w.H, 0), dtype=np.int64),
            np.zeros((w.H, 0), dtype=np.int64), np.tile(np.arange(20), (w.H, 1))]
    # reference with the valid sequences' own offsets
    ref_inp = dict(inp)
    ref_inp["cu"] = np.array([0, 10, 10, 20, 40], dtype=np.int32)
    _check_varlen(w, ref_inp, out, True, rows, skip=(1, 2))
