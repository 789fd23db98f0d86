"""Properties of the kernels that hold at any size, checked bit for bit at
the full size of the benchmark workloads and in their launch configuration
(the persistent launch and the XCD-aware work order included):

* causality of the forward: replacing K and V from token p on (p inside a
  key tile and a query tile) leaves O and LSE of every query before p
  unchanged, and changes rows from p on;
* causality of the backward: with q, o, lse and dO held fixed, replacing K
  and V from token p on leaves dQ, dK and dV of every token before p
  unchanged (dQ_i sums over keys j <= i; dK_j and dV_j sum P_ij, dP_ij and
  D_i over queries i >= j, all of which depend on K_j and V_j and on the
  fixed inputs only);
* independence of the (batch, head) problems: replacing one problem's K
  and V leaves every other problem's O and LSE unchanged; with grouped
  K/V heads, replacing K/V head g changes exactly the query heads that
  read it; with packed sequences, replacing one sequence's K and V changes
  that sequence's rows only.

Each follows from the definition of causal attention (a query attends to
the keys at or before it, and each (batch, head) is its own problem), so
no oracle value is involved; the kernels are deterministic (two identical
calls are bitwise equal, test_parity_gpu.py), which makes a bitwise
comparison meaningful.
"""

import numpy as np
import pytest
import torch

import exact_attention_tile_amd as eat
from parity_common import Guarded, dev_u16, dev_u8, require_gpu, run_bf16, run_fp8
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def _replacement(inp, dtype, sl, seed):
    """inp with K and V replaced on the index expression sl by other seeded
    values of the same kind (finite bf16 normals, or finite e4m3 codes; the
    fp8 descales stay)."""
    rng = np.random.default_rng(seed)
    out = dict(inp)
    for name in ("k", "v"):
        a = inp[name].copy()
        shape = a[sl].shape
        if dtype == "fp8":
            codes = rng.integers(0, 256, size=shape, dtype=np.uint8)
            codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN codes
            a[sl] = codes
        else:
            vals = rng.standard_normal(size=shape).astype(np.float32)
            a[sl] = (vals.view(np.uint32) >> 16).astype(np.uint16)
        out[name] = a
    return out


def _forward(w, inp, causal):
    print("case %s B=%d H=%d N=%d d=%d causal=%d" % (w.name, w.B, w.H, w.N, w.d, causal), flush=True)
    run = run_fp8 if w.dtype == "fp8" else run_bf16
    out = run(inp, w.B, w.H, w.N, w.d, causal, w.scale)
    assert out.guards_intact()
    o = out.o().view(torch.int16)
    return o, out.lse().view(torch.int32)


@pytest.mark.parametrize("name,causal", [("long8k", True), ("long8k64", True), ("ctx32k", True),
                                         ("fp8_8k", True)])
def test_forward_causal_prefix(name, causal):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    p = w.N // 2 + 37                       # inside a key tile and a query tile
    o0, l0 = _forward(w, inp, causal)
    o1, l1 = _forward(w, _replacement(inp, w.dtype, np.s_[:, p:], 901), causal)
    assert torch.equal(o0[:, :p], o1[:, :p]), "O of a query before p changed"
    assert torch.equal(l0[:, :, :p], l1[:, :, :p]), "LSE of a query before p changed"
    assert not torch.equal(o0[:, p:], o1[:, p:]), "rows from p on did not see the new keys"


@pytest.mark.parametrize("name,causal", [("long8k", True), ("fp8_8k", False), ("mha2k", False)])
def test_forward_problem_independence(name, causal):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    b, h = w.B - 1, 3
    o0, l0 = _forward(w, inp, causal)
    o1, l1 = _forward(w, _replacement(inp, w.dtype, np.s_[b, :, h], 902), causal)
    keep_o = torch.ones(o0.shape[0], o0.shape[2], dtype=torch.bool, device=o0.device)
    keep_o[b, h] = False
    oa, ob = o0.permute(0, 2, 1, 3), o1.permute(0, 2, 1, 3)      # [B][H][N][d]
    assert torch.equal(oa[keep_o], ob[keep_o]), "another problem's O changed"
    assert torch.equal(l0[keep_o], l1[keep_o]), "another problem's LSE changed"
    assert not torch.equal(oa[b, h], ob[b, h]), "the replaced problem's O did not change"


def _backward(w, inp, o, lse, do, causal):
    B, N, H, d = w.B, w.N, w.H, w.d
    print("case bwd %s B=%d H=%d N=%d d=%d causal=%d" % (w.name, B, H, N, d, causal), flush=True)
    q, k, v = dev_u16(inp["q"]), dev_u16(inp["k"]), dev_u16(inp["v"])
    grads = [torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    delta = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    eat.attn_bwd(q, k, v, o, lse, do, grads[0], grads[1], grads[2], delta, B, H, N, d, int(causal),
                 w.scale, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return [g.view(torch.int16) for g in grads]


@pytest.mark.parametrize("name", ["long8k", "long8k64"])
def test_backward_causal_prefix(name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    B, N, H, d = w.B, w.N, w.H, w.d
    q, k, v = dev_u16(inp["q"]), dev_u16(inp["k"]), dev_u16(inp["v"])
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    eat.attn_fwd(q, k, v, o, lse, B, H, N, d, 1, w.scale, torch.cuda.current_stream())
    rng = np.random.default_rng(903)
    do_bits = (rng.standard_normal(size=(B, N, H, d)).astype(np.float32).view(np.uint32)
               >> 16).astype(np.uint16)
    do = dev_u16(do_bits)
    p = N // 2 + 37
    g0 = _backward(w, inp, o, lse, do, True)
    g1 = _backward(w, _replacement(inp, "bf16", np.s_[:, p:], 904), o, lse, do, True)
    for name_g, a, b in zip(("dQ", "dK", "dV"), g0, g1):
        assert torch.equal(a[:, :p], b[:, :p]), "%s of a token before p changed" % name_g
    assert not torch.equal(g0[0][:, p:], g1[0][:, p:]), "dQ from p on did not see the new keys"


def _run_grouped(w, inp, causal):
    """gqa8k / varlen (bf16) through attn_fwd_gqa / attn_fwd_varlen; O and
    LSE as integer views, O as [B or 1][tokens][H][d]."""
    q, k, v = dev_u16(inp["q"]), dev_u16(inp["k"]), dev_u16(inp["v"])
    s = torch.cuda.current_stream()
    if w.varlen:
        cu = torch.from_numpy(np.asarray(inp["cu"], dtype=np.int32)).cuda()
        nseq = len(inp["cu"]) - 1
        print("case %s sequences=%d total=%d H=%d Hkv=%d d=%d causal=%d" %
              (w.name, nseq, w.total, w.H, w.kv_heads, w.d, causal), flush=True)
        out = Guarded(1, w.total, w.H, w.d)
        eat.attn_fwd_varlen(q, k, v, out.o_ptr, out.l_ptr, cu, nseq, w.total, w.N, w.H,
                            w.kv_heads, w.d, int(causal), w.scale, s)
    else:
        print("case %s B=%d H=%d Hkv=%d N=%d d=%d causal=%d" %
              (w.name, w.B, w.H, w.kv_heads, w.N, w.d, causal), flush=True)
        out = Guarded(w.B, w.N, w.H, w.d)
        eat.attn_fwd_gqa(q, k, v, out.o_ptr, out.l_ptr, w.B, w.H, w.kv_heads, w.N, w.d,
                         int(causal), w.scale, s)
    torch.cuda.synchronize()
    assert out.guards_intact()
    return out.o().view(torch.int16), out.lse().view(torch.int32)


def test_grouped_kv_head_independence():
    w = WORKLOADS["gqa8k"]
    inp = make_inputs(w)
    g = 5
    o0, l0 = _run_grouped(w, inp, True)
    o1, l1 = _run_grouped(w, _replacement(inp, "bf16", np.s_[:, :, g], 905), True)
    group = w.H // w.kv_heads
    for h in range(w.H):
        same_o = torch.equal(o0[:, :, h], o1[:, :, h])
        same_l = torch.equal(l0[:, h], l1[:, h])
        if h // group == g:
            assert not same_o, "query head %d did not see its new K/V head" % h
        else:
            assert same_o and same_l, "query head %d changed with K/V head %d" % (h, g)


def test_varlen_sequence_independence():
    w = WORKLOADS["varlen"]
    inp = make_inputs(w)
    cu = [int(x) for x in inp["cu"]]
    lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    s_rep = int(np.argsort(lens)[len(lens) // 2])       # a sequence of middling length
    o0, l0 = _run_grouped(w, inp, True)
    o1, l1 = _run_grouped(w, _replacement(inp, "bf16", np.s_[:, cu[s_rep]:cu[s_rep + 1]], 906),
                          True)
    for sq in range(len(lens)):
        a, b = cu[sq], cu[sq + 1]
        same = torch.equal(o0[:, a:b], o1[:, a:b]) and torch.equal(l0[:, :, a:b], l1[:, :, a:b])
        if sq == s_rep:
            assert lens[sq] == 0 or not torch.equal(o0[:, a:b], o1[:, a:b]), \
                "the replaced sequence did not change"
        else:
            assert same, "sequence %d changed with sequence %d" % (sq, s_rep)
