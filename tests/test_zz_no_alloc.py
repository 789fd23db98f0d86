"""attn_bwd_noalloc -- the backward pass with its D workspace in the
library's static device array, for callers that cannot allocate -- against
attn_bwd with a caller-allocated workspace, through the C ABI.

Both run the same kernels, so the gradients must agree bit for bit; the
check runs two calls in a row on one GPU (the second with a smaller input,
so it reuses the array the first one filled), each compared with attn_bwd on
the same inputs.  The first pair is also checked against the fp64 gradient
oracle (oracle.attention_backward) to the backward tolerances.
"""

import numpy as np
import pytest
import torch

import exact_attention_tile_amd as eat
from parity_common import dev_u16, require_gpu
from workloads import Workload, make_dout, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def _forward_and_grads(w, causal):
    inp, do_bits = make_inputs(w), make_dout(w)
    q, k, v = dev_u16(inp["q"]), dev_u16(inp["k"]), dev_u16(inp["v"])
    do = dev_u16(do_bits)
    s = torch.cuda.current_stream()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    eat.attn_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.d, int(causal), w.scale, s)
    ref = [torch.full_like(q, float("nan")) for _ in range(3)]
    delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    eat.attn_bwd(q, k, v, o, lse, do, ref[0], ref[1], ref[2], delta, w.B, w.H, w.N, w.d,
                 int(causal), w.scale, s)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    eat.attn_bwd_noalloc(q, k, v, o, lse, do, got[0], got[1], got[2], w.B, w.H, w.N, w.d,
                         int(causal), w.scale, s)
    torch.cuda.synchronize()
    return inp, do_bits, ref, got


def test_noalloc_matches_attn_bwd_on_two_calls_in_a_row():
    cases = [Workload("noalloc_a", 95, 2, 4, 700, 128, "bf16", (True,)),
             Workload("noalloc_b", 96, 1, 3, 300, 64, "bf16", (False,))]
    assert cases[1].B * cases[1].H * cases[1].N < cases[0].B * cases[0].H * cases[0].N
    for i, w in enumerate(cases):
        causal = w.modes[0]
        print("case %s B=%d H=%d N=%d d=%d causal=%d" % (w.name, w.B, w.H, w.N, w.d, causal),
              flush=True)
        inp, do_bits, ref, got = _forward_and_grads(w, causal)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        if i == 0:
            from test_parity_bwd import check_bwd
            grads = [x.float().cpu().numpy().astype(np.float64) for x in got]
            check_bwd(inp, do_bits, grads, causal, w.scale, "noalloc %s" % w.name)


def test_noalloc_rejects_an_oversized_call_and_launches_nothing():
    w = Workload("noalloc_c", 97, 1, 2, 64, 64, "bf16", (False,))
    inp = make_inputs(w)
    q = dev_u16(inp["q"])
    out = torch.full_like(q, 1.0)
    n = eat.ATTN_BWD_NOALLOC_MAX_ROWS // 2 + 1
    st = eat.attn_bwd_noalloc(q, q, q, q, out, q, out, out, out, 1, 2, n, 64, 0, 0.125,
                              torch.cuda.current_stream(), check=False)
    torch.cuda.synchronize()
    assert st == eat.ATTN_ERR_UNSUPPORTED
    assert bool((out == 1.0).all())
