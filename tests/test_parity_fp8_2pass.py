"""GPU parity of the two-pass FP8 forward (attn_fwd_fp8_2pass) against the
fp64 oracle on the dequantised inputs, and its accuracy next to the
single-pass kernel.

The two-pass form ("FlashAttention-3" page, section on FP8 stability) first
finds each row's exact score maximum, then exponentiates against it with a
static scale on P.  It computes the same attention, so the bar is the FP8
one of the single pass (O relative RMS <= 3e-2, the per-row LSE bound).
Cases: ragged shapes (N = 1, 17, 257, 300), both head dimensions and
masks, grouped-query heads, the fp8_8k workload at full size on sampled
rows, guard bands, and bitwise determinism.  The accuracy comparison
prints both kernels' errors on the outlier workload and requires the
two-pass error to be no larger.
"""

import numpy as np
import pytest
import torch

import exact_attention_tile_amd as eat
from oracle import attention_forward, dequantize_e4m3
from parity_common import (Guarded, assert_fp8_ok, dev_u8, errors, fp8_lse_bound, reference,
                           require_gpu, run_fp8)
from workloads import WORKLOADS, Workload, make_inputs, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def run_2pass(inp, B, H, Hkv, N, d, causal, scale):
    print("case fp8 2-pass B=%d H=%d Hkv=%d N=%d d=%d causal=%d" % (B, H, Hkv, N, d, causal),
          flush=True)
    q, k, v = dev_u8(inp["q"]), dev_u8(inp["k"]), dev_u8(inp["v"])
    dq = torch.from_numpy(inp["dq"]).reshape(-1).cuda()
    dk = torch.from_numpy(inp["dk"]).reshape(-1).cuda()
    dv = torch.from_numpy(inp["dv"]).reshape(-1).cuda()
    out = Guarded(B, N, H, d)
    eat.attn_fwd_fp8_2pass(q, k, v, out.o_ptr, out.l_ptr, dq, dk, dv, B, H, Hkv, N, d, int(causal),
                           scale, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert out.guards_intact()
    return out


def _gqa_reference(inp, causal, scale, rows=None):
    q = dequantize_e4m3(inp["q"], inp["dq"])
    k = dequantize_e4m3(inp["k"], inp["dk"])
    v = dequantize_e4m3(inp["v"], inp["dv"])
    rep = q.shape[2] // k.shape[2]
    k, v = np.repeat(k, rep, axis=2), np.repeat(v, rep, axis=2)
    return attention_forward(q, k, v, scale, causal, rows=rows), (q, k, v)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,d", [(1, 2, 2, 1, 128), (1, 2, 2, 17, 64), (2, 3, 3, 300, 128),
                                         (1, 2, 2, 257, 64), (2, 8, 2, 200, 128), (1, 4, 1, 130, 64)])
def test_two_pass_shapes(B, H, Hkv, N, d, causal):
    w = Workload("t", 51, B, H, N, d, "fp8", (causal,), outliers=True, Hkv=Hkv)
    inp = make_inputs(w)
    out = run_2pass(inp, B, H, Hkv, N, d, causal, w.scale)
    (ro, rl), _ = _gqa_reference(inp, causal, w.scale)
    err = errors(out, ro, rl, lse_bound=fp8_lse_bound(inp, causal, w.scale))
    assert_fp8_ok(err, "2-pass B=%d H=%d Hkv=%d N=%d d=%d causal=%d" % (B, H, Hkv, N, d, causal))


def test_two_pass_full_size_and_accuracy():
    w = WORKLOADS["fp8_8k"]
    inp = make_inputs(w)
    rows = sample_rows(w)
    ro, rl = reference(inp, "fp8", False, w.scale, rows=rows)
    bound = fp8_lse_bound(inp, False, w.scale, rows)
    two = errors(run_2pass(inp, w.B, w.H, w.H, w.N, w.d, False, w.scale), ro, rl, rows,
                 lse_bound=bound)
    assert_fp8_ok(two, "fp8_8k 2-pass")
    one = errors(run_fp8(inp, w.B, w.H, w.N, w.d, False, w.scale), ro, rl, rows, lse_bound=bound)
    assert_fp8_ok(one, "fp8_8k 1-pass")
    print("fp8_8k O rel RMS: single pass %.4e, two pass %.4e (ratio %.2f)"
          % (one[1], two[1], one[1] / two[1]), flush=True)
    assert two[1] <= one[1]


def test_two_pass_deterministic():
    w = Workload("t", 52, 2, 4, 700, 128, "fp8", (True,), outliers=True)
    inp = make_inputs(w)
    a = run_2pass(inp, 2, 4, 4, 700, 128, True, w.scale)
    b = run_2pass(inp, 2, 4, 4, 700, 128, True, w.scale)
    assert torch.equal(a.o_raw, b.o_raw) and torch.equal(a.l_raw, b.l_raw)
