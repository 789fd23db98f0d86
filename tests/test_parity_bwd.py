"""GPU parity of the backward pass (attn_bwd) against the fp64 oracle
gradients (oracle.attention_backward) on the same seeded bf16 inputs; O and
lse come from the library's own forward, as they would in training.

Tolerance (no target is stated for the backward pass; derived from the
arithmetic): per gradient tensor, relative RMS <= 1e-2 and max-abs <= 2e-2
times the largest reference magnitude.  The kernels round P and dS to bf16
(relative error <= 2^-9 ~ 2e-3 per element) for the MFMA products and
accumulate in fp32; the forward's bf16 O and its lse enter through D and P.
Summed over many keys the relative RMS error is a few 1e-3; 1e-2 leaves a
margin of about 3.

Cases: ragged and degenerate shapes (N = 17, 257, 300, 520, 1000; grids that
are not a multiple of 8, and head counts B*H divisible by 8, which the short
causal calls run in tile-major order), both head dimensions, both masks, a negative and a
zero scale, a 2048-token case, the long8k workload at full size (B = 2,
H = 16, N = 8192, d = 128, causal, as the benchmark times it) checked on two
whole heads, untouched guard bands around every gradient, and bitwise
determinism of two identical calls.
"""

import numpy as np
import pytest
import torch

import exact_attention_tile_amd as eat
from oracle import attention_backward, attention_backward_head, bf16_bits_to_float64
from parity_common import SENTINEL_BF16, dev_u16, require_gpu
from workloads import WORKLOADS, Workload, make_dout, make_inputs

pytestmark = pytest.mark.gpu

BWD_RELRMS = 1e-2
BWD_MAXABS_REL = 2e-2
GUARD = 4096


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def _guarded(n):
    return torch.full((n + 2 * GUARD,), SENTINEL_BF16, dtype=torch.int16, device="cuda")


def _inner(buf, n, shape):
    return buf[GUARD:GUARD + n].view(torch.bfloat16).view(shape)


def run_bwd(inp, do_bits, B, H, N, d, causal, scale):
    print("case bwd B=%d H=%d N=%d d=%d causal=%d scale=%g" % (B, H, N, d, causal, scale), flush=True)
    q, k, v = dev_u16(inp["q"]), dev_u16(inp["k"]), dev_u16(inp["v"])
    do = dev_u16(do_bits)
    n = B * N * H * d
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    delta = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    eat.attn_fwd(q, k, v, o, lse, B, H, N, d, int(causal), scale, s)
    bufs = [_guarded(n) for _ in range(3)]
    ptrs = [b.data_ptr() + 2 * GUARD for b in bufs]
    eat.attn_bwd(q, k, v, o, lse, do, ptrs[0], ptrs[1], ptrs[2], delta, B, H, N, d, int(causal),
                 scale, s)
    torch.cuda.synchronize()
    for b in bufs:
        assert bool((b[:GUARD] == SENTINEL_BF16).all()) and bool((b[GUARD + n:] == SENTINEL_BF16).all())
    return [_inner(b, n, (B, N, H, d)).float().cpu().numpy().astype(np.float64) for b in bufs], bufs


def check_bwd(inp, do_bits, grads, causal, scale, label):
    q, k, v = (bf16_bits_to_float64(inp[x]) for x in ("q", "k", "v"))
    ref = attention_backward(q, k, v, bf16_bits_to_float64(do_bits), scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        diff = g - r
        scale_r = max(float(np.abs(r).max()), 1e-30)
        max_rel = float(np.abs(diff).max()) / scale_r
        denom = float((r ** 2).sum())
        rel_rms = float(np.sqrt((diff ** 2).sum() / denom)) if denom > 0 else float(np.abs(diff).max())
        msg = "%s %s: rel_rms=%.3e max_abs/max_ref=%.3e" % (label, name, rel_rms, max_rel)
        print(msg, flush=True)
        assert rel_rms <= BWD_RELRMS, msg
        assert max_rel <= BWD_MAXABS_REL, msg


BWD_SHAPES = [(1, 2, 128, 64), (2, 3, 300, 128), (1, 2, 1000, 64), (1, 1, 17, 128),
              (3, 1, 257, 64), (1, 4, 2048, 128),
              # B*H divisible by 8: the causal calls take the tile-major block order
              (2, 4, 1000, 64), (1, 8, 520, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", BWD_SHAPES)
def test_backward_shapes(B, H, N, d, causal):
    w = Workload("bwd", 70 + N % 13, B, H, N, d, "bf16", (causal,))
    inp, dob = make_inputs(w), make_dout(w)
    grads, _ = run_bwd(inp, dob, B, H, N, d, causal, w.scale)
    check_bwd(inp, dob, grads, causal, w.scale, "bwd B=%d H=%d N=%d d=%d causal=%d" %
              (B, H, N, d, causal))


@pytest.mark.parametrize("scale", [-0.125, 0.0])
def test_backward_scale_sign_and_zero(scale):
    w = Workload("bwd_s", 77, 1, 2, 333, 128, "bf16", (True,))
    inp, dob = make_inputs(w), make_dout(w)
    grads, _ = run_bwd(inp, dob, 1, 2, 333, 128, True, scale)
    if scale == 0.0:
        # P uniform over the visible keys: dQ and dK are exactly zero
        assert np.array_equal(grads[0], np.zeros_like(grads[0]))
        assert np.array_equal(grads[1], np.zeros_like(grads[1]))
    check_bwd(inp, dob, grads, True, scale, "bwd scale=%g" % scale)


def test_backward_bitwise_deterministic():
    w = Workload("bwd_det", 78, 2, 2, 700, 128, "bf16", (True,))
    inp, dob = make_inputs(w), make_dout(w)
    _, b1 = run_bwd(inp, dob, 2, 2, 700, 128, True, w.scale)
    _, b2 = run_bwd(inp, dob, 2, 2, 700, 128, True, w.scale)
    for x, y in zip(b1, b2):
        assert torch.equal(x, y)


def test_backward_full_size_sampled_heads():
    w = WORKLOADS["long8k"]
    B, H, N, d, causal = w.B, w.H, w.N, w.d, True
    inp, dob = make_inputs(w), make_dout(w)
    grads, _ = run_bwd(inp, dob, B, H, N, d, causal, w.scale)
    q, k, v = (bf16_bits_to_float64(inp[x]) for x in ("q", "k", "v"))
    do = bf16_bits_to_float64(dob)
    for b, h in ((0, 3), (1, 12)):
        ref = attention_backward_head(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], w.scale,
                                      causal)
        for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
            diff = g[b, :, h] - r
            max_rel = float(np.abs(diff).max()) / max(float(np.abs(r).max()), 1e-30)
            rel_rms = float(np.sqrt((diff ** 2).sum() / (r ** 2).sum()))
            msg = "long8k b=%d h=%d %s: rel_rms=%.3e max_abs/max_ref=%.3e" % (b, h, name, rel_rms,
                                                                             max_rel)
            print(msg, flush=True)
            assert rel_rms <= BWD_RELRMS, msg
            assert max_rel <= BWD_MAXABS_REL, msg
