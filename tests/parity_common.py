"""Helpers for the GPU parity tests: run the HIP library through its C ABI
on seeded inputs and compare with the CPU oracle.

Tolerances:
  bf16 : O max-abs <= 2e-2, O relative RMS <= 5e-3, LSE max-abs <= 1e-3
         (the method's stated accuracy target)
  fp8  : O relative RMS <= 3e-2 (stated target).  No LSE target is stated;
         the bound is derived from the matrix cores' error model:
           |lse_gpu - lse_ref| <= 1e-3 + EPS_E4M3_MFMA * (d / 64) * M_i,
           M_i = |scale| * max_j max_c |q_ic k_jc| over the visible keys j
         (q, k the dequantised inputs).
         Derivation.  The kernel's score of (i, j) is the fp32 chain of d/64
         e4m3 instructions on the codes, times |scale| dq dk.  Each
         instruction's error is at most EPS_E4M3_MFMA times the binade of its
         largest product, 2^floor(log2 max_c |a_c b_c|) <= max_c |a_c b_c|,
         plus binary32 rounding of the accumulator (the model
         tests/test_mfma_accuracy.py checks on the hardware; EPS_E4M3_MFMA is
         the largest ratio seen, rounded up to a power of two).  Scaled by
         the descales to natural-log units, the score error is at most
         EPS_E4M3_MFMA * (d / 64) * |scale| * max_c |q_ic k_jc|.  The
         log-sum-exp is monotone and shifts with a constant added to all its
         arguments, so the row's LSE moves by at most the largest score
         error, which is at most EPS_E4M3_MFMA * (d / 64) * M_i.  The 1e-3
         covers the remaining fp32 steps (exponentials, the row sum, the
         logarithm) as for bf16.  Both the absolute error and its ratio to
         the bound are printed.
relative RMS = ||O_gpu - O_ref||_2 / ||O_ref||_2 over every checked element.
"""

import numpy as np
import torch

import exact_attention_tile_amd as eat
from oracle import attention_forward, bf16_bits_to_float64, dequantize_e4m3

BF16_MAXABS = 2e-2
BF16_RELRMS = 5e-3
LSE_MAXABS = 1e-3
FP8_RELRMS = 3e-2
# Error model of one matrix-core instruction beyond binary32 rounding of the
# accumulator: |D - D_exact| <= EPS * 2^floor(log2 max_k |a_k b_k|), EPS the
# largest ratio tests/test_mfma_accuracy.py measures on the workloads'
# operand distributions (2^-11.04 for e4m3, 2^-22.07 for bf16), rounded up
# to a power of two; that test fails if the hardware exceeds it.
EPS_E4M3_MFMA = 2.0 ** -11
EPS_BF16_MFMA = 2.0 ** -22

GUARD = 4096          # sentinel elements on each side of O and LSE
SENTINEL_BF16 = 0x7FC1  # a NaN pattern the kernel never writes
SENTINEL_F32 = 0x7FC00001


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    eat.load_library()


def dev_u16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_u8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


class Guarded:
    """O (bf16) and LSE (fp32) buffers with sentinel-filled margins."""

    def __init__(self, B, N, H, d):
        self.no = B * N * H * d
        self.nl = B * H * N
        self.o_raw = torch.full((self.no + 2 * GUARD,), SENTINEL_BF16, dtype=torch.int16,
                                device="cuda")
        self.l_raw = torch.full((self.nl + 2 * GUARD,), SENTINEL_F32, dtype=torch.int32,
                                device="cuda")
        self.shape = (B, N, H, d)
        self.lshape = (B, H, N)

    @property
    def o_ptr(self):
        return self.o_raw.data_ptr() + 2 * GUARD

    @property
    def l_ptr(self):
        return self.l_raw.data_ptr() + 4 * GUARD

    def o(self):
        return self.o_raw[GUARD:GUARD + self.no].view(torch.bfloat16).view(self.shape)

    def lse(self):
        return self.l_raw[GUARD:GUARD + self.nl].view(torch.float32).view(self.lshape)

    def guards_intact(self):
        o_ok = bool((self.o_raw[:GUARD] == SENTINEL_BF16).all() and
                    (self.o_raw[GUARD + self.no:] == SENTINEL_BF16).all())
        l_ok = bool((self.l_raw[:GUARD] == SENTINEL_F32).all() and
                    (self.l_raw[GUARD + self.nl:] == SENTINEL_F32).all())
        return o_ok and l_ok


def run_bf16(inp, B, H, N, d, causal, scale):
    q, k, v = dev_u16(inp["q"]), dev_u16(inp["k"]), dev_u16(inp["v"])
    out = Guarded(B, N, H, d)
    eat.attn_fwd(q, k, v, out.o_ptr, out.l_ptr, B, H, N, d, int(causal), scale,
                 torch.cuda.current_stream())
    torch.cuda.synchronize()
    return out


def run_fp8(inp, B, H, N, d, causal, scale):
    q, k, v = dev_u8(inp["q"]), dev_u8(inp["k"]), dev_u8(inp["v"])
    dq = torch.from_numpy(inp["dq"]).reshape(-1).cuda()
    dk = torch.from_numpy(inp["dk"]).reshape(-1).cuda()
    dv = torch.from_numpy(inp["dv"]).reshape(-1).cuda()
    out = Guarded(B, N, H, d)
    eat.attn_fwd_fp8(q, k, v, out.o_ptr, out.l_ptr, dq, dk, dv, B, H, N, d, int(causal), scale,
                     torch.cuda.current_stream())
    torch.cuda.synchronize()
    return out


def reference(inp, dtype, causal, scale, rows=None):
    if dtype == "fp8":
        q = dequantize_e4m3(inp["q"], inp["dq"])
        k = dequantize_e4m3(inp["k"], inp["dk"])
        v = dequantize_e4m3(inp["v"], inp["dv"])
    else:
        q = bf16_bits_to_float64(inp["q"])
        k = bf16_bits_to_float64(inp["k"])
        v = bf16_bits_to_float64(inp["v"])
    return attention_forward(q, k, v, scale, causal, rows=rows)


def lse_bound_rows(q, k, scale, causal, rows):
    """fp8 LSE tolerance 1e-3 + EPS_E4M3_MFMA * (d / 64) * M_i (module
    docstring) for the query rows ``rows`` of one head: q [n][d], k [n][d]
    float64 dequantised inputs of that head (its K/V head for grouped
    queries).  max_j max_c |q_ic k_jc| = max_c |q_ic| * max_j |k_jc|, the
    inner maximum over the visible keys (a running maximum when causal)."""
    rows = np.asarray(rows)
    kabs = np.abs(k)
    if causal:
        kmax = np.maximum.accumulate(kabs, axis=0)[np.minimum(rows, k.shape[0] - 1)]
    else:
        kmax = kabs.max(axis=0)[None, :]
    m = abs(scale) * (np.abs(q[rows]) * kmax).max(axis=1)
    return LSE_MAXABS + EPS_E4M3_MFMA * (q.shape[1] // 64) * m


def fp8_lse_bound(inp, causal, scale, rows=None):
    """The per-row fp8 LSE tolerance of a fixed-length fp8 input set (q
    [B][N][H][d], k [B][N][H_kv][d] codes with descales), shaped like the
    oracle's lse: [B][H][N], or [B][H][R] for sampled ``rows``."""
    q = dequantize_e4m3(inp["q"], inp["dq"])
    k = dequantize_e4m3(inp["k"], inp["dk"])
    B, N, H, d = q.shape
    g = H // k.shape[2]
    R = N if rows is None else rows.shape[2]
    bound = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            r = np.arange(N) if rows is None else rows[b, h]
            bound[b, h] = lse_bound_rows(q[b, :, h, :], k[b, :, h // g, :], scale, causal, r)
    return bound


def errors(out, ref_o, ref_lse, rows=None, lse_bound=None):
    """Errors on the checked rows: (max_abs_O, rel_rms_O, max_abs_LSE), and
    with a per-row ``lse_bound`` also the largest ratio |LSE err| / bound
    as a fourth entry (the check is then that ratio <= 1)."""
    o = out.o().float().cpu().numpy().astype(np.float64)      # [B][N][H][d]
    lse = out.lse().cpu().numpy().astype(np.float64)          # [B][H][N]
    if rows is None:
        go, gl = o, lse
    else:
        B, H, R = rows.shape
        go = np.empty(ref_o.shape)
        gl = np.empty(ref_lse.shape)
        for b in range(B):
            for h in range(H):
                go[b, h] = o[b, rows[b, h], h, :]
                gl[b, h] = lse[b, h, rows[b, h]]
    return error_figures(go, ref_o, gl, ref_lse, lse_bound)


def error_figures(go, ref_o, gl, ref_lse, lse_bound=None):
    """The error tuple of ``errors`` from gathered GPU and oracle arrays."""
    diff = go - ref_o
    max_abs = float(np.abs(diff).max())
    rel_rms = float(np.sqrt((diff ** 2).sum() / (ref_o ** 2).sum()))
    lerr = np.abs(gl - ref_lse)
    if lse_bound is None:
        return max_abs, rel_rms, float(lerr.max())
    return max_abs, rel_rms, float(lerr.max()), float((lerr / lse_bound).max())


def assert_bf16_ok(err, label):
    max_abs, rel_rms, lse_abs = err
    msg = "%s: max_abs=%.3e rel_rms=%.3e lse=%.3e" % (label, max_abs, rel_rms, lse_abs)
    print(msg, flush=True)
    assert max_abs <= BF16_MAXABS, msg
    assert rel_rms <= BF16_RELRMS, msg
    assert lse_abs <= LSE_MAXABS, msg


def assert_fp8_ok(err, label):
    """``err`` must come from errors(..., lse_bound=...) (four entries)."""
    max_abs, rel_rms, lse_abs, lse_ratio = err
    msg = ("%s: max_abs=%.3e rel_rms=%.3e lse_abs=%.3e lse_err/bound=%.3f"
           % (label, max_abs, rel_rms, lse_abs, lse_ratio))
    print(msg, flush=True)
    assert rel_rms <= FP8_RELRMS, msg
    assert lse_ratio <= 1.0, msg
