"""Throughput of the tiled exact attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--workload ctx32k]
                    [--no-cpu-baseline] [--copy-calibration]

A step is one pass of the whole hot path -- one attn_fwd (or attn_fwd_fp8)
launch: Q/K/V tile loads, both MFMA products, the online softmax with its
gated rescale, causal masking, and the O/LSE epilogue -- over one batch of
seeded synthetic inputs already resident in HBM.  W untimed steps, then K
steps timed with HIP events on the stream the kernel is launched on (torch's
current stream).  Prints ONE JSON line.

Default workload ctx32k: B=1, H=32, N=32768, d=128, bf16, causal, scale
1/sqrt(d), 1% of each head's K rows scaled by 8 -- the largest configuration
the throughput target is stated for (N >= 8192, d = 128) that fits one GPU.
Other workloads (--workload: long8k, fp8_8k, ...) are timed the same way;
the parity tests cover all of them.

TFLOPS = 4*B*H*N^2*d (halved when causal) / time per step.

Other passes (--pass), each timed the same way with its own JSON line:
  fwd2   the two-pass fp8 forward (attn_fwd_fp8_2pass), fp8 workloads;
  bwd    the backward pass (attn_bwd), bf16 workloads, TFLOPS counted as
         2.5 x the forward's;
  quant  the E4M3 quantisation of Q, K (rotated) and V (attn_fp8_quantize),
         fp8 workloads, GB/s of algorithmic bytes against the HBM peak.
Each line carries the oracle timed on the host beside it (cpu_baseline),
unless --no-cpu-baseline.
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2}   # 256 CU x 2.4 GHz dense MFMA
METRIC = "attn fwd TFLOPS (4BHN²d, causal halved) + % of MI355X MFMA peak, 1 GPU"
METRIC_BWD = "attn bwd TFLOPS (2.5 x 4BHN²d, causal halved) + % of MI355X MFMA peak, 1 GPU"
METRIC_QUANT = ("fp8 input quantisation GB/s (Q, K rotated + V; 3 B per element: bf16 in, "
                "e4m3 out) + % of MI355X HBM peak, 1 GPU")
PEAK_HBM_GBS = 8000.0
METRIC_FWD2 = ("attn fwd fp8 two-pass TFLOPS (4BHN²d, causal halved; the row-maximum pass is "
               "not counted) + % of MI355X MFMA peak, 1 GPU")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.txt")
MICROBENCH_FILE = os.path.join(ROOT, "profiles", "gfx950_microbench.md")
CUS, SIMDS, XCDS, CLOCK_GHZ = 256, 1024, 8, 2.4
SQ_FIELDS = ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
             "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]


KERNEL_SOURCES = {"quant": ("attn_quant.hip", "attn_kernels.hpp", "attn_api.cpp"),
                  "bf16": ("attn_fwd_bf16.hip", "attn_kernels.hpp", "attn_api.cpp"),
                  "fp8": ("attn_fwd_fp8.hip", "attn_kernels.hpp", "attn_api.cpp"),
                  "bwd": ("attn_bwd_bf16.hip", "attn_kernels.hpp", "attn_api.cpp")}


def kernel_source_hash(dtype):
    """Hash of the sources the dtype's kernel is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_tile_amd", "csrc")
    for name in KERNEL_SOURCES[dtype]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, dtype, causal, key=None):
    """HBM bytes per launch (per step for the quantiser) from the committed
    rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE, each scaled by what it
    reads for a plain copy), if they were taken on the current kernel
    sources; else None."""
    if key is None:
        key = "%s_%s" % (workload, "causal" if causal else "noncausal")
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                fields = line.split()
                if len(fields) == 7 and fields[0] == key:
                    if fields[1] != kernel_source_hash(dtype):
                        return None
                    return int(fields[6])
    except (OSError, ValueError):
        return None
    return None


def measured_counters(key, dtype):
    """Figures derived from the committed SQ counter run of the kernel
    (profiles/counters.txt, per-launch averages), if it was taken on the
    current kernel sources; else None:
      mfma_busy      SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x engine cycles
                     per XCD): the fraction of the launch the matrix cores
                     were busy, at the clock the chip held;
      valu_per_mfma  (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA (the
                     counter of vector instructions includes the MFMAs);
      lds_per_mfma   SQ_INSTS_LDS / SQ_INSTS_MFMA;
      clock_mhz      GRBM_GUI_ACTIVE / 8 XCDs / the launch's duration under
                     counters (the engine clock held over the launch);
      lds_bank_conflict_cycles."""
    try:
        with open(COUNTERS_FILE) as f:
            for line in f:
                fields = line.split()
                if len(fields) == 2 + len(SQ_FIELDS) + 1 and fields[0] == key:
                    if fields[1] != kernel_source_hash(dtype):
                        return None
                    v = dict(zip(SQ_FIELDS, map(float, fields[2:2 + len(SQ_FIELDS)])))
                    dur_ns = float(fields[-1])
                    cycles = v["GRBM_GUI_ACTIVE"] / XCDS
                    return {
                        "source": "profiles/counters.txt (rocprofv3 --pmc, key %s)" % key,
                        "mfma_busy": round(v["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cycles), 4),
                        "valu_per_mfma": round((v["SQ_INSTS_VALU"] - v["SQ_INSTS_MFMA"]) /
                                               v["SQ_INSTS_MFMA"], 3),
                        "lds_per_mfma": round(v["SQ_INSTS_LDS"] / v["SQ_INSTS_MFMA"], 3),
                        "clock_mhz": round(cycles / dur_ns * 1e3, 1),
                        "lds_bank_conflict_cycles": v["SQ_LDS_BANK_CONFLICT"],
                        "sq_insts_valu": v["SQ_INSTS_VALU"] - v["SQ_INSTS_MFMA"],
                    }
    except (OSError, ValueError):
        return None
    return None


def microbench_figures():
    """From the committed microbenchmark table (profiles/gfx950_microbench.md):
    cycles per v_fma_f32 per SIMD with four waves per SIMD, and LDS bytes read
    per cycle per compute unit by ds_read_b128 and ds_read_b64_tr_b16 with
    16 waves.  None where the table is missing."""
    out = {"valu_cycles": None, "lds_b128": None, "lds_tr16": None}
    try:
        with open(MICROBENCH_FILE) as f:
            for line in f:
                cells = [c.strip() for c in line.strip().strip("|").split("|")]
                if len(cells) < 4:
                    continue
                try:
                    num = float(cells[3].split()[0])
                except (ValueError, IndexError):
                    continue
                if cells[0] == "valu" and cells[1] == "v_fma_f32" and cells[2].startswith("4 "):
                    out["valu_cycles"] = num
                elif cells[0] == "lds" and cells[2].startswith("16 "):
                    if cells[1] == "ds_read_b128":
                        out["lds_b128"] = num
                    elif cells[1] == "ds_read_b64_tr_b16":
                        out["lds_tr16"] = num
    except OSError:
        pass
    return out


def algorithmic_bytes(w):
    """HBM bytes one forward launch must move: Q, K, V read once, O and LSE
    written once."""
    e = 1 if w.dtype == "fp8" else 2
    T = w.total
    return T * w.d * (w.H * e + 2 * w.kv_heads * e + w.H * 2) + T * w.H * 4


def algorithmic_bytes_bwd(w):
    """HBM bytes one backward call must move: q, k, v, o and dO read once,
    dQ, dK and dV written once (bf16), lse read once, and the fp32 D
    workspace written once and read once."""
    T = w.total
    return T * w.d * 2 * (4 * w.H + 4 * w.kv_heads) + T * w.H * 4 * 3


def secondary_roofs(w, flops, achieved, ctr, mb):
    """The two on-chip roofs beside the matrix-core peak, in TFLOP/s of the
    metric's flops (each at the nominal 2.4 GHz, like the peak):
      valu  the launch's vector ALU instructions other than MFMAs
            (SQ_INSTS_VALU - SQ_INSTS_MFMA) issued back to back at the measured
            cycles per v_fma_f32 with four waves per SIMD (the SIMD's full
            rate), spread over the 1024 SIMDs;
      lds   the K and V operand reads from LDS: each 32-query wave reads the
            whole K and V tile for every tile it visits, 2 * d * e bytes per
            key, i.e. e / 64 bytes per flop (e = 2 bf16, 1 fp8), against the
            measured ds_read bandwidth (ds_read_b128 for K, the transposing
            read for V: their mean)."""
    out = {}
    if ctr is not None and mb["valu_cycles"]:
        t = ctr["sq_insts_valu"] / SIMDS * mb["valu_cycles"] / (CLOCK_GHZ * 1e9)
        roof = flops / t / 1e12
        out["valu"] = {"roof": round(roof, 1), "frac": round(achieved / roof, 4),
                       "basis": "SQ_INSTS_VALU x %.2f cycles / 1024 SIMDs at 2.4 GHz"
                                % mb["valu_cycles"]}
    if mb["lds_b128"] and mb["lds_tr16"]:
        e = 1 if w.dtype == "fp8" else 2
        bw = 0.5 * (mb["lds_b128"] + mb["lds_tr16"]) * CUS * CLOCK_GHZ * 1e9
        roof = bw / (e / 64.0) / 1e12
        out["lds"] = {"roof": round(roof, 1), "frac": round(achieved / roof, 4),
                      "basis": "%.3f LDS bytes per flop at %.1f B/clk/CU" % (
                          e / 64.0, 0.5 * (mb["lds_b128"] + mb["lds_tr16"]))}
    return out or None


def _head_problem(w, inp, b, h):
    """float64 q, k, v [n][d] of (batch or sequence b, query head h), exactly
    as the GPU sees them (the K/V head is h // (H / Hkv))."""
    from oracle import bf16_bits_to_float64, dequantize_e4m3
    hk = h // (w.H // w.kv_heads)
    if w.varlen:
        s0, s1 = int(inp["cu"][b]), int(inp["cu"][b + 1])
        sl, bi = (slice(0, 1), slice(s0, s1)), 0
    else:
        sl, bi = (slice(b, b + 1), slice(None)), b
    if w.dtype == "fp8":
        def deq(name, head):
            return dequantize_e4m3(inp[name][sl[0], sl[1], head:head + 1, :],
                                   inp["d" + name][b:b + 1, head:head + 1])[0, :, 0, :]
        return deq("q", h), deq("k", hk), deq("v", hk)
    return (bf16_bits_to_float64(inp["q"][bi, sl[1], h, :]),
            bf16_bits_to_float64(inp["k"][bi, sl[1], hk, :]),
            bf16_bits_to_float64(inp["v"][bi, sl[1], hk, :]))


def _one_head(w, inp, causal, b, h, rows):
    from oracle import attention_head_rows
    q, k, v = _head_problem(w, inp, b, h)
    return attention_head_rows(q, k, v, w.scale, causal, rows)


def _rows_for(w, count, b, h, n):
    """``count`` seeded query rows of a length-n problem (all when n <= count)."""
    if n <= count:
        return np.arange(n)
    g = np.random.default_rng(1000 * w.wid + 7 + 131 * b + h)
    return np.concatenate([[0, n - 1], np.sort(g.choice(np.arange(1, n - 1), count - 2,
                                                        replace=False))])


def cpu_baseline(w, inp, causal, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the same workload:
    seeded query rows of every (batch or sequence, head) problem, as many per
    problem as fit in about ``budget_s`` seconds.  A 512-row probe sizes a
    first pass; a pass that ends in under half the budget is discarded and
    repeated with the row count scaled up (at most twice)."""
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    lens = list(w.lengths) if w.varlen else [w.N] * w.B
    heads = [(b, h) for b in range(len(lens)) for h in range(w.H) if lens[b] > 0]
    b0 = max(range(len(lens)), key=lambda b: lens[b])
    probe = _rows_for(w, min(512, lens[b0]), b0, 0, lens[b0])
    _one_head(w, inp, causal, b0, 0, probe)                 # thread pools warm up
    t0 = time.perf_counter()
    _one_head(w, inp, causal, b0, 0, probe)
    per_row = (time.perf_counter() - t0) / probe.shape[0]
    count = int(min(max(lens), max(512, budget_s / max(per_row, 1e-9) / len(heads))))
    for attempt in range(3):
        flops = 0.0
        done = 0
        nrows = 0
        t0 = time.perf_counter()
        for (b, h) in heads:
            r = _rows_for(w, count, b, h, lens[b])
            _one_head(w, inp, causal, b, h, r)
            vis = (r + 1) if causal else np.full(r.shape, lens[b])
            flops += float(4.0 * w.d * vis.sum())
            done += 1
            nrows += r.shape[0]
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        if dt >= 0.5 * budget_s or count >= max(lens) or attempt == 2:
            break
        count = int(min(max(lens), count * budget_s / max(dt, 1e-3)))
    rate = flops / dt
    return {
        "value": rate / 1e12,
        "unit": "TFLOPS",
        "cores": int(cores),
        "kind": "oracle",
        "sample": "fp64 NumPy oracle on up to %d seeded query rows of each of %d/%d (batch, head) "
                  "problems (%d rows, %.2f GFLOP counted with the metric's 4*d*visible_keys per "
                  "row, %.1f s)" % (count, done, len(heads), nrows, flops / 1e9, dt),
        "extrapolated_full_config_s": round(w.flops(causal) / rate, 1),
        "extrapolation": "an extrapolation, not a measurement: the whole workload's flops "
                         "(%.4g) at the sample's rate" % w.flops(causal),
    }


def bwd_cpu_baseline(w, inp, dout_bits, causal, budget_s=12.0):
    """The gradient oracle, as it stands, on whole (batch, head) problems of
    the same workload taken in order until about ``budget_s`` seconds have
    passed (at least one), counted with the metric's 2.5 x 4 d N^2 per head
    (halved when causal)."""
    from oracle import attention_backward_head, bf16_bits_to_float64
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    per_head = 2.5 * 4.0 * w.d * w.N * w.N / (2.0 if causal else 1.0)
    done = 0
    t0 = time.perf_counter()
    for (b, h) in heads:
        q, k, v, do = (bf16_bits_to_float64(x[b, :, h, :]) for x in
                       (inp["q"], inp["k"], inp["v"], dout_bits))
        attention_backward_head(q, k, v, do, w.scale, causal)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": per_head * done / dt / 1e12,
        "unit": "TFLOPS",
        "cores": int(cores),
        "kind": "oracle",
        "sample": "fp64 NumPy gradient oracle on %d of %d whole (batch, head) problems "
                  "(N=%d, d=%d, %.1f s)" % (done, len(heads), w.N, w.d, dt),
    }


def quant_line(args, w, ms_per_step, avg_launch_ms, src_elems):
    """The JSON line of --pass quant: bytes are algorithmic (each bf16 input
    element read once, each code written once); the second read pass of the
    two-pass quantiser is overhead, visible in the measured traffic."""
    nbytes = 3.0 * src_elems
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_launch_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC_QUANT, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded, workloads/)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "pass": "quant",
                   "rotation": "Q and K (random Hadamard), V plain"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(w.name, "quant", False, key=w.name + "_quant"),
                     "kernel_avg_ms": round(avg_launch_ms, 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = quant_cpu_baseline(w)
    return out


def quant_cpu_baseline(w):
    """The oracle's quantiser (rotation on) on one (batch, head) of Q at the
    full sequence length, scaled to GB/s of the same algorithmic bytes."""
    from oracle import bf16_bits_to_float64, quantize_e4m3
    from workloads import make_bf16, rotation_signs
    x = bf16_bits_to_float64(make_bf16(w)["q"][:1, :, :1, :])
    signs, _ = rotation_signs(w)
    t0 = time.perf_counter()
    reps = 0
    while True:
        quantize_e4m3(x, signs)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 50:
            break
    gbs = 3.0 * x.size * reps / el / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "one (batch, head) of Q, %d rows x d=%d, rotation on, %d repetitions"
                      % (w.N, w.d, reps)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="ctx32k")
    ap.add_argument("--causal", type=int, default=None, help="override the workload's mode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=["fwd", "fwd2", "bwd", "quant"], default="fwd",
                    help="time the forward (default), the two-pass fp8 forward (fwd2), the "
                         "backward pass (bf16 workloads) or the E4M3 quantisation of the "
                         "inputs (fp8 workloads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run a plain 1 GiB device copy (for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the work would shard by (batch, head) with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_tile_amd as eat
    from workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    eat.load_library()
    w = WORKLOADS[args.workload]
    causal = bool(w.modes[0] if args.causal is None else args.causal)
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    Hkv, T = w.kv_heads, w.total
    if w.varlen:
        cu = torch.from_numpy(inp["cu"]).to(dev)
    if w.dtype == "fp8":
        q = torch.from_numpy(inp["q"]).to(dev)
        k = torch.from_numpy(inp["k"]).to(dev)
        v = torch.from_numpy(inp["v"]).to(dev)
        dq = torch.from_numpy(inp["dq"]).reshape(-1).to(dev)
        dk = torch.from_numpy(inp["dk"]).reshape(-1).to(dev)
        dv = torch.from_numpy(inp["dv"]).reshape(-1).to(dev)

        if args.which == "fwd2":
            if w.varlen:
                print("--pass fwd2 takes a fixed-length fp8 workload", file=sys.stderr)
                sys.exit(2)

            def step():
                eat.attn_fwd_fp8_2pass(q, k, v, o, lse, dq, dk, dv, w.B, w.H, Hkv, w.N, w.d,
                                       int(causal), w.scale, stream)
        elif w.varlen:
            def step():
                eat.attn_fwd_fp8_varlen(q, k, v, o, lse, dq, dk, dv, cu, w.B, T, w.N, w.H, Hkv,
                                        w.d, int(causal), w.scale, stream)
        else:
            def step():
                eat.attn_fwd_fp8_gqa(q, k, v, o, lse, dq, dk, dv, w.B, w.H, Hkv, w.N, w.d,
                                     int(causal), w.scale, stream)
    else:
        if args.which == "fwd2":
            print("--pass fwd2 takes an fp8 workload", file=sys.stderr)
            sys.exit(2)

        def dev16(x):
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        q, k, v = dev16(inp["q"]), dev16(inp["k"]), dev16(inp["v"])

        if w.varlen:
            def step():
                eat.attn_fwd_varlen(q, k, v, o, lse, cu, w.B, T, w.N, w.H, Hkv, w.d, int(causal),
                                    w.scale, stream)
        elif Hkv != w.H:
            def step():
                eat.attn_fwd_gqa(q, k, v, o, lse, w.B, w.H, Hkv, w.N, w.d, int(causal), w.scale,
                                 stream)
        else:
            def step():
                eat.attn_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.d, int(causal), w.scale, stream)

    o = torch.empty((T, w.H, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.H, T) if w.varlen else (w.B, w.H, w.N), dtype=torch.float32, device=dev)
    if args.which == "bwd":
        if w.dtype != "bf16" or w.varlen or Hkv != w.H:
            print("--pass bwd takes a bf16 multi-head workload", file=sys.stderr)
            sys.exit(2)
        from workloads import make_dout
        step()                                     # O and lse of the forward
        torch.cuda.synchronize()
        do_bits = make_dout(w)
        do = dev16(do_bits)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def step():
            eat.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, w.B, w.H, w.N, w.d, int(causal),
                         w.scale, stream)

    if args.which == "quant":
        if w.dtype != "fp8" or w.varlen:
            print("--pass quant takes a fixed-length fp8 workload", file=sys.stderr)
            sys.exit(2)
        from workloads import make_bf16, rotation_signs
        src = make_bf16(w)
        qb, kb, vb = (torch.from_numpy(src[n].view(np.int16)).to(dev).view(torch.bfloat16)
                      for n in "qkv")
        del src
        _, words = rotation_signs(w)
        sw = torch.from_numpy(words.view(np.int32)).to(dev)
        for t in (q, k, v, dq, dk, dv):
            t.zero_()

        def step():
            eat.attn_fp8_quantize(qb, q, dq, sw, w.B, w.N, w.H, w.d, stream)
            eat.attn_fp8_quantize(kb, k, dk, sw, w.B, w.N, Hkv, w.d, stream)
            eat.attn_fp8_quantize(vb, v, dv, None, w.B, w.N, Hkv, w.d, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = total_ms / args.steps
    avg_launch_ms = sum(launch_ms) / len(launch_ms)

    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    outs = [lse, o] + ([dq, dk, dv] if args.which == "bwd" else [])
    if args.which == "quant":
        outs = [dq, dk, dv]
        if not all(bool((x > 0).all()) for x in outs):
            print("quantiser wrote no descale", file=sys.stderr)
            sys.exit(1)
    if not all(bool(torch.isfinite(x.float()).all()) for x in outs):
        print("non-finite output", file=sys.stderr)
        sys.exit(1)

    if args.which == "quant":
        print(json.dumps(quant_line(args, w, ms_per_step, avg_launch_ms, src_elems=(
            w.B * w.N * (w.H + 2 * Hkv) * w.d))), flush=True)
        return

    flops = w.flops(causal) * (2.5 if args.which == "bwd" else 1.0)
    peak = PEAK_TFLOPS[w.dtype]
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": METRIC if args.which == "fwd" else METRIC_BWD,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, workloads/)",
        "config": dict({"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                        "causal": causal, "scale": w.scale,
                        "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)"},
                       **({"H_kv": Hkv} if Hkv != w.H else {}),
                       **({"seq_lens": list(w.lengths), "total_tokens": T} if w.varlen else {})),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(w.name, w.dtype, causal),
                     "kernel_avg_ms": round(avg_launch_ms, 4),
                     "kernel_median_ms": round(statistics.median(launch_ms), 4),
                     "kernel_min_ms": round(min(launch_ms), 4)},
    }
    rf = out["roofline"]
    if args.which == "fwd":
        rf["algorithmic_bytes"] = algorithmic_bytes(w)
        rf["traffic_ratio"] = (round(rf["traffic"] / rf["algorithmic_bytes"], 3)
                               if rf["traffic"] else None)
        key = "%s_%s" % (w.name, "causal" if causal else "noncausal")
        ctr = measured_counters(key, w.dtype)
        rf["counters"] = ctr
        rf["secondary"] = secondary_roofs(w, flops, achieved, ctr, microbench_figures())
        if ctr is not None:
            del ctr["sq_insts_valu"]
    if args.which in ("bwd", "fwd2"):
        out["config"]["pass"] = args.which
        rf["traffic"] = None
    if args.which == "bwd":
        # per call (the three kernels), like achieved
        rf["traffic"] = measured_traffic(w.name, "bwd", causal,
                                         key="%s_bwd%s" % (w.name, "" if causal else "_noncausal"))
        rf["algorithmic_bytes"] = algorithmic_bytes_bwd(w)
        rf["traffic_ratio"] = (round(rf["traffic"] / rf["algorithmic_bytes"], 3)
                               if rf["traffic"] else None)
    if args.which == "fwd2":
        out["metric"] = METRIC_FWD2
    if not args.no_cpu_baseline and args.which in ("fwd", "fwd2"):
        out["cpu_baseline"] = cpu_baseline(w, inp, causal)
    if not args.no_cpu_baseline and args.which == "bwd":
        out["cpu_baseline"] = bwd_cpu_baseline(w, inp, do_bits, causal)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
