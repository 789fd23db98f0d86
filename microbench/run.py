"""Runs the gfx950 microbenchmarks of ``mb_kernels.hip`` on cuda:0 and
prints a Markdown table (also written to ``--out``).

    python -m microbench.run [--out FILE] [--quick]

Every figure is in cycles of the shader clock (s_memtime), taken per wave
around the timed loop; one work-group per compute unit.  The clock each run
held is the shader cycles over the real-time counter (100 MHz).

Rows:
  valu      cycles per vector instruction per SIMD, for 16 independent chains
            of one operation (fma, exp, add, cvt_pk_bf16) or a softmax mix,
            with 1, 2 or 4 waves per SIMD;
  mfma      cycles per v_mfma_f32_32x32x16_bf16 per SIMD (4 independent
            accumulators), accumulators in VGPRs or AGPRs, alone and with a
            softmax-mix wave on the same SIMD (and that wave's cycles per
            vector instruction);
  mfma+valu in one wave
            cycles per MFMA when one wave per SIMD issues its MFMAs with 0-5
            independent vector instructions after each, the A operand from
            registers or LDS;
  lds       LDS bytes read per cycle per compute unit (ds_read_b128,
            ds_read_b64, ds_read_b64_tr_b16) with 4, 8 or 16 waves;
  mfma+lds  cycles per MFMA when its A operand is a 1 KiB ds_read_b128
            fragment, as in the attention kernels' matrix-core phase;
  atomics   fp32 atomic adds in the pattern a backward pass would need to
            accumulate dQ across key tiles (long8k's 32 heads, N = 8192,
            d = 128), against plain stores of the same addresses.
"""

import argparse
import os
import statistics
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _stamps(buf, waves):
    # [grid][waves][c0, c1, r0, r1, hw_id, xcc_id, -, -]
    return buf.cpu().numpy().reshape(-1, waves, 8)


def _placement(s):
    """Work-groups per compute unit (max over units), from each work-group's
    first wave: HW_ID bits 15:8 (engine, array, CU) and XCC_ID."""
    hw = s[:, 0, 4].astype(np.int64)
    xcc = s[:, 0, 5].astype(np.int64)
    key = (xcc & 0xF) * 256 + ((hw >> 8) & 0xFF)
    _, counts = np.unique(key, return_counts=True)
    return int(counts.max())


class Runner:
    def __init__(self, grid):
        import torch
        import microbench
        self.torch = torch
        self.lib = microbench.load()
        self.grid = grid
        self.stream = torch.cuda.current_stream().cuda_stream
        self.stamps = torch.zeros(grid * 16 * 8, dtype=torch.int64, device="cuda")
        self.max_per_cu = 0
        self.sink = torch.zeros(grid * 1024, dtype=torch.float32, device="cuda")

    def _launch(self, fn, *args):
        for _ in range(2):                       # the first launch warms up
            st = fn(*args, self.stamps.data_ptr(), self.sink.data_ptr(), self.stream)
            if st != 0:
                raise RuntimeError("launch failed: hipError %d" % st)
        self.torch.cuda.synchronize()

    def _read(self, waves):
        s = _stamps(self.stamps[:self.grid * waves * 8], waves)
        self.max_per_cu = max(self.max_per_cu, _placement(s))
        return (s[:, :, 1] - s[:, :, 0]).astype(np.float64), (s[:, :, 3] - s[:, :, 2]).astype(
            np.float64)

    def valu(self, op, waves, iters):
        self._launch(self.lib.mb_valu_rate, op, self.grid, waves, iters)
        return self._read(waves)

    def pair(self, acc, mfma_waves, valu, iters):
        self._launch(self.lib.mb_mfma_pair, acc, self.grid, mfma_waves, valu, iters)
        return self._read(8)

    def lds(self, kind, waves, iters):
        self._launch(self.lib.mb_lds_read, kind, self.grid, waves, iters)
        return self._read(waves)

    def mfma_lds(self, mfma_waves, valu, iters):
        self._launch(self.lib.mb_mfma_lds, self.grid, mfma_waves, valu, iters)
        return self._read(8)

    def tile_loads(self, kind, per_wave, loaders, iters):
        if not hasattr(self, "src"):
            self.src = self.torch.zeros(512 << 20, dtype=self.torch.uint8, device="cuda")
        for _ in range(2):
            st = self.lib.mb_tile_loads(kind, per_wave, loaders, self.grid, iters,
                                        self.src.data_ptr(), self.src.numel(),
                                        self.stamps.data_ptr(), self.sink.data_ptr(), self.stream)
            if st != 0:
                raise RuntimeError("launch failed: hipError %d" % st)
        self.torch.cuda.synchronize()
        s = _stamps(self.stamps[:self.grid * 8 * 8], 8)
        return (s[:, :loaders, 0].astype(np.float64), s[:, :loaders, 1].astype(np.float64),
                s[:, :loaders, 2].astype(np.float64))

    def inwave(self, m, ldsr, iters, waves=4):
        self._launch(self.lib.mb_mfma_inwave, m, ldsr, waves, self.grid, iters)
        return self._read(waves)

    def chain(self, nch, waves, iters):
        self._launch(self.lib.mb_mfma_chain, nch, waves, self.grid, iters)
        return self._read(waves)

    def lds_latency(self, kind, iters):
        self._launch(self.lib.mb_lds_latency, kind, self.grid, iters)
        return self._read(4)

    def dq_atomics(self, bh, n, reps):
        """ms per launch of the atomic and the plain-store form, and the
        number of elements whose atomic sum (one launch from zero) differs
        from the exact value."""
        torch = self.torch
        acc = torch.zeros(bh * n * 128, dtype=torch.float32, device="cuda")
        out = {}
        for mode in (1, 0):
            for _ in range(2):
                if self.lib.mb_dq_atomics(mode, bh, n, acc.data_ptr(), 1.0, self.stream) != 0:
                    raise RuntimeError("mb_dq_atomics failed")
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                self.lib.mb_dq_atomics(mode, bh, n, acc.data_ptr(), 1.0, self.stream)
            b.record()
            torch.cuda.synchronize()
            out[mode] = a.elapsed_time(b) / reps
        acc.zero_()
        if self.lib.mb_dq_atomics(0, bh, n, acc.data_ptr(), 1.0, self.stream) != 0:
            raise RuntimeError("mb_dq_atomics failed")
        torch.cuda.synchronize()
        got = acc.view(bh, n, 128).cpu().numpy()
        row = np.arange(n)
        x = row % 32
        want = ((row // 64) // 2 + 1) * (4 * (x // 8) + x % 4 + 1)
        bad = int((got != want[None, :, None].astype(np.float32)).sum())
        return out[0], out[1], bad


def _mhz(cyc, rt):
    ok = rt > 0
    return float(np.median(cyc[ok] / (rt[ok] * 10e-9) / 1e6)) if ok.any() else float("nan")


VALU_OPS = [(0, "v_fma_f32", 16), (1, "v_exp_f32", 16), (2, "v_add_f32", 16),
            (3, "v_cvt_pk_bf16_f32", 8), (5, "v_exp_f32 and v_fma_f32 alternating", 16),
            (4, "softmax mix (fma, exp, add, cvt, xor)", 57)]


def run(quick=False, only=None):
    """All rows, or (only = list of "chain", "ldslat", "atomics") just those groups."""
    import torch

    def want(name):
        return only is None or name in only
    props = torch.cuda.get_device_properties(0)
    grid = props.multi_processor_count
    r = Runner(grid)
    k = 4 if quick else 1
    rows = []

    # MFMA dependency chains: cycles per MFMA with 1-4 chains per wave
    if want("chain"):
        for waves in (4, 8):
            for nch in (1, 2, 3, 4):
                iters = 2000 // k
                cyc, rt = r.chain(nch, waves, iters)
                mf = np.median(cyc.max(axis=1)) / (iters * 8 * nch * (waves // 4))
                rows.append(("mfma chains", "32x32x16 bf16, %d chain(s) per wave" % nch,
                             "%d wave(s)/SIMD" % (waves // 4),
                             "%.2f cycles per MFMA per SIMD" % mf, _mhz(cyc, rt)))

    # LDS read latency (dependent reads, one wave per SIMD)
    if want("ldslat"):
        for kind, name in ((0, "ds_read_b32"), (1, "ds_read_b128")):
            iters = 2000 // k
            cyc, rt = r.lds_latency(kind, iters)
            rows.append(("lds latency", name, "1 wave/SIMD, dependent reads",
                         "%.1f cycles per read" % (np.median(cyc) / (iters * 16)),
                         _mhz(cyc, rt)))
    # fp32 atomics in the pattern of a causal backward accumulating dQ (32 heads,
    # N = 8192, d = 128: every 128-key tile adds into the rows of the queries it sees)
    if want("atomics"):
        bh, n = 32, 8192
        tiles = bh * sum(n // 64 - 2 * kt for kt in range(n // 128))
        gb = tiles * 64 * 128 * 4 / 1e9
        t_at, t_st, bad = r.dq_atomics(bh, n, 3 if quick else 5)
        rows.append(("atomics", "global_atomic_add_f32 (agent scope, no return), "
                     "%.2f GB of fp32 adds" % gb, "4 waves per work-group, %d work-groups" % (
                         bh * n // 128),
                     "%.3f ms = %.0f GB/s (plain stores of the same addresses: %.3f ms = %.0f "
                     "GB/s); exact sums, %d elements differ" % (t_at, gb / t_at * 1e3, t_st,
                                                               gb / t_st * 1e3, bad),
                     float("nan")))
    if only:
        return props, rows, r.max_per_cu

    # vector ALU issue rates
    for op, name, per in VALU_OPS:
        for waves in (4, 8, 16):
            iters = 20000 // k
            cyc, rt = r.valu(op, waves, iters)
            per_simd = waves // 4
            # the slowest wave of each work-group bounds its SIMDs
            v = np.median(cyc.max(axis=1)) / (iters * per * per_simd)
            rows.append(("valu", name, "%d wave(s)/SIMD" % per_simd,
                         "%.2f cycles per instruction per SIMD" % v, _mhz(cyc, rt)))

    # MFMA rate, alone and beside a vector wave
    for acc, accname in ((0, "VGPR acc"), (1, "AGPR acc")):
        iters = 4000 // k
        cyc, rt = r.pair(acc, 4, 0, iters)
        mf_alone = np.median(cyc[:, :4]) / (iters * 32)
        rows.append(("mfma", "32x32x16 bf16, " + accname, "1 MFMA wave/SIMD",
                     "%.2f cycles per MFMA" % mf_alone, _mhz(cyc[:, :4], rt[:, :4])))
        cyc, rt = r.pair(acc, 8, 0, iters)
        mf2 = np.median(cyc.max(axis=1)) / (iters * 32 * 2)
        rows.append(("mfma", "32x32x16 bf16, " + accname, "2 MFMA waves/SIMD",
                     "%.2f cycles per MFMA per SIMD" % mf2, _mhz(cyc, rt)))
        cyc, rt = r.pair(acc, 4, 1, iters)
        mf = np.median(cyc[:, :4]) / (iters * 32)
        va = np.median(cyc[:, 4:]) / (2 * iters * 57)
        rows.append(("mfma", "32x32x16 bf16, " + accname, "+1 softmax wave/SIMD",
                     "%.2f cycles per MFMA; partner %.2f cycles per vector instruction "
                     "(114 per 32 MFMAs)" % (mf, va), _mhz(cyc, rt)))
    cyc, rt = r.pair(0, 0, 1, 4000 // k)
    va = np.median(cyc[:, 4:]) / (2 * (4000 // k) * 57)
    rows.append(("mfma", "(softmax wave alone)", "1 wave/SIMD",
                 "%.2f cycles per vector instruction" % va, _mhz(cyc[:, 4:], rt[:, 4:])))

    # one or two waves per SIMD, each interleaving its own MFMAs and vector work
    for waves in (4, 8):
        for ldsr, lname in ((0, "A in registers"), (1, "A from LDS, 1 read per MFMA"),
                            (2, "A from LDS, 1 read per 2 MFMAs")):
            for m in (0, 4, 6, 8, 10):
                iters = 8000 // k
                cyc, rt = r.inwave(m, ldsr, iters, waves)
                mf = np.median(cyc.max(axis=1)) / (iters * 16 * (waves // 4))
                rows.append(("mfma+valu in one wave", "32x32x16 bf16, " + lname,
                             "%d wave(s)/SIMD, %d vector per MFMA" % (waves // 4, m // 2),
                             "%.2f cycles per MFMA per SIMD" % mf, _mhz(cyc, rt)))

    # tile loads: 32 KiB per round per work-group, as the attention kernels load a K/V tile
    for kind, per_wave, loaders in ((0, 8, 4), (0, 4, 8), (0, 2, 8), (1, 8, 4), (1, 4, 8)):
        iters = 400 // k
        iss, drn, lgkm = r.tile_loads(kind, per_wave, loaders, iters)
        name = "global_load_lds_dwordx4 (to LDS)" if kind == 0 else "global_load_dwordx4 (to VGPRs)"
        txt = ("issue %.0f, then an lgkmcnt(0) wait %.0f, then the vmcnt(0) drain %.0f cycles "
               "per wave per round" % (np.median(iss) / iters, np.median(lgkm) / iters,
                                       np.median(drn) / iters)
               if kind == 0 else "issue and wait %.0f cycles per wave per round"
               % (np.median(iss) / iters))
        rows.append(("tile loads", name, "%d loader waves x %d KiB" % (loaders, per_wave), txt,
                     float("nan")))

    # LDS read bandwidth
    for kind, name, nbytes in ((0, "ds_read_b128", 1024), (1, "ds_read_b64", 512),
                               (2, "ds_read_b64_tr_b16", 512)):
        for waves in (4, 8, 16):
            iters = 8000 // k
            cyc, rt = r.lds(kind, waves, iters)
            bpc = waves * iters * 8 * nbytes / cyc.max(axis=1)
            rows.append(("lds", name, "%d waves/CU" % waves,
                         "%.1f bytes per cycle per CU" % float(np.median(bpc)), _mhz(cyc, rt)))

    # MFMA with its A operand from LDS
    iters = 8000 // k
    for mw, valu, label in ((4, 0, "1 MFMA wave/SIMD"), (8, 0, "2 MFMA waves/SIMD"),
                            (4, 1, "1 MFMA wave + 1 softmax wave/SIMD")):
        cyc, rt = r.mfma_lds(mw, valu, iters)
        per_simd = mw // 4
        mf = np.median(cyc[:, :mw].max(axis=1)) / (iters * 16 * per_simd)
        txt = "%.2f cycles per MFMA per SIMD (%.1f LDS bytes per cycle per CU)" % (
            mf, 4 * 1024 / mf)
        if valu:
            va = np.median(cyc[:, 4:]) / (iters * 57)
            txt += "; partner %.2f cycles per vector instruction (57 per 16 MFMAs)" % va
        rows.append(("mfma+lds", "32x32x16 bf16, A from ds_read_b128", label, txt,
                     _mhz(cyc, rt)))
    return props, rows, r.max_per_cu


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    ap.add_argument("--quick", action="store_true", help="a quarter of the iterations")
    ap.add_argument("--only", default=None,
                    help="comma-separated groups to run alone: chain, ldslat, atomics")
    args = ap.parse_args()
    import torch
    if not torch.cuda.is_available():
        print("microbench needs a GPU", file=sys.stderr)
        sys.exit(1)
    props, rows, per_cu = run(args.quick, args.only.split(",") if args.only else None)
    lines = ["# gfx950 microbenchmarks", "",
             "Command: `python -m microbench.run%s`" % (" --quick" if args.quick else ""), "",
             "Device: %s, %d compute units; one work-group per compute unit; figures in shader "
             "clock cycles (s_memtime), median over work-groups; at most %d work-group(s) "
             "shared a compute unit in any run (HW_ID / XCC_ID)." % (
                 props.name, props.multi_processor_count, per_cu),
             "", "| unit | what | waves | result | clock MHz |", "|---|---|---|---|---|"]
    for row in rows:
        lines.append("| %s | %s | %s | %s | %.0f |" % row)
    text = "\n".join(lines) + "\n"
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)


if __name__ == "__main__":
    main()
