"""Summaries of rocprofv3 runs of bench.py, as committed under profiles/.

    python bench_profiles.py trace    --dir D --kernel SUB --bench-log L --cmd C --title T --out F
    python bench_profiles.py counters --sq D1 --fetch D2 --write D3 --kernel SUB --workload W
                                      --dtype bf16|fp8 --key K --cmds F --title T --out F
    python bench_profiles.py traffic  --fetch D2 --write D3 --kernel SUB --key K --dtype quant
                                      --steps-total S --cmds F --title T --out F [--note F]
    python bench_profiles.py mix      --sq D1 --kernel SUB --dtype bwd --cmds F --title T --out F

``trace`` reads the ``*_kernel_stats.csv`` of a ``rocprofv3 --kernel-trace
--stats --output-format csv`` run and the bench JSON line the same run
printed, and writes the kernel's calls and average / min / max duration next
to bench.py's own HIP-event figures.

``mix`` reads one SQ run and tabulates each matching kernel (the backward
pass's three).  ``traffic`` reads only the FETCH_SIZE and WRITE_SIZE runs (for the HBM-bound
quantiser) and reports them per kernel and per step.

``counters`` reads three ``rocprofv3 --pmc`` runs (the SQ instruction and
busy counters with GRBM_GUI_ACTIVE; FETCH_SIZE; WRITE_SIZE, the last two
with bench.py's --copy-calibration), writes the per-launch averages, the
derived figures (matrix-core busy fraction, vector instructions per MFMA,
achieved clock) and the HBM bytes per launch (each counter scaled by what
it reads for the plain 1 GiB device copy in the same run), and updates the
key's line in profiles/hbm_traffic.txt and profiles/counters.txt, stamped
with bench.kernel_source_hash(dtype) so that bench.py stops quoting them
once the kernel's sources change.
"""

import argparse
import collections
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2516.6, "fp8": 5033.2}
SQ = ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
      "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]
XCDS = 8
SIMDS = 1024          # 256 compute units x 4 SIMDs
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.txt")


def _one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit("no file matches %s" % pattern)
    return hits[-1]


def bench_line(path):
    lines = [l for l in open(path) if l.startswith("{")]
    if not lines:
        raise SystemExit("no bench JSON line in %s" % path)
    return json.loads(lines[-1])


def kernel_stats(d):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*_kernel_stats.csv")))))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    return rows, total


def counter_rows(d):
    """{kernel name: {counter: [value per dispatch]}} and {kernel: [duration ns]}."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in csv.DictReader(open(_one(os.path.join(d, "**", "*_counter_collection.csv")))):
        per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[r["Kernel_Name"]][r["Dispatch_Id"]] = (float(r["End_Timestamp"]) -
                                                   float(r["Start_Timestamp"]))
    return per, {k: list(v.values()) for k, v in dur.items()}


def _avg(per, sub, name):
    vals = [v for k, c in per.items() if sub in k for v in c.get(name, [])]
    if not vals:
        raise SystemExit("no %s values for kernels matching %r" % (name, sub))
    return sum(vals) / len(vals)


def _copy_counter(per, name):
    vals = [max(c[name]) for k, c in per.items() if "copy" in k.lower() and name in c]
    if not vals:
        raise SystemExit("no device-copy dispatch with %s (run bench.py with --copy-calibration)"
                         % name)
    return max(vals)


def cmd_trace(a):
    rows, total = kernel_stats(a.dir)
    out = ["# " + a.title, "", "Command (from the repository root, library built):", "", "```",
           a.cmd, "```", "", "| kernel | calls | average µs | min µs | max µs |",
           "|---|---|---|---|---|"]
    # GPU time per step: each matching kernel's average times its launches
    # per step (its calls over the run's warm-up and timed steps)
    b = bench_line(a.bench_log)
    nsteps = b["steps"] + b["warmup"]
    share, kavg, nmatch = 0.0, 0.0, 0
    for r in rows:
        if a.kernel in r["Name"]:
            out.append("| `%s` | %s | %.1f | %.1f | %.1f |" % (
                r["Name"], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3))
            share += float(r["TotalDurationNs"])
            kavg += float(r["AverageNs"]) / 1e3 * round(float(r["Calls"]) / nsteps)
            nmatch += 1
    if not nmatch:
        raise SystemExit("no kernel matches %r" % a.kernel)
    rf = b["roofline"]
    out += ["", "Matching kernels: %.2f%% of all GPU time in the run (the rest is input upload "
            "and the finiteness check). The calls include the %d warm-up launches."
            % (100 * share / total, b["warmup"]), "",
            "The same run's bench line, with HIP events on the launch stream over the %d timed "
            "launches:" % b["steps"], ""]
    if "kernel_avg_ms" in rf:
        what = ("profiler average above" if nmatch == 1 else
                "the %d kernels' profiler averages above times their launches per step" % nmatch)
        out.append("- average step %.1f µs (%s: %.1f µs, ratio %.3f)" % (
            rf["kernel_avg_ms"] * 1e3, what, kavg, rf["kernel_avg_ms"] * 1e3 / kavg))
    out.append("- %.1f %s per launch = %.3f of the peak (%.1f %s)" % (
        rf["achieved"], rf["unit"], rf["frac"], rf["peak"], rf["unit"]))
    out.append("- whole-run value %.1f %s, %.4f ms per step" % (b["value"], b["unit"],
                                                              b["ms_per_step"]))
    if "cpu_baseline" in b:
        cb = b["cpu_baseline"]
        out.append("- oracle on the host beside it: %.4g %s on %d threads (%s)" % (
            cb["value"], cb["unit"], cb["cores"], cb["sample"]))
    with open(a.out, "w") as f:
        f.write("\n".join(out) + "\n")
    print("wrote", a.out)


def _update(path, key, fields, header):
    lines = open(path).read().splitlines() if os.path.exists(path) else header
    new = " ".join([key] + [str(x) for x in fields])
    done = False
    for i, l in enumerate(lines):
        if l.split()[:1] == [key]:
            lines[i] = new
            done = True
    if not done:
        lines.append(new)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


SQ_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + " ".join(SQ) +
          " --kernel-trace -d <out>/sq_{w} -o sq --output-format csv -- python3 /root/repo/bench.py"
          " --workload {w} --steps 3 --warmup 1 --no-cpu-baseline{x}")
CTR_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --kernel-trace -d <out>/{n}_{w} "
           "-o {n} --output-format csv -- python3 /root/repo/bench.py --workload {w} --steps 3 "
           "--warmup 1 --no-cpu-baseline --copy-calibration{x}")


def cmd_lines(a):
    if a.cmds:
        return [l.rstrip("\n") for l in open(a.cmds) if l.strip()]
    x = (" " + a.bench_args) if a.bench_args else ""
    return [SQ_CMD.format(w=a.workload, x=x),
            CTR_CMD.format(c="FETCH_SIZE", n="fetch", w=a.workload, x=x),
            CTR_CMD.format(c="WRITE_SIZE", n="write", w=a.workload, x=x)]


def cmd_counters(a):
    import bench
    sq, sq_dur = counter_rows(a.sq)
    fe, _ = counter_rows(a.fetch)
    wr, _ = counter_rows(a.write)
    cf, cw = _copy_counter(fe, "FETCH_SIZE"), _copy_counter(wr, "WRITE_SIZE")
    ff, fw = 1048576.0 / cf, 1048576.0 / cw
    fk, wk = _avg(fe, a.kernel, "FETCH_SIZE"), _avg(wr, a.kernel, "WRITE_SIZE")
    hbm = int(round((fk * ff + wk * fw) * 1024))
    vals = {c: _avg(sq, a.kernel, c) for c in SQ}
    durs = [v for k, d in sq_dur.items() if a.kernel in k for v in d]
    dur_ns = sum(durs) / len(durs)
    cycles = vals["GRBM_GUI_ACTIVE"] / XCDS
    busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cycles)
    # SQ_INSTS_VALU counts the MFMAs too
    vpm = (vals["SQ_INSTS_VALU"] - vals["SQ_INSTS_MFMA"]) / vals["SQ_INSTS_MFMA"]
    clock = cycles / dur_ns * 1e3
    src = bench.kernel_source_hash(a.dtype)
    out = ["# " + a.title, "",
           "Three runs, one counter group each (counters are never combined with a trace "
           "other than the kernel trace):", "", "```"] + \
          cmd_lines(a) + \
          ["```", "", "## Instruction mix and matrix-core activity (average per launch)", "",
           "| counter | value |", "|---|---|"]
    for c in SQ:
        out.append("| %s | %s |" % (c, "%d" % vals[c] if c == "SQ_WAVES" else "%.4g" % vals[c]))
    out += ["", "Derived (the SQ run; counters slow the kernel, whose average duration there "
            "was %.1f µs):" % (dur_ns / 1e3), "",
            "- GRBM_GUI_ACTIVE is summed over the %d XCDs: %.4g cycles per XCD per launch, "
            "%.0f MHz over the launch (the counter window is slightly longer than the kernel, "
            "so this is a lower bound on the clock it held)" % (XCDS, cycles, clock),
            "- matrix cores busy: SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x cycles per XCD) = "
            "%.3f (%.1f busy cycles per MFMA instruction)" % (
                SIMDS, busy, vals["SQ_VALU_MFMA_BUSY_CYCLES"] / vals["SQ_INSTS_MFMA"]),
            "- vector ALU instructions (other than MFMAs) per MFMA: %.2f; LDS instructions per "
            "MFMA: %.2f" % (
                vpm, vals["SQ_INSTS_LDS"] / vals["SQ_INSTS_MFMA"]),
            "", "## HBM traffic per launch", "",
            "The 1 GiB device copy that `--copy-calibration` runs after the timed region reads "
            "%.0f KiB with FETCH_SIZE and %.0f KiB with WRITE_SIZE, so the scale factors are "
            "%.4f and %.4f." % (cf, cw, ff, fw), "",
            "| | counter KiB | scaled MiB |", "|---|---|---|",
            "| FETCH_SIZE | %.1f | %.1f |" % (fk, fk * ff / 1024),
            "| WRITE_SIZE | %.1f | %.1f |" % (wk, wk * fw / 1024),
            "| total | | %.1f |" % (hbm / 2 ** 20), "",
            "Kernel source hash (bench.py `kernel_source_hash('%s')`): `%s`" % (a.dtype, src)]
    with open(a.out, "w") as f:
        f.write("\n".join(out) + "\n")
    _update(TRAFFIC_FILE, a.key, [src, "%.1f" % fk, "%.5f" % ff, "%.1f" % wk, "%.5f" % fw, hbm],
            ["# HBM bytes per launch of the attention kernels, from rocprofv3 FETCH_SIZE and",
             "# WRITE_SIZE runs, each counter scaled by what it reads for a plain 1 GiB device",
             "# copy in the same run (written by bench_profiles.py counters).",
             "# key kernel_source_hash fetch_KiB fetch_factor write_KiB write_factor hbm_bytes"])
    _update(COUNTERS_FILE, a.key, [src] + ["%.6g" % vals[c] for c in SQ] + ["%.1f" % dur_ns],
            ["# Per-launch averages of the SQ counters of the attention kernels (rocprofv3",
             "# --pmc, written by bench_profiles.py counters), with the launch's duration",
             "# under counters.",
             "# key kernel_source_hash " + " ".join(SQ) + " duration_ns"])
    print("wrote", a.out, "hbm", hbm, "busy %.3f valu/mfma %.2f clock %.0f" % (busy, vpm, clock))


def cmd_traffic(a):
    """HBM traffic only (FETCH_SIZE and WRITE_SIZE runs, no SQ run): per
    kernel per dispatch, and per step for a multi-launch entry point."""
    import bench
    fe, _ = counter_rows(a.fetch)
    wr, _ = counter_rows(a.write)
    cf, cw = _copy_counter(fe, "FETCH_SIZE"), _copy_counter(wr, "WRITE_SIZE")
    ff, fw = 1048576.0 / cf, 1048576.0 / cw
    rows, tf, tw = [], 0.0, 0.0
    for name in sorted(k for k in fe if a.kernel in k):
        f = sum(fe[name]["FETCH_SIZE"]) / len(fe[name]["FETCH_SIZE"])
        w = sum(wr[name]["WRITE_SIZE"]) / len(wr[name]["WRITE_SIZE"])
        per_step = round(len(fe[name]["FETCH_SIZE"]) / a.steps_total)
        rows.append((name, f, w, per_step))
        tf += f * per_step
        tw += w * per_step
    if not rows:
        raise SystemExit("no kernel matches %r" % a.kernel)
    hbm = int(round((tf * ff + tw * fw) * 1024))
    src = bench.kernel_source_hash(a.dtype)
    cmds = [l.rstrip("\n") for l in open(a.cmds) if l.strip()]
    out = ["# " + a.title, "", "Two runs, one counter each (never combined with traces other "
           "than the kernel trace):", "", "```"] + cmds + ["```", ""]
    if a.note:
        out += [open(a.note).read().strip(), ""]
    out += ["The 1 GiB device copy after the timed region calibrates the counters: FETCH_SIZE "
            "reads %.0f KiB for it (scale factor %.4f), WRITE_SIZE %.0f KiB (%.4f)." % (
                cf, ff, cw, fw), "",
            "| kernel | launches per step | FETCH_SIZE KiB per launch | WRITE_SIZE KiB per launch |",
            "|---|---|---|---|"]
    for name, f, w, n in rows:
        out.append("| `%s` | %d | %.1f | %.1f |" % (name, n, f, w))
    out += ["", "Per step, scaled: %.1f MiB fetched + %.1f MiB written = %.1f MiB." % (
        tf * ff / 1024, tw * fw / 1024, hbm / 2 ** 20), "",
            "Kernel source hash (bench.py `kernel_source_hash('%s')`): `%s`" % (a.dtype, src)]
    with open(a.out, "w") as f:
        f.write("\n".join(out) + "\n")
    _update(TRAFFIC_FILE, a.key, [src, "%.1f" % tf, "%.5f" % ff, "%.1f" % tw, "%.5f" % fw, hbm],
            ["# key kernel_source_hash fetch_KiB fetch_factor write_KiB write_factor hbm_bytes"])
    print("wrote", a.out, "hbm", hbm)


def cmd_mix(a):
    """SQ instruction mix only (one run), kernel by kernel: for a
    multi-kernel entry point such as the backward pass."""
    import bench
    sq, sq_dur = counter_rows(a.sq)
    cmds = [l.rstrip("\n") for l in open(a.cmds) if l.strip()]
    out = ["# " + a.title, "", "One run of the SQ counter group (never combined with traces "
           "other than the kernel trace):", "", "```"] + cmds + ["```", "",
           "| kernel | µs under counters | MHz | matrix cores busy | VALU per MFMA | "
           "LDS per MFMA | LDS bank conflicts |", "|---|---|---|---|---|---|---|"]
    for name in sorted(k for k in sq if a.kernel in k):
        v = {c: sum(sq[name][c]) / len(sq[name][c]) for c in SQ}
        dur = sum(sq_dur[name]) / len(sq_dur[name])
        cyc = v["GRBM_GUI_ACTIVE"] / XCDS
        mf = v["SQ_INSTS_MFMA"]
        per = (lambda x: "%.2f" % (x / mf)) if mf > 0 else (lambda x: "-")
        out.append("| `%s` | %.1f | %.0f | %.3f | %s | %s | %.3g |" % (
            name, dur / 1e3, cyc / dur * 1e3, v["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cyc),
            per(v["SQ_INSTS_VALU"] - mf), per(v["SQ_INSTS_LDS"]), v["SQ_LDS_BANK_CONFLICT"]))
    out += ["", "Matrix cores busy: SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x GRBM_GUI_ACTIVE "
            "per XCD); VALU per MFMA excludes the MFMAs (SQ_INSTS_VALU counts them); the clock "
            "is GRBM_GUI_ACTIVE per XCD over the kernel's duration (a lower bound, and meaningless "
            "for a kernel as short as the counter window's overhead)." % SIMDS, "",
            "Kernel source hash (bench.py `kernel_source_hash('%s')`): `%s`" % (
                a.dtype, bench.kernel_source_hash(a.dtype))]
    with open(a.out, "w") as f:
        f.write("\n".join(out) + "\n")
    print("wrote", a.out)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--bench-log", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    for n in ("--sq", "--fetch", "--write", "--kernel", "--workload", "--key", "--title", "--out"):
        c.add_argument(n, required=True)
    c.add_argument("--cmds", default=None,
                   help="file with the three rocprofv3 commands (default: the standard ones for "
                        "--workload and --bench-args)")
    c.add_argument("--bench-args", default="", help="extra bench.py arguments of the runs")
    c.add_argument("--dtype", required=True, choices=["bf16", "fp8", "quant", "bwd"])
    r = sub.add_parser("traffic")
    for n in ("--fetch", "--write", "--kernel", "--key", "--title", "--out", "--cmds"):
        r.add_argument(n, required=True)
    r.add_argument("--steps-total", type=int, required=True,
                   help="warm-up plus timed steps of the counter runs")
    r.add_argument("--note", default=None, help="file with a paragraph for the summary")
    r.add_argument("--dtype", required=True, choices=["bf16", "fp8", "quant", "bwd"])
    m = sub.add_parser("mix")
    for n in ("--sq", "--kernel", "--title", "--out", "--cmds"):
        m.add_argument(n, required=True)
    m.add_argument("--dtype", required=True, choices=["bf16", "fp8", "quant", "bwd"])
    a = ap.parse_args()
    {"trace": cmd_trace, "counters": cmd_counters, "traffic": cmd_traffic, "mix": cmd_mix}[a.what](a)


if __name__ == "__main__":
    main()
