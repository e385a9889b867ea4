"""Hardware counters of the library's kernels, read with rocprofv3 on an MI355X.

    python -m precision_attention_amd.counters {directp,directp_anchored,bwd,quant,project,nvfp4,bf16,causal,fp8route} OUTDIR

runs bench.py's single-kernel mode for the chosen path under rocprofv3, one process per pass
(a kernel trace, two passes of eight SQ counters, FETCH_SIZE and WRITE_SIZE, and the two byte
counters on a plain 256 MiB device copy for calibration), then prints a Markdown summary per
kernel: average duration, MFMA busy, VALU and transcendental shares, LDS bank conflicts, and
HBM bytes and GB/s. Every pass stays within the per-block counter limits of one rocprofv3 run
and runs under its own time limit. The GPU is touched only by the child processes.
"""
from __future__ import annotations

import collections
import csv
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CU_NUM, SIMD_NUM = 256, 1024
CLOCK_GHZ = 2.4

KT_WARMUP, TIMED_LAUNCHES = 300, 50  # kernel-trace pass: warm-up launches, then the timed ones
MODES = {"directp": ["--only-kernel"], "directp_anchored": ["--only-kernel", "--anchored"], "bwd": ["--only-bwd"],
         "quant": ["--only-quant"], "project": ["--only-project"],
         "project_train": ["--only-project-train"],
         "nvfp4": ["--only-nvfp4"], "bf16": ["--only-bf16"], "causal": ["--only-causal"],
         "fp8route": ["--only-fp8route"]}
PASSES = {
    "sq1": ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
            "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"],
    "sq2": ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_LDS",
            "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_SALU"],
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    # GPU clock cycles while busy, per XCC (rocprofv3 sums its 8 XCC instances), per dispatch;
    # with the dispatch's own timestamps in the same file they give the clock the kernel ran at.
    # The counters also run over a few microseconds around the kernel, so this pass times a long
    # kernel of the same kind (CLOCK_ARGS), where that window is under 1 % of the duration.
    "clk": ["GRBM_GUI_ACTIVE", "GRBM_COUNT"],
}
N_XCC = 8
CLOCK_ARGS = {"directp": ["--n", "16384"], "directp_anchored": ["--n", "16384"]}
CLOCK_LAUNCHES, CLOCK_WARMUP = 10, 40
# peak of each profiled kernel's MFMA format at the published 2.4 GHz (TFLOP/s) and its FLOPs per
# launch, for the fraction of peak at the datasheet clock and at the measured one
PEAK_TFLOPS = {"directp": 10100.0, "directp_anchored": 10100.0, "project": 2500.0, "project_train": 2500.0,
               "nvfp4": 2.0 / (1.0 / 2500.0 + 1.0 / 10100.0), "bf16": 2500.0,
               "causal": 2.0 / (1.0 / 10100.0 + 1.0 / 5030.0), "fp8route": 2.0 / (1.0 / 10100.0 + 1.0 / 5030.0)}
FLOPS_PER_LAUNCH = {"directp": 4.0 * 16 * 4096 * 4096 * 128, "directp_anchored": 4.0 * 16 * 4096 * 4096 * 128,
                    "project": 2.0 * 4096 * 2048 * 6144, "project_train": 2.0 * 8192 * 4096 * 6144, "nvfp4": 4.0 * 16 * 4096 * 4096 * 128,
                    "bf16": 4.0 * 16 * 4096 * 4096 * 128, "causal": 2.0 * 32 * 8192 * 8192 * 128,
                    "fp8route": 4.0 * 16 * 4096 * 4096 * 128}


def _bench(mode_args, steps, warmup):
    return [sys.executable, os.path.join(ROOT, "bench.py"), *mode_args, "--steps", str(steps), "--warmup",
            str(warmup)]


def _run(cmd, log, limit):
    print("+", " ".join(cmd), file=sys.stderr, flush=True)
    with open(log, "w") as f:
        r = subprocess.run(["timeout", "-s", "KILL", str(limit), *cmd], cwd=ROOT, stdout=f, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise SystemExit("pass failed (exit %d), see %s" % (r.returncode, log))


def collect(mode, out, steps=3, warmup=1):
    os.makedirs(out, exist_ok=True)
    kt = os.path.join(out, mode + "_kt")
    _run(["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", kt, "-o", "kt", "--",
          *_bench(MODES[mode], TIMED_LAUNCHES, KT_WARMUP)], kt + ".log", 180)
    for name, counters in PASSES.items():
        d = os.path.join(out, "%s_%s" % (mode, name))
        if name == "clk":
            if mode not in CLOCK_ARGS:
                continue
            cmd = _bench(MODES[mode] + CLOCK_ARGS[mode], CLOCK_LAUNCHES, CLOCK_WARMUP)
        else:
            cmd = _bench(MODES[mode], steps, warmup)
        _run(["rocprofv3", "--pmc", *counters, "--output-format", "csv", "-d", d, "-o", "p", "--", *cmd], d + ".log",
             180 if name == "clk" else 90)
    for name in ("fetch", "write"):
        d = os.path.join(out, "copy_" + name)
        if not glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            _run(["rocprofv3", "--pmc", *PASSES[name], "--output-format", "csv", "-d", d, "-o", "p", "--",
                  *_bench(["--copy-calibration"], steps, warmup)], d + ".log", 90)


def _csv(d, suffix):
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit("no %s under %s" % (suffix, d))
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counters(d):
    """{kernel: {counter: mean value per dispatch}}"""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _csv(d, "counter_collection.csv"):
        acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def _short(name):
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def _dispatches(d):
    """{kernel: [duration in ns of each dispatch, in launch order]} from a kernel trace, or from a
    counter collection (which carries the same timestamps, one row per counter)."""
    per = collections.defaultdict(dict)
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    rows = _csv(d, "kernel_trace.csv") if files else _csv(d, "counter_collection.csv")
    for r in rows:
        per[r["Kernel_Name"]][int(r.get("Dispatch_Id", r.get("Correlation_Id", 0)))] = (
            int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return {k: [ns for _, ns in sorted(v.values())] for k, v in per.items()}


def _durations(d, last=TIMED_LAUNCHES):
    """{kernel: mean duration in ns of its last `last` dispatches}: the timed launches that follow
    the warm-up launches (the GPU's clocks rise during the first tens of milliseconds of work)."""
    return {k: sum(v[-last:]) / len(v[-last:]) for k, v in _dispatches(d).items()}


def trace_table(mode, out):
    """Markdown table of the kernel-trace pass: every dispatch, and the timed ones."""
    lines = ["| Kernel | Dispatches | Average (ns) | Min (ns) | Max (ns) | Last %d: average (ns) | min | max |"
             % TIMED_LAUNCHES, "|---|---|---|---|---|---|---|---|"]
    for k, v in sorted(_dispatches(os.path.join(out, mode + "_kt")).items(), key=lambda kv: -sum(kv[1])):
        t = v[-TIMED_LAUNCHES:]
        lines.append("| %s | %d | %.0f | %d | %d | %.0f | %d | %d |" % (
            _short(k), len(v), sum(v) / len(v), min(v), max(v), sum(t) / len(t), min(t), max(t)))
    return "\n".join(lines)


def commands(mode):
    """The rocprofv3 commands collect() runs for this mode."""
    out = ["rocprofv3 --kernel-trace --stats --output-format csv -d <out>/%s_kt -o kt -- python bench.py %s"
           " --steps %d --warmup %d" % (mode, " ".join(MODES[mode]), TIMED_LAUNCHES, KT_WARMUP)]
    for name, counters in PASSES.items():
        if name == "clk":
            if mode not in CLOCK_ARGS:
                continue
            args, st, wu = MODES[mode] + CLOCK_ARGS[mode], CLOCK_LAUNCHES, CLOCK_WARMUP
        else:
            args, st, wu = MODES[mode], 3, 1
        out.append("rocprofv3 --pmc %s --output-format csv -d <out>/%s_%s -o p -- python bench.py %s --steps %d"
                   " --warmup %d" % (" ".join(counters), mode, name, " ".join(args), st, wu))
    for name in ("fetch", "write"):
        out.append("rocprofv3 --pmc %s --output-format csv -d <out>/copy_%s -o p -- python bench.py"
                   " --copy-calibration --steps 3 --warmup 1" % (" ".join(PASSES[name]), name))
    return out


def _clock_ghz(d, last=CLOCK_LAUNCHES):
    """{kernel: (GRBM_GUI_ACTIVE / dispatch duration in ns, GRBM_COUNT / duration)} per XCC,
    averaged over its last `last` dispatches in the clock pass: cycles per ns = GHz."""
    per = collections.defaultdict(dict)
    for r in _csv(d, "counter_collection.csv"):
        key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
        per[key][r["Counter_Name"]] = float(r["Counter_Value"])
        per[key]["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    byk = collections.defaultdict(list)
    for (k, did), c in sorted(per.items(), key=lambda kv: kv[0][1]):
        if c.get("ns", 0) > 0 and "GRBM_GUI_ACTIVE" in c:
            byk[k].append((c["GRBM_GUI_ACTIVE"] / N_XCC / c["ns"], c.get("GRBM_COUNT", 0.0) / N_XCC / c["ns"]))
    return {k: tuple(sum(x[i] for x in v[-last:]) / len(v[-last:]) for i in range(2)) for k, v in byk.items()}


def summarize(mode, out):
    dur = _durations(os.path.join(out, mode + "_kt"))
    sq = {}
    for name in ("sq1", "sq2", "fetch", "write"):
        for k, cs in _counters(os.path.join(out, "%s_%s" % (mode, name))).items():
            sq.setdefault(k, {}).update(cs)
    cf = list(_counters(os.path.join(out, "copy_fetch")).values())
    cw = list(_counters(os.path.join(out, "copy_write")).values())
    copy_kib = 256 * 1024
    # the copy kernel is the dispatch with the largest byte counts
    f_scale = copy_kib / max(c["FETCH_SIZE"] for c in cf)
    w_scale = copy_kib / max(c["WRITE_SIZE"] for c in cw)
    lines = ["| Kernel | us | MFMA busy | VALU issue | trans / VALU | LDS bank conflict | waits (any / inst) |"
             " HBM MB read / written | HBM GB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for k, c in sorted(sq.items(), key=lambda kv: -dur.get(kv[0], 0.0)):
        if k not in dur or "SQ_WAVES" not in c:
            continue
        us = dur[k] / 1e3
        cyc = us * 1e3 * CLOCK_GHZ  # kernel cycles at the published clock
        mfma = 100.0 * c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * SIMD_NUM)
        valu = 100.0 * 4 * c.get("SQ_ACTIVE_INST_VALU", 0.0) / (cyc * SIMD_NUM)
        trans = 100.0 * c.get("SQ_INSTS_VALU_TRANS_F32", 0.0) / max(c.get("SQ_INSTS_VALU", 1.0), 1.0)
        lds = 100.0 * c.get("SQ_LDS_BANK_CONFLICT", 0.0) / (cyc * CU_NUM)
        wc = max(c.get("SQ_WAVE_CYCLES", 1.0), 1.0)
        wa, wi = 100.0 * c.get("SQ_WAIT_ANY", 0.0) / wc, 100.0 * c.get("SQ_WAIT_INST_ANY", 0.0) / wc
        rd = c.get("FETCH_SIZE", 0.0) * f_scale * 1024 / 1e6
        wr = c.get("WRITE_SIZE", 0.0) * w_scale * 1024 / 1e6
        lines.append("| %s | %.1f | %.1f %% | %.1f %% | %.1f %% | %.2f %% | %.0f %% / %.0f %% | %.1f / %.1f | %.0f |" % (
            _short(k), us, mfma, valu, trans, lds, wa, wi, rd, wr, (rd + wr) / us * 1e3))
    notes = [
        "",
        "Kernel cycles = average duration of the last %d dispatches in the kernel trace (the timed launches after"
        " %d warm-up launches) x %.1f GHz. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /"
        " (cycles x %d SIMDs); VALU issue = 4 x SQ_ACTIVE_INST_VALU / (cycles x %d SIMDs) (quad-cycles in which a"
        " wave issued VALU work, summed over the waves of a SIMD); trans / VALU = SQ_INSTS_VALU_TRANS_F32 /"
        " SQ_INSTS_VALU; LDS bank conflict = SQ_LDS_BANK_CONFLICT / (cycles x %d CUs); waits = SQ_WAIT_ANY and"
        " SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES; HBM bytes = FETCH_SIZE x %.3f and WRITE_SIZE x %.3f (KiB per"
        " dispatch, each scaled by what the counter reads for a plain 256 MiB device copy). Counters are averages"
        " over the profiled dispatches." % (TIMED_LAUNCHES, KT_WARMUP, CLOCK_GHZ, SIMD_NUM, SIMD_NUM, CU_NUM, f_scale, w_scale),
    ]
    clk_dir = os.path.join(out, "%s_clk" % mode)
    if glob.glob(os.path.join(clk_dir, "**", "*counter_collection.csv"), recursive=True):
        notes += ["", "Clock (GRBM_GUI_ACTIVE and GRBM_COUNT per XCC per dispatch over the dispatch's own duration, last"
                  " %d of %d launches of the same kernel with bench.py %s):" % (
                      CLOCK_LAUNCHES, CLOCK_LAUNCHES + CLOCK_WARMUP, " ".join(MODES[mode] + CLOCK_ARGS.get(mode, []))),
                  ""]
        clocks = _clock_ghz(clk_dir)
        # the pass runs the profiled kernel at a long size; other dispatches in it (a set-up launch)
        # are too short for the counters' window and are left out
        longest = max(clocks, key=lambda k: _durations(clk_dir, CLOCK_LAUNCHES).get(k, 0.0)) if clocks else None
        for k, (act, cnt) in clocks.items():
            if k != longest:
                continue
            line = "- %s: %.3f GHz busy (GRBM_GUI_ACTIVE), %.3f GHz (GRBM_COUNT)" % (_short(k), act, cnt)
            if mode in PEAK_TFLOPS and dur:
                kd = max(dur, key=dur.get)
                tf = FLOPS_PER_LAUNCH[mode] / dur[kd] / 1e3
                line += ("; at the headline size %.0f TFLOP/s = %.1f %% of the peak at %.1f GHz, %.1f %% of the"
                         " peak scaled to %.3f GHz" % (tf, 100 * tf / PEAK_TFLOPS[mode], CLOCK_GHZ,
                                                      100 * tf / (PEAK_TFLOPS[mode] * act / CLOCK_GHZ), act))
            notes.append(line)
    raw = ["", "Raw counters (per dispatch):", ""]
    for k, c in sorted(sq.items(), key=lambda kv: -dur.get(kv[0], 0.0)):
        if k in dur:
            raw.append("- %s: %s" % (_short(k), ", ".join("%s %.0f" % (n, v) for n, v in sorted(c.items()))))
    return "\n".join(lines + notes + raw)


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    if len(argv) < 2 or argv[0] not in MODES:
        raise SystemExit("usage: python -m precision_attention_amd.counters {%s} OUTDIR [--summary-only]"
                         % ",".join(MODES))
    mode, out = argv[0], os.path.abspath(argv[1])
    if "--summary-only" not in argv:
        collect(mode, out)
    print("Produced by `python -m precision_attention_amd.counters %s <out>` (from the repository root), which"
          " runs each of these as its own process under `timeout -s KILL`:\n" % mode)
    print("\n".join("    " + c for c in commands(mode)))
    print("\n## Kernel trace\n")
    print(trace_table(mode, out))
    print("\n## Counters\n")
    print(summarize(mode, out))


if __name__ == "__main__":
    main()
