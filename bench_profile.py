"""rocprofv3 passes behind the benchmark's kernel figures; writes summaries
into profiles/.

  python bench_profile.py [--out gpurun_out/prof] [--workload NAME]
  python bench_profile.py --decode NAME     (a decode workload: trace + traffic)

Summaries are written to <out>/summaries/ (copy them into profiles/ to
commit them). Runs, each as its own rocprofv3 process over bench.py (the
program directly after ``--``):
  1. --kernel-trace --stats: per-kernel call counts and average durations
     -> profiles/kernel_trace_<workload>.md
  2. --pmc FETCH_SIZE, then 3. --pmc WRITE_SIZE over the same command, and
  4./5. the same two counters over a plain device copy of known size (the
     scale that turns the counters' KiB into bytes)
     -> profiles/hbm_traffic_<workload>.md and, for the dominant kernel,
        profiles/attn_bwd_main_gpt2_124m_traffic.json (read by bench.py,
        keyed by a hash of the kernel source so a stale figure is dropped).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

CALIB_MIB = 256

# SQ counter passes (at most 8 SQ and 2 GRBM counters per rocprofv3 run).
SQ_PASSES = [
    ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
     "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"],
    ["SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_LDS",
     "SQ_ACTIVE_INST_VALU", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_ANY",
     "SQ_VALU_MFMA_COEXEC_CYCLES"],
    ["SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU_CVT", "SQ_INSTS_SALU", "SQ_ACTIVE_INST_VMEM",
     "SQ_INSTS_VMEM_RD", "SQ_LDS_ADDR_CONFLICT", "SQ_INSTS_LDS_LOAD_BANDWIDTH",
     "SQ_INSTS_BRANCH"],
]


def portable(cmd):
    """The command as text, with the interpreter as python3 and paths relative
    to the repository root."""
    text = " ".join(cmd).replace(sys.executable, "python3")
    return text.replace(ROOT + "/", "")


def log(msg):
    print(f"[bench_profile {time.strftime('%H:%M:%S')}] {msg}", flush=True)


SUMMARIZE_ONLY = False


def run_rocprof(flags, prog_args, out_dir, timeout_s):
    os.makedirs(out_dir, exist_ok=True)
    cmd = ["timeout", "-s", "KILL", str(timeout_s), "rocprofv3", *flags, "-d", out_dir,
           "-o", "run", "--output-format", "csv", "--", sys.executable, *prog_args]
    if SUMMARIZE_ONLY:
        return cmd, 0
    log("running: " + " ".join(cmd))
    env = dict(os.environ, TMPDIR="/tmp")
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    with open(os.path.join(out_dir, "console.log"), "w") as f:
        f.write(r.stdout)
        f.write(r.stderr)
    log(f"exit {r.returncode}; last output: {r.stdout.strip().splitlines()[-1:]}")
    # rocprofv3 may exit non-zero after a complete run; the CSVs decide.
    return cmd, r.returncode


def find_csv(out_dir, suffix):
    hits = sorted(glob.glob(os.path.join(out_dir, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {out_dir}")
    return hits[-1]


def read_rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def col(row, *names):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in {list(row)}")


KERNELS = ("attn_fwd_kernel", "attn_bwd_prep_kernel", "attn_bwd_main_kernel",
           "attn_bwd_dkdv_kernel", "attn_bwd_dq_kernel",
           "attn_decode_split_kernel", "attn_decode_merge_kernel", "dropout_mask_kernel",
           "attn_fwd_f32_kernel", "attn_bwd_prep_f32_kernel", "attn_bwd_dkdv_f32_kernel",
           "attn_bwd_dq_f32_kernel", "sclk_probe_kernel")


def short_name(kernel_name):
    for key in KERNELS:
        if key in kernel_name:
            return key
    return kernel_name.split("(")[0][:80]


def counter_per_dispatch(path, counter):
    """Average counter value per dispatch, per kernel (short name)."""
    per = {}
    for row in read_rows(path):
        if col(row, "Counter_Name") != counter:
            continue
        k = short_name(col(row, "Kernel_Name"))
        per.setdefault(k, []).append(float(col(row, "Counter_Value")))
    return {k: (sum(v) / len(v), len(v)) for k, v in per.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "prof"))
    ap.add_argument("--workload", default=bench.DEFAULT_WORKLOAD)
    ap.add_argument("--skip-trace", action="store_true")
    ap.add_argument("--skip-pmc", action="store_true")
    ap.add_argument("--sq", action="store_true",
                    help="run only the SQ counter passes -> sq_counters_<workload>.md")
    ap.add_argument("--summarize-only", action="store_true",
                    help="rebuild the summaries from CSVs already under --out")
    ap.add_argument("--decode", default=None, metavar="NAME",
                    help="profile bench.py --mode decode on decode workload NAME instead")
    args = ap.parse_args()
    global SUMMARIZE_ONLY
    SUMMARIZE_ONLY = args.summarize_only
    out = os.path.abspath(args.out)
    bench_py = os.path.join(ROOT, "bench.py")
    if args.decode:
        return profile_decode(args.decode, out, bench_py)
    from causal_self_attention_amd.inputs import WORKLOADS
    w = WORKLOADS[args.workload]
    short = args.workload
    prof_dir = os.path.join(out, "summaries")
    os.makedirs(prof_dir, exist_ok=True)

    if args.sq:
        prog = [bench_py, "--workload", args.workload, "--steps", "2", "--warmup", "1",
                "--no-cpu-baseline"]
        table, cmds = {}, []
        for i, counters in enumerate(SQ_PASSES):
            d = os.path.join(out, f"sq_pass{i}")
            cmd, _ = run_rocprof(["--pmc", *counters], prog, d, 60)
            cmds.append(portable(cmd[4:]))
            path = find_csv(d, "counter_collection.csv")
            for c in counters:
                for kname, (val, n) in counter_per_dispatch(path, c).items():
                    if kname in KERNELS:
                        table.setdefault(kname, {})[c] = val
        lines = [f"# SQ counters per dispatch: {args.workload}", "",
                 "Average per dispatch over the profiled steps (values as rocprofv3 reports "
                 "them, summed over the counter's instances).", "",
                 "Commands (run from /tmp with TMPDIR=/tmp; paths relative to the repository "
                 "root):", ""] + [f"    {c}" for c in cmds] + [""]
        names = sorted(table)
        lines.append("| counter | " + " | ".join(names) + " |")
        lines.append("|---|" + "---|" * len(names))
        for counters in SQ_PASSES:
            for c in counters:
                lines.append(f"| {c} | " + " | ".join(
                    f"{table[k].get(c, float('nan')):.4g}" for k in names) + " |")
        with open(os.path.join(prof_dir, f"sq_counters_{short}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        log("SQ counter summary written")
        return 0

    if not args.skip_trace:
        prog = [bench_py, "--workload", args.workload, "--steps", "20", "--warmup", "5",
                "--no-cpu-baseline"]
        cmd, _ = run_rocprof(["--kernel-trace", "--stats"], prog, os.path.join(out, "trace"),
                             300)
        stats = read_rows(find_csv(os.path.join(out, "trace"), "kernel_stats.csv"))
        lines = [f"# Kernel trace: {args.workload}", "",
                 f"Workload: B={w.B} H={w.H} T={w.T} D={w.D} {w.dtype}, causal. bench.py with "
                 "--steps 20 --warmup 5: 5 warm-up steps (one step = forward, backward prep, "
                 "backward main), then runs of 20 steps whole and cut after each kernel for "
                 "the per-kernel times, 20 back-to-back backward-main launches for the "
                 "roofline, and the 20 timed steps, each step and launch on the next of the "
                 "rotated copies of the step's data (at least 1 GiB in all, so none finds its "
                 "data in the 256 MB Infinity Cache); every launch of each kernel is counted "
                 "below.", "", "Command (run from /tmp with TMPDIR=/tmp; paths relative to the repository root):", "",
                 "    " + portable(cmd[4:]), "",
                 "| kernel | calls | avg us | min us | max us | share of GPU time |",
                 "|---|---|---|---|---|---|"]
        for row in stats:
            lines.append("| {} | {} | {:.2f} | {:.2f} | {:.2f} | {:.1f}% |".format(
                short_name(col(row, "Name", "KernelName", "Kernel_Name")), col(row, "Calls"),
                float(col(row, "AverageNs")) / 1e3, float(col(row, "MinNs")) / 1e3,
                float(col(row, "MaxNs")) / 1e3, float(col(row, "Percentage"))))
        with open(os.path.join(prof_dir, f"kernel_trace_{short}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        log("kernel trace summary written")

    if args.skip_pmc:
        return 0
    prog = [bench_py, "--workload", args.workload, "--steps", "3", "--warmup", "1",
            "--no-cpu-baseline"]
    calib = [bench_py, "--calibrate-copy-mib", str(CALIB_MIB)]
    res, cmds = {}, {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        for label, p in (("attn", prog), ("copy", calib)):
            d = os.path.join(out, f"pmc_{counter}_{label}")
            cmd, _ = run_rocprof(["--pmc", counter], p, d, 120)
            cmds[(counter, label)] = portable(cmd[4:])
            res[(counter, label)] = counter_per_dispatch(find_csv(d, "counter_collection.csv"),
                                                         counter)
    copy_bytes = CALIB_MIB << 20

    def copy_kib(counter):
        vals = [v for k, (v, n) in res[(counter, "copy")].items()]
        return max(vals)  # the copy kernel is the only large dispatch in that run

    f_fetch = copy_bytes / (copy_kib("FETCH_SIZE") * 1024.0)
    f_write = copy_bytes / (copy_kib("WRITE_SIZE") * 1024.0)
    fwd_flop, bwd_flop = bench.flops(w)
    E = w.B * w.H * w.T * w.D
    R = w.B * w.H * w.T
    stats = 32 * w.B * w.H * ((w.T + 127) // 128)  # per-chunk maxima in the workspace
    zero_dq = 4 * E if w.D <= 64 else 0  # the main phase accumulates dQ at D <= 64 only
    algo = {  # compulsory bytes per launch of the plain calls, 16-bit inputs, fp32 gradients
        "attn_fwd_kernel": 3 * 2 * E + 2 * E + 4 * R,                    # q,k,v in; o, lse out
        "attn_bwd_prep_kernel": 3 * 2 * E + 4 * R + zero_dq + stats,     # q,o,dout in; delta,
        "attn_bwd_main_kernel": 4 * 2 * E + 8 * R + 3 * 4 * E + stats,   # (dq=0), maxima out;
        "attn_bwd_dkdv_kernel": 4 * 2 * E + 8 * R + 2 * 4 * E + stats,   # q,k,v,dout,lse,delta,
        "attn_bwd_dq_kernel": 4 * 2 * E + 8 * R + 4 * E + stats,         # maxima in; dq,dk,dv
    }                                                                    # (their share) out
    lines = [f"# HBM traffic per dispatch: {args.workload}", "",
             f"Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one rocprofv3 --pmc run "
             f"each), scaled by what the same counters read for a plain {CALIB_MIB} MiB "
             f"device copy: fetch x{f_fetch:.4f}, write x{f_write:.4f}.", "",
             "Commands (run from /tmp with TMPDIR=/tmp; paths relative to the repository "
             "root):", ""]
    for (c, l), cmd in cmds.items():
        lines.append(f"    {cmd}")
    lines += ["", "| kernel | fetch MB | write MB | total MB | algorithmic MB | ratio |",
              "|---|---|---|---|---|---|"]
    per_kernel = {}
    for k in sorted(res[("FETCH_SIZE", "attn")]):
        fk = res[("FETCH_SIZE", "attn")][k][0] * 1024 * f_fetch
        wk = res[("WRITE_SIZE", "attn")].get(k, (0.0, 0))[0] * 1024 * f_write
        per_kernel[k] = (fk, wk)
        a = algo.get(k)
        lines.append("| {} | {:.2f} | {:.2f} | {:.2f} | {} | {} |".format(
            k, fk / 1e6, wk / 1e6, (fk + wk) / 1e6, f"{a / 1e6:.2f}" if a else "-",
            f"{(fk + wk) / a:.2f}" if a else "-"))
    with open(os.path.join(prof_dir, f"hbm_traffic_{short}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    dk = bench.DOMINANT_KERNEL
    if dk in per_kernel and args.workload == bench.DEFAULT_WORKLOAD:
        fk, wk = per_kernel[dk]
        rec = {"kernel": dk, "workload": args.workload,
               "kernel_source_sha256_16": bench.kernel_source_hash(),
               "fetch_bytes_per_launch": round(fk), "write_bytes_per_launch": round(wk),
               "hbm_bytes_per_launch": round(fk + wk),
               "algorithmic_bytes_per_launch": algo[dk],
               "copy_scale": {"fetch": f_fetch, "write": f_write, "copy_bytes": copy_bytes},
               "commands": [cmds[k] for k in sorted(cmds)]}
        with open(os.path.join(prof_dir, os.path.basename(bench.TRAFFIC_FILE)), "w") as f:
            json.dump(rec, f, indent=1)
    log("traffic summaries written")
    return 0


def copy_scales(out, bench_py):
    """FETCH_SIZE and WRITE_SIZE of a plain device copy of known size: the
    factors that turn the counters' KiB into bytes, and their commands."""
    calib = [bench_py, "--calibrate-copy-mib", str(CALIB_MIB)]
    scale, cmds = {}, []
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(out, f"pmc_{counter}_copy")
        cmd, _ = run_rocprof(["--pmc", counter], calib, d, 120)
        cmds.append(portable(cmd[4:]))
        kib = max(v for v, n in counter_per_dispatch(find_csv(d, "counter_collection.csv"),
                                                      counter).values())
        scale[counter] = (CALIB_MIB << 20) / (kib * 1024.0)
    return scale, cmds


def profile_decode(name, out, bench_py):
    """Kernel trace and HBM traffic of bench.py --mode decode on one decode
    workload -> kernel_trace_<name>.md, hbm_traffic_<name>.md."""
    from causal_self_attention_amd.inputs import DECODE_WORKLOADS, decode_inputs
    w = DECODE_WORKLOADS[name]
    prof_dir = os.path.join(out, "summaries")
    os.makedirs(prof_dir, exist_ok=True)
    base = [bench_py, "--mode", "decode", "--workload", name, "--no-cpu-baseline"]
    tprog = base + ["--steps", "50", "--warmup", "10"]
    d = os.path.join(out, f"trace_{name}")
    cmd, _ = run_rocprof(["--kernel-trace", "--stats"], tprog, d, 300)
    lines = [f"# Kernel trace: {name}", "",
             f"Decode workload: B={w.B} sequences, H={w.H}, cache L={w.L}, D={w.D}, {w.dtype}"
             f"{', lengths uniform in 1..L' if w.ragged else ''}. bench.py --mode decode: 10 "
             "warm-up calls, then 50 timed calls (one call = split kernel + merge kernel), "
             "each on the next of the rotated copies of the cache (at least 1 GiB in all, so "
             "none is found in the 256 MB Infinity Cache).",
             "", "Command (run from /tmp with TMPDIR=/tmp; paths relative to the repository "
             "root):", "", "    " + portable(cmd[4:]), "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for row in read_rows(find_csv(d, "kernel_stats.csv")):
        lines.append("| {} | {} | {:.2f} | {:.2f} | {:.2f} | {:.1f}% |".format(
            short_name(col(row, "Name", "KernelName", "Kernel_Name")), col(row, "Calls"),
            float(col(row, "AverageNs")) / 1e3, float(col(row, "MinNs")) / 1e3,
            float(col(row, "MaxNs")) / 1e3, float(col(row, "Percentage"))))
    with open(os.path.join(prof_dir, f"kernel_trace_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    log("decode kernel trace summary written")

    scale, cmds = copy_scales(out, bench_py)
    pprog = base + ["--steps", "3", "--warmup", "1"]
    res = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(out, f"pmc_{counter}_{name}")
        cmd, _ = run_rocprof(["--pmc", counter], pprog, d, 120)
        cmds.append(portable(cmd[4:]))
        res[counter] = counter_per_dispatch(find_csv(d, "counter_collection.csv"), counter)
    nbytes = bench.decode_bytes(w, decode_inputs(w, seed=0)["lengths"].tolist())
    lines = [f"# HBM traffic per dispatch: {name}", "",
             "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one rocprofv3 --pmc run "
             f"each), scaled by what the same counters read for a plain {CALIB_MIB} MiB "
             f"device copy: fetch x{scale['FETCH_SIZE']:.4f}, write x{scale['WRITE_SIZE']:.4f}. "
             f"Algorithmic bytes of one call (split + merge): the cache rows read plus q, O "
             f"and LSE, {nbytes / 1e6:.2f} MB.", "",
             "Commands (run from /tmp with TMPDIR=/tmp; paths relative to the repository "
             "root):", ""] + [f"    {c}" for c in cmds] + [
             "", "| kernel | fetch MB | write MB | total MB |", "|---|---|---|---|"]
    for k in sorted(res["FETCH_SIZE"]):
        if k not in KERNELS:
            continue
        fk = res["FETCH_SIZE"][k][0] * 1024 * scale["FETCH_SIZE"]
        wk = res["WRITE_SIZE"].get(k, (0.0, 0))[0] * 1024 * scale["WRITE_SIZE"]
        lines.append(f"| {k} | {fk / 1e6:.2f} | {wk / 1e6:.2f} | {(fk + wk) / 1e6:.2f} |")
    with open(os.path.join(prof_dir, f"hbm_traffic_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    log("decode traffic summary written")
    return 0


if __name__ == "__main__":
    sys.exit(main())
