"""Benchmark: causal attention forward + backward TFLOP/s on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: gpt_attn_fwd (O, o_lo, LSE), then the backward's
two phases gpt_attn_bwd_prep (delta, dQ zero-fill) and gpt_attn_bwd_main
(dQ, dK, dV), all through the C ABI on torch's current stream. With
``--layout fused`` the same step runs through the strided entry points on the
attention layer's own buffers: q, k, v read from one [B, T, 3C] projection
output, dO from and O into [B, T, C], fp32 dQ, dK, dV into one [B, T, 3C].
``--dropout P`` applies attention dropout at rate P in the forward and the
backward (the keep mask regenerated in both); the FLOP count is unchanged.

Data sets: MI355X keeps a 256 MB Infinity Cache in front of HBM, which one
layer's attention tensors fit. A training step or a decode step of a real
model touches each layer's tensors once, so consecutive steps here rotate
over ``--sets`` independent copies of the inputs and outputs (by default as
many as make at least 1 GiB), and no step finds its data left in that cache
by the step before; ``--sets 1`` reuses one copy (a warm-cache figure).

Timing: the timed region holds only the step's three launches, ``--steps``
times, between two HIP events (nothing recorded between launches, since an
event between two kernels adds a gap; ``--graph`` replays the step from a
HIP graph instead, which measured slower than plain launches on this
runtime). Per-kernel durations come from three more runs of ``--steps``
back-to-back eager steps, each between two events: cut after the forward,
cut after the preprocess, and whole; a kernel's duration is what it adds to
the step.

FLOPs are the causal algorithmic count: only the T(T+1)/2 unmasked (query,
key) pairs per head, 4*D per pair forward (QK^T and PV) and 10*D per pair
backward (QK^T recompute, dP, dV, dK, dQ).

``--mode decode`` measures the inference path instead: one step = one
gpt_attn_decode call (one new query per sequence and head against a
key/value cache) on a decode workload; the metric is cache bytes read per
second against the HBM roofline.

Prints one JSON line. ``roofline`` describes the dominant kernel (the
backward main kernel): its algorithmic FLOPs per launch over its average
launch duration, from ``--steps`` back-to-back launches of it between two
HIP events on the launch stream. ``cpu_baseline`` times the fp64 oracle on a bounded sample of the
same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA, published
PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 1 << 30  # data rotated over per run: 4x the 256 MB Infinity Cache
DEFAULT_WORKLOAD = "gpt2_124m_bf16_b12_h12_t1024"
DEFAULT_DECODE_WORKLOAD = "gpt2_124m_decode_bf16_b64_h12_l1024"
DOMINANT_KERNEL = "attn_bwd_main_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bwd_main_gpt2_124m_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "causal_self_attention_amd", "csrc", f)
                  for f in ("attn_bwd.hip", "attn_common.h", "attn_launch.h", "attn_dropout.h")]


def flops(w):
    pairs = w.B * w.H * w.T * (w.T + 1) // 2
    return 4 * w.D * pairs, 10 * w.D * pairs


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(n_launch_flop: int):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is missing or was taken on other kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, max_heads: int, threads: int):
    """Oracle (fp64, plain C, threads over heads) on the first max_heads heads
    (by default all of them) of the same inputs: forward plus backward. Scaled to TFLOP/s with the
    same algorithmic FLOP count as the GPU figure."""
    import oracle
    n_heads = w.B * w.H
    heads = min(max_heads, n_heads)
    arr = {n: inp[n].double().numpy().reshape(n_heads, w.T, w.D)[:heads].copy()
           for n in ("q", "k", "v", "do")}
    oracle._load()
    t0 = time.perf_counter()
    oracle.attn_fwd(arr["q"], arr["k"], arr["v"], nthreads=threads)
    oracle.attn_bwd(arr["q"], arr["k"], arr["v"], arr["do"], nthreads=threads)
    dt = time.perf_counter() - t0
    pairs = heads * w.T * (w.T + 1) // 2
    fl = 14 * w.D * pairs
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": min(threads, heads),
            "kind": "oracle",
            "sample": (f"all {n_heads} heads" if heads == n_heads else
                       f"{heads} of {n_heads} heads") +
                      f" (T={w.T}, D={w.D}), forward + backward, fp64, {dt:.2f} s wall"}


def n_sets(requested: int, set_bytes: int) -> int:
    """Copies of the data to rotate over: ``requested`` if positive, else the
    fewest whose total reaches ROTATE_BYTES (at most 16)."""
    if requested > 0:
        return requested
    return max(1, min(16, -(-ROTATE_BYTES // max(1, set_bytes))))


def decode_bytes(w, lengths) -> int:
    """Algorithmic bytes of one decode call: every cached K and V row up to
    each sequence's length, q, O (input dtype) and LSE (fp32)."""
    esize = 4 if w.dtype == "f32" else 2
    rows = int(sum(int(n) for n in lengths)) * w.H
    return rows * w.D * 2 * esize + 2 * w.B * w.H * w.D * esize + 4 * w.B * w.H


def run_decode(args) -> int:
    import torch
    import causal_self_attention_amd as gattn
    from causal_self_attention_amd.inputs import DECODE_WORKLOADS, decode_inputs

    if not os.path.exists(gattn.library_path()):
        from causal_self_attention_amd import build
        build.build()
    name = args.workload if args.workload in DECODE_WORKLOADS else DEFAULT_DECODE_WORKLOAD
    w = DECODE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp = decode_inputs(w, seed=args.seed)
    lengths = inp["lengths"].to(dev) if w.ragged else None
    esize = 4 if w.dtype == "f32" else 2
    ns = n_sets(args.sets, 2 * w.B * w.H * w.L * w.D * esize)
    sets = []
    for _ in range(ns):
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty(w.B, w.H, dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, gattn.gpt_attn_decode_workspace_bytes(w.dtype, w.B, w.H, w.L,
                                                                      w.D) // 4),
                         dtype=torch.float32, device=dev)
        sets.append((q, k, v, o, lse, ws))
    stream = torch.cuda.current_stream(dev)

    def call(i):
        q, k, v, o, lse, ws = sets[i % ns]
        gattn.gpt_attn_decode(q, k, v, lengths, o, lse, ws, stream)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    # One step is one call (split + merge kernels): back-to-back calls between
    # two HIP events on the launch stream, so the per-call duration behind
    # the roofline is the timed region's time per step.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        call(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    avg = ms_per_step
    nbytes = decode_bytes(w, inp["lengths"].tolist())
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg * 1e-3) / 1e9
    o, lse = sets[(args.steps - 1) % ns][3:5]
    if not (torch.isfinite(o.float()).all() and torch.isfinite(lse).all()):
        print("non-finite outputs", file=sys.stderr)
        return 1
    out = {
        "metric": "causal attn decode step GB/s (KV cache read), GPT-2 124M layer",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "D": w.D,
                   "ragged": w.ragged, "seed": args.seed, "bytes_per_step": nbytes,
                   "data_sets": ns},
        "roofline": {"kernel": "attn_decode_split_kernel + attn_decode_merge_kernel",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "avg_launch_ms": round(avg, 5), "bytes_per_launch": nbytes,
                     "traffic": None},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle._load()
        t = time.perf_counter()
        oracle.attn_decode(inp["q"], inp["k"], inp["v"], inp["lengths"].numpy())
        dt = time.perf_counter() - t
        out["cpu_baseline"] = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"all {w.B * w.H} heads, one fp64 thread, "
                                         f"{dt:.2f} s wall"}
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sets", type=int, default=0,
                    help="copies of the step's data to rotate over (0: enough for 1 GiB, so "
                         "no step finds its data in the 256 MB Infinity Cache; 1: warm cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run 5 plain device-to-device copies of this many MiB (the "
                         "known-size reference for HBM byte counters) and exit")
    ap.add_argument("--cpu-heads", type=int, default=1 << 30,
                    help="heads of the workload the oracle baseline runs")
    ap.add_argument("--cpu-threads", type=int, default=16)
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="attention dropout rate (Philox keep mask, seed 1234, offset 0)")
    ap.add_argument("--mode", choices=("train", "decode"), default="train",
                    help="train: forward + backward (the headline); decode: one query per "
                         "sequence against a key/value cache")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured in a HIP graph")
    ap.add_argument("--layout", choices=("bhtd", "fused"), default="bhtd",
                    help="bhtd: contiguous [B, H, T, D] operands; fused: views of the "
                         "projection's [B, T, 3C] output and of [B, T, C] buffers")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): the attention heads are independent, so a multi-GPU run is the "
              f"same kernel on each GPU's share of the heads.", file=sys.stderr)
        return 2

    import torch

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return 0

    if args.mode == "decode":
        return run_decode(args)

    import causal_self_attention_amd as gattn
    from causal_self_attention_amd.inputs import WORKLOADS, workload_inputs

    if not os.path.exists(gattn.library_path()):
        from causal_self_attention_amd import build
        build.build()
    w = WORKLOADS[args.workload]
    if w.dtype == "f32":
        print("bench.py times the matrix-core path; pick a bf16 or f16 workload",
              file=sys.stderr)
        return 2
    from causal_self_attention_amd.inputs import torch_dtype
    td = torch_dtype(w.dtype)
    dev = torch.device("cuda:0")
    inp = workload_inputs(w, seed=args.seed)
    fused = args.layout == "fused"
    E, R = w.B * w.H * w.T * w.D, w.B * w.H * w.T
    esize = 2
    # q, k, v, dO, O, o_lo (input type), fp32 dQ, dK, dV, LSE and delta.
    ns = n_sets(args.sets, 6 * E * esize + 3 * E * 4 + 2 * R * 4)

    def make_set():
        if fused:
            C = w.H * w.D
            qkv = torch.empty(w.B, w.T, 3 * C, dtype=td, device=dev)
            q, k, v = gattn.split_qkv_heads(qkv, w.H)
            for view, name in ((q, "q"), (k, "k"), (v, "v")):
                view.copy_(inp[name].to(dev))
            do = gattn.merged_heads_view(torch.empty(w.B, w.T, C, dtype=td, device=dev), w.H)
            do.copy_(inp["do"].to(dev))
            o = gattn.merged_heads_view(torch.empty(w.B, w.T, C, dtype=td, device=dev), w.H)
            dq, dk, dv = gattn.split_qkv_heads(
                torch.empty(w.B, w.T, 3 * C, dtype=torch.float32, device=dev), w.H)
        else:
            q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
            o = torch.empty_like(q)
            dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
            dk = torch.empty_like(dq)
            dv = torch.empty_like(dq)
        o_lo = torch.empty(q.shape, dtype=td, device=dev)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        ws = torch.empty(gattn.gpt_attn_bwd_workspace_bytes(w.dtype, w.B, w.H, w.T, w.D) // 4,
                         dtype=torch.float32, device=dev)
        return dict(q=q, k=k, v=v, do=do, o=o, o_lo=o_lo, lse=lse, dq=dq, dk=dk, dv=dv, ws=ws)

    sets = [make_set() for _ in range(ns)]
    if fused:
        fwd_call = gattn.gpt_attn_fwd_strided
        prep_call = gattn.gpt_attn_bwd_prep_strided
        main_call = gattn.gpt_attn_bwd_main_strided
    else:
        fwd_call, prep_call, main_call = (gattn.gpt_attn_fwd, gattn.gpt_attn_bwd_prep,
                                          gattn.gpt_attn_bwd_main)
    if args.dropout > 0.0:
        import functools
        drop = (args.dropout, 1234, 0)
        fwd_call = functools.partial(gattn.gpt_attn_fwd_strided, dropout=drop)
        prep_call = gattn.gpt_attn_bwd_prep_strided
        main_call = functools.partial(gattn.gpt_attn_bwd_main_strided, dropout=drop)
    stream = torch.cuda.current_stream(dev)

    def step(i, upto=3):
        """Step i's launches on the current stream (the capture stream while
        capturing), on data set i mod ns; upto < 3 launches only the first
        `upto` kernels."""
        d = sets[i % ns]
        st = torch.cuda.current_stream(dev)
        fwd_call(d["q"], d["k"], d["v"], d["o"], d["o_lo"], d["lse"], st)
        if upto > 1:
            prep_call(d["o"], d["o_lo"], d["do"], d["dq"], d["ws"], st)
        if upto > 2:
            main_call(d["q"], d["k"], d["v"], d["do"], d["lse"], d["dq"], d["dk"], d["dv"],
                      d["ws"], st)

    def main_only(i):
        d = sets[i % ns]
        main_call(d["q"], d["k"], d["v"], d["do"], d["lse"], d["dq"], d["dk"], d["dv"], d["ws"],
                  stream)

    def timed(fn, n):
        """ms per call of fn(i), i = 0..n-1, over n back-to-back calls, from two
        HIP events on the launch stream around them (nothing recorded in
        between)."""
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    for i in range(max(args.warmup, ns)):
        step(i)
    torch.cuda.synchronize()

    graphs = None
    if args.graph:
        # One graph per data set, each holding that set's step.
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for j in range(ns):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(j)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % ns].replay()
        torch.cuda.synchronize()

    # Per-kernel durations by difference (before the timed region, which they
    # also keep the clocks warm for): the same number of back-to-back eager
    # steps cut after the forward, after the preprocess, and whole; each
    # kernel's time is what it adds to its step (its launch gap included).
    timed(step, args.steps)  # not used: brings the clocks to their working level
    t_f = timed(lambda i: step(i, 1), args.steps)
    t_fp = timed(lambda i: step(i, 2), args.steps)
    t_all = timed(step, args.steps)
    avg = {"fwd": t_f, "prep": t_fp - t_f, "main": t_all - t_fp}
    # The dominant kernel alone: back-to-back launches between two events,
    # rotating over the data sets like the steps (each set's inputs are from
    # its last step; each launch adds into that set's dQ again).
    t_main = timed(main_only, args.steps)

    # The timed region: --steps whole steps, launches only.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        if graphs is not None:
            graphs[i % ns].replay()
        else:
            step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    fwd_flop, bwd_flop = flops(w)
    value = (fwd_flop + bwd_flop) / (ms_per_step * 1e-3) / 1e12
    last = sets[(args.steps - 1) % ns]
    if not (torch.isfinite(last["dq"]).all() and torch.isfinite(last["o"].float()).all()):
        print("non-finite outputs", file=sys.stderr)
        return 1

    main_tflops = bwd_flop / (t_main * 1e-3) / 1e12
    traffic = (None if (fused or args.dropout > 0.0 or w.name != DEFAULT_WORKLOAD)
               else load_traffic(bwd_flop))
    out = {
        "metric": "causal attn fwd+bwd TFLOP/s and % bf16 MFMA peak, GPT-2 124M shape",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "D": w.D,
                   "causal": True, "scale": 1.0 / w.D ** 0.5, "seed": args.seed,
                   "layout": "B,T,3C views" if fused else "BHTD", "dropout": args.dropout,
                   "launch": "eager" if graphs is None else "hip_graph",
                   "data_sets": ns,
                   "pct_of_peak": round(100 * value / PEAK_MFMA_TFLOPS, 2)},
        "fwd": {"ms": round(avg["fwd"], 5),
                "tflops": round(fwd_flop / (avg["fwd"] * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * fwd_flop / (avg["fwd"] * 1e-3) / 1e12 /
                                  PEAK_MFMA_TFLOPS, 2)},
        "bwd": {"ms": round(avg["prep"] + avg["main"], 5), "prep_ms": round(avg["prep"], 5),
                "main_ms": round(avg["main"], 5),
                "tflops": round(bwd_flop / ((avg["prep"] + avg["main"]) * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * bwd_flop / ((avg["prep"] + avg["main"]) * 1e-3) /
                                  1e12 / PEAK_MFMA_TFLOPS, 2)},
        "roofline": {"kernel": DOMINANT_KERNEL, "bound": "mfma",
                     "achieved": round(main_tflops, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(main_tflops / PEAK_MFMA_TFLOPS, 4),
                     "avg_launch_ms": round(t_main, 5),
                     "flop_per_launch": bwd_flop, "traffic": traffic},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_heads, args.cpu_threads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
