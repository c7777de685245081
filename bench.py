"""Benchmark: causal attention forward + backward TFLOP/s on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: gpt_attn_fwd (O, LSE), then the backward's two
phases gpt_attn_bwd_prep (delta, per-chunk maxima, dQ zero-fill) and
gpt_attn_bwd_main (dQ, dK, dV), all through the C ABI on torch's current
stream. By default these are the plain entry points; ``--o-lo`` runs the
strided ones with the forward's low part of O passed to the backward (what
the sharp-softmax workload needs for its dQ), and ``--layout fused`` runs the
strided ones on the attention layer's own buffers: q, k, v read from one
[B, T, 3C] projection output, dO from and O into [B, T, C], fp32 dQ, dK, dV
into one [B, T, 3C]. ``--dropout P`` applies attention dropout at rate P in
the forward and the backward (the keep mask regenerated in both); the FLOP
count is unchanged.

Data sets: MI355X keeps a 256 MB Infinity Cache in front of HBM, which one
layer's attention tensors fit. A training step or a decode step of a real
model touches each layer's tensors once, so consecutive steps here rotate
over ``--sets`` independent copies of the inputs and outputs (by default as
many as make at least 1 GiB), and no step finds its data left in that cache
by the step before; ``--sets 1`` reuses one copy (a warm-cache figure).

Timing: after the warm-up steps, whole steps run back to back for a fixed
``--settle-ms`` of wall time (whatever ``--steps`` is), so the clocks reach
their working level under load before anything is measured. Each kernel is
then timed alone, ``--reps`` times over ``--steps`` back-to-back launches
between two HIP events on the launch stream, and reported as the median and
the minimum of those per-launch averages; what each kernel adds to a step
comes from runs of whole steps and of steps cut after the forward and after
the preprocess. Last comes the timed region: exactly ``--steps`` whole steps
between two HIP events (nothing recorded between launches, since an event
between two kernels adds a gap; ``--graph`` replays the step from a HIP
graph instead), bracketed by device synchronizations. ``value`` is the
algorithmic FLOPs of those steps over that region. ``sclk_mhz`` is the
shader clock the steps ran at: the same steps once more, beside a one-wave
probe kernel that counts shader cycles against the 100 MHz real-time
counter (``causal_self_attention_amd/probe``).

FLOPs are the causal algorithmic count: only the T(T+1)/2 unmasked (query,
key) pairs per head, 4*D per pair forward (QK^T and PV) and 10*D per pair
backward (QK^T recompute, dP, dV, dK, dQ).

``--all-configs`` prints one line per benchmark configuration (the
Shakespeare-char layer in fp32 and bf16, the GPT-2 124M, 350M, 774M and
1558M layers, the last also at T = 2048, and the 774M layer's width as 10
heads of 128), each with the max-abs and mean-abs error of every output
against the fp64 oracle on all heads.

``--mode decode`` measures the inference path instead: one step = one
gpt_attn_decode call (one new query per sequence and head against a
key/value cache) on a decode workload; the metric is cache bytes read per
second against the HBM roofline.

Prints one JSON line. ``roofline`` describes the dominant kernel (the
backward main kernel): its algorithmic FLOPs per launch over its median
launch duration. ``cpu_baseline`` times the fp64 oracle on the same workload
on the host cores (``cores``: the threads it used), with the host's CPU
model and core count and a one-thread figure on the Shakespeare-char fp32
layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA, published
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector, published
PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 1 << 30  # data rotated over per run: 4x the 256 MB Infinity Cache
DEFAULT_WORKLOAD = "gpt2_124m_bf16_b12_h12_t1024"
DEFAULT_DECODE_WORKLOAD = "gpt2_124m_decode_bf16_b64_h12_l1024"
ALL_CONFIGS = ("shakespeare_char_f32_b1_h6_t256", "shakespeare_char_bf16_b64_h6_t256",
               "gpt2_124m_bf16_b12_h12_t1024", "gpt2_350m_bf16_b12_h16_t1024",
               "gpt2_774m_sharp_bf16_b8_h20_t1024", "gpt2_1558m_bf16_b4_h25_t1024",
               "gpt2_1558m_long_bf16_b2_h25_t2048", "gpt2_774m_d128_bf16_b8_h10_t1024")
ONE_THREAD_WORKLOAD = "shakespeare_char_f32_b1_h6_t256"
DOMINANT_KERNEL = "attn_bwd_main_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bwd_main_gpt2_124m_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "causal_self_attention_amd", "csrc", f)
                  for f in ("attn_bwd.hip", "attn_common.h", "attn_launch.h", "attn_dropout.h")]


PROBE_LIB = os.path.join(ROOT, "causal_self_attention_amd", "libsclkprobe.so")


def sclk_during(run_steps, span_ms: float, dev):
    """Shader clock (MHz) while run_steps() runs: a one-wave probe on a stream
    of its own counts shader cycles (s_memtime) against the 100 MHz real-time
    counter over about 80% of span_ms, started just before the steps are
    launched. The probe holds one wave slot of one CU; the clock it reads is
    that CU's. None when the probe library is not built."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    lib.sclk_probe_launch.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_void_p]
    lib.sclk_probe_launch.restype = ctypes.c_int
    out = torch.zeros(2, dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(dev)  # default priority
    ticks = max(1, int(0.8 * span_ms * 1e5))
    torch.cuda.synchronize()
    if lib.sclk_probe_launch(ctypes.c_void_p(out.data_ptr()), ticks,
                             ctypes.c_void_p(side.cuda_stream)) != 0:
        return None
    run_steps()
    torch.cuda.synchronize()
    cycles, real = (int(x) for x in out.tolist())
    return round(cycles / real * 100.0, 1) if real > 0 else None


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


def host_cpu():
    """CPU model, logical CPUs this process may run on, and physical cores
    among them (from /proc/cpuinfo)."""
    model, cores, cur = None, set(), {}
    try:
        allowed = os.sched_getaffinity(0)
    except AttributeError:
        allowed = set(range(os.cpu_count() or 1))
    try:
        with open("/proc/cpuinfo") as f:
            for line in f.read().split("\n") + [""]:
                if not line.strip():
                    if cur.get("processor") is not None and int(cur["processor"]) in allowed:
                        cores.add((cur.get("physical id", "0"), cur.get("core id",
                                                                       cur["processor"])))
                    cur = {}
                    continue
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                cur[k] = v
                if k == "model name" and model is None:
                    model = v
    except OSError:
        pass
    return {"cpu_model": model or "unknown", "logical_cpus": len(allowed),
            "physical_cores": len(cores) or None}


def default_threads() -> int:
    """The oracle's threads: the CPUs this process may use, at most 16 (one
    GPU's share of a GPU node's host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_time(w, inp, heads: int, threads: int) -> float:
    import oracle
    n_heads = w.B * w.H
    arr = {n: inp[n].double().numpy().reshape(n_heads, w.T, w.D)[:heads].copy()
           for n in ("q", "k", "v", "do")}
    oracle._load()
    t0 = time.perf_counter()
    oracle.attn_fwd(arr["q"], arr["k"], arr["v"], nthreads=threads)
    oracle.attn_bwd(arr["q"], arr["k"], arr["v"], arr["do"], nthreads=threads)
    return time.perf_counter() - t0


def cpu_baseline(w, inp, max_heads: int, threads: int):
    """Oracle (fp64, plain C, one thread per head at a time) on the first
    max_heads heads (by default all of them) of the same inputs: forward plus
    backward, scaled to TFLOP/s with the same algorithmic FLOP count as the
    GPU figure. Also the oracle with one thread on the Shakespeare-char fp32
    layer (a per-core rate) and the host's CPU model and core count."""
    from causal_self_attention_amd.inputs import WORKLOADS, workload_inputs
    n_heads = w.B * w.H
    heads = min(max_heads, n_heads)
    used = min(threads, heads)
    dt = _oracle_time(w, inp, heads, used)
    pairs = heads * w.T * (w.T + 1) // 2
    fl = 14 * w.D * pairs
    w1 = WORKLOADS[ONE_THREAD_WORKLOAD]
    dt1 = _oracle_time(w1, workload_inputs(w1, seed=0), w1.B * w1.H, 1)
    f1 = sum(flops(w1))
    out = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
           "sample": (f"all {n_heads} heads" if heads == n_heads else
                      f"{heads} of {n_heads} heads") +
                     f" (T={w.T}, D={w.D}), forward + backward, fp64, {used} threads, "
                     f"{dt:.2f} s wall",
           "one_thread": {"workload": ONE_THREAD_WORKLOAD, "seconds": round(dt1, 4),
                          "gflops": round(f1 / dt1 / 1e9, 4)}}
    out.update(host_cpu())
    return out


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


def _errors(gpu: dict, ref: dict) -> dict:
    import numpy as np
    out = {}
    for name, r in ref.items():
        d = np.abs(gpu[name].double().cpu().numpy().reshape(r.shape) - r)
        out[name] = {"max_abs": float(d.max()), "mean_abs": float(d.mean())}
    return out


def run_train(w, args, with_errors: bool = False, cpu_base: bool = True):
    """Measure one training workload; returns the JSON record."""
    import torch
    import causal_self_attention_amd as gattn
    from causal_self_attention_amd.inputs import torch_dtype, workload_inputs

    td = torch_dtype(w.dtype)
    dev = torch.device("cuda:0")
    inp = workload_inputs(w, seed=args.seed)
    fused = args.layout == "fused"
    use_lo = (args.o_lo or (with_errors and w.qk_scale != 1.0)) and w.dtype != "f32"
    strided = fused or use_lo or args.dropout > 0.0
    E, R = w.B * w.H * w.T * w.D, w.B * w.H * w.T
    esize = 4 if w.dtype == "f32" else 2
    ws_bytes = gattn.gpt_attn_bwd_workspace_bytes(w.B, w.H, w.T, w.D)
    # q, k, v, dO, O (and o_lo), fp32 dQ, dK, dV, LSE and the workspace.
    set_bytes = (5 + use_lo) * E * esize + 3 * E * 4 + R * 4 + ws_bytes
    ns = n_sets(args.sets, set_bytes)

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
        o_lo = torch.empty(q.shape, dtype=td, device=dev) if use_lo else None
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device=dev)
        return dict(q=q, k=k, v=v, do=do, o=o, o_lo=o_lo, lse=lse, dq=dq, dk=dk, dv=dv, ws=ws)

    sets = [make_set() for _ in range(ns)]
    drop = (args.dropout, 1234, 0) if args.dropout > 0.0 else None

    def fwd(d, st):
        if strided:
            gattn.gpt_attn_fwd_strided(d["q"], d["k"], d["v"], d["o"], d["o_lo"], d["lse"], st,
                                       drop)
        else:
            gattn.gpt_attn_fwd(d["q"], d["k"], d["v"], d["o"], d["lse"], st)

    def prep(d, st):
        if strided:
            gattn.gpt_attn_bwd_prep_strided(d["q"], d["o"], d["o_lo"], d["do"], d["dq"], d["ws"],
                                            st)
        else:
            gattn.gpt_attn_bwd_prep(d["q"], d["o"], d["do"], d["dq"], d["ws"], st)

    def bmain(d, st):
        if strided:
            gattn.gpt_attn_bwd_main_strided(d["q"], d["k"], d["v"], d["do"], d["lse"], d["dq"],
                                            d["dk"], d["dv"], d["ws"], st, drop)
        else:
            gattn.gpt_attn_bwd_main(d["q"], d["k"], d["v"], d["do"], d["lse"], d["dq"],
                                    d["dk"], d["dv"], d["ws"], st)

    stream = torch.cuda.current_stream(dev)

    def step(i, upto=3):
        """Step i's launches on the current stream (the capture stream while
        capturing), on data set i mod ns; upto < 3 launches only the first
        `upto` kernels."""
        d = sets[i % ns]
        st = torch.cuda.current_stream(dev)
        fwd(d, st)
        if upto > 1:
            prep(d, st)
        if upto > 2:
            bmain(d, st)

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

    if with_errors:
        # The last warm-up step ran set (max(warmup, ns) - 1) % ns: outputs of
        # the same inputs as every other set.
        import oracle
        d = sets[(max(args.warmup, ns) - 1) % ns]
        gpu = {n: d[n] for n in ("o", "lse", "dq", "dk", "dv")}
        gpu = {n: (t.contiguous().cpu() if n != "lse" else t.cpu()) for n, t in gpu.items()}
        ro, rl = oracle.attn_fwd(inp["q"], inp["k"], inp["v"])
        rdq, rdk, rdv = oracle.attn_bwd(inp["q"], inp["k"], inp["v"], inp["do"])
        errs = _errors(gpu, {"o": ro, "lse": rl, "dq": rdq, "dk": rdk, "dv": rdv})

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

    # Clock settling: whole steps back to back for a fixed wall time.
    t_settle = time.perf_counter()
    i = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(8):
            step(i)
            i += 1
        torch.cuda.synchronize()

    # Each kernel alone, --reps runs of --steps back-to-back launches: median
    # and minimum of the per-launch averages. Every launch is on the next
    # data set (each set's inputs are from its last step; the main kernel
    # adds into that set's dQ again).
    alone = {"fwd": lambda i: fwd(sets[i % ns], stream),
             "prep": lambda i: prep(sets[i % ns], stream),
             "main": lambda i: bmain(sets[i % ns], stream)}
    per_kernel = {}
    for name, fn in alone.items():
        runs = [timed(fn, args.steps) for _ in range(args.reps)]
        per_kernel[name] = {"median_ms": round(statistics.median(runs), 5),
                            "min_ms": round(min(runs), 5)}
    # What each kernel adds to a step (its launch gap included).
    t_f = timed(lambda i: step(i, 1), args.steps)
    t_fp = timed(lambda i: step(i, 2), args.steps)
    t_all = timed(step, args.steps)
    in_step = {"fwd": t_f, "prep": t_fp - t_f, "main": t_all - t_fp}

    # The timed region: exactly --steps whole steps, launches only.
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
        raise RuntimeError("non-finite outputs")

    # After the timed region, the same steps again beside the clock probe.
    def again():
        for i in range(args.steps):
            if graphs is not None:
                graphs[i % ns].replay()
            else:
                step(i)
    sclk = sclk_during(again, ms_per_step * args.steps, dev)

    peak = PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_MFMA_TFLOPS

    def tf(fl, ms):
        return fl / (ms * 1e-3) / 1e12

    t_main = per_kernel["main"]["median_ms"]
    t_fwd = per_kernel["fwd"]["median_ms"]
    t_bwd = per_kernel["prep"]["median_ms"] + t_main
    main_tflops = tf(bwd_flop, t_main)
    traffic = (None if (fused or use_lo or args.dropout > 0.0 or w.name != DEFAULT_WORKLOAD)
               else load_traffic(bwd_flop))
    path = ("strided, fused [B,T,3C] layout" if fused else
            "strided, o_lo" if use_lo else "strided" if strided else "plain")
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
                   "entry_points": path, "o_lo": use_lo,
                   "layout": "B,T,3C views" if fused else "BHTD", "dropout": args.dropout,
                   "launch": "eager" if graphs is None else "hip_graph",
                   "data_sets": ns, "settle_ms": args.settle_ms, "reps": args.reps,
                   "pct_of_peak": round(100 * value / peak, 2)},
        "fwd": {"ms": t_fwd, "min_ms": per_kernel["fwd"]["min_ms"],
                "in_step_ms": round(in_step["fwd"], 5),
                "tflops": round(tf(fwd_flop, t_fwd), 2),
                "pct_peak": round(100 * tf(fwd_flop, t_fwd) / peak, 2)},
        "bwd": {"ms": round(t_bwd, 5), "prep_ms": per_kernel["prep"]["median_ms"],
                "prep_min_ms": per_kernel["prep"]["min_ms"], "main_ms": t_main,
                "main_min_ms": per_kernel["main"]["min_ms"],
                "in_step_ms": round(in_step["prep"] + in_step["main"], 5),
                "tflops": round(tf(bwd_flop, t_bwd), 2),
                "pct_peak": round(100 * tf(bwd_flop, t_bwd) / peak, 2)},
        "roofline": {"kernel": ("attn_bwd_dkdv_f32_kernel + attn_bwd_dq_f32_kernel"
                                if w.dtype == "f32" else
                                "attn_bwd_dkdv_kernel + attn_bwd_dq_kernel" if w.D == 128
                                else DOMINANT_KERNEL),
                     "bound": "mfma" if w.dtype != "f32" else "alu",
                     "achieved": round(main_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(main_tflops / peak, 4),
                     "avg_launch_ms": t_main, "flop_per_launch": bwd_flop,
                     "traffic": traffic},
        "wall_s_timed": round(wall, 4),
        "sclk_mhz": sclk,
    }
    if with_errors:
        out["errors_vs_oracle"] = errs
        out["oracle_heads"] = w.B * w.H
    if cpu_base and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_heads,
                                           args.cpu_threads or default_threads())
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=5,
                    help="repetitions of each kernel's back-to-back timing (median, min)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="wall time of whole steps run before any measurement")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all-configs", action="store_true",
                    help="one line per benchmark configuration, with errors vs the oracle")
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
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (0: the CPUs this process may use, at most 16)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="attention dropout rate (Philox keep mask, seed 1234, offset 0)")
    ap.add_argument("--o-lo", action="store_true",
                    help="strided entry points, with the forward's o_lo passed to the backward")
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
    from causal_self_attention_amd.inputs import WORKLOADS

    if not os.path.exists(gattn.library_path()):
        from causal_self_attention_amd import build
        build.build()
    if args.all_configs:
        for name in ALL_CONFIGS:
            rec = run_train(WORKLOADS[name], args, with_errors=True,
                            cpu_base=name == DEFAULT_WORKLOAD)
            print(json.dumps(rec), flush=True)
        return 0
    w = WORKLOADS[args.workload]
    print(json.dumps(run_train(w, args)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
