#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step = one attn_fwd (or attn_fwd_chunked) call over one set of synthetic
inputs already resident in HBM.  Inputs rotate over enough sets that the timed
footprint exceeds the 256 MB Infinity Cache, so short workloads measure HBM,
not the cache; the set index runs on across repeats, so every set is timed.
Prints ONE JSON line (rank 0, N = 1):

  value        counted TFLOP/s = 4*B*H*S_q*S_kv*D (halved when causal) / time
  ms_per_step  mean time per call over the timed region (HIP events)
  roofline     the kernel against its binding MI355X peak (MFMA or HBM)
  cpu_baseline the fp64 oracle on a bounded sample of the same workload, on
               this host's cores
  per_config   the other workloads (c1 .. c4, every dtype), each with its own
               ms/call, TFLOP/s, roofline and cpu_baseline, and as context
               library_sdpa: torch's scaled_dot_product_attention (flash or
               memory-efficient backend) timed on the same inputs

Default workload: the long-context causal chunked workload (B=16, H=16,
S=98,304, D=64, bf16, 4,096-row query windows against the K/V cache), the
largest of the five workloads; --workload NAME times one other workload alone.
"""
from __future__ import annotations

import argparse
import statistics
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % of MFMA peak (ms/call) at 1 GPU, per config"
PEAK = {  # MI355X datasheet, dense
    "mfma_f32": 157.3, "mfma_f16": 2516.6, "mfma_bf16": 2516.6,  # TFLOP/s
    "hbm": 8000.0,  # GB/s
}
ROTATE_BYTES = 1 << 30  # timed footprint target (> 256 MB Infinity Cache)
HEADLINE = "c5_long_causal_chunked"
# The other workloads, every dtype: reported under per_config.
PER_CONFIG = [("c1_single_head_f32", "f32"), ("c2_mha_s512", "f32"), ("c2_mha_s512", "f16"),
              ("c3_causal_s2048", "bf16"), ("c3_causal_s2048", "f16"), ("c4_large_batch_s1024", "bf16")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: enough for about 0.5 s of GPU time, 10 .. 20000)")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--repeats", type=int, default=5,
                    help="the timed steps are split into this many back-to-back repeats (median reported)")
    ap.add_argument("--no-aa", action="store_true", help="skip the A/A control (a second timing of the same steps)")
    ap.add_argument("--workload", default=HEADLINE,
                    help="the workload of the headline line (default: the long-context chunked workload); "
                         "the per-config block is added only for the default")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time the headline workload alone (no per_config block)")
    ap.add_argument("--per-config-seconds", type=float, default=0.25,
                    help="GPU time per per-config entry (its step count follows from a short estimate)")
    ap.add_argument("--per-config-cpu-seconds", type=float, default=3.0,
                    help="oracle time per per-config entry's cpu_baseline")
    ap.add_argument("--dtype", default=None, help="f32 | f16 | bf16 (default: the workload's first)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sdpa", action="store_true",
                    help="skip the per-config library_sdpa context (torch's scaled_dot_product_attention timed "
                         "on the same inputs)")
    ap.add_argument("--eager", action="store_true",
                    help="launch each timed step from Python instead of replaying a captured HIP graph")
    ap.add_argument("--stream", action="store_true",
                    help="chunked workloads: one step runs every query window in order, appending the "
                         "window's K/V rows to a cache (attn_kv_append) and attending its queries to the "
                         "grown cache (attn_fwd_chunked)")
    ap.add_argument("--varlen", action="store_true",
                    help="attn_fwd_varlen with per-sequence key lengths drawn uniform on [S_kv/4, S_kv] "
                         "(seeded); value counts only the visible (row, key) pairs")
    ap.add_argument("--decode", type=int, default=None, metavar="R",
                    help="R query rows (the last R positions) against the workload's whole K/V cache through "
                         "attn_fwd_splitkv (keys split over workgroup ranges and merged)")
    ap.add_argument("--qkv", action="store_true",
                    help="the fused Q/K/V projection (attn_qkv_proj) of a [B, S, 64H] input with synthetic "
                         "weights [3d, d] and bias; value is its TFLOP/s (2 * B*S * 3d * d per call)")
    ap.add_argument("--n-split", type=int, default=0,
                    help="key ranges for --decode (0: attn_splitkv_choose for this GPU)")
    ap.add_argument("--cpu-sample-seconds", type=float, default=15.0)
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--copy-mb", type=float, default=None,
                    help="instead of attention, time a plain device copy of this many MB per step "
                         "(reference kernel of known traffic for scaling HBM counters)")
    return ap.parse_args()


def copy_calibration(args):
    """A plain copy kernel of known size: each step reads and writes copy_mb MB."""
    import torch
    dev = torch.device("cuda:0")
    n = int(args.copy_mb * 1e6) // 4
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    line = {"metric": "device copy GB/s (read + write)", "value": round(2 * n * 4 / (ms * 1e-3) / 1e9, 2),
            "unit": "GB/s", "bytes_read_per_step": n * 4, "bytes_written_per_step": n * 4,
            "ms_per_step": round(ms, 6), "steps": args.steps}
    print(json.dumps(line), flush=True)


def varlen_work(w, lens, dtype):
    """Counted FLOPs (4*D per visible (row, key) pair) and algorithmic HBM
    bytes (Q and O once, each sequence's first L_b K/V rows once) of one
    attn_fwd_varlen call with per-sequence lengths `lens`."""
    import torch
    e = torch.finfo(getattr(torch, {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}[dtype])).bits // 8
    pairs, kv_rows = 0, 0
    for L in (min(max(int(x), 0), w.S_kv) for x in lens):
        kv_rows += L
        if w.causal:  # row i sees min(L, max(0, L - S_q + i + 1)) keys
            pairs += sum(min(L, max(0, L - w.S_q + i + 1)) for i in range(w.S_q))
        else:
            pairs += w.S_q * L
    flops = 4.0 * w.D * pairs * w.H
    nbytes = (2 * w.S_q * w.B + 2 * kv_rows) * w.D * e * w.H
    return flops, nbytes


def roofline_for(w, dtype, sec_per_call, work=None):
    flops, nbytes = work if work is not None else (w.flops(), w.bytes(dtype))
    t_mfma = flops / (PEAK[f"mfma_{dtype}"] * 1e12)
    t_hbm = nbytes / (PEAK["hbm"] * 1e9)
    if t_hbm > t_mfma:
        ach = nbytes / sec_per_call / 1e9
        return {"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK["hbm"], "unit": "GB/s",
                "frac": round(ach / PEAK["hbm"], 4), "traffic": None}
    ach = flops / sec_per_call / 1e12
    pk = PEAK[f"mfma_{dtype}"]
    return {"bound": "mfma", "achieved": round(ach, 3), "peak": pk, "unit": "TFLOP/s",
            "frac": round(ach / pk, 4), "traffic": None}


def code_key(paths):
    """sha256 prefix of C++/HIP sources (one path or a list, concatenated)
    with comments removed and whitespace collapsed: it changes when the code
    changes, not when a comment does.  (The kernel sources hold no string
    literal with a comment marker.)"""
    import hashlib
    import re
    src = ""
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(path) as f:
            src += f.read() + "\n"
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def measured_traffic(workload, dtype):
    """HBM bytes per launch from the committed counter runs (profiles/traffic.json),
    or None when there is no entry or the kernel code changed since."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            t = json.load(f)
        srcs = t["kernel_source"]
        key = code_key([os.path.join(ROOT, x) for x in ([srcs] if isinstance(srcs, str) else srcs)])
    except (OSError, KeyError, ValueError):
        return None
    e = t.get("entries", {}).get(f"{workload}/{dtype}")
    if e is None or key != t.get("code_sha256_16"):
        return None
    return e["traffic_bytes"]


def cpu_baseline(w, dtype, budget_s):
    """Time the fp64 oracle on a bounded sample of the workload's query rows."""
    import numpy as np
    import oracle
    import workloads as W
    threads = len(os.sched_getaffinity(0))
    small = w.S_q * w.S_kv * w.B * w.H <= (1 << 27) and w.B * w.H * (w.S_q + 2 * w.S_kv) * w.D <= (1 << 27)
    if small:
        q, k, v = W.make_inputs(w, dtype)
    else:  # one (b,h) head of the workload's shape
        one = W.Workload(w.name, 1, 1, w.S_q, w.S_kv, w.D, w.causal, w.dtypes, w.sigma, w.seed,
                         w.outlier_frac, w.outlier_mult)
        q, k, v = W.make_inputs(one, dtype)
    heads = q.shape[0] * q.shape[1]
    # Time batches of randomly drawn query rows (all heads of the sample) until
    # the budget is used; a sample that covers every row repeats whole runs.
    rng = np.random.default_rng(0)
    order = rng.permutation(w.S_q)
    batch = max(1, min(w.S_q, (1 << 26) // (w.S_kv * heads)))  # ~2^26 (row, key) pairs per batch
    done, reps, pos = [], 0, 0
    t0 = time.perf_counter()
    while True:
        rows = np.sort(order[pos:pos + batch])
        oracle.attention(q, k, v, causal=w.causal, scale=w.scale, rows=rows, threads=threads)
        done.append(rows)
        pos += batch
        if pos >= w.S_q:
            pos, reps = 0, reps + 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    r = np.concatenate(done)
    # counted FLOPs of the sampled rows: 4*D per visible (row, key) pair
    shift = w.S_kv - w.S_q
    vis = (np.minimum(r + shift + 1, w.S_kv) if w.causal else np.full(len(r), w.S_kv)).sum()
    flops = 4.0 * w.D * float(vis) * heads
    rate = flops / el
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} head(s) x {len(r)} query-row evaluations (rows of {w.S_q}, in random order) "
                      f"({flops / 1e9:.2f} GFLOP counted, {el:.1f} s, fp64)",
            "seconds": round(el, 3), "gflop_per_s": round(rate / 1e9, 3),
            "us_per_row_per_head": round(el / (len(r) * heads) * 1e6, 3),
            "extrapolated_full_workload_s": round(w.flops() / rate, 1),
            "extrapolation_note": "counted FLOPs of the whole workload / the sample's rate (not measured)"}


def gpu_clock_mhz(dev, n_wg=256, iters=4096):
    """Shader clock (MHz) while a short busy kernel runs: median over waves of
    100 MHz * shader cycles / reference ticks (attn_clock_probe).  None if the
    probe library is missing."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "transformer_attention_04_amd", "libattn_clock.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.attn_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    out = torch.zeros(2 * n_wg, dtype=torch.int64, device=dev)
    st = lib.attn_clock_probe(out.data_ptr(), n_wg, iters, ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    if st != 0:
        return None
    torch.cuda.synchronize()
    c = out.view(n_wg, 2).cpu().double()
    mhz = 100.0 * c[:, 0] / c[:, 1].clamp(min=1)
    return round(float(mhz.median()), 1)


def measured_peak(dev, bound, dtype):
    """The ceiling this box sustains for the roof that binds: a pure MFMA loop
    (attn_mfma_probe, two waves per SIMD, 16 MFMAs per iteration in four
    chains) in TFLOP/s, or a 1 GiB streaming copy (attn_copy_probe, read +
    write) in GB/s.  Median of 5 timed launches after one warmup.  None if the
    probe library is missing."""
    import ctypes
    import torch
    stream = torch.cuda.current_stream(dev)
    times = []
    if bound == "mfma":
        path = os.path.join(ROOT, "transformer_attention_04_amd", "libattn_clock.so")
        if not os.path.exists(path):
            return None
        lib = ctypes.CDLL(path)
        lib.attn_mfma_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
        n_wg = 2 * torch.cuda.get_device_properties(dev).multi_processor_count  # 8 waves per CU
        iters = 32768 if code else 8192  # ~15-20 ms per launch: long enough for the clock to settle
        out = torch.empty(4 * n_wg, dtype=torch.float32, device=dev)
        flops = n_wg * 4 * iters * 16 * (4096 if code == 0 else 32768)
        for r in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = lib.attn_mfma_probe(out.data_ptr(), n_wg, iters, code, ctypes.c_void_p(stream.cuda_stream))
            e1.record(stream)
            if st != 0:
                return None
            torch.cuda.synchronize(dev)
            if r:
                times.append(e0.elapsed_time(e1) * 1e-3)
        return {"peak": round(flops / statistics.median(times) / 1e12, 1), "unit": "TFLOP/s",
                "how": f"{dtype} 32x32 MFMA loop, 4 chains, 2 waves per SIMD (attn_mfma_probe)"}
    path = os.path.join(ROOT, "transformer_attention_04_amd", "libattn_clock.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.attn_copy_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    nbytes = 1 << 30
    try:
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
    except torch.cuda.OutOfMemoryError:
        return None
    n_wg = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    for r in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.attn_copy_probe(src.data_ptr(), dst.data_ptr(), nbytes, n_wg, ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        if st != 0:
            return None
        torch.cuda.synchronize(dev)
        if r:
            times.append(e0.elapsed_time(e1) * 1e-3)
    del src, dst
    return {"peak": round(2 * nbytes / statistics.median(times) / 1e9, 1), "unit": "GB/s",
            "how": "streaming copy of 1 GiB, 16 B per lane, bytes read + written (attn_copy_probe)"}


def environment(dev):
    """What the numbers were measured on: versions, GPU, host CPU, build."""
    import platform
    import torch
    props = torch.cuda.get_device_properties(dev)
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    info = {}
    try:
        with open(os.path.join(ROOT, "transformer_attention_04_amd", "build_info.json")) as f:
            info = json.load(f)
    except (OSError, ValueError):
        pass
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None), "cu": props.multi_processor_count,
            "torch": torch.__version__, "hip": torch.version.hip, "python": platform.python_version(),
            "host_cpu": cpu, "host_cores": len(os.sched_getaffinity(0)),
            "git_rev": info.get("git_rev"), "tree_modified_at_build": info.get("tree_modified"),
            "hipcc": info.get("hipcc")}


def split_steps(k, r):
    """Split k steps into r back-to-back repeats (sizes differ by at most one)."""
    r = max(1, min(r, k))
    return [k // r + (1 if i < k % r else 0) for i in range(r)]


def repeat_bases(sizes):
    """First global step index of each repeat: the input-set index runs on
    from one repeat to the next, so k steps touch min(k, n_sets) sets."""
    out, b = [], 0
    for n in sizes:
        out.append(b)
        b += n
    return out


def sets_timed(k, n_sets):
    """Distinct input sets that k steps over n_sets rotating sets touch."""
    return min(k, n_sets)


class Timer:
    """Exactly `steps` steps in back-to-back repeats, timed with HIP events on
    the launch stream.  Repeat r runs global steps base_r .. base_r + n_r - 1
    (step(i) picks input set i mod n_sets), captured once into a HIP graph and
    replayed (eager: launched from Python), so the timed region holds exactly
    the steps' kernels."""

    def __init__(self, step, steps, repeats, eager, stream, replay_once=True):
        import torch
        self.stream = stream
        self.sizes = split_steps(steps, repeats)
        self.bases = repeat_bases(self.sizes)
        self.step = step
        self.graphs = []
        if not eager:
            for b, n in zip(self.bases, self.sizes):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(b, b + n):
                        step(i)
                if replay_once:
                    g.replay()  # one untimed replay
                self.graphs.append(g)
            torch.cuda.synchronize()

    @property
    def launch(self):
        return "hip_graph_replay" if self.graphs else "eager"

    def run(self):
        """Returns (total ms, [ms per step of each repeat])."""
        import torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(self.sizes) + 1)]
        ev[0].record(self.stream)
        for r, (b, n) in enumerate(zip(self.bases, self.sizes)):
            if self.graphs:
                self.graphs[r].replay()
            else:
                for i in range(b, b + n):
                    self.step(i)
            ev[r + 1].record(self.stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[-1]), [ev[r].elapsed_time(ev[r + 1]) / n for r, n in enumerate(self.sizes)]


def estimate_ms(step, stream, n):
    """Mean eager ms per step over n steps (after the warmup)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def bench_qkv(args, w, dtype):
    """Time attn_qkv_proj on the workload's batch, sequence and heads."""
    import torch
    import workloads as W
    import transformer_attention_04_amd as A
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, S, H = w.B, w.S_q, w.H
    d = 64 * H
    t = W.DTYPES[dtype]
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 700)
    wt = (torch.randn((3 * d, d), generator=g, device=dev) / d ** 0.5).to(t)
    bias = (torch.randn((3 * d,), generator=g, device=dev) * 0.1).to(t)
    x0 = torch.randn((B, S, d), generator=g, device=dev).to(t)
    per_set = 4 * B * S * d * 2
    n_sets = max(1, min(64, math.ceil(ROTATE_BYTES / per_set)))
    sets = [(x0 if i == 0 else x0.clone(), tuple(torch.empty((B, H, S, 64), dtype=t, device=dev) for _ in range(3)))
            for i in range(n_sets)]
    flops = 2.0 * B * S * 3 * d * d
    nbytes = (B * S * d + 3 * d * d + 3 * d + 3 * B * S * d) * 2
    log(f"[bench] qkv projection B={B} S={S} d={d} {dtype}: {flops / 1e9:.1f} GFLOP per call, {n_sets} sets")

    def step(i):
        x, outs = sets[i % n_sets]
        A.attn_qkv_proj(x, wt, bias, out=outs)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    if args.steps is None:
        est = estimate_ms(step, stream, 10)
        args.steps = int(min(20000, max(10, math.ceil(500.0 / max(est, 1e-3)))))
    tm = Timer(step, args.steps, args.repeats, args.eager, stream)
    clk0 = gpu_clock_mhz(dev)
    total_ms, rep_ms = tm.run()
    clk1 = gpu_clock_mhz(dev)
    ms = total_ms / args.steps
    sec = ms / 1e3
    tflops = flops / sec / 1e12
    pk = PEAK[f"mfma_{dtype}"]
    log(f"[bench] qkv projection {ms * 1e3:.2f} us/call, {tflops:.1f} TFLOP/s ({100 * tflops / pk:.1f}% of peak)")
    line = {
        "metric": "fused Q/K/V projection TFLOP/s + % of MFMA peak (ms/call) at 1 GPU", "value": round(tflops, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}_qkv_projection", "B": B, "S": S, "H": H, "d": d, "bias": True,
                   "rotating_sets": n_sets, "sets_timed": sets_timed(args.steps, n_sets),
                   "mode": "attn_qkv_proj: x [B,S,d] @ W^T [d,3d] + b -> q,k,v [B,H,S,64]",
                   "launch": tm.launch},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": pk, "unit": "TFLOP/s",
                     "frac": round(tflops / pk, 4), "traffic": None,
                     "algorithmic_bytes": nbytes, "peak_source": "datasheet"},
        "timing": {"repeats": len(rep_ms), "steps_per_repeat": tm.sizes,
                   "ms_per_step_each_repeat": [round(x, 6) for x in rep_ms],
                   "median_ms_per_step": round(sorted(rep_ms)[len(rep_ms) // 2], 6),
                   "gpu_clock_mhz": {"before": clk0, "after": clk1}},
        "environment": environment(dev),
        "cpu_baseline": None,
    }
    mp = measured_peak(dev, "mfma", dtype)
    if mp is not None:
        mp["frac"] = round(tflops / mp["peak"], 4)
    line["roofline"]["measured"] = mp
    emit(args, line)


def emit(args, line):
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(s + "\n")


def clock_block(clk0, clk1):
    return {"before": clk0, "after": clk1,
            "after_over_before": round(clk1 / clk0, 4) if clk0 and clk1 else None,
            "below_85pct": (clk1 < 0.85 * clk0) if clk0 and clk1 else None}


def make_sets(w, dtype, dev, log_name=True):
    """The rotating input sets of a workload: distinct buffers holding the same
    seeded values, enough of them (at most 64, within 90% of the free device
    memory) that their footprint exceeds the Infinity Cache.  Large workloads
    are drawn on the device (one set).  Exits with status 3 when one set does
    not fit."""
    import torch
    import workloads as W
    footprint = w.bytes(dtype)
    n_sets = max(1, min(64, math.ceil(ROTATE_BYTES / footprint)))
    free_b, _ = torch.cuda.mem_get_info(dev)
    if footprint > 0.9 * free_b:
        print(f"bench.py: workload {w.name} needs {footprint / 2**30:.1f} GiB of device memory, "
              f"{free_b / 2**30:.1f} GiB are free", file=sys.stderr)
        sys.exit(3)
    n_sets = max(1, min(n_sets, int(0.9 * free_b // footprint)))
    sets = []
    if w.S_q * w.S_kv * w.B * w.H > (1 << 32) or w.B * w.H * w.S_kv * w.D > (1 << 28):  # large: draw on the device
        q, k, v = W.make_device_inputs(w, dtype, dev)
        sets.append((q, k, v, torch.empty_like(q)))
    else:
        q0, k0, v0 = (x.to(dev) for x in W.make_inputs(w, dtype))
        for i in range(n_sets):
            if i == 0:
                q, k, v = q0, k0, v0
            else:  # distinct buffers, same values: the cache cannot hold them all
                q, k, v = q0.clone(), k0.clone(), v0.clone()
            sets.append((q, k, v, torch.empty_like(q)))
    if log_name:
        log(f"[bench] workload {w.name} dtype {dtype}: {footprint / 1e6:.1f} MB per set, {len(sets)} sets")
    return sets


def library_sdpa(args, w, sets, steps, stream, ours_ms):
    """Context, not the product: torch's scaled_dot_product_attention (its flash
    or memory-efficient backend; the math backend is never run) on the same
    rotating sets, timed like our call, and its largest difference from our
    output on set 0.  The pages measure their kernel against this library
    call.  Square workloads only (its causal mask is top-left aligned, which
    equals the bottom-right one only when S_q = S_kv)."""
    import warnings
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import sdpa_kernel, SDPBackend
    if w.S_q != w.S_kv:
        return None
    notes = {}
    for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            with sdpa_kernel([be]), warnings.catch_warnings():
                warnings.simplefilter("ignore", UserWarning)  # the backends' notes on unsupported dtypes
                def step(i):
                    q, k, v, _ = sets[i % len(sets)]
                    F.scaled_dot_product_attention(q, k, v, is_causal=w.causal, scale=w.scale)

                q, k, v, o = sets[0]
                diff = (F.scaled_dot_product_attention(q, k, v, is_causal=w.causal, scale=w.scale).float()
                        - o.float()).abs().max().item()
                n = max(len(sets), min(steps, 500))  # bounds the graph memory of the library's outputs
                tm = Timer(step, n, args.repeats, args.eager, stream)
                total_ms, _ = tm.run()
                del tm
        except RuntimeError as ex:  # no kernel of this backend for the dtype or shape
            notes[be.name] = str(ex).splitlines()[0][:120]
            continue
        ms = total_ms / n
        log(f"[bench] per-config {w.name}: torch SDPA ({be.name}) {ms * 1e3:.2f} us/call, ours "
            f"{ours_ms * 1e3:.2f} us ({ms / ours_ms:.2f}x)")
        return {"backend": be.name, "ms_per_call": round(ms, 6), "tflops": round(w.flops() / (ms / 1e3) / 1e12, 4),
                "steps": n, "ours_speedup": round(ms / ours_ms, 3), "max_abs_diff_vs_ours": diff}
    return {"unavailable": notes}


def per_config_entry(args, name, dtype, dev, stream, peaks):
    """One per-config result: the workload's single call (attn_fwd, or
    attn_fwd_chunked for a chunked workload) over rotating sets, timed like the
    headline but for about --per-config-seconds of GPU time."""
    import torch
    import workloads as W
    import transformer_attention_04_amd as A
    w = W.BY_NAME[name]
    sets = make_sets(w, dtype, dev)

    def step(i):
        q, k, v, o = sets[i % len(sets)]
        if w.chunk:
            A.attn_fwd_chunked(q, k, v, chunk=w.chunk, causal=w.causal, scale=w.scale, out=o)
        else:
            A.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o)

    for i in range(20):
        step(i)
    torch.cuda.synchronize()
    est = estimate_ms(step, stream, 20)
    steps = int(min(20000, max(len(sets), math.ceil(args.per_config_seconds * 1e3 / max(est, 1e-3)))))
    tm = Timer(step, steps, args.repeats, args.eager, stream)
    clk0 = gpu_clock_mhz(dev)
    total_ms, rep_ms = tm.run()
    clk1 = gpu_clock_mhz(dev)
    ms = total_ms / steps
    sec = ms / 1e3
    tflops = w.flops() / sec / 1e12
    roof = roofline_for(w, dtype, sec)
    roof["traffic"] = measured_traffic(w.name, dtype)
    roof["peak_source"] = "datasheet"
    key = (roof["bound"], dtype if roof["bound"] == "mfma" else "hbm")
    if key not in peaks:
        peaks[key] = measured_peak(dev, roof["bound"], dtype)
    mp = dict(peaks[key]) if peaks[key] else None
    if mp is not None:
        mp["frac"] = round(roof["achieved"] / mp["peak"], 4)
    roof["measured"] = mp
    med = sorted(rep_ms)[len(rep_ms) // 2]
    log(f"[bench] per-config {name} {dtype}: {ms * 1e3:.2f} us/call, {tflops:.2f} TFLOP/s, "
        f"{roof['bound']} frac {roof['frac']}")
    e = torch.finfo(W.DTYPES[dtype]).bits // 8
    entry = {
        "workload": name, "dtype": dtype, "ms_per_call": round(ms, 6), "median_ms_per_call": round(med, 6),
        "tflops": round(tflops, 4), "steps": steps, "rotating_sets": len(sets),
        "sets_timed": sets_timed(steps, len(sets)), "launch": tm.launch,
        "shape": {"B": w.B, "H": w.H, "S_q": w.S_q, "S_kv": w.S_kv, "D_h": w.D, "causal": w.causal,
                  "chunk": w.chunk},
        "roofline": roof,
        "bandwidth": {"algorithmic_bytes": int(w.bytes(dtype)), "gbps": round(w.bytes(dtype) / sec / 1e9, 2)},
        "timing": {"repeats": len(rep_ms), "steps_per_repeat": tm.sizes,
                   "ms_per_step_each_repeat": [round(x, 6) for x in rep_ms],
                   "gpu_clock_mhz": clock_block(clk0, clk1)},
    }
    assert e in (2, 4)
    del tm
    entry["library_sdpa"] = None if (args.no_sdpa or w.chunk) else library_sdpa(args, w, sets, steps, stream, ms)
    del sets
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        entry["cpu_baseline"] = cpu_baseline(w, dtype, args.per_config_cpu_seconds)
    else:
        entry["cpu_baseline"] = None
    return entry


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(no multi-GPU path exists in this library)", file=sys.stderr)
        sys.exit(2)
    if args.copy_mb:
        copy_calibration(args)
        return
    import torch
    import workloads as W
    import transformer_attention_04_amd as A

    w = W.BY_NAME[args.workload]
    dtype = args.dtype or w.dtypes[0]
    if args.qkv:
        if args.varlen or args.stream or args.decode or dtype == "f32":
            print("--qkv takes a 16-bit dtype and neither --varlen, --stream nor --decode", file=sys.stderr)
            sys.exit(2)
        return bench_qkv(args, w, dtype)
    special = bool(args.decode or args.varlen or args.stream)
    with_per_config = not args.no_per_config and not special and args.workload == HEADLINE and args.dtype is None
    if args.decode:
        if args.varlen or args.stream:
            print("--decode takes neither --varlen nor --stream", file=sys.stderr)
            sys.exit(2)
        import dataclasses
        w = dataclasses.replace(w, name=f"{w.name}_decode{args.decode}", S_q=args.decode, chunk=None,
                                sample_rows=None)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets = make_sets(w, dtype, dev)
    chunk = w.chunk
    work = None
    if args.decode:
        R, kvl = w.S_q, w.S_kv
        pairs = sum(min(kvl, max(0, kvl - R + i + 1)) for i in range(R)) if w.causal else R * kvl
        e = torch.finfo(W.DTYPES[dtype]).bits // 8
        work = (4.0 * w.D * pairs * w.B * w.H, (2 * R + 2 * kvl) * w.D * e * w.B * w.H)
        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        n_split = args.n_split or A.splitkv_choose(w.B, w.H, R, kvl, n_cu)
        ws = torch.empty(max(16, A.splitkv_workspace_bytes(w.B, w.H, R, n_split)), dtype=torch.uint8, device=dev)
        log(f"[bench] decode: {R} row(s) x {kvl} keys per head, n_split {n_split}")
    if args.varlen:
        if chunk or args.stream:
            print("--varlen takes a single-call workload", file=sys.stderr)
            sys.exit(2)
        lens_cpu = W.varlen_lengths(w.B, w.S_kv, seed=w.seed + 900, edges=False)
        lens = lens_cpu.to(dev)
        work = varlen_work(w, lens_cpu.tolist(), dtype)
        log(f"[bench] varlen: lengths {lens_cpu.tolist()[:8]}..., "
            f"{work[0] / w.flops():.3f} of the full-length work")
    if args.stream:
        if not chunk:
            print("--stream needs a chunked workload", file=sys.stderr)
            sys.exit(2)
        # The window's new K/V rows and queries arrive as separate buffers;
        # the cache holds NaN past kv_len (never read).
        q, k, v, o = sets[0]
        bounds = [(s, min(w.S_q, s + chunk)) for s in range(0, w.S_q, chunk)]
        win = [tuple(x[:, :, a:b].contiguous() for x in (q, k, v, o)) for a, b in bounds]
        kc = torch.full_like(k, float("nan"))
        vc = torch.full_like(v, float("nan"))
        del sets[:], q, k, v, o
        log(f"[bench] streaming: {len(bounds)} windows of {chunk} rows")
    n_sets = 1 if args.stream else len(sets)

    def step(i):
        if args.stream:
            kv = 0
            for qw, kw, vw, ow in win:
                kv = A.attn_kv_append(kc, vc, kw, vw, kv)
                A.attn_fwd_chunked(qw, kc, vc, chunk=chunk, kv_len=kv, causal=w.causal, scale=w.scale, out=ow)
            return
        q, k, v, o = sets[i % len(sets)]
        if args.decode:
            A.attn_fwd_splitkv(q, k, v, causal=w.causal, scale=w.scale, n_split=n_split, out=o, workspace=ws)
        elif args.varlen:
            A.attn_fwd_varlen(q, k, v, lens, causal=w.causal, scale=w.scale, out=o)
        elif chunk:
            A.attn_fwd_chunked(q, k, v, chunk=chunk, causal=w.causal, scale=w.scale, out=o)
        else:
            A.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    long_steps = bool(args.stream or chunk)
    if args.steps is None:  # about 0.5 s of GPU time (long workloads: 10 steps), from a short eager estimate
        est = estimate_ms(step, stream, 3 if long_steps else 20)
        args.steps = int(min(20000, max(10, math.ceil(500.0 / max(est, 1e-3)))))
        if long_steps:
            args.steps = min(args.steps, 10)
        log(f"[bench] ~{est * 1e3:.1f} us per eager step: timing {args.steps} steps")
    # Steps of ~0.3 s need no untimed replay of each graph before the timing.
    tm = Timer(step, args.steps, args.repeats, args.eager, stream, replay_once=not long_steps)

    clk0 = gpu_clock_mhz(dev)
    t0 = time.perf_counter()
    total_ms, rep_ms = tm.run()
    wall = time.perf_counter() - t0
    clk1 = gpu_clock_mhz(dev)
    ms = total_ms / args.steps
    sec = ms / 1e3
    tflops = (work[0] if work else w.flops()) / sec / 1e12
    med = sorted(rep_ms)[len(rep_ms) // 2]
    log(f"[bench] {ms * 1e3:.2f} us/call (median of {len(rep_ms)} repeats {med * 1e3:.2f}), "
        f"{tflops:.2f} TFLOP/s, wall {wall:.3f} s, clock {clk0} -> {clk1} MHz")
    aa = None
    if not args.no_aa:  # A/A control: the same steps timed again in this process
        total2, _ = tm.run()
        aa = round(total2 / total_ms, 4)
        log(f"[bench] A/A: second timing / first = {aa}")

    line = {
        "metric": METRIC, "value": round(tflops, 4), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S_q": w.S_q, "S_kv": w.S_kv, "D_h": w.D,
                   "causal": w.causal, "chunk": w.chunk, "rotating_sets": n_sets,
                   "sets_timed": sets_timed(args.steps, n_sets),
                   "mode": (f"decode: {w.S_q} query row(s) against the whole cache, keys split over "
                            f"{n_split} workgroup range(s) (attn_fwd_splitkv)" if args.decode else
                            "stream: append + attend per window" if args.stream else
                            "varlen: per-sequence key lengths uniform on [S_kv/4, S_kv], visible pairs counted"
                            if args.varlen else
                            f"single attn_fwd_chunked call, {-(-w.S_q // chunk)} windows of {chunk} query rows"
                            if chunk else "single attn_fwd call"),
                   "launch": tm.launch},
        "roofline": roofline_for(w, dtype, sec, work),
        "timing": {"repeats": len(rep_ms), "steps_per_repeat": tm.sizes,
                   "ms_per_step_each_repeat": [round(x, 6) for x in rep_ms],
                   "median_ms_per_step": round(med, 6),
                   "gpu_clock_mhz": clock_block(clk0, clk1),
                   "aa_ratio": aa},
        "environment": environment(dev),
    }
    alg_bytes = work[1] if work else w.bytes(dtype)
    line["bandwidth"] = {"algorithmic_bytes": int(alg_bytes), "gbps": round(alg_bytes / sec / 1e9, 2),
                         "note": "Q, K, V read once and O written once per call, over the measured time"}
    if args.varlen:
        line["config"]["kv_lens"] = lens_cpu.tolist()
    line["roofline"]["traffic"] = None if special else measured_traffic(w.name, dtype)
    # The datasheet peak is the headline; the ceiling measured on this machine is
    # reported beside it, labelled.
    peaks = {}
    bound = line["roofline"]["bound"]
    peaks[(bound, dtype if bound == "mfma" else "hbm")] = mp = measured_peak(dev, bound, dtype)
    mp = dict(mp) if mp else None
    if mp is not None:
        mp["frac"] = round(line["roofline"]["achieved"] / mp["peak"], 4)
    line["roofline"]["peak_source"] = "datasheet"
    line["roofline"]["measured"] = mp
    del tm, sets
    if args.stream:
        del win, kc, vc
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        line["cpu_baseline"] = cpu_baseline(w, dtype, args.cpu_sample_seconds)
    else:
        line["cpu_baseline"] = None
    if with_per_config:
        line["per_config"] = [per_config_entry(args, name, dt, dev, stream, peaks) for name, dt in PER_CONFIG]
        line["per_config_note"] = ("each entry times its workload alone for about --per-config-seconds of GPU "
                                   "time (its own step count, 5 repeats, graph replay, rotating sets), "
                                   "independent of --steps and --warmup, which set the headline's steps; "
                                   "library_sdpa is context, not this library: torch's scaled_dot_product_attention "
                                   "(flash or memory-efficient backend) timed the same way on the same inputs")
    emit(args, line)


if __name__ == "__main__":
    main()
