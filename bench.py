#!/usr/bin/env python3
"""Benchmark of the modal-SSM Hyena hot path on one MI355X.

Default line (no arguments): the 24-layer projected stack at 1.3B width
(B=64, D=2048, 16 heads, d=16, 2048-token prompt, 512 generated tokens fed
back), which is the largest workload that fits one GPU.  A step is one pass
of the whole hot path over one batch of synthetic input:
  1. the prompt through all layers: per layer, the in_proj GEMM with the
     per-token RMS fused, the modal prefill (64-step sub-blocks on the matrix
     cores) and the out_proj GEMM;
  2. S generated tokens, each through all layers (per layer: the gate kernel
     -- in_proj with the RMS fused, u = k v, y = q (D u + rho), the next
     layer's prepare riding along -- and the out_proj kernel), one HIP graph
     per token captured once and replayed.
Two operator workloads ride along in ``sub_workloads``, each timed the same
way (filter taps, prefill, S decode steps as one graph replay):
  batch256-decode-bf16 (the decode step that must stream HBM) and
  long64k-f32 (the 64k-token prefill).
``--config N`` runs a single workload (1-5) instead.  Counter runs use
``--decode-mode eager --calibrate-copy`` (operator workloads) or
``--token-counters N`` (the stack's generated token) or ``--prefill-counters``
(the stack's prompt GEMMs), and ``--traffic-from``
turns their output into the committed traffic summaries.

Inputs are resident in HBM before any timed region.  Every time comes from
HIP events on the stream the library's kernels run on.  The ``roofline``
object covers the unit of work that dominates each step; ``cpu_baseline``
times the float64 oracle on this host over a bounded sample of the same
workload, and the same oracle outputs give ``parity`` (max |err| / max
|oracle| of the GPU's outputs on that sample).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/sec and prefill tokens/sec at 1 GPU; % of HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores
VALU_F32_PEAK_TFLOPS = 78.6    # 256 CU x 64 lanes x 2 flop (FMA) x 2.4 GHz, unpacked float32
TOL = {"f32": 1e-4, "bf16": 2e-2}

PROFILES = os.path.join(ROOT, "profiles")
PKG = os.path.join(ROOT, "distilled_modal_ssm_amd")
CSRC = os.path.join(PKG, "csrc")
# Sources whose change invalidates a hardware-counter measurement of a kernel:
# the kernel's own file (its code and launch configuration), the shared
# device header and, where it adds flags for that file, the build script.
KERNEL_SOURCES = {
    "decode_step_fixed": ["decode.hip", "hm_internal.hpp", "../build.py"],
    "chunk_mfma_kernel": ["prefill_mfma.hip", "prefill.hip", "hm_internal.hpp"],
    "chunk_scan_kernel": ["prefill.hip", "hm_internal.hpp"],
    # the projected stack's generated token: the gate (with the next layer's
    # prepare riding along) and out_proj, both streaming GEMMs of dense.hip
    "stack_token": ["dense.hip", "hm_internal.hpp"],
    # the stack's prompt GEMMs (in_proj with the row scale, out_proj), both gemm_dl8_kernel
    "stack_prompt_gemm": ["dense.hip", "hm_internal.hpp"],
}
# Dispatches that make up one generated token of the stack, per layer (names as
# the profiler prints them, matched by prefix).
STACK_TOKEN_KERNELS = {
    "gate": "gemm_stream_lds_kernel<3, 1, true, 32, -1,",
    "out_proj": "gemm_stream_dl_kernel<6>",
}
# Prompt GEMM dispatches of one layer's prefill: in_proj and out_proj, one each
STACK_PROMPT_GEMM_KERNELS = {"in_proj + out_proj": ("gemm_dl8_kernel", 2)}
COPY_BYTES = 1 << 30  # the calibration copy: 1 GiB read, 1 GiB written


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ provenance


def source_fingerprint() -> str:
    """sha256 (16 hex digits) over the library sources, the header, the Python
    package and this file: identifies the code a result line came from, also
    where no git metadata travels with the tree."""
    files = sorted(glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h")) +
                   glob.glob(os.path.join(PKG, "*.py")) + [os.path.abspath(__file__)])
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def git_sha():
    """HEAD's commit from .git when the tree has one (None elsewhere)."""
    try:
        head = open(os.path.join(ROOT, ".git", "HEAD")).read().strip()
        if head.startswith("ref: "):
            ref = head[5:]
            p = os.path.join(ROOT, ".git", ref)
            if os.path.exists(p):
                return open(p).read().strip()
            for line in open(os.path.join(ROOT, ".git", "packed-refs")):
                if line.strip().endswith(ref):
                    return line.split()[0]
            return None
        return head
    except OSError:
        return None


def build_info() -> dict:
    """The commit the library was built from, as the build recorded it."""
    try:
        with open(os.path.join(PKG, "build_info.json")) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def provenance() -> dict:
    b = build_info()
    return {"git_sha": git_sha(), "built_from_git_sha": b.get("git_sha"),
            "built_sources_modified": b.get("sources_modified"), "source_fingerprint": source_fingerprint()}


# ------------------------------------------------------------------ counter traffic


def kernel_fingerprint(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(PROFILES, f"{kernel}.{workload}.traffic.txt")


def read_traffic(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch of `kernel` on `workload`, from the
    committed summary, or None when there is none or the kernel's sources have
    changed since the counters were taken."""
    p = traffic_path(kernel, workload)
    if kernel not in KERNEL_SOURCES or not os.path.exists(p):
        return None
    kv = {}
    with open(p) as fh:
        for line in fh:
            if ":" in line and not line[0].isspace() and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("fingerprint") != kernel_fingerprint(kernel):
        return None
    return int(kv["traffic_bytes_per_launch"])


def calibration_copy():
    """One plain device copy of COPY_BYTES (three times), run only for counter
    collection: its FETCH_SIZE / WRITE_SIZE readings scale the kernel's."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _counter_rows(directory: str, counter: str):
    rows = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    if not rows:
        raise SystemExit(f"no {counter} rows under {directory}")
    return rows


def write_traffic(args):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    of this benchmark with --calibrate-copy (or, for the stack's generated
    token, of --token-counters) into the per-launch traffic summary."""
    from workloads import get_config
    cfg = get_config(args.config)
    kernel = args.traffic_kernel
    fetch_dir, write_dir = args.traffic_from
    # kernel name patterns and launches per unit: one dispatch of the kernel,
    # or for the stack's token every layer's gate and out_proj
    if kernel == "stack_token":
        parts = {k: (v, cfg.layers) for k, v in STACK_TOKEN_KERNELS.items()}
    elif kernel == "stack_prompt_gemm":
        parts = dict(STACK_PROMPT_GEMM_KERNELS)  # per layer: the mean dispatch x 2
    else:
        parts = {kernel: (kernel, 1)}
    out = {}
    per_part = []
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, name)
        copies = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        if not copies:
            raise SystemExit(f"{name}: no dispatch of the calibration copy in {d}")
        cal = max(copies)  # the 1 GiB copy is by far the largest copy dispatch
        factor = COPY_BYTES / (cal * 1024.0)
        kib = 0.0
        for part, (pat, per_unit) in parts.items():
            k = np.array([float(r["Counter_Value"]) for r in rows if pat in r["Kernel_Name"]])
            if len(k) == 0:
                raise SystemExit(f"{name}: no dispatches of {pat} in {d}")
            kib += per_unit * k.mean()
            per_part.append(f"# {name} {part} ({pat}...): {len(k)} dispatches, mean {k.mean():.1f} KiB "
                            f"(min {k.min():.1f}, max {k.max():.1f}) x {per_unit} per launch")
        out[name] = dict(kib=kib, copy_kib=cal, factor=factor, bytes=kib * 1024.0 * factor)
    sb = cfg.act_bytes
    if kernel == "stack_token":
        alg = stack_token_bytes(cfg)
    elif kernel == "stack_prompt_gemm":
        alg = stack_prompt_gemm_bytes(cfg)
    elif kernel.startswith("decode"):
        alg = cfg.B * cfg.D * (16 * cfg.d + 4 * sb)
    else:
        alg = 4 * sb * cfg.B * cfg.L * cfg.D + 8 * cfg.B * cfg.D * cfg.d
    total = int(round(out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]))
    cmd = args.traffic_cmd or "(commands not recorded)"
    lines = [
        f"# HBM traffic per launch of {kernel}, workload {cfg.name} ({cfg.describe()})",
        "#",
        "# Commands (repository root, one MI355X):",
    ] + [f"#     {c}" for c in cmd.split(" ;; ")] + [
        "#",
        "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by",
        f"# {COPY_BYTES} bytes / (what the same counter reads for a plain {COPY_BYTES >> 30} GiB device copy).",
        "#",
    ]
    lines += per_part + ["#"]
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        o = out[name]
        lines.append(f"# {name}: {o['kib']:.1f} KiB per launch; copy reads {o['copy_kib']:.1f} KiB -> "
                     f"factor {o['factor']:.4f} -> {o['bytes'] / 1e6:.3f} MB")
    lines += [
        "#",
        f"kernel: {kernel}",
        f"workload: {cfg.name}",
        f"fingerprint: {kernel_fingerprint(kernel)}",
        f"fetch_factor: {out['FETCH_SIZE']['factor']:.6f}",
        f"write_factor: {out['WRITE_SIZE']['factor']:.6f}",
        f"traffic_bytes_per_launch: {total}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {total / alg:.4f}",
    ]
    os.makedirs(PROFILES, exist_ok=True)
    path = traffic_path(kernel, cfg.name)
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(open(path).read())


def write_trace_summary(args):
    """Turn a rocprofv3 --kernel-trace --stats run of this benchmark into the
    committed text summary: per-kernel calls and durations, plus the command."""
    src, dst = args.summarize_trace
    files = glob.glob(os.path.join(src, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {src}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    agg = {}
    for r in rows:
        a = agg.setdefault(r["Name"], [0, 0.0, float("inf"), 0.0])
        n = int(r["Calls"])
        a[0] += n
        a[1] += float(r["TotalDurationNs"])
        a[2] = min(a[2], float(r["MinNs"]))
        a[3] = max(a[3], float(r["MaxNs"]))
    total = sum(a[1] for a in agg.values())
    lines = [f"# {args.summary_title or 'rocprofv3 kernel statistics'}", "",
             "Command (run from the repository root on one MI355X):", "", f"    {args.traffic_cmd or '(not recorded)'}",
             "", "rocprofv3 kernel statistics (durations per dispatch):", "",
             f"{'kernel':<72s} {'calls':>7s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_ms':>9s} {'pct':>6s}"]
    for name, a in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        short = name if len(name) <= 72 else name[:69] + "..."
        lines.append(f"{short:<72s} {a[0]:>7d} {a[1] / a[0] / 1e3:>10.2f} {a[2] / 1e3:>10.2f} {a[3] / 1e3:>10.2f} "
                     f"{a[1] / 1e6:>9.3f} {100 * a[1] / total:>6.2f}")
    with open(dst, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(open(dst).read())


# ------------------------------------------------------------------ arguments


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=5, help="headline workload (1-5; 5 = projected stack)")
    ap.add_argument("--sub", default=None,
                    help="comma-separated operator workloads timed beside the headline "
                         "(default: 3,4 with the stack headline, none otherwise; '' for none)")
    ap.add_argument("--decode-mode", choices=["graph", "eager"], default="graph",
                    help="generated steps as HIP graph replays (timing) or eager launches (counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-1thread", type=int, default=None, metavar="CONFIG",
                    help=argparse.SUPPRESS)  # child process of the one-thread CPU baseline
    ap.add_argument("--no-extras", "--no-fir", dest="no_extras", action="store_true",
                    help="skip the distillation, FFT-prefill and explicit-filter baselines")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--fingerprint", action="store_true", help="print the source fingerprint and exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="no GPU: write the traffic summary of --traffic-kernel from two rocprofv3 --pmc runs")
    ap.add_argument("--traffic-kernel", default="decode_step_fixed",
                    help="decode_step_fixed, chunk_mfma_kernel, chunk_scan_kernel, stack_token or stack_prompt_gemm")
    ap.add_argument("--prefill-counters", action="store_true",
                    help="for counter runs of the stack's prompt GEMMs: the calibration copy, then one "
                         "eager prefill of the prompt through all layers")
    ap.add_argument("--token-counters", type=int, default=None, metavar="N",
                    help="for counter runs of the stack's generated token: the calibration copy, then N "
                         "generated tokens launched eagerly from a synthetic state (no prompt, no graphs)")
    ap.add_argument("--traffic-cmd", default=None, help="the profiling commands, ' ;; '-separated, for the summary")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT_TXT"), default=None,
                    help="no GPU: write a text summary of a rocprofv3 --kernel-trace --stats run "
                         "(command from --traffic-cmd, title from --summary-title)")
    ap.add_argument("--summary-title", default=None)
    return ap.parse_args()


# ------------------------------------------------------------------ shared helpers


def pct(x):
    return {"p10": float(np.percentile(x, 10)), "p50": float(np.median(x)), "p90": float(np.percentile(x, 90))}


def rel_err(got, ref) -> float:
    scale = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(got))) if np.size(got) else 0.0
    return float(np.max(np.abs(got - ref))) / scale


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def state_channels(state_t, chans, P) -> np.ndarray:
    """[B][H][d][P][2] device state -> [B][len(chans)][d][2] float64 (the oracle's layout)."""
    st = state_t.detach().cpu().numpy().astype(np.float64)
    ch = np.asarray(chans)
    return np.ascontiguousarray(st[:, ch // P, :, ch % P, :].transpose(1, 0, 2, 3))


def channel_sample(cfg, budget):
    """Evenly spaced channels so that the oracle's full step on them costs about
    ``budget`` mode-steps (all channels when the budget allows)."""
    per_channel = cfg.B * (cfg.L + cfg.S) * cfg.d
    n_sel = int(min(cfg.D, max(1, budget // per_channel)))
    if n_sel >= cfg.D:
        return np.arange(cfg.D, dtype=np.int64)
    return np.linspace(0, cfg.D - 1, n_sel).round().astype(np.int64)


def timed_events(stream, fn, n):
    """n calls of fn bracketed by HIP events on `stream`; ms per call."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for e in ev:
        e[0].record(stream)
        fn()
        e[1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


# ------------------------------------------------------------------ operator workloads


def operator_cpu_baseline(cfg, params, inp, dec, gpu_sample, min_seconds: float = 10.0):
    """The float64 oracle (as it stands) on this host over the same workload: the
    full step (filter, prefill, decode steps) repeated until ``min_seconds`` of
    CPU time have passed (at most 100 repetitions), on an evenly spaced channel
    subset when one repetition of the whole width would be too long.  The first
    repetition's outputs are compared with the GPU's on the same channels."""
    import oracle
    chans = channel_sample(cfg, 6e9)  # ~1 s per repetition on 16 cores
    sel = None if len(chans) == cfg.D else chans
    reps, first = 0, None
    t0 = time.perf_counter()
    while reps < 100 and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.filter_taps(params, cfg.L)
        y, st = oracle.modal_scan(params, inp["q"], inp["k"], inp["v"], channels=sel)
        yd, st2 = oracle.modal_scan(params, dec["q"], dec["k"], dec["v"], state=st, channels=sel,
                                    batch_axis=1, time_axis=0)
        if first is None:
            first = (y, yd, st2)
        reps += 1
    dt = time.perf_counter() - t0
    tokens = cfg.B * (cfg.L + cfg.S) * (len(chans) / cfg.D) * reps
    sample = (f"full step (filter, prefill L={cfg.L}, {cfg.S} decode steps) for "
              f"{'all' if sel is None else len(chans)} of {cfg.D} channels x {cfg.B} rows, {reps} repetition(s), "
              f"{dt:.1f} s; tokens scaled by the channel fraction")
    base = {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": sample}
    g_y, g_yd, g_st = gpu_sample(chans)
    tol = TOL[cfg.act]
    parity = {"sample": f"the cpu_baseline's first repetition: {len(chans)} channels x all {cfg.B} rows, "
                        f"every prompt position and generated step",
              "prefill_y": rel_err(g_y, first[0]), "decode_y": rel_err(g_yd, first[1]),
              "final_state": rel_err(g_st, first[2]), "tolerance": tol}
    parity["pass"] = bool(max(parity["prefill_y"], parity["decode_y"], parity["final_state"]) <= tol)
    return base, parity


def cpu_one_thread(ci: int, min_seconds: float = 5.0):
    """Child process of the CPU baseline (started with OMP_NUM_THREADS=1, no
    GPU use): the oracle's full step on one batch row and an evenly spaced
    channel subset, repeated for ``min_seconds``; prints one JSON line."""
    import dataclasses

    import oracle
    from workloads import decode_inputs, get_config, modal_params, prompt_inputs
    cfg = get_config(ci)
    params = modal_params(cfg)
    inp = prompt_inputs(cfg, batches=[0])
    dec = decode_inputs(cfg)
    dec = {k: np.ascontiguousarray(v[:, :1]) for k, v in dec.items()}
    one = dataclasses.replace(cfg, B=1)
    chans = channel_sample(one, 2e8)
    sel = None if len(chans) == cfg.D else chans
    reps, t0 = 0, time.perf_counter()
    while reps < 100 and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.filter_taps(params, cfg.L)
        _, st = oracle.modal_scan(params, inp["q"], inp["k"], inp["v"], channels=sel)
        oracle.modal_scan(params, dec["q"], dec["k"], dec["v"], state=st, channels=sel,
                          batch_axis=1, time_axis=0)
        reps += 1
    dt = time.perf_counter() - t0
    print(json.dumps({"value": (cfg.L + cfg.S) * (len(chans) / cfg.D) * reps / dt, "unit": "tokens/s",
                      "cores": oracle.threads(),
                      "sample": f"full step for batch row 0, {len(chans)} of {cfg.D} channels, {reps} "
                                f"repetition(s), {dt:.1f} s; tokens scaled by the channel fraction"}))


def cpu_baseline_one_thread(cfg):
    """The same oracle step on one thread, in a child process (the thread count
    of the oracle's OpenMP runtime is fixed when it loads)."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-1thread", str(cfg.index)],
                           env=env, capture_output=True, text=True, timeout=300)
        return json.loads(r.stdout.strip().splitlines()[-1])
    except Exception as e:  # reported, never fatal to the benchmark line
        return {"error": f"{type(e).__name__}: {e}"}


def run_operator(args, cfg, dev) -> dict:
    """One operator workload: filter taps, prefill, S decode steps per step."""
    import torch
    from distilled_modal_ssm_amd import ModalHyena
    from distilled_modal_ssm_amd import binding as hb
    from workloads import decode_inputs, modal_params, prompt_inputs

    log(f"[bench] workload {cfg.index} {cfg.describe()}: inputs")
    params = modal_params(cfg)
    inp = prompt_inputs(cfg)
    dec = decode_inputs(cfg)

    def to_dev(a):
        if cfg.act == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = (to_dev(inp[n]) for n in "qkv")
    dq, dk, dv = (to_dev(dec[n]) for n in "qkv")
    op = ModalHyena(params.poles, params.residues, params.skip, cfg.B, cfg.D, cfg.act, device=dev)
    tdt = op.tdtype
    y = torch.empty((cfg.B, cfg.L, cfg.D), dtype=tdt, device=dev)
    ys = torch.empty((cfg.S, cfg.B, cfg.D), dtype=tdt, device=dev)
    state = op.new_state()
    h = torch.empty((cfg.H, cfg.L), dtype=torch.float32, device=dev)
    op.workspace(cfg.L)  # allocate once, outside the timed region
    stream = torch.cuda.current_stream()

    def filter_call():
        hb.hyena_filter_materialize(op.desc, cfg.L, h)

    def prefill_call():
        op.prefill(q, k, v, y=y, state_out=state)

    def decode_eager():
        for s in range(cfg.S):
            op.decode_step(dq[s], dk[s], dv[s], state, y=ys[s])

    log(f"[bench] workload {cfg.index}: timing")
    if args.decode_mode == "graph":
        prefill_call()
        decode_eager()  # warm the launch path before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_eager()
        torch.cuda.synchronize()
        decode_call = graph.replay
    else:
        decode_call = decode_eager

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        filter_call()
        if ev:
            ev[1].record(stream)
        prefill_call()
        if ev:
            ev[2].record(stream)
        decode_call()
        if ev:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    ph = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in evs])
    ms_filter, ms_prefill, ms_decode = (float(np.median(ph[:, i])) for i in range(3))
    ms_decode_launch = ms_decode / cfg.S

    # outside the timed region: spreads of the prefill call and of the decode block
    pf_ms = timed_events(stream, prefill_call, 20 if cfg.L * cfg.B * cfg.D < 2 ** 30 else 5)
    dec_us = timed_events(stream, decode_call, 10) * 1e3 / cfg.S

    E = cfg.B * cfg.L * cfg.D
    sb = cfg.act_bytes
    decode_bytes = cfg.B * cfg.D * (16 * cfg.d + 4 * sb)
    prefill_bytes = 4 * sb * E + 8 * cfg.B * cfg.D * cfg.d
    prefill_flops = (12 * cfg.d + 5) * E
    plan = op.plan(cfg.L)
    if plan["algo"] == "mfma":
        # matrix-core sub-blocks: the products are a few % of the MFMA peak and
        # the pass streams q, k, v and y once, so HBM bounds it
        prefill_roof = dict(bound="hbm", unit="GB/s", per_launch=prefill_bytes, peak=HBM_PEAK_GBS,
                            kernel="chunk_mfma_kernel")
        prefill_rates = {"hbm_GBs": prefill_bytes / ms_prefill * 1e-6,
                         "hbm_frac": prefill_bytes / ms_prefill * 1e-6 / HBM_PEAK_GBS}
    else:
        # vector scan: one complex FMA pair per mode and step, on the vector ALUs
        prefill_roof = dict(bound="alu", unit="TFLOP/s", per_launch=prefill_flops, peak=VALU_F32_PEAK_TFLOPS,
                            kernel="chunk_scan_kernel")
        prefill_rates = {"alu_TFLOPs": prefill_flops / ms_prefill * 1e-9,
                         "alu_frac": prefill_flops / ms_prefill * 1e-9 / VALU_F32_PEAK_TFLOPS,
                         "hbm_GBs": prefill_bytes / ms_prefill * 1e-6,
                         "hbm_frac": prefill_bytes / ms_prefill * 1e-6 / HBM_PEAK_GBS}
    units = {
        "decode_step": dict(bound="hbm", unit="GB/s", per_launch=decode_bytes, ms=ms_decode_launch,
                            total_ms=ms_decode, peak=HBM_PEAK_GBS, kernel="decode_step_fixed"),
        "prefill": dict(ms=ms_prefill, total_ms=ms_prefill, **prefill_roof),
    }
    dom = units[max(units, key=lambda n: units[n]["total_ms"])]
    scale = 1e-6 if dom["unit"] == "GB/s" else 1e-9  # bytes/ms -> GB/s ; flops/ms -> TFLOP/s
    achieved = dom["per_launch"] / dom["ms"] * scale
    roofline = {"bound": dom["bound"], "achieved": round(achieved, 3), "peak": dom["peak"],
                "unit": dom["unit"], "frac": round(achieved / dom["peak"], 4),
                "traffic": read_traffic(dom["kernel"], cfg.name),
                "kernel": dom["kernel"], "launch_ms": round(dom["ms"], 6),
                ("algorithmic_bytes_per_launch" if dom["unit"] == "GB/s" else "algorithmic_flops_per_launch"):
                    dom["per_launch"]}
    notes = []
    if cfg.act == "f32" and plan["algo"] == "mfma":
        notes.append("float32 activations and state; the prefill's matrix-core products take every operand "
                     "as a sum of three bfloat16 parts (hi + mid + lo) with float32 accumulation")
    if decode_bytes < 64e6:
        notes.append("the decode step's state and activations fit in L2 and the Infinity Cache: its time is "
                     "set by dispatch latency, not HBM")
    res = {
        "workload": f"{cfg.name}: {cfg.describe()}",
        "config": {"workload": cfg.name, "B": cfg.B, "D": cfg.D, "H": cfg.H, "d": cfg.d, "L": cfg.L, "S": cfg.S,
                   "act_dtype": cfg.act, "decode_mode": args.decode_mode},
        "dtype": cfg.act,
        "tokens_per_s": cfg.B * (cfg.L + cfg.S) / (ms_step / 1e3),
        "ms_per_step": ms_step,
        "prefill_plan": plan,
        "prefill_tokens_per_s": cfg.B * cfg.L / (ms_prefill / 1e3),
        "decode_tokens_per_s": cfg.B / (ms_decode_launch / 1e3),
        "phase_ms": {"filter": ms_filter, "prefill": ms_prefill, "decode_total": ms_decode,
                     "decode_per_step": ms_decode_launch},
        "decode_step_us_per_replay": pct(dec_us),
        "prefill_ms_per_call": pct(pf_ms),
        "prefill_rates": prefill_rates,
        "decode_rates": {"hbm_GBs": decode_bytes / ms_decode_launch * 1e-6,
                         "hbm_frac": decode_bytes / ms_decode_launch * 1e-6 / HBM_PEAK_GBS},
        "roofline": roofline,
        "notes": notes,
    }
    if not args.no_extras:
        res["distill"] = distill_bench(cfg, params, stream)
        res["fft_prefill"] = fft_prefill_baseline(cfg, op, q, k, v, ms_prefill, stream)
        for window in (0, 256):
            res[f"fir_baseline_w{window}"] = fir_baseline(cfg, op, k, v, dq, dk, dv, window,
                                                          ms_decode_launch, stream)
    if args.calibrate_copy:
        calibration_copy()
    if not args.no_cpu_baseline:
        # one more whole step, so that y, ys and state hold exactly one step's
        # outputs (the spreads above replayed the decode block on top of it)
        step()
        torch.cuda.synchronize()

        def gpu_sample(chans):
            ct = torch.as_tensor(chans, device=dev)
            return (to_f64(y.index_select(2, ct)), to_f64(ys.index_select(2, ct)).transpose(1, 0, 2),
                    state_channels(state, chans, cfg.P))

        log(f"[bench] workload {cfg.index}: cpu baseline (float64 oracle) and parity")
        res["cpu_baseline"], res["parity"] = operator_cpu_baseline(cfg, params, inp, dec, gpu_sample)
        res["cpu_baseline"]["one_thread"] = cpu_baseline_one_thread(cfg)
    del q, k, v, dq, dk, dv, y, ys
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ projected stack


def stack_prompt_gemm_bytes(cfg) -> int:
    """HBM bytes one layer's two prompt GEMMs must move: in_proj reads the
    layer input [B L][D] and W_in [3D][D] and writes q, k, v [B L][3D]; out_proj
    reads the operator output [B L][D] and W_out [D][D] and writes [B L][D]
    (bf16 throughout; the row scales, 4 bytes a row, are left out)."""
    M, D = cfg.B * cfg.L, cfg.D
    return 2 * (M * D + 3 * D * D + 3 * M * D) + 2 * (M * D + D * D + M * D)


def stack_token_bytes(cfg) -> int:
    """HBM bytes a generated token of the projected stack must move: per layer the
    bf16 weights (W_in 3D x D, W_out D x D), the modal state read and written
    (16 d bytes per row and channel), and the bf16 activations: the layer input
    read, the operator output written and read back by out_proj, the layer
    output written (q, k, v stay on chip in the fused step)."""
    D, B = cfg.D, cfg.B
    return cfg.layers * (4 * D * D * 2 + B * D * 16 * cfg.d + 4 * B * D * 2)


def stack_cpu_baseline(cfg, layers, rec_prompt, rec_steps, rows, min_seconds: float = 10.0):
    """The float64 oracle on a bounded sample of the stack: layers 0, 1, ... in
    turn (until ``min_seconds`` have passed, at least two) for the recorded
    batch rows, each layer teacher-forced on the inputs the GPU's layer
    received (the prompt and all S generated steps).  Tokens are scaled by the
    row and layer fractions; the same outputs give the per-layer parity of the
    GPU's layer outputs."""
    import oracle
    errs = []
    t0 = time.perf_counter()
    for l in range(cfg.layers):
        if l >= 2 and time.perf_counter() - t0 >= min_seconds:
            break
        p, w_in, w_out = layers[l]
        out_p, out_s, _, _ = oracle.stack_layer(p, oracle.bf16_to_f64(w_in), oracle.bf16_to_f64(w_out),
                                                rec_prompt[l], rec_steps[l])
        errs.append((rel_err(oracle.bf16_to_f64(rec_prompt[l + 1]), out_p),
                     rel_err(oracle.bf16_to_f64(rec_steps[l + 1]), out_s)))
    dt = time.perf_counter() - t0
    nl = len(errs)
    tokens = len(rows) * (cfg.L + cfg.S) * nl / cfg.layers
    sample = (f"batch rows {list(map(int, rows))} of {cfg.B}, layers 0-{nl - 1} of {cfg.layers}, each "
              f"teacher-forced on the GPU's inputs over the {cfg.L}-token prompt and {cfg.S} generated steps")
    base = {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{sample}, {dt:.1f} s; tokens scaled by the row and layer fractions"}
    worst = max(max(e) for e in errs)
    parity = {"sample": sample,
              "per_layer": [{"layer": l, "prompt_out": e[0], "generated_out": e[1]} for l, e in enumerate(errs)],
              "worst": worst, "tolerance": TOL["bf16"], "pass": bool(worst <= TOL["bf16"])}
    return base, parity


def run_stack(args, cfg, dev) -> dict:
    """Projected stack: prefill through all layers, then S generated tokens per
    batch row (one HIP graph per generated token, replayed; or eager)."""
    import torch
    from distilled_modal_ssm_amd.stack import HyenaStack
    from workloads import dense_weights, modal_params, stack_prompt

    log(f"[bench] workload {cfg.index} {cfg.describe()}: weights and prompt")
    with ThreadPoolExecutor(8) as ex:
        ws = list(ex.map(lambda l: dense_weights(cfg, l), range(cfg.layers)))
    layers = [(modal_params(cfg, l), *ws[l]) for l in range(cfg.layers)]
    del ws
    st = HyenaStack(layers, cfg.B, cfg.L, device=dev)
    x0 = stack_prompt(cfg)
    X = torch.from_numpy(x0.view(np.int16)).view(torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream()

    log(f"[bench] workload {cfg.index}: timing ({args.decode_mode} generation)")
    out = st.prefill(X)
    st.start_generation(out)
    st.decode_step()
    torch.cuda.synchronize()
    if args.decode_mode == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            st.decode_step()
        torch.cuda.synchronize()
        token_call = graph.replay
    else:
        token_call = st.decode_step

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        o = st.prefill(X)
        st.start_generation(o)
        if ev:
            ev[1].record(stream)
        for _ in range(cfg.S):
            token_call()
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    ph = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in evs])
    ms_prefill, ms_decode = float(np.median(ph[:, 0])), float(np.median(ph[:, 1]))
    ms_tok = ms_decode / cfg.S

    M, D = cfg.B * cfg.L, cfg.D
    gemm_flops = cfg.layers * 2 * M * D * 4 * D          # in_proj (3D) + out_proj (D)
    hyena_flops = cfg.layers * (12 * cfg.d + 5) * M * D
    token_bytes = stack_token_bytes(cfg)
    decode_gbs = token_bytes / ms_tok * 1e-6
    gemm_tf = gemm_flops / ms_prefill * 1e-9
    if ms_prefill >= ms_decode:
        roof = {"bound": "mfma", "achieved": round(gemm_tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "kernel": "prompt through all layers (in_proj/out_proj GEMMs dominant)",
                "launch_ms": round(ms_prefill, 4), "algorithmic_flops_per_launch": gemm_flops}
    else:
        roof = {"bound": "hbm", "achieved": round(decode_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "kernel": f"generated token: one graph launch of {cfg.layers} x (gate with the next layer's "
                          f"prepare, out_proj)",
                "launch_ms": round(ms_tok, 5), "algorithmic_bytes_per_launch": token_bytes}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    # counter-measured HBM bytes of the dominant phase's kernels: the token's
    # gates and out_projs, or the prompt GEMMs (summary per layer; the mfma
    # roofline counts the prompt through all layers)
    if roof["bound"] == "hbm":
        roof["traffic"] = read_traffic("stack_token", cfg.name)
    else:
        t = read_traffic("stack_prompt_gemm", cfg.name)
        roof["traffic"] = t * cfg.layers if t is not None else None

    # outside the timed region: the generation kernels alone, each captured
    # 24 times over the layers (cache-cold weights, as in the stack) and
    # replayed; the prompt GEMMs of one layer eagerly
    kern = stack_kernel_breakdown(cfg, st, X, stream)

    res = {
        "workload": f"{cfg.name}: {cfg.describe()}",
        "config": {"workload": cfg.name, "B": cfg.B, "D": cfg.D, "H": cfg.H, "d": cfg.d, "L": cfg.L, "S": cfg.S,
                   "layers": cfg.layers, "act_dtype": cfg.act,
                   "decode_mode": "graph per generated token" if args.decode_mode == "graph" else "eager"},
        "dtype": "bf16",
        "tokens_per_s": cfg.B * (cfg.L + cfg.S) / (ms_step / 1e3),
        "ms_per_step": ms_step,
        "prefill_tokens_per_s": M / (ms_prefill / 1e3),
        "decode_tokens_per_s": cfg.B / (ms_tok / 1e3),
        "phase_ms": {"prefill": ms_prefill, "decode_total": ms_decode, "decode_per_token": ms_tok},
        "prefill_rates": {"gemm_TFLOPs": gemm_tf, "gemm_mfma_frac": gemm_tf / MFMA_BF16_PEAK_TFLOPS,
                          "all_TFLOPs": (gemm_flops + hyena_flops) / ms_prefill * 1e-9},
        "decode_rates": {"hbm_GBs": decode_gbs, "hbm_frac": decode_gbs / HBM_PEAK_GBS,
                         "algorithmic_bytes_per_token": token_bytes},
        "kernels": kern,
        "roofline": roof,
    }
    if args.calibrate_copy:
        calibration_copy()
    if not args.no_cpu_baseline:
        log(f"[bench] workload {cfg.index}: recording layer inputs for the oracle sample")
        rows = np.array([5, 58])
        rec_p, rec_s = stack_record(cfg, st, X, rows, cfg.layers)
        log(f"[bench] workload {cfg.index}: cpu baseline (float64 oracle, sampled) and parity")
        res["cpu_baseline"], res["parity"] = stack_cpu_baseline(cfg, layers, rec_p, rec_s, rows)
    del st, X
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def token_counter_run(cfg, dev, n_tokens: int) -> None:
    """Counter collection for the stack's generated token: the 1 GiB calibration
    copy, then ``n_tokens`` generated tokens launched eagerly (the per-layer
    gate with its ride-along prepare, and out_proj).  The state and the first
    input are synthetic (no prompt pass); the kernels and their bytes are those
    of the timed generation."""
    import torch
    from distilled_modal_ssm_amd.stack import HyenaStack
    from workloads import dense_weights, modal_params

    if not cfg.layers:
        raise SystemExit("--token-counters needs the stack workload (--config 5)")
    log(f"[bench] workload {cfg.index}: weights for the token counter run")
    with ThreadPoolExecutor(8) as ex:
        ws = list(ex.map(lambda l: dense_weights(cfg, l), range(cfg.layers)))
    layers = [(modal_params(cfg, l), *ws[l]) for l in range(cfg.layers)]
    del ws
    st = HyenaStack(layers, cfg.B, 1, device=dev)
    if not st.deferred:
        raise SystemExit("the stack's shape does not take the deferred generation path")
    g = torch.Generator(device=dev).manual_seed(11)
    for s in st.states:
        s.copy_(0.01 * torch.randn(s.shape, device=dev, generator=g))
    st.start_generation(torch.randn(cfg.B, cfg.D, device=dev, generator=g).to(torch.bfloat16))
    torch.cuda.synchronize()
    calibration_copy()
    for t in range(n_tokens):
        log(f"[bench] token {t}")
        st.decode_step()
        torch.cuda.synchronize()
    print(json.dumps({"token_counter_run": cfg.name, "tokens": n_tokens, "layers": cfg.layers}), flush=True)


def prefill_counter_run(cfg, dev) -> None:
    """Counter collection for the stack's prompt GEMMs: the 1 GiB calibration
    copy, then one prefill of the prompt through all layers (eager), whose
    in_proj and out_proj are the kernels and shapes of the timed prefill."""
    import torch
    from distilled_modal_ssm_amd.stack import HyenaStack
    from workloads import dense_weights, modal_params, stack_prompt

    if not cfg.layers:
        raise SystemExit("--prefill-counters needs the stack workload (--config 5)")
    log(f"[bench] workload {cfg.index}: weights and prompt for the prefill counter run")
    with ThreadPoolExecutor(8) as ex:
        ws = list(ex.map(lambda l: dense_weights(cfg, l), range(cfg.layers)))
    layers = [(modal_params(cfg, l), *ws[l]) for l in range(cfg.layers)]
    del ws
    st = HyenaStack(layers, cfg.B, cfg.L, device=dev)
    X = torch.from_numpy(stack_prompt(cfg).view(np.int16)).view(torch.bfloat16).to(dev)
    torch.cuda.synchronize()
    calibration_copy()
    log("[bench] prefill")
    st.prefill(X)
    torch.cuda.synchronize()
    print(json.dumps({"prefill_counter_run": cfg.name, "layers": cfg.layers}), flush=True)


def stack_record(cfg, st, X, rows, nl):
    """One untimed pass (prompt, then S generated tokens, eager) that copies the
    inputs of layers 0..nl (the outputs of layers 0..nl-1) for ``rows``."""
    import torch
    rt = torch.as_tensor(rows, device=X.device)
    L, D, S = cfg.L, cfg.D, cfg.S
    rec_p = torch.empty((nl + 1, len(rows), L, D), dtype=torch.bfloat16, device=X.device)
    rec_s = torch.empty((nl + 1, S, len(rows), D), dtype=torch.bfloat16, device=X.device)

    def rp(l, x):
        if l <= nl:
            rec_p[l] = x.view(cfg.B, L, D).index_select(0, rt)

    out = st.prefill(X, record=rp)
    if nl >= cfg.layers:
        rec_p[nl] = out.view(cfg.B, L, D).index_select(0, rt)
    st.start_generation(out)
    for s in range(S):
        def rd(l, x, s=s):
            if l <= nl:
                rec_s[l, s] = x.index_select(0, rt)
        y = st.decode_step(record=rd)
        if nl >= cfg.layers:
            rec_s[nl, s] = y.index_select(0, rt)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    return bits(rec_p), bits(rec_s)


def stack_kernel_breakdown(cfg, st, X, stream) -> dict:
    """Per-kernel times of the stack with HIP events: the generation step's two
    kernels, each launched once per layer (24 distinct weights, so the weights
    come from HBM as in the stack) inside one captured graph, replayed 10
    times; and the prompt's two GEMMs of layer 0, eagerly."""
    import torch
    from distilled_modal_ssm_amd import binding as hb
    from distilled_modal_ssm_amd.stack import RMS_EPS
    B, D, L, nl = cfg.B, cfg.D, cfg.L, cfg.layers
    out = {}
    fusable = st.w_in_packed is not None and hb.hyena_layer_step_bf16(
        st.ops[0].desc, st.xd, D, st.w_in_packed[0], RMS_EPS, st.states[0], st.yd, D) == hb.HM_OK
    gens = []
    if st.deferred:
        def gate():
            for l in range(nl):
                n = (l + 1) % nl
                hb.hyena_layer_gate_bf16(st.ops[l].desc, st.xd, st.xd.stride(0), st.w_in_packed[l], RMS_EPS,
                                         st.rho[l], st.u_prev[l], st.yd, st.yd.stride(0), st.ops[n].desc,
                                         st.states[n], st.u_prev[n], st.rho[n])

        def outp():
            for l in range(nl):
                hb.hyena_dense_bf16(B, D, D, st.yd, st.yd.stride(0), st.w_out[l], st.w_out[l].stride(0), None,
                                    st.xd_mid[0], st.xd_mid[0].stride(0), workspace=st.ws)

        # gate + the next layer's prepare: W_in, the layer input read, y written, rho read and u_prev
        # written; the next layer's state read and written, its u_prev read and rho written
        gens = [("gate_in_proj_prepare", gate,
                 3 * D * D * 2 + 2 * B * D * 2 + 2 * B * D * 4 + B * D * 16 * cfg.d + 2 * B * D * 4),
                ("out_proj", outp, D * D * 2 + 2 * B * D * 2)]
    elif fusable:
        def fused():
            for l in range(nl):
                hb.hyena_layer_step_bf16(st.ops[l].desc, st.xd, st.xd.stride(0), st.w_in_packed[l], RMS_EPS,
                                         st.states[l], st.yd, st.yd.stride(0))

        def outp():
            for l in range(nl):
                hb.hyena_dense_bf16(B, D, D, st.yd, st.yd.stride(0), st.w_out[l], st.w_out[l].stride(0), None,
                                    st.xd_mid[0], st.xd_mid[0].stride(0), workspace=st.ws)

        gens = [("fused_in_proj_decode", fused, 3 * D * D * 2 + B * D * 16 * cfg.d + 2 * B * D * 2),
                ("out_proj", outp, D * D * 2 + 2 * B * D * 2)]
    if gens:
        for name, fn, byts in gens:
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            torch.cuda.synchronize()
            us = timed_events(stream, g.replay, 10) * 1e3 / nl
            out[name] = {"us_per_launch": pct(us), "algorithmic_bytes_per_launch": byts,
                         "hbm_GBs": byts / np.median(us) * 1e-3,
                         "hbm_frac": byts / np.median(us) * 1e-3 / HBM_PEAK_GBS}
            del g
    M = B * L
    x = X.reshape(M, D)

    def in_proj():  # as the stack's prompt: the row RMS pass, then the projection with the row scale
        hb.hyena_row_rms(x, M, D, D, RMS_EPS, st.inv_rms)
        hb.hyena_dense_bf16(M, 3 * D, D, x, D, st.w_in[0], D, st.inv_rms, st.qkv, 3 * D)

    def out_proj_p():
        hb.hyena_dense_bf16(M, D, D, st.y, D, st.w_out[0], D, None, st.x[0], D)

    for name, fn, flops in (("prompt_in_proj", in_proj, 2 * M * 3 * D * D), ("prompt_out_proj", out_proj_p, 2 * M * D * D)):
        fn()
        ms = timed_events(stream, fn, 5)
        out[name] = {"ms_per_launch": pct(ms), "algorithmic_flops_per_launch": flops,
                     "TFLOPs": flops / np.median(ms) * 1e-9,
                     "mfma_frac": flops / np.median(ms) * 1e-9 / MFMA_BF16_PEAK_TFLOPS}
    return out


# ------------------------------------------------------------------ f2-f4 baselines


def distill_bench(cfg, params, stream, steps=300):
    """Distillation of d-mode filters from a richer target: the filters of a
    2d-mode system (this workload's modes plus d more, radii scaled by 0.98 and
    residues halved), materialised by the library.  Iterations (objective,
    gradient, Adam step) captured in a HIP graph and timed; the loss over the
    run is reported."""
    import torch
    from distilled_modal_ssm_amd import ModalHyena
    from distilled_modal_ssm_amd.distill import ModalDistiller
    log("[bench] distillation iterations")
    poles = np.concatenate([params.poles, params.poles[:, ::-1] * np.float32(0.98)], 1)
    res = np.concatenate([params.residues, params.residues * np.float32(0.5)], 1)
    rich = ModalHyena(poles, res, params.skip, 1, cfg.H, "f32")
    target = rich.filter(cfg.L)
    dist = ModalDistiller(target, cfg.d)
    hist = torch.empty((steps, cfg.H), dtype=torch.float32, device="cuda")
    dist.step(1e-2, loss=hist[0], stream=stream)  # warm
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(1, steps):
            dist.step(1e-2, loss=hist[i])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (steps - 1)
    h = hist.sum(1).cpu().numpy()
    del graph
    out = {"heads": cfg.H, "modes": cfg.d, "taps": cfg.L, "target_modes": 2 * cfg.d, "iterations": steps,
           "us_per_iteration": us, "loss_first": float(h[0]), "loss_last": float(h[-1])}
    # the Prony-type start (host: Hankel order, matrix pencil, least squares), then Adam
    from distilled_modal_ssm_amd.distill import hankel_order
    t0 = time.perf_counter()
    order = hankel_order(target, 64, 1e-6)
    fit = ModalDistiller(target, cfg.d, init="fit")
    t_init = time.perf_counter() - t0
    first = float(fit.objective().sum().item())
    hist2 = torch.empty((steps, cfg.H), dtype=torch.float32, device="cuda")
    for i in range(steps):
        fit.step(1e-5, loss=hist2[i], stream=stream)
    last = float(fit.objective().sum().item())
    out["fit_start"] = {"hankel_order_at_1e-6": [int(o) for o in order], "host_init_s": t_init,
                        "loss_at_start": first, "adam_lr": 1e-5, "loss_after_adam": last,
                        "below_default_start_first": float(h[0]) / max(last, 1e-30)}
    return out


def fft_prefill_baseline(cfg, op, q, k, v, ms_modal_prefill, stream):
    """The same prompt through the FFT convolution (Hyena's own prefill), timed
    with HIP events outside the timed step (20 calls; 5 past 4096 steps, where
    the transforms run in three passes over HBM)."""
    import torch
    from distilled_modal_ssm_amd import binding as hb
    log("[bench] FFT prefill baseline")
    n = hb.hyena_fft_prefill_workspace(op.desc, cfg.L)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=op.device)
    yf = torch.empty((cfg.B, cfg.L, cfg.D), dtype=op.tdtype, device=op.device)

    def call():
        hb.hyena_fft_prefill(op.desc, cfg.L, q, k, v, cfg.D, yf, cfg.D, ws, n, stream)

    call()
    torch.cuda.synchronize()
    multipass = cfg.L > 4096
    ms = float(np.median(timed_events(stream, call, 5 if multipass else 20)))
    byts = 4 * cfg.act_bytes * cfg.B * cfg.L * cfg.D
    del ws, yf
    torch.cuda.empty_cache()
    return {"ms": ms, "tokens_per_s": cfg.B * cfg.L / (ms / 1e3),
            "transforms": "three passes over HBM" if multipass else "in LDS",
            "operator_GBs": byts / ms * 1e-6, "modal_prefill_speedup": ms / ms_modal_prefill}


def fir_baseline(cfg, op, k, v, dq, dk, dv, window, ms_modal_step, stream):
    """The non-distilled decode on the same workload, outside the timed step:
    the prompt's u cached (not timed), then S generated tokens through the
    explicit filter (window 0 = every past step), captured in a HIP graph."""
    import torch
    from distilled_modal_ssm_amd import binding as hb
    log(f"[bench] explicit-filter decode baseline, window {window or 'full'}")
    fir = hb.FirHyena(op, cfg.L + cfg.S)
    fir.fill(k, v)
    h = op.filter(cfg.L + cfg.S)
    yf = torch.empty((cfg.S, cfg.B, cfg.D), dtype=op.tdtype, device=op.device)

    def run():
        for s in range(cfg.S):
            fir.step(h, cfg.L + s, dq[s], dk[s], dv[s], window=window, y=yf[s])

    run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    graph.replay()
    torch.cuda.synchronize()
    ms_step = float(timed_events(stream, graph.replay, 1)[0]) / cfg.S
    sb = cfg.act_bytes
    rows = [min(cfg.L + s, window - 1 if window else cfg.L + s) for s in range(cfg.S)]
    byts = float(np.mean([cfg.B * cfg.D * (r * sb + 5 * sb) for r in rows]))
    del graph, fir, yf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    gbs = byts / ms_step * 1e-6
    return {"window": window, "decode_us_per_step": ms_step * 1e3,
            "decode_tokens_per_s": cfg.B / (ms_step / 1e3),
            "algorithmic_bytes_per_step": byts, "hbm_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "modal_decode_speedup": ms_step / ms_modal_step}


# ------------------------------------------------------------------ main


def _json_default(o):
    if isinstance(o, np.generic):
        return o.item()
    if isinstance(o, np.ndarray):
        return o.tolist()
    raise TypeError(f"not JSON serialisable: {type(o).__name__}")


def emit(args, res):
    line = json.dumps(res, default=_json_default)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


def main():
    args = parse()
    if args.fingerprint:
        print(json.dumps(provenance()))
        return
    if args.traffic_from:
        return write_traffic(args)
    if args.summarize_trace:
        return write_trace_summary(args)
    if args.cpu_1thread is not None:
        return cpu_one_thread(args.cpu_1thread)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path would shard by batch rows and heads, with no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import get_config

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = get_config(args.config)
    if args.token_counters is not None:
        return token_counter_run(cfg, dev, args.token_counters)
    if args.prefill_counters:
        return prefill_counter_run(cfg, dev)
    subs = args.sub if args.sub is not None else ("3,4" if cfg.layers else "")
    subs = [int(s) for s in subs.split(",") if s.strip()]
    t_wall = time.perf_counter()
    head = run_stack(args, cfg, dev) if cfg.layers else run_operator(args, cfg, dev)
    res = {
        "metric": METRIC,
        "value": head.pop("tokens_per_s"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.pop("dtype"),
        "data": "synthetic",
        "config": head.pop("config"),
    }
    res["config"]["workload"] = head.pop("workload")
    res.update(head)
    res["provenance"] = provenance()
    if subs:
        res["sub_workloads"] = {}
        for ci in subs:
            sc = get_config(ci)
            r = run_operator(args, sc, dev)
            r["provenance"] = res["provenance"]
            r["steps"], r["warmup"] = args.steps, args.warmup
            res["sub_workloads"][sc.name] = r
    res["wall_s"] = time.perf_counter() - t_wall
    emit(args, res)


if __name__ == "__main__":
    main()
