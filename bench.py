#!/usr/bin/env python3
"""Benchmark of the modal-SSM Hyena hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  1. materialise the first L filter taps of every head,
  2. prefill over the L-token prompt -> y and the modal state: 64-step
     sub-blocks as per-head Toeplitz / readout / Vandermonde products on the
     matrix cores (the prompt split into chunks joined by a carry scan only when
     batch x heads are too few to fill the GPU), or the vector-ALU modal scan for
     shapes outside that path,
  3. S generation steps (one decode launch per token, captured once in a HIP
     graph and replayed), consuming the prefill state.
Inputs are resident in HBM before the timed region starts.

Printed: one JSON line (last line of stdout).  value = whole-step tokens/s,
B*(L+S) / step time; prefill and decode rates are reported beside it.
The roofline object covers the kernel that dominates the step, measured live
with HIP events on the stream the kernels run on; cpu_baseline times the float64
oracle on this host's cores over the same workload (rank 0, N = 1 only).
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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
VALU_F32_PEAK_TFLOPS = 78.6    # 256 CU x 64 lanes x 2 flop (FMA) x 2.4 GHz, unpacked float32

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "distilled_modal_ssm_amd", "csrc")
# Sources whose change invalidates a hardware-counter measurement of a kernel:
# the kernel's own file (its code and launch configuration), the shared
# device header and, where it adds flags for that file, the build script.
KERNEL_SOURCES = {
    "decode_step_fixed": ["decode.hip", "hm_internal.hpp", "../build.py"],
    "chunk_mfma_kernel": ["prefill_mfma.hip", "prefill.hip", "hm_internal.hpp"],
    "chunk_scan_kernel": ["prefill.hip", "hm_internal.hpp"],
}
COPY_BYTES = 1 << 30  # the calibration copy: 1 GiB read, 1 GiB written


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
    of this benchmark with --calibrate-copy into the per-launch traffic summary."""
    from workloads import get_config
    cfg = get_config(args.config)
    kernel = args.traffic_kernel
    fetch_dir, write_dir = args.traffic_from
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, name)
        k = np.array([float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]])
        copies = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        if len(k) == 0 or not copies:
            raise SystemExit(f"{name}: no dispatches of {kernel} or of the calibration copy in {d}")
        cal = max(copies)  # the 1 GiB copy is by far the largest copy dispatch
        factor = COPY_BYTES / (cal * 1024.0)
        out[name] = dict(n=len(k), mean=k.mean(), lo=k.min(), hi=k.max(), copy_kib=cal, factor=factor,
                         bytes=k.mean() * 1024.0 * factor)
    sb = cfg.act_bytes
    if kernel.startswith("decode"):
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
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        o = out[name]
        lines.append(f"# {name}: {o['n']} dispatches, mean {o['mean']:.1f} KiB (min {o['lo']:.1f}, max {o['hi']:.1f}); "
                     f"copy reads {o['copy_kib']:.1f} KiB -> factor {o['factor']:.4f} -> {o['bytes'] / 1e6:.3f} MB")
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=2, help="workload index (1-5; 5 = projected stack)")
    ap.add_argument("--decode-mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-1thread", type=int, default=None, metavar="CONFIG",
                    help=argparse.SUPPRESS)  # child process of the one-thread CPU baseline
    ap.add_argument("--no-fir", action="store_true", help="skip the explicit-filter decode baseline")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="no GPU: write the traffic summary of --traffic-kernel from two rocprofv3 --pmc runs")
    ap.add_argument("--traffic-kernel", default="decode_step_fixed")
    ap.add_argument("--traffic-cmd", default=None, help="the profiling commands, ' ;; '-separated, for the summary")
    return ap.parse_args()


def cpu_baseline(cfg, params, inp, dec, min_seconds: float = 10.0):
    """The float64 oracle (as it stands) on this host over the same workload:
    the full step (filter, prefill, decode steps) repeated until ``min_seconds``
    of CPU time have passed (at most 100 repetitions), on an evenly spaced
    channel subset when one repetition of the whole width would be too long."""
    import oracle
    budget = 6e9  # mode-steps per repetition, ~1 s on 16 cores
    per_channel = cfg.B * (cfg.L + cfg.S) * cfg.d
    n_sel = int(min(cfg.D, max(1, budget // per_channel)))
    chans = np.linspace(0, cfg.D - 1, n_sel).round().astype(np.int64) if n_sel < cfg.D else None
    reps = 0
    t0 = time.perf_counter()
    while reps < 100 and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.filter_taps(params, cfg.L)
        _, st = oracle.modal_scan(params, inp["q"], inp["k"], inp["v"], channels=chans)
        oracle.modal_scan(params, dec["q"], dec["k"], dec["v"], state=st, channels=chans,
                          batch_axis=1, time_axis=0)
        reps += 1
    dt = time.perf_counter() - t0
    tokens = cfg.B * (cfg.L + cfg.S) * (n_sel / cfg.D) * reps
    sample = (f"full step (filter, prefill L={cfg.L}, {cfg.S} decode steps) for "
              f"{'all' if n_sel == cfg.D else n_sel} of {cfg.D} channels x {cfg.B} rows, {reps} repetition(s), "
              f"{dt:.1f} s; tokens scaled by the channel fraction")
    return {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": sample}


def emit(args, res):
    line = json.dumps(res)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


def stack_cpu_baseline(cfg, layers, x0):
    """The float64 oracle on a bounded sample of the stack: one batch row through
    the first two layers, over the prompt and then all S generated steps whose
    inputs are that sample's own outputs fed back (as on the GPU)."""
    import oracle
    nl, steps, D = 2, cfg.S, cfg.D
    w64 = [(oracle.bf16_to_f64(w_in), oracle.bf16_to_f64(w_out)) for _, w_in, w_out in layers[:nl]]
    t0 = time.perf_counter()
    cur, states = x0[:1], []
    for l in range(nl):
        out, _, st, _ = oracle.stack_layer(layers[l][0], w64[l][0], w64[l][1], cur)
        states.append(st)
        cur = out
    xt = cur[:, -1, :]
    for _ in range(steps):
        for l in range(nl):
            qkv = oracle.dense(xt, w64[l][0]) * oracle.rms_inv(xt)[..., None]
            q, k, v = (np.ascontiguousarray(qkv[:, None, i * D:(i + 1) * D]) for i in range(3))
            y, states[l] = oracle.modal_scan(layers[l][0], q, k, v, state=states[l])
            xt = oracle.dense(y[:, 0, :], w64[l][1])
    dt = time.perf_counter() - t0
    tokens = (cfg.L + steps) * nl / cfg.layers  # one row, scaled by the layer fraction
    return {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"1 of {cfg.B} batch rows, layers 0-1 of {cfg.layers}, {cfg.L}-token prompt + {steps} "
                      f"generated steps, {dt:.1f} s; tokens scaled by the layer fraction"}


def stack_token_bytes(cfg) -> int:
    """HBM bytes a generated token of the projected stack must move: per layer the
    bf16 weights (W_in 3D x D, W_out D x D), the modal state read and written
    (16 d bytes per row and channel), and the bf16 activations: the layer input
    read, the operator output written and read back by out_proj, the layer
    output written (q, k, v stay on chip in the fused step)."""
    D, B = cfg.D, cfg.B
    return cfg.layers * (4 * D * D * 2 + B * D * 16 * cfg.d + 4 * B * D * 2)


def bench_stack(args, cfg, dev):
    """Projected stack: prefill through all layers, then S generated tokens per
    batch row (one HIP graph per generated token, replayed)."""
    import torch
    from distilled_modal_ssm_amd.stack import HyenaStack
    from workloads import dense_weights, modal_params, stack_prompt
    layers = [(modal_params(cfg, l), *dense_weights(cfg, l)) for l in range(cfg.layers)]
    st = HyenaStack(layers, cfg.B, cfg.L, device=dev)
    x0 = stack_prompt(cfg)
    X = torch.from_numpy(x0.view(np.int16)).view(torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream()

    # capture one generated token (all layers) once
    out = st.prefill(X)
    st.start_generation(out)
    st.decode_step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.decode_step()
    torch.cuda.synchronize()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        o = st.prefill(X)
        st.start_generation(o)
        if ev:
            ev[1].record(stream)
        for _ in range(cfg.S):
            graph.replay()
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
    M = cfg.B * cfg.L
    D = cfg.D
    gemm_flops = cfg.layers * 2 * M * D * 4 * D          # in_proj (3D) + out_proj (D)
    hyena_flops = cfg.layers * (12 * cfg.d + 5) * M * D
    decode_bytes = stack_token_bytes(cfg)
    prefill_tf = (gemm_flops + hyena_flops) / ms_prefill * 1e-9
    decode_gbs = decode_bytes / ms_tok * 1e-6
    if ms_prefill >= ms_decode:
        roof = {"bound": "mfma", "achieved": round(gemm_flops / ms_prefill * 1e-9, 2), "peak": 2500.0,
                "unit": "TFLOP/s", "kernel": "prefill (gemm_tiled dominant)", "launch_ms": round(ms_prefill, 4)}
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    else:
        roof = {"bound": "hbm", "achieved": round(decode_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "kernel": "generated token (weights + state stream)", "launch_ms": round(ms_tok, 5)}
        roof["frac"] = round(decode_gbs / HBM_PEAK_GBS, 4)
    roof["traffic"] = None
    res = {
        "metric": "decode tokens/sec and prefill tokens/sec at 1 GPU; % of HBM roofline",
        "value": cfg.B * (cfg.L + cfg.S) / (ms_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.describe()}", "B": cfg.B, "D": cfg.D, "H": cfg.H, "d": cfg.d,
                   "L": cfg.L, "S": cfg.S, "layers": cfg.layers, "act_dtype": cfg.act,
                   "decode_mode": "graph per generated token"},
        "prefill_tokens_per_s": M / (ms_prefill / 1e3),
        "decode_tokens_per_s": cfg.B / (ms_tok / 1e3),
        "phase_ms": {"prefill": ms_prefill, "decode_total": ms_decode, "decode_per_token": ms_tok},
        "prefill_rates": {"TFLOPs": prefill_tf, "mfma_frac_of_gemm_flops": gemm_flops / ms_prefill * 1e-9 / 2500.0},
        "decode_rates": {"hbm_GBs": decode_gbs, "hbm_frac": decode_gbs / HBM_PEAK_GBS},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (float64 oracle, sampled)")
        res["cpu_baseline"] = stack_cpu_baseline(cfg, layers, x0)
    emit(args, res)


def cpu_one_thread(ci: int, min_seconds: float = 5.0):
    """Child process of the CPU baseline (started with OMP_NUM_THREADS=1, no
    GPU use): the oracle's full step on an evenly spaced channel subset,
    repeated for ``min_seconds``; prints one JSON line."""
    import oracle
    from workloads import decode_inputs, get_config, modal_params, prompt_inputs
    cfg = get_config(ci)
    params = modal_params(cfg)
    inp, dec = prompt_inputs(cfg), decode_inputs(cfg)
    per_channel = cfg.B * (cfg.L + cfg.S) * cfg.d
    n_sel = int(min(cfg.D, max(1, 2e8 // per_channel)))
    chans = np.linspace(0, cfg.D - 1, n_sel).round().astype(np.int64) if n_sel < cfg.D else None
    reps, t0 = 0, time.perf_counter()
    while reps < 100 and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.filter_taps(params, cfg.L)
        _, st = oracle.modal_scan(params, inp["q"], inp["k"], inp["v"], channels=chans)
        oracle.modal_scan(params, dec["q"], dec["k"], dec["v"], state=st, channels=chans,
                          batch_axis=1, time_axis=0)
        reps += 1
    dt = time.perf_counter() - t0
    print(json.dumps({"value": cfg.B * (cfg.L + cfg.S) * (n_sel / cfg.D) * reps / dt, "unit": "tokens/s",
                      "cores": oracle.threads(),
                      "sample": f"full step for {n_sel} of {cfg.D} channels x {cfg.B} rows, {reps} repetition(s), "
                                f"{dt:.1f} s; tokens scaled by the channel fraction"}))


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


def main():
    args = parse()
    if args.traffic_from:
        return write_traffic(args)
    if args.cpu_1thread is not None:
        return cpu_one_thread(args.cpu_1thread)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path would shard by batch rows and heads, with no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from distilled_modal_ssm_amd import ModalHyena
    from workloads import decode_inputs, get_config, modal_params, prompt_inputs

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {cfg.index} {cfg.describe()}")
    if cfg.layers:
        return bench_stack(args, cfg, dev)

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

    from distilled_modal_ssm_amd import binding as hb

    def filter_call():
        hb.hyena_filter_materialize(op.desc, cfg.L, h)

    def prefill_call():
        op.prefill(q, k, v, y=y, state_out=state)

    def decode_eager():
        for s in range(cfg.S):
            op.decode_step(dq[s], dk[s], dv[s], state, y=ys[s])

    stream = torch.cuda.current_stream()
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
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    ph = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in evs])
    ms_filter, ms_prefill, ms_decode = (float(np.median(ph[:, i])) for i in range(3))
    ms_decode_launch = ms_decode / cfg.S

    # outside the timed region: 20 prefill calls alone, and 10 replays of the
    # S-step decode graph (per-launch spread of the decode kernel: see the
    # rocprofv3 kernel-trace summaries, which time every dispatch)
    torch.cuda.synchronize()
    pf_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(20)]
    for e in pf_ev:
        e[0].record(stream)
        prefill_call()
        e[1].record(stream)
    dg_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
    for e in dg_ev:
        e[0].record(stream)
        decode_call()
        e[1].record(stream)
    torch.cuda.synchronize()
    pf_ms = np.array([a.elapsed_time(b) for a, b in pf_ev])
    dec_us = np.array([a.elapsed_time(b) * 1e3 / cfg.S for a, b in dg_ev])
    pct = lambda x: {"p10": float(np.percentile(x, 10)), "p50": float(np.median(x)), "p90": float(np.percentile(x, 90))}

    E = cfg.B * cfg.L * cfg.D
    sb = cfg.act_bytes
    decode_bytes = cfg.B * cfg.D * (16 * cfg.d + 4 * sb)
    prefill_flops = (12 * cfg.d + 5) * E
    prefill_bytes = 4 * sb * E + 8 * cfg.B * cfg.D * cfg.d
    plan = op.plan(cfg.L)
    if plan["algo"] == "mfma":
        # matrix-core sub-blocks: the products are a few % of the bf16 MFMA peak;
        # the pass streams q, k, v, y once, so HBM bounds it
        prefill_roof = dict(bound="hbm", unit="GB/s", per_launch=prefill_bytes, peak=HBM_PEAK_GBS)
    else:
        # vector scan: one complex FMA pair per mode and step, on the vector ALUs
        prefill_roof = dict(bound="alu", unit="TFLOP/s", per_launch=prefill_flops, peak=VALU_F32_PEAK_TFLOPS)
    kernels = {
        "decode_step": dict(bound="hbm", unit="GB/s", per_launch=decode_bytes, ms=ms_decode_launch,
                            total_ms=ms_decode, peak=HBM_PEAK_GBS),
        "prefill": dict(ms=ms_prefill, total_ms=ms_prefill, **prefill_roof),
    }
    dom_name = max(kernels, key=lambda n: kernels[n]["total_ms"])
    dom = kernels[dom_name]
    scale = 1e-6 if dom["unit"] == "GB/s" else 1e-9  # bytes/ms -> GB/s ; flops/ms -> TFLOP/s
    achieved = dom["per_launch"] / dom["ms"] * scale
    kname = "decode_step_fixed" if dom_name == "decode_step" else (
        "chunk_mfma_kernel" if plan["algo"] == "mfma" else "chunk_scan_kernel")
    roofline = {"bound": dom["bound"], "achieved": round(achieved, 3), "peak": dom["peak"],
                "unit": dom["unit"], "frac": round(achieved / dom["peak"], 4),
                "traffic": read_traffic(kname, cfg.name),
                "kernel": kname, "launch_ms": round(dom["ms"], 6),
                "algorithmic_bytes_per_launch": decode_bytes if dom_name == "decode_step" else prefill_bytes}

    tokens = cfg.B * (cfg.L + cfg.S)
    res = {
        "metric": "decode tokens/sec and prefill tokens/sec at 1 GPU; % of HBM roofline",
        "value": tokens / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.describe()}", "B": cfg.B, "D": cfg.D, "H": cfg.H,
                   "d": cfg.d, "L": cfg.L, "S": cfg.S, "act_dtype": cfg.act,
                   "decode_mode": args.decode_mode},
        "prefill_plan": plan,
        "prefill_tokens_per_s": cfg.B * cfg.L / (ms_prefill / 1e3),
        "decode_tokens_per_s": cfg.B / (ms_decode_launch / 1e3),
        "phase_ms": {"filter": ms_filter, "prefill": ms_prefill, "decode_total": ms_decode,
                     "decode_per_step": ms_decode_launch},
        "decode_step_us_per_replay": pct(dec_us),
        "prefill_ms_20_calls": pct(pf_ms),
        "prefill_rates": {"alu_TFLOPs": prefill_flops / ms_prefill * 1e-9,
                          "alu_frac": prefill_flops / ms_prefill * 1e-9 / VALU_F32_PEAK_TFLOPS,
                          "hbm_GBs": prefill_bytes / ms_prefill * 1e-6,
                          "hbm_frac": prefill_bytes / ms_prefill * 1e-6 / HBM_PEAK_GBS},
        "decode_rates": {"hbm_GBs": decode_bytes / ms_decode_launch * 1e-6,
                         "hbm_frac": decode_bytes / ms_decode_launch * 1e-6 / HBM_PEAK_GBS},
        "wall_s_timed": t_wall,
        "roofline": roofline,
    }
    if not args.no_fir:
        res["distill"] = distill_bench(cfg, params, stream)
        res["fft_prefill"] = fft_prefill_baseline(cfg, op, q, k, v, ms_prefill, stream)
        for window in (0, 256):
            res[f"fir_baseline_w{window}"] = fir_baseline(cfg, op, k, v, dq, dk, dv, window,
                                                          ms_decode_launch, stream)
    if args.calibrate_copy:
        calibration_copy()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (float64 oracle)")
        res["cpu_baseline"] = cpu_baseline(cfg, params, inp, dec)
        res["cpu_baseline"]["one_thread"] = cpu_baseline_one_thread(cfg)
    emit(args, res)


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
    return {"heads": cfg.H, "modes": cfg.d, "taps": cfg.L, "target_modes": 2 * cfg.d, "iterations": steps,
            "us_per_iteration": us, "loss_first": float(h[0]), "loss_last": float(h[-1])}


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
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5 if multipass else 20)]
    for e in ev:
        e[0].record(stream)
        call()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / cfg.S
    sb = cfg.act_bytes
    rows = [min(cfg.L + s, window - 1 if window else cfg.L + s) for s in range(cfg.S)]
    byts = float(np.mean([cfg.B * cfg.D * (r * sb + 5 * sb) for r in rows]))
    del graph, fir, yf
    torch.cuda.synchronize()
    gbs = byts / ms_step * 1e-6
    return {"window": window, "decode_us_per_step": ms_step * 1e3,
            "decode_tokens_per_s": cfg.B / (ms_step / 1e3),
            "algorithmic_bytes_per_step": byts, "hbm_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "modal_decode_speedup": ms_step / ms_modal_step}


if __name__ == "__main__":
    main()
