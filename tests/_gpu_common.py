"""Helpers shared by the GPU tests: moving seeded inputs to the device, state
layout mapping and error measures.  No arithmetic of the operator lives here."""

from __future__ import annotations

import json
import os
import sys

import numpy as np

from workloads import bf16_bits_to_f32


def log(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu():
    import pytest
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    return torch


def to_dev(arr: np.ndarray, act: str, device="cuda"):
    """numpy float32 (act f32) or bfloat16 bit patterns (act bf16) -> device tensor."""
    import torch
    if act == "bf16":
        assert arr.dtype == np.uint16
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        assert arr.dtype == np.float32
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def to_np64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def act_to_f64(arr: np.ndarray) -> np.ndarray:
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return arr.astype(np.float64)


def state_for_channels(state_t, channels, P: int) -> np.ndarray:
    """GPU state [B][H][d][P][2] -> oracle layout [B][len(channels)][d][2]."""
    st = state_t.detach().cpu().numpy().astype(np.float64)
    ch = np.asarray(channels)
    return np.ascontiguousarray(st[:, ch // P, :, ch % P, :].transpose(1, 0, 2, 3))


def state_to_gpu_layout(st_oracle: np.ndarray, H: int, P: int) -> np.ndarray:
    """Oracle state for ALL channels [B][D][d][2] -> GPU layout [B][H][d][P][2] float32."""
    B, D, d, _ = st_oracle.shape
    return np.ascontiguousarray(st_oracle.reshape(B, H, P, d, 2).transpose(0, 1, 3, 2, 4)).astype(np.float32)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref)))
    if scale == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref))) / scale


TOL = {"f32": 1e-4, "bf16": 2e-2}


# Parity margins of the full-size cases: every recorded (case, phase) error is
# printed in pytest's terminal summary (so a -q run shows it) and appended to
# gpurun_out/parity_margins.jsonl when that folder can be written.
MARGINS: list = []


def record_margin(case: str, phase: str, err: float, tol: float) -> None:
    row = {"case": case, "phase": phase, "max_err_over_max_ref": float(err), "tol": tol,
           "margin": (tol / err) if err > 0 else None}
    MARGINS.append(row)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = os.path.join(root, "gpurun_out")
    try:
        os.makedirs(out, exist_ok=True)
        with open(os.path.join(out, "parity_margins.jsonl"), "a") as f:
            f.write(json.dumps(row) + "\n")
    except OSError:
        pass
