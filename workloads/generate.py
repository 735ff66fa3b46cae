"""Seeded generators for the synthetic workloads.

Recipe (every draw is float64 from numpy's PCG64, then rounded once to the
storage type with round-to-nearest-even):

* Modal parameters of layer ``l``: one stream keyed ``[seed, 0, l]`` drawing, in
  this order, pole radii r[H][d] ~ U(r_lo, r_hi), pole angles th[H][d] ~ U(0, pi),
  Re R[H][d] and Im R[H][d] ~ N(0, 1/(2d)) (so R is circular complex normal
  with E|R|^2 = 1/d), and the per-head skip D_h[H] ~ N(0, 1).  The pole is
  r*(cos th + i sin th) in float64; its two components, R and D_h are then
  rounded to float32.
* Prompt activations q, k, v ([B][L][D]): tensor ids 1, 2, 3.  Row block ``i``
  (time steps 256*i ... 256*i+255) of batch row ``b`` comes from the stream
  keyed ``[seed, id, b, i]`` as N(0, 1) in row-major (time, channel) order.
* Generated-step activations q, k, v ([S][B][D]): tensor ids 4, 5, 6; step ``s``
  comes from the stream keyed ``[seed, id, s]``.
* Projected stack: layer-0 prompt input X ([B][L][D], id 7, blocked like the
  prompt), W_in[l] ([3D][D], id 8) and W_out[l] ([D][D], id 9) from streams
  keyed ``[seed, id, l]``, N(0, w_std^2).

``seed`` is 1000 + the workload index.  Blocks are independent streams so that
large tensors can be drawn in parallel and a subset of rows can be drawn alone.
Activations come back as float32 arrays, or, for bf16 workloads, as uint16
arrays holding bfloat16 bit patterns.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .configs import Config

BLOCK_ROWS = 256

_ID_PARAMS = 0
_ID_PROMPT = {"q": 1, "k": 2, "v": 3}
_ID_DECODE = {"q": 4, "k": 5, "v": 6}
_ID_STACK_X = 7
_ID_W_IN = 8
_ID_W_OUT = 9


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- rounding


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even); return bit patterns.

    bfloat16 keeps 8 significant bits and the float32 exponent range.  The
    significand m of x = m * 2**e (0.5 <= |m| < 1) is scaled by 2**8 and rounded
    to an integer with numpy's half-to-even rounding, which is exact in float64.
    Values must lie in the normal float32 range (or be zero).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.round(m * 256.0), e - 8)
    a = np.abs(r)
    if not np.all(np.isfinite(r)) or np.any((a != 0) & ((a < 2.0 ** -126) | (a > 3.3e38))):
        raise ValueError("value outside the normal bfloat16 range")
    f = r.astype(np.float32)  # exact: r has 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _to_act(x64: np.ndarray, act: str) -> np.ndarray:
    if act == "bf16":
        return round_to_bf16_bits(x64)
    if act == "f32":
        return x64.astype(np.float32)
    raise ValueError(f"unknown activation dtype {act!r}")


def act_numpy_dtype(act: str):
    return np.uint16 if act == "bf16" else np.float32


# ---------------------------------------------------------------- modal params


@dataclass
class ModalParams:
    """Per-head tables, float32.

    poles, residues: [H][d][2] (real, imaginary); skip: [H].
    """

    poles: np.ndarray
    residues: np.ndarray
    skip: np.ndarray

    @property
    def H(self) -> int:
        return self.poles.shape[0]

    @property
    def d(self) -> int:
        return self.poles.shape[1]

    def f64(self):
        return (self.poles.astype(np.float64), self.residues.astype(np.float64),
                self.skip.astype(np.float64))


def modal_params(cfg: Config, layer: int = 0) -> ModalParams:
    H, d = cfg.H, cfg.d
    g = _rng(cfg.seed, _ID_PARAMS, layer)
    r = g.uniform(cfg.r_lo, cfg.r_hi, size=(H, d))
    th = g.uniform(0.0, np.pi, size=(H, d))
    sd = np.sqrt(1.0 / (2.0 * d))
    re_r = g.normal(0.0, sd, size=(H, d))
    im_r = g.normal(0.0, sd, size=(H, d))
    skip = g.normal(0.0, 1.0, size=(H,))
    poles = np.stack([r * np.cos(th), r * np.sin(th)], axis=-1).astype(np.float32)
    residues = np.stack([re_r, im_r], axis=-1).astype(np.float32)
    mag = np.hypot(poles[..., 0].astype(np.float64), poles[..., 1].astype(np.float64))
    if not np.all(mag < 1.0):
        raise AssertionError("a rounded pole left the unit disc")
    return ModalParams(poles=poles, residues=residues, skip=skip.astype(np.float32))


# ---------------------------------------------------------------- activations


def _fill_blocked(out: np.ndarray, seed: int, tid: int, batches, act: str, std: float = 1.0):
    """Fill out[bi] ([T][D]) for bi, b in enumerate(batches) block by block."""
    T, D = out.shape[1], out.shape[2]
    nblk = (T + BLOCK_ROWS - 1) // BLOCK_ROWS

    def job(args):
        bi, b, i = args
        t0 = i * BLOCK_ROWS
        t1 = min(T, t0 + BLOCK_ROWS)
        x = _rng(seed, tid, b, i).standard_normal((t1 - t0, D))
        if std != 1.0:
            x *= std
        out[bi, t0:t1, :] = _to_act(x, act)

    jobs = [(bi, b, i) for bi, b in enumerate(batches) for i in range(nblk)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, jobs))


def prompt_inputs(cfg: Config, names=("q", "k", "v"), batches=None) -> dict:
    """Prompt activations [len(batches)][L][D] for each requested tensor."""
    batches = list(range(cfg.B)) if batches is None else list(batches)
    res = {}
    for nm in names:
        out = np.empty((len(batches), cfg.L, cfg.D), dtype=act_numpy_dtype(cfg.act))
        _fill_blocked(out, cfg.seed, _ID_PROMPT[nm], batches, cfg.act)
        res[nm] = out
    return res


def decode_inputs(cfg: Config, names=("q", "k", "v"), steps=None) -> dict:
    """Generated-step activations [len(steps)][B][D] for each requested tensor."""
    steps = list(range(cfg.S)) if steps is None else list(steps)
    res = {}
    for nm in names:
        out = np.empty((len(steps), cfg.B, cfg.D), dtype=act_numpy_dtype(cfg.act))

        def job(args, out=out, nm=nm):
            si, s = args
            x = _rng(cfg.seed, _ID_DECODE[nm], s).standard_normal((cfg.B, cfg.D))
            out[si] = _to_act(x, cfg.act)

        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(job, list(enumerate(steps))))
        res[nm] = out
    return res


def stack_prompt(cfg: Config, batches=None) -> np.ndarray:
    """Layer-0 prompt input X [len(batches)][L][D] of the projected stack (bf16 bits)."""
    batches = list(range(cfg.B)) if batches is None else list(batches)
    out = np.empty((len(batches), cfg.L, cfg.D), dtype=act_numpy_dtype(cfg.act))
    _fill_blocked(out, cfg.seed, _ID_STACK_X, batches, cfg.act)
    return out


def dense_weights(cfg: Config, layer: int):
    """(W_in [3D][D], W_out [D][D]) of one layer as bfloat16 bit patterns."""
    D = cfg.D
    w_in = _rng(cfg.seed, _ID_W_IN, layer).normal(0.0, cfg.w_std, size=(3 * D, D))
    w_out = _rng(cfg.seed, _ID_W_OUT, layer).normal(0.0, cfg.w_std, size=(D, D))
    return round_to_bf16_bits(w_in), round_to_bf16_bits(w_out)
