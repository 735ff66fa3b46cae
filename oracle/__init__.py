"""Float64 CPU oracle of the modal-SSM Hyena operator (test infrastructure).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product library never does, and
this package imports nothing from it.

Contents
--------
build()                 compile ``modal_oracle.c`` with gcc (OpenMP, no fast-math,
                        no FP contraction) into ``liboracle.so``.
filter_taps()           h[g][t], t < L, from the closed form of the modal filter.
modal_scan()            the recurrence (prefill with a zero state, or decode steps
                        from a given state), float64.
rms_inv(), dense()      the projected stack's per-token inverse RMS and a float64
                        matrix product (numpy's matmul as the library primitive).
stack_layer()           one layer of the projected stack, teacher-forced on a given
                        input sequence (see ``stack_layer``'s docstring).
distill_loss_grad()     the filter discrepancy of a modal filter against target
                        taps and its analytic gradient (the distillation objective);
                        hankel_singular_values() of a filter; modal_fit_init(), the
                        matrix-pencil / least-squares initial fit.
fir_conv()              the same operator with an explicit (possibly truncated)
                        filter over a cache of u rounded to the activation dtype:
                        the non-distilled decode baseline.

The operator, its readings and its pins are described at the top of
``modal_oracle.c``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "modal_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DT_F32, DT_BF16, DT_F64 = 0, 1, 2
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc.  Returns the library path."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_filter.argtypes = [i64, i64, p, p, p, i64, p]
    lib.oracle_filter.restype = ctypes.c_int
    lib.oracle_modal_scan.argtypes = [i64, i64, i64, i64, p, p, p, i64, ctypes.c_int,
                                      p, p, p, i64, i64, i64, p, p, p]
    lib.oracle_modal_scan.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            _lib = _bind(_LIB_PATH)
    return _lib


def threads() -> int:
    """OpenMP threads the oracle uses on this host."""
    return int(_load().oracle_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _tables(params):
    poles = np.ascontiguousarray(params.poles, dtype=np.float64)
    res = np.ascontiguousarray(params.residues, dtype=np.float64)
    skip = np.ascontiguousarray(params.skip, dtype=np.float64)
    return poles, res, skip


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float64:
        return DT_F64
    raise TypeError(f"unsupported activation dtype {a.dtype}")


def filter_taps(params, L: int, _lib_handle=None) -> np.ndarray:
    """h [H][L] float64: h[g,0] = D_g, h[g,t] = Re sum_n R_gn lambda_gn^(t-1)."""
    lib = _lib_handle or _load()
    poles, res, skip = _tables(params)
    H, d = poles.shape[0], poles.shape[1]
    h = np.empty((H, L), dtype=np.float64)
    rc = lib.oracle_filter(H, d, _ptr(poles), _ptr(res), _ptr(skip), L, _ptr(h))
    if rc:
        raise ValueError("oracle_filter rejected its arguments")
    return h


def modal_scan(params, q, k, v, state=None, channels=None, batch_axis=0, time_axis=1,
               _lib_handle=None):
    """Run the recurrence over every time step of q, k, v.

    q, k, v: 3-D arrays (float32, bfloat16 bit patterns as uint16, or float64) of
    identical shape and dtype, C-contiguous, with the channel axis last.  The
    batch and time axes are given by ``batch_axis``/``time_axis`` (0/1 for
    [B][T][D] prompts, 1/0 for [S][B][D] generated steps).
    state: [B][n_sel][d][2] float64 initial state (None: zero).
    channels: optional channel indices to compute (default: all).
    Returns (y [B][T][n_sel] float64, final state [B][n_sel][d][2] float64).
    """
    lib = _lib_handle or _load()
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    if not (q.shape == k.shape == v.shape) or q.ndim != 3:
        raise ValueError("q, k, v must share one 3-D shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    poles, res, skip = _tables(params)
    H, d = poles.shape[0], poles.shape[1]
    D = q.shape[2]
    B, T = q.shape[batch_axis], q.shape[time_axis]
    strides = [q.strides[i] // q.itemsize for i in range(3)]
    sb, st = strides[batch_axis], strides[time_axis]
    if channels is None:
        n_sel, sel_ptr, sel = D, None, None
    else:
        sel = np.ascontiguousarray(channels, dtype=np.int64)
        if sel.size and (sel.min() < 0 or sel.max() >= D):
            raise ValueError("channel index out of range")
        n_sel, sel_ptr = sel.size, _ptr(sel)
    y = np.empty((B, T, n_sel), dtype=np.float64)
    if state is None:
        state = np.zeros((B, n_sel, d, 2), dtype=np.float64)
    else:
        state = np.array(state, dtype=np.float64, order="C", copy=True)
        if state.shape != (B, n_sel, d, 2):
            raise ValueError(f"state shape {state.shape} != {(B, n_sel, d, 2)}")
    rc = lib.oracle_modal_scan(B, D, H, d, _ptr(poles), _ptr(res), _ptr(skip), T,
                               _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), sb, st,
                               n_sel, sel_ptr, _ptr(y), _ptr(state))
    if rc:
        raise ValueError("oracle_modal_scan rejected its arguments")
    return y, state


# ------------------------------------------------------------ explicit-filter (FIR) Hyena


def round_to_act(x, act: str) -> np.ndarray:
    """Round float64 values once to the activation dtype (IEEE round to nearest
    even) and return them widened back to float64.  act: "f64" (no rounding),
    "f32", or "bf16" (the top 16 bits of the float32 pattern, rounded on the
    lower 16 with ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    if act == "f64":
        return x.copy()
    f = x.astype(np.float32)  # round to nearest even, once
    if act == "f32":
        return f.astype(np.float64)
    if act != "bf16":
        raise ValueError(act)
    if not np.array_equal(f.astype(np.float64), x):
        raise ValueError("bf16 rounding expects float32-exact inputs (products of bf16 values are)")
    bits = f.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def _widen(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


def fir_conv(h, q, k, v, act: str, window: int = 0, t_from: int = 0, heads=None) -> np.ndarray:
    """The non-distilled Hyena operator evaluated as an explicit finite filter.

    y[b,t,c] = q[b,t,c] * sum_{j=0}^{min(t, W-1)} h[g(c), j] * u[b, t-j, c],   t >= t_from,
    with u = k v rounded once to the activation dtype ``act`` (an FIR cache keeps
    past u in that dtype) and W = ``window`` (<= 0: every past step).
    h: [H][>= T] float64 taps; q, k, v: [B][T][C] float32, bfloat16 bit patterns
    (uint16) or float64; heads: the head of each of the C channels (default
    c // (C / H)).  Returns y [B][T - t_from][C] float64.
    """
    h = np.asarray(h, dtype=np.float64)
    q64, k64, v64 = _widen(q), _widen(k), _widen(v)
    B, T, C = q64.shape
    if heads is None:
        heads = np.arange(C) // (C // h.shape[0])
    W = T if window <= 0 else min(int(window), T)
    if h.shape[1] < W:
        raise ValueError("filter shorter than the window")
    u = round_to_act(k64 * v64, act)
    taps = h[np.asarray(heads)]  # [C][Lh]
    y = np.zeros((B, T - t_from, C))
    for j in range(W):
        t0 = max(j, t_from)
        if t0 >= T:
            continue
        y[:, t0 - t_from:, :] += taps[:, j][None, None, :] * u[:, t0 - j:T - j, :]
    return y * q64[:, t_from:, :]


# ------------------------------------------------------------ distillation objective


def distill_loss_grad(params, h_target, L: int):
    """Filter discrepancy of a modal filter against target taps and its
    gradient, float64 (the objective modal distillation minimises):

        J_g = sum_{t<L} (hhat_g[t] - h_g[t])^2,
        hhat_g[0] = D_g,  hhat_g[t] = Re sum_n R_gn lambda_gn^(t-1).

    With e = hhat - h and p_t = lambda^(t-1):
        dJ/dD       = 2 e[0]
        dJ/dRe R_n  = 2 sum_{t>=1} e[t] Re p_t,   dJ/dIm R_n = -2 sum e[t] Im p_t
        dJ/dRe l_n  = 2 sum_{t>=2} e[t] Re(R_n (t-1) l_n^(t-2)),
        dJ/dIm l_n  = -2 sum_{t>=2} e[t] Im(R_n (t-1) l_n^(t-2))
    (hhat is the real part of a holomorphic function of lambda).
    Returns (loss [H], g_poles [H][d][2], g_res [H][d][2], g_skip [H])."""
    h_target = np.asarray(h_target, dtype=np.float64)
    lam = params.poles[..., 0].astype(np.float64) + 1j * params.poles[..., 1].astype(np.float64)
    R = params.residues[..., 0].astype(np.float64) + 1j * params.residues[..., 1].astype(np.float64)
    H, d = lam.shape
    hhat = filter_taps(params, L)
    e = hhat - h_target[:, :L]
    loss = np.sum(e * e, axis=1)
    t = np.arange(1, L)
    pw = lam[:, :, None] ** (t - 1)[None, None, :]                 # lambda^(t-1), t >= 1
    et = e[:, None, 1:]
    g_res = np.stack([2 * np.sum(et * pw.real, -1), -2 * np.sum(et * pw.imag, -1)], -1)
    dl = np.zeros_like(pw)
    if L > 2:
        dl[:, :, 1:] = R[:, :, None] * (t[1:] - 1)[None, None, :] * lam[:, :, None] ** (t[1:] - 2)[None, None, :]
    g_poles = np.stack([2 * np.sum(et * dl.real, -1), -2 * np.sum(et * dl.imag, -1)], -1)
    g_skip = 2 * e[:, 0]
    return loss, g_poles, g_res, g_skip


def modal_fit_init(h, d: int, r_max: float = 0.9999):
    """Initial modal fit of each filter h [H][L] (float64): poles by the matrix
    pencil method of Hua and Sarkar (IEEE Trans. ASSP, 1990), residues by
    linear least squares, skip = h[0] -- the Prony-type reduction the
    distillation review describes (提出的方法: modal truncation with a
    Prony-like parametrisation).

    For each head, with x_k = h[1 + k] (k < N = L - 1) and M = 2d real
    exponentials (d complex modes and their conjugates):
      1. window length n = min(2M + 8, N // 2), rows = min(N - n + 1, 2n);
         Hankel data matrix Y[i][j] = x[i + j] (rows x n);
      2. V = the top-M right singular vectors of Y (n x M);
      3. Psi = least-squares solution of V[:-1] Psi = V[1:]; its eigenvalues
         are the poles (the shifted windows span the same space);
      4. modes: poles with Im > 0 (one of each conjugate pair) and real poles,
         each scaled back to radius r_max if outside it;
      5. residues R minimising sum_{t >= 1} (Re sum_n R_n lambda_n^(t-1) - h[t])^2
         over all taps (columns Re lambda^(t-1) and -Im lambda^(t-1));
      6. more than d modes: keep the d with the largest |R|^2 / (1 - |lambda|^2)
         and solve step 5 again; fewer: pad with zero-residue poles at 0.
    Returns (poles [H][d][2], residues [H][d][2], skip [H]) float64."""
    h = np.atleast_2d(np.asarray(h, dtype=np.float64))
    H, L = h.shape
    N, M = L - 1, 2 * d
    n = min(2 * M + 8, N // 2)
    rows = min(N - n + 1, 2 * n)
    t = np.arange(L - 1)

    def residues_for(lam, taps):
        pw = lam[None, :] ** t[:, None]                       # lambda^(t-1), t = 1 .. L-1
        cols = np.concatenate([pw.real, -pw.imag], axis=1)
        keep = np.any(cols != 0.0, axis=0)                    # a real pole has no imaginary column
        sol = np.zeros(2 * lam.size)
        sol[keep] = np.linalg.lstsq(cols[:, keep], taps, rcond=None)[0]
        return sol[:lam.size] + 1j * sol[lam.size:]

    poles = np.zeros((H, d, 2))
    res = np.zeros((H, d, 2))
    for g in range(H):
        x = h[g, 1:]
        Y = x[np.arange(rows)[:, None] + np.arange(n)[None, :]]
        V = np.linalg.svd(Y)[2][:M].T
        Psi = np.linalg.lstsq(V[:-1], V[1:], rcond=None)[0]
        z = np.linalg.eigvals(Psi)
        tol = 1e-9 * np.maximum(1.0, np.abs(z))
        lam = np.concatenate([z[z.imag > tol], z[np.abs(z.imag) <= tol].real + 0j])
        big = np.abs(lam) > r_max
        lam[big] *= r_max / np.abs(lam[big])
        R = residues_for(lam, x)
        if lam.size > d:
            energy = np.abs(R) ** 2 / np.maximum(1e-12, 1.0 - np.abs(lam) ** 2)
            lam = lam[np.argsort(-energy)[:d]]
            R = residues_for(lam, x)
        k = lam.size
        poles[g, :k] = np.stack([lam.real, lam.imag], -1)
        res[g, :k] = np.stack([R.real, R.imag], -1)
    return poles, res, h[:, 0].copy()


def hankel_singular_values(h_row, n: int) -> np.ndarray:
    """Singular values of the n x n Hankel matrix [h[i + j + 1]] of one filter
    (taps from t = 1; the skip term h[0] is not part of the SSM's Hankel)."""
    h_row = np.asarray(h_row, dtype=np.float64)
    idx = np.arange(n)[:, None] + np.arange(n)[None, :] + 1
    return np.linalg.svd(h_row[idx], compute_uv=False)


# ------------------------------------------------------------ projected stack


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rms_inv(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """1 / sqrt(mean(x^2) + eps) over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)


def dense(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x @ w^T in float64 (w stored [out][in])."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def stack_layer(params, w_in, w_out, x_prompt, x_steps=None, eps: float = 1e-6, _scan=None):
    """One layer of the projected stack in float64, teacher-forced.

    Layer input x (per token, width D) -> s = 1/rms(x) -> [q|k|v] = (x W_in^T) s
    (contiguous thirds) -> y = q * (h conv (k v)) through the modal recurrence ->
    layer output y W_out^T.  No bias, no residual.

    x_prompt: [B][L][D] layer input over the prompt; x_steps: optional
    [S][B][D] layer inputs of the generated steps (each one the actual input the
    layer received at that step).  Returns (out_prompt [B][L][D],
    out_steps [S][B][D] or None, state after the prompt, final state).
    The generated steps continue the recurrence from the state the prompt left
    (the decode step of the operator), so over prompt + steps the layer is the
    same causal convolution as over one sequence of L + S tokens.
    """
    scan = _scan or modal_scan
    D = x_prompt.shape[-1]
    w_in = bf16_to_f64(w_in) if w_in.dtype == np.uint16 else np.asarray(w_in, np.float64)
    w_out = bf16_to_f64(w_out) if w_out.dtype == np.uint16 else np.asarray(w_out, np.float64)

    def project(x):
        x = bf16_to_f64(x) if x.dtype == np.uint16 else np.asarray(x, np.float64)
        qkv = dense(x, w_in) * rms_inv(x, eps)[..., None]
        return (np.ascontiguousarray(qkv[..., :D]), np.ascontiguousarray(qkv[..., D:2 * D]),
                np.ascontiguousarray(qkv[..., 2 * D:]))

    q, k, v = project(x_prompt)
    y, st_prompt = scan(params, q, k, v)
    out_prompt = dense(y, w_out)
    out_steps, st = None, st_prompt
    if x_steps is not None:
        q, k, v = project(x_steps)
        ys, st = scan(params, q, k, v, state=st_prompt, batch_axis=1, time_axis=0)
        # ys is [B][S][D]; return step-major like the inputs
        out_steps = dense(np.ascontiguousarray(ys.transpose(1, 0, 2)), w_out)
    return out_prompt, out_steps, st_prompt, st


class Bound:
    """The oracle's functions bound to another build of ``modal_oracle.c``.

    Used by the tests that plant mistakes in a copy of the oracle source to show
    that the pins catch them.
    """

    def __init__(self, lib_path: str):
        self._h = _bind(lib_path)

    def filter_taps(self, params, L):
        return filter_taps(params, L, _lib_handle=self._h)

    def modal_scan(self, *a, **kw):
        return modal_scan(*a, _lib_handle=self._h, **kw)

    def stack_layer(self, *a, **kw):
        return stack_layer(*a, _scan=self.modal_scan, **kw)
