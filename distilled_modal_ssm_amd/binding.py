"""ctypes binding of ``libhyena_modal.so`` (the C ABI in include/hyena_modal.h).

Argument marshalling only: every computation runs in the library's HIP kernels.
Pointer arguments accept an ``int`` device address, ``None`` (NULL) or any
object with ``data_ptr()`` (a torch tensor); ``stream`` accepts an ``int``
hipStream_t, ``None`` (the current torch stream when torch is loaded, else the
default stream) or a torch stream.

The library must have been built in-tree (``distilled_modal_ssm_amd/build.py``);
if it is missing, loading raises :class:`LibraryMissing` -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhyena_modal.so")

HM_ABI_VERSION = 1
HM_MAX_MODES = 64
HM_F32, HM_BF16 = 0, 1
HM_OK, HM_ERR_INVALID_ARG, HM_ERR_UNSUPPORTED, HM_ERR_WORKSPACE, HM_ERR_HIP = range(5)
HM_PREFILL_AUTO, HM_PREFILL_SCAN, HM_PREFILL_MFMA = 0, 1, 2
HM_NOALLOC_SCRATCH_BYTES = 16 << 20  # per-GPU scratch of hyena_modal_prefill_noalloc
ALGOS = {"auto": HM_PREFILL_AUTO, "scan": HM_PREFILL_SCAN, "mfma": HM_PREFILL_MFMA}

EXPORTS = (
    "hm_abi_version",
    "hm_status_string",
    "hyena_modal_prefill_workspace",
    "hyena_modal_prefill_workspace_ex",
    "hyena_modal_prefill_plan",
    "hyena_modal_prefill",
    "hyena_modal_prefill_ex",
    "hyena_modal_prefill_noalloc",
    "hyena_modal_decode_step",
    "hyena_filter_materialize",
    "hyena_row_rms",
    "hyena_dense_bf16",
    "hyena_dense_rms_bf16",
    "hyena_dense_workspace",
    "hyena_dense_bf16_ex",
    "hyena_dense_rms_bf16_ex",
    "hyena_layer_step_bf16",
    "hyena_pack_in_proj_bf16",
    "hyena_fir_workspace",
    "hyena_fir_decode_step",
    "hyena_fir_decode_step_ex",
    "hyena_fir_cache_fill",
    "hyena_fft_prefill_workspace",
    "hyena_fft_prefill",
    "hyena_distill_workspace",
    "hyena_distill_grad",
    "hyena_distill_adam_step",
    "hyena_decode_prepare",
    "hyena_layer_gate_bf16",
    "hyena_hankel_singular_values",
    "hyena_modal_order",
    "hyena_modal_fit_init",
)


class LibraryMissing(RuntimeError):
    pass


class HMError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class hm_desc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int64),
        ("channels", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("modes", ctypes.c_int64),
        ("poles", ctypes.c_void_p),
        ("residues", ctypes.c_void_p),
        ("skip", ctypes.c_void_p),
    ]


class hm_prefill_opts(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int64), ("algo", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class hm_prefill_info(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32), ("channel_tile", ctypes.c_int32), ("chunk", ctypes.c_int64),
                ("n_chunks", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once (raises LibraryMissing if it was not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise LibraryMissing(
                f"{path} not found: build it with `python -m distilled_modal_ssm_amd.build` "
                "(or __graft_entry__.build()); there is no CPU fallback")
        lib = ctypes.CDLL(path)
        i64, p, sz, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
        D = ctypes.POINTER(hm_desc)
        sig = {
            "hm_abi_version": ([], ctypes.c_int),
            "hm_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "hyena_modal_prefill_workspace": ([D, i64, ctypes.POINTER(sz)], ctypes.c_int),
            "hyena_modal_prefill_workspace_ex": ([D, i64, ctypes.POINTER(hm_prefill_opts), ctypes.POINTER(sz)],
                                                 ctypes.c_int),
            "hyena_modal_prefill_plan": ([D, i64, ctypes.POINTER(hm_prefill_opts), ctypes.POINTER(hm_prefill_info)],
                                         ctypes.c_int),
            "hyena_modal_prefill": ([D, i64, p, p, p, i64, p, i64, p, p, p, sz, p], ctypes.c_int),
            "hyena_modal_prefill_ex": ([D, i64, p, p, p, i64, p, i64, p, p, p, sz,
                                        ctypes.POINTER(hm_prefill_opts), p], ctypes.c_int),
            "hyena_modal_prefill_noalloc": ([D, i64, p, p, p, i64, p, i64, p, p,
                                             ctypes.POINTER(hm_prefill_opts), p], ctypes.c_int),
            "hyena_modal_decode_step": ([D, p, p, p, i64, p, i64, p, p], ctypes.c_int),
            "hyena_filter_materialize": ([D, i64, p, p], ctypes.c_int),
            "hyena_row_rms": ([p, i64, i64, i64, ctypes.c_float, p, p], ctypes.c_int),
            "hyena_dense_bf16": ([i64, i64, i64, p, i64, p, i64, p, p, i64, p], ctypes.c_int),
            "hyena_dense_rms_bf16": ([i64, i64, i64, p, i64, p, i64, ctypes.c_float, p, i64, p], ctypes.c_int),
            "hyena_dense_workspace": ([i64, i64, i64, ctypes.POINTER(sz)], ctypes.c_int),
            "hyena_fir_workspace": ([D, ctypes.POINTER(sz)], ctypes.c_int),
            "hyena_fir_decode_step": ([D, p, i64, i64, i64, p, p, p, i64, p, i64, p, i64, p, sz, p], ctypes.c_int),
            "hyena_fir_decode_step_ex": ([D, p, i64, i64, i64, p, p, p, i64, p, i64, p, i64, p, sz, ctypes.c_int32, p],
                                         ctypes.c_int),
            "hyena_fir_cache_fill": ([D, i64, p, p, i64, p, i64, p], ctypes.c_int),
            "hyena_fft_prefill_workspace": ([D, i64, ctypes.POINTER(sz)], ctypes.c_int),
            "hyena_fft_prefill": ([D, i64, p, p, p, i64, p, i64, p, sz, p], ctypes.c_int),
            "hyena_distill_workspace": ([D, i64, ctypes.POINTER(sz)], ctypes.c_int),
            "hyena_distill_grad": ([D, i64, p, p, p, p, p, p, sz, p], ctypes.c_int),
            "hyena_distill_adam_step": ([i64, i64, p, p, p, p, p, p, p, p, i64, f32, f32, f32, f32, f32, p],
                                        ctypes.c_int),
            "hyena_dense_bf16_ex": ([i64, i64, i64, p, i64, p, i64, p, p, i64, p, sz, p], ctypes.c_int),
            "hyena_dense_rms_bf16_ex": ([i64, i64, i64, p, i64, p, i64, ctypes.c_float, p, i64, p, sz, p],
                                        ctypes.c_int),
            "hyena_layer_step_bf16": ([D, p, i64, p, ctypes.c_float, p, p, i64, p], ctypes.c_int),
            "hyena_pack_in_proj_bf16": ([i64, i64, p, i64, p, p], ctypes.c_int),
            "hyena_decode_prepare": ([D, p, p, p, p], ctypes.c_int),
            "hyena_layer_gate_bf16": ([D, p, i64, p, ctypes.c_float, p, p, p, i64, D, p, p, p, p], ctypes.c_int),
            "hyena_hankel_singular_values": ([p, i64, i64, p], ctypes.c_int),
            "hyena_modal_order": ([p, i64, i64, i64, ctypes.c_double, p], ctypes.c_int),
            "hyena_modal_fit_init": ([p, i64, i64, i64, f32, p, p, p], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        if lib.hm_abi_version() != HM_ABI_VERSION:
            raise LibraryMissing("libhyena_modal.so has a different ABI version")
        _lib = lib
        return lib


def status_string(status: int) -> str:
    try:
        return load().hm_status_string(status).decode()
    except LibraryMissing:
        return f"status {status}"


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s):
    if s is None:
        import sys
        torch = sys.modules.get("torch")
        if torch is not None and torch.cuda.is_initialized():
            return int(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _check(status: int, where: str):
    if status != HM_OK:
        raise HMError(status, where)


def make_desc(batch, channels, heads, modes, act_dtype, poles, residues, skip) -> hm_desc:
    return hm_desc(HM_ABI_VERSION, act_dtype, batch, channels, heads, modes,
                   _ptr(poles), _ptr(residues), _ptr(skip))


# ----------------------------------------------------------------- raw entry points


def hm_abi_version() -> int:
    return load().hm_abi_version()


def _opts(chunk, algo):
    a = ALGOS[algo] if isinstance(algo, str) else int(algo)
    return hm_prefill_opts(int(chunk), a, 0)


def hyena_modal_prefill_workspace(desc: hm_desc, L: int, chunk: int = 0, algo="auto") -> int:
    n = ctypes.c_size_t(0)
    if chunk or algo not in ("auto", HM_PREFILL_AUTO):
        o = _opts(chunk, algo)
        st = load().hyena_modal_prefill_workspace_ex(ctypes.byref(desc), L, ctypes.byref(o), ctypes.byref(n))
    else:
        st = load().hyena_modal_prefill_workspace(ctypes.byref(desc), L, ctypes.byref(n))
    _check(st, "hyena_modal_prefill_workspace")
    return n.value


def hyena_modal_prefill_plan(desc: hm_desc, L: int, chunk: int = 0, algo="auto") -> dict:
    """What a prefill would run: {"algo": "scan"|"mfma", "channel_tile", "chunk", "n_chunks",
    "workspace_bytes"}."""
    o = _opts(chunk, algo)
    info = hm_prefill_info()
    _check(load().hyena_modal_prefill_plan(ctypes.byref(desc), L, ctypes.byref(o), ctypes.byref(info)),
           "hyena_modal_prefill_plan")
    names = {HM_PREFILL_SCAN: "scan", HM_PREFILL_MFMA: "mfma"}
    return {"algo": names[info.algo], "channel_tile": info.channel_tile, "chunk": info.chunk,
            "n_chunks": info.n_chunks, "workspace_bytes": info.workspace_bytes}


def hyena_modal_prefill(desc: hm_desc, L, q, k, v, ld_in, y, ld_y, state_in, state_out,
                        workspace, ws_bytes, stream=None, chunk: int = 0, algo="auto") -> None:
    lib = load()
    args = (ctypes.byref(desc), L, _ptr(q), _ptr(k), _ptr(v), ld_in, _ptr(y), ld_y,
            _ptr(state_in), _ptr(state_out), _ptr(workspace), ws_bytes)
    if chunk or algo not in ("auto", HM_PREFILL_AUTO):
        o = _opts(chunk, algo)
        st = lib.hyena_modal_prefill_ex(*args, ctypes.byref(o), _stream(stream))
    else:
        st = lib.hyena_modal_prefill(*args, _stream(stream))
    _check(st, "hyena_modal_prefill")


def hyena_modal_prefill_noalloc(desc: hm_desc, L, q, k, v, ld_in, y, ld_y, state_in, state_out,
                                stream=None, chunk: int = 0, algo="auto") -> None:
    """The prefill with the library's own per-GPU scratch as its workspace
    (no allocation; calls that overlap on one GPU race)."""
    o = _opts(chunk, algo)
    st = load().hyena_modal_prefill_noalloc(ctypes.byref(desc), L, _ptr(q), _ptr(k), _ptr(v), ld_in, _ptr(y),
                                            ld_y, _ptr(state_in), _ptr(state_out), ctypes.byref(o),
                                            _stream(stream))
    _check(st, "hyena_modal_prefill_noalloc")


def hyena_modal_decode_step(desc: hm_desc, q, k, v, ld_in, y, ld_y, state, stream=None) -> None:
    st = load().hyena_modal_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), ld_in,
                                        _ptr(y), ld_y, _ptr(state), _stream(stream))
    _check(st, "hyena_modal_decode_step")


def hyena_filter_materialize(desc: hm_desc, L, h_out, stream=None) -> None:
    st = load().hyena_filter_materialize(ctypes.byref(desc), L, _ptr(h_out), _stream(stream))
    _check(st, "hyena_filter_materialize")


def hyena_row_rms(x, M, D, ld, eps, inv_rms, stream=None) -> None:
    st = load().hyena_row_rms(_ptr(x), M, D, ld, eps, _ptr(inv_rms), _stream(stream))
    _check(st, "hyena_row_rms")


def _ws_bytes(workspace, ws_bytes):
    if ws_bytes is not None:
        return int(ws_bytes)
    return workspace.numel() * workspace.element_size() if workspace is not None else 0


def hyena_dense_bf16(M, N, K, A, lda, W, ldw, row_scale, C, ldc, stream=None, workspace=None,
                     ws_bytes=None) -> None:
    """C = row_scale * A W^T; with a workspace, small M takes the split-K path."""
    if workspace is None:
        st = load().hyena_dense_bf16(M, N, K, _ptr(A), lda, _ptr(W), ldw, _ptr(row_scale), _ptr(C), ldc,
                                     _stream(stream))
    else:
        st = load().hyena_dense_bf16_ex(M, N, K, _ptr(A), lda, _ptr(W), ldw, _ptr(row_scale), _ptr(C), ldc,
                                        _ptr(workspace), _ws_bytes(workspace, ws_bytes), _stream(stream))
    _check(st, "hyena_dense_bf16")


def hyena_dense_rms_bf16(M, N, K, A, lda, W, ldw, eps, C, ldc, stream=None, workspace=None,
                         ws_bytes=None) -> None:
    if workspace is None:
        st = load().hyena_dense_rms_bf16(M, N, K, _ptr(A), lda, _ptr(W), ldw, eps, _ptr(C), ldc,
                                         _stream(stream))
    else:
        st = load().hyena_dense_rms_bf16_ex(M, N, K, _ptr(A), lda, _ptr(W), ldw, eps, _ptr(C), ldc,
                                            _ptr(workspace), _ws_bytes(workspace, ws_bytes), _stream(stream))
    _check(st, "hyena_dense_rms_bf16")


def hyena_dense_workspace(M, N, K) -> int:
    n = ctypes.c_size_t(0)
    _check(load().hyena_dense_workspace(M, N, K, ctypes.byref(n)), "hyena_dense_workspace")
    return n.value


def hyena_pack_in_proj_bf16(D, K, w_in, ldw, w_packed, stream=None) -> None:
    """w_packed row 48 G + 16 j + i = w_in row j D + 16 G + i (q, k, v rows of a 16-channel group adjacent)."""
    _check(load().hyena_pack_in_proj_bf16(D, K, _ptr(w_in), ldw, _ptr(w_packed), _stream(stream)),
           "hyena_pack_in_proj_bf16")


def hyena_layer_step_bf16(desc: hm_desc, x, ldx, w_packed, eps, state, y, ld_y, stream=None) -> int:
    """Fused generation step of a projected layer (in_proj with RMS + decode step).

    Returns the library status without raising for HM_ERR_UNSUPPORTED, so a
    caller can fall back to the two separate calls; other errors raise."""
    st = load().hyena_layer_step_bf16(ctypes.byref(desc), _ptr(x), ldx, _ptr(w_packed), eps, _ptr(state), _ptr(y),
                                      ld_y, _stream(stream))
    if st != HM_ERR_UNSUPPORTED:
        _check(st, "hyena_layer_step_bf16")
    return st


def hyena_fir_workspace(desc: hm_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().hyena_fir_workspace(ctypes.byref(desc), ctypes.byref(n)), "hyena_fir_workspace")
    return n.value


HM_FIR_LOADS_AUTO, HM_FIR_LOADS_PLAIN, HM_FIR_LOADS_NONTEMPORAL = 0, 1, 2


def hyena_fir_decode_step(desc: hm_desc, h, h_len, window, t, q, k, v, ld_in, y, ld_y, u_cache, cache_len,
                          workspace, ws_bytes=None, stream=None, loads=None) -> None:
    """loads: None for the library's default; else HM_FIR_LOADS_* (hyena_fir_decode_step_ex)."""
    if loads is None:
        st = load().hyena_fir_decode_step(ctypes.byref(desc), _ptr(h), h_len, window, t, _ptr(q), _ptr(k),
                                          _ptr(v), ld_in, _ptr(y), ld_y, _ptr(u_cache), cache_len,
                                          _ptr(workspace), _ws_bytes(workspace, ws_bytes), _stream(stream))
    else:
        st = load().hyena_fir_decode_step_ex(ctypes.byref(desc), _ptr(h), h_len, window, t, _ptr(q), _ptr(k),
                                             _ptr(v), ld_in, _ptr(y), ld_y, _ptr(u_cache), cache_len,
                                             _ptr(workspace), _ws_bytes(workspace, ws_bytes), int(loads),
                                             _stream(stream))
    _check(st, "hyena_fir_decode_step")


def hyena_fir_cache_fill(desc: hm_desc, L, k, v, ld_in, u_cache, cache_len, stream=None) -> None:
    st = load().hyena_fir_cache_fill(ctypes.byref(desc), L, _ptr(k), _ptr(v), ld_in, _ptr(u_cache), cache_len,
                                     _stream(stream))
    _check(st, "hyena_fir_cache_fill")


def hyena_fft_prefill_workspace(desc: hm_desc, L: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().hyena_fft_prefill_workspace(ctypes.byref(desc), L, ctypes.byref(n)),
           "hyena_fft_prefill_workspace")
    return n.value


def hyena_fft_prefill(desc: hm_desc, L, q, k, v, ld_in, y, ld_y, workspace, ws_bytes=None, stream=None) -> None:
    st = load().hyena_fft_prefill(ctypes.byref(desc), L, _ptr(q), _ptr(k), _ptr(v), ld_in, _ptr(y), ld_y,
                                  _ptr(workspace), _ws_bytes(workspace, ws_bytes), _stream(stream))
    _check(st, "hyena_fft_prefill")


def hyena_distill_workspace(desc: hm_desc, L: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().hyena_distill_workspace(ctypes.byref(desc), L, ctypes.byref(n)), "hyena_distill_workspace")
    return n.value


def hyena_distill_grad(desc: hm_desc, L, h_target, loss, g_poles, g_res, g_skip, workspace, ws_bytes=None,
                       stream=None) -> None:
    st = load().hyena_distill_grad(ctypes.byref(desc), L, _ptr(h_target), _ptr(loss), _ptr(g_poles), _ptr(g_res),
                                   _ptr(g_skip), _ptr(workspace), _ws_bytes(workspace, ws_bytes), _stream(stream))
    _check(st, "hyena_distill_grad")


def hyena_distill_adam_step(H, d, poles, residues, skip, g_poles, g_res, g_skip, m, v, step, lr, beta1=0.9,
                            beta2=0.999, eps=1e-8, r_max=0.9999, stream=None) -> None:
    st = load().hyena_distill_adam_step(H, d, _ptr(poles), _ptr(residues), _ptr(skip), _ptr(g_poles), _ptr(g_res),
                                        _ptr(g_skip), _ptr(m), _ptr(v), step, lr, beta1, beta2, eps, r_max,
                                        _stream(stream))
    _check(st, "hyena_distill_adam_step")


# ----------------------------------------------------------------- generation step, deferred state


def hyena_decode_prepare(desc: hm_desc, state, u_prev, rho, stream=None) -> None:
    _check(load().hyena_decode_prepare(ctypes.byref(desc), _ptr(state), _ptr(u_prev), _ptr(rho), _stream(stream)),
           "hyena_decode_prepare")


def hyena_layer_gate_bf16(desc: hm_desc, x, ldx, w_packed, eps, rho, u_prev, y, ld_y, next_desc=None,
                          next_state=None, next_u_prev=None, next_rho=None, stream=None) -> int:
    """Returns the status (HM_ERR_UNSUPPORTED lets a caller fall back)."""
    nd = ctypes.byref(next_desc) if next_desc is not None else None
    st = load().hyena_layer_gate_bf16(ctypes.byref(desc), _ptr(x), ldx, _ptr(w_packed), eps, _ptr(rho), _ptr(u_prev),
                                      _ptr(y), ld_y, nd, _ptr(next_state), _ptr(next_u_prev), _ptr(next_rho),
                                      _stream(stream))
    if st not in (HM_OK, HM_ERR_UNSUPPORTED):
        _check(st, "hyena_layer_gate_bf16")
    return st


# ----------------------------------------------------------------- host-side fit set-up


def _host_f32(a):
    import numpy as np
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def hyena_hankel_singular_values(h, n: int):
    """Singular values (decreasing) of the n x n Hankel matrix of one filter's taps h[1:]."""
    import numpy as np
    h = _host_f32(h)
    sv = np.empty(n, dtype=np.float64)
    _check(load().hyena_hankel_singular_values(h.ctypes.data, h.size, n, sv.ctypes.data),
           "hyena_hankel_singular_values")
    return sv


def hyena_modal_order(h, n: int, rel_tol: float):
    """Per head of h [H][L]: Hankel singular values above rel_tol x the largest."""
    import numpy as np
    h = _host_f32(h)
    out = np.empty(h.shape[0], dtype=np.int64)
    _check(load().hyena_modal_order(h.ctypes.data, h.shape[0], h.shape[1], n, rel_tol, out.ctypes.data),
           "hyena_modal_order")
    return out


def hyena_modal_fit_init(h, d: int, r_max: float = 0.9999):
    """Matrix-pencil / least-squares initial fit of h [H][L] (host arrays):
    returns (poles [H][d][2], residues [H][d][2], skip [H]) float32."""
    import numpy as np
    h = _host_f32(h)
    H, L = h.shape
    poles = np.empty((H, d, 2), dtype=np.float32)
    res = np.empty((H, d, 2), dtype=np.float32)
    skip = np.empty(H, dtype=np.float32)
    _check(load().hyena_modal_fit_init(h.ctypes.data, H, L, d, r_max, poles.ctypes.data, res.ctypes.data,
                                       skip.ctypes.data), "hyena_modal_fit_init")
    return poles, res, skip


# ----------------------------------------------------------------- tensor helpers


def _row_stride(t, same):
    """Row stride ld of a [B][L][D] view laid out as (b*L + t)*ld + c; checks peers."""
    if t.dim() != 3 or (t.shape[2] > 1 and t.stride(2) != 1):
        raise ValueError("activations must be [B][L][D] views with unit channel stride")
    B, L = t.shape[0], t.shape[1]
    ld = t.stride(1) if L > 1 else (t.stride(0) if B > 1 else t.shape[2])
    if B > 1 and L > 0 and t.stride(0) != L * ld:
        raise ValueError("batch rows must be contiguous runs of L rows (stride(0) == L*stride(1))")
    for o in same:
        if o.shape != t.shape or (L > 1 and o.stride(1) != ld) or (B > 1 and L > 0 and o.stride(0) != t.stride(0)):
            raise ValueError("q, k, v must share shape and strides")
    return ld


class ModalHyena:
    """Device tables of one operator plus calls on torch tensors.

    poles, residues: [H][d][2] float32; skip: [H] float32 (host arrays or
    tensors; copied to ``device``).  Activations are torch tensors of dtype
    float32 or bfloat16 on the same device; outputs are allocated with torch
    (device memory is torch's job, the arithmetic is the library's).
    """

    def __init__(self, poles, residues, skip, batch: int, channels: int, act: str, device="cuda"):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        t = lambda a: torch.as_tensor(a, dtype=torch.float32).contiguous().to(self.device)
        self.poles, self.residues, self.skip = t(poles), t(residues), t(skip)
        self.H, self.d = int(self.poles.shape[0]), int(self.poles.shape[1])
        self.B, self.D = int(batch), int(channels)
        self.P = self.D // self.H
        self.act = act
        self.tdtype = torch.bfloat16 if act == "bf16" else torch.float32
        self.desc = make_desc(self.B, self.D, self.H, self.d, HM_BF16 if act == "bf16" else HM_F32,
                              self.poles, self.residues, self.skip)
        self._ws = None

    def new_state(self):
        return self.torch.zeros((self.B, self.H, self.d, self.P, 2), dtype=self.torch.float32,
                                device=self.device)

    def workspace(self, L: int, chunk: int = 0, algo="auto"):
        n = hyena_modal_prefill_workspace(self.desc, L, chunk, algo)
        if self._ws is None or self._ws.numel() < n:
            self._ws = self.torch.empty(max(n, 256), dtype=self.torch.uint8, device=self.device)
        return self._ws, n

    def plan(self, L: int, chunk: int = 0, algo="auto") -> dict:
        return hyena_modal_prefill_plan(self.desc, L, chunk, algo)

    def prefill(self, q, k, v, y=None, state_in=None, state_out=None, chunk: int = 0, algo="auto",
                stream=None):
        """q, k, v: [B][L][ld] views with unit channel stride.  Returns (y, state).

        algo: "auto", "scan" (vector-ALU modal scan) or "mfma" (matrix-core sub-blocks).
        """
        B, L = q.shape[0], q.shape[1]
        if y is None:
            y = self.torch.empty((B, L, self.D), dtype=self.tdtype, device=self.device)
        if state_out is None:
            state_out = self.new_state()
        ld_in = _row_stride(q, (k, v))
        ld_y = _row_stride(y, ())
        ws, n = self.workspace(L, chunk, algo)
        hyena_modal_prefill(self.desc, L, q, k, v, ld_in, y, ld_y, state_in, state_out, ws, n,
                            stream, chunk, algo)
        return y, state_out

    def fft_prefill(self, q, k, v, y=None, stream=None):
        """The prompt through the FFT convolution (no state).  q, k, v: [B][L][ld] views."""
        L = int(q.shape[1])
        if y is None:
            y = self.torch.empty((self.B, L, self.D), dtype=self.tdtype, device=self.device)
        ld_in = _row_stride(q, (k, v))
        n = hyena_fft_prefill_workspace(self.desc, L)
        ws = self.torch.empty(max(n, 256), dtype=self.torch.uint8, device=self.device)
        hyena_fft_prefill(self.desc, L, q, k, v, ld_in, y, _row_stride(y, ()), ws, n, stream)
        return y

    def decode_step(self, q, k, v, state, y=None, stream=None):
        """q, k, v: [B][ld] rows.  Updates state in place; returns y [B][D]."""
        if y is None:
            y = self.torch.empty((self.B, self.D), dtype=self.tdtype, device=self.device)
        for t in (q, k, v, y):
            if t.dim() != 2 or t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) != q.stride(0) and t is not y):
                raise ValueError("decode_step needs [B][D] rows with unit channel stride and one row stride for q, k, v")
        hyena_modal_decode_step(self.desc, q, k, v, q.stride(0), y, y.stride(0), state, stream)
        return y

    def filter(self, L: int, stream=None):
        h = self.torch.empty((self.H, L), dtype=self.torch.float32, device=self.device)
        hyena_filter_materialize(self.desc, L, h, stream)
        return h


class FirHyena:
    """The explicit-filter (non-distilled) decode baseline on the same shapes as
    a :class:`ModalHyena`: a u cache [B][cache_len][D] in the activation dtype
    and the pass-1 workspace, allocated once with torch."""

    def __init__(self, op: ModalHyena, cache_len: int):
        torch = op.torch
        self.op, self.torch = op, torch
        self.cache_len = int(cache_len)
        self.cache = torch.zeros((op.B, self.cache_len, op.D), dtype=op.tdtype, device=op.device)
        n = hyena_fir_workspace(op.desc)
        self.ws = torch.empty(max(n, 256), dtype=torch.uint8, device=op.device)

    def fill(self, k, v, stream=None):
        """Cache rows 0 .. L-1 from a prompt's k, v [B][L][ld] views."""
        L = int(k.shape[1])
        ld = _row_stride(k, (v,))
        hyena_fir_cache_fill(self.op.desc, L, k, v, ld, self.cache, self.cache_len, stream)

    def step(self, h, t: int, q, k, v, window: int = 0, y=None, stream=None, loads=None):
        """One generated token at position t through the taps h [H][>= min(t+1, W)];
        q, k, v: [B][ld] rows with one row stride.  loads: None (the library's
        choice by window size) or HM_FIR_LOADS_PLAIN / HM_FIR_LOADS_NONTEMPORAL."""
        if y is None:
            y = self.torch.empty((self.op.B, self.op.D), dtype=self.op.tdtype, device=self.op.device)
        for x in (q, k, v, y):
            if x.dim() != 2 or x.stride(1) != 1 or (x.shape[0] > 1 and x is not y and x.stride(0) != q.stride(0)):
                raise ValueError("FIR step needs [B][D] rows with unit channel stride and one row stride for q, k, v")
        hyena_fir_decode_step(self.op.desc, h, int(h.shape[-1]), window, t, q, k, v, q.stride(0), y,
                              y.stride(0), self.cache, self.cache_len, self.ws, stream=stream, loads=loads)
        return y
