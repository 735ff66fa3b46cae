"""GPU parity of the HIP path against the float64 oracle (through the C ABI).

Tolerances (max |err| over the compared tensor, relative to its max |oracle|):
1e-4 for float32 activations, 2e-2 for bfloat16 activations; the same rule is
applied to the modal states and, at 1e-4, to the materialised filter.
Large workloads run at full size on the GPU, in the launch configuration the
benchmark uses (automatic chunking); the oracle then recomputes a seeded sample
of channels (channels are independent, so each sampled channel is exact).
"""

import zlib

import numpy as np
import pytest

import oracle
from _gpu_common import (TOL, act_to_f64, log, record_margin, rel_err, require_gpu, state_for_channels,
                         state_to_gpu_layout, to_dev, to_np64)
from distilled_modal_ssm_amd import ModalHyena
from distilled_modal_ssm_amd import binding as hb
from workloads import decode_inputs, get_config, modal_params, prompt_inputs
from workloads.generate import ModalParams

pytestmark = pytest.mark.gpu


def _op(params, B, D, act):
    return ModalHyena(params.poles, params.residues, params.skip, B, D, act)


def _sample_channels(cfg, n_random, seed):
    rng = np.random.default_rng(seed)
    P = cfg.P
    fixed = [0, P - 1, P, cfg.D - 1]
    extra = rng.choice(cfg.D, size=n_random, replace=False)
    return np.unique(np.concatenate([fixed, extra])).astype(np.int64)


def _rand_params(rng, H, d, r_lo=0.5, r_hi=0.99):
    r = rng.uniform(r_lo, r_hi, (H, d))
    th = rng.uniform(0, np.pi, (H, d))
    poles = np.stack([r * np.cos(th), r * np.sin(th)], -1).astype(np.float32)
    res = (rng.standard_normal((H, d, 2)) / np.sqrt(2 * d)).astype(np.float32)
    return ModalParams(poles, res, rng.standard_normal(H).astype(np.float32))


def _rand_act(rng, shape, act):
    from workloads import round_to_bf16_bits
    x = rng.standard_normal(shape)
    return round_to_bf16_bits(x) if act == "bf16" else x.astype(np.float32)


# ------------------------------------------------------------------ filter


@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5])
def test_filter_materialize(ci):
    torch = require_gpu()
    cfg = get_config(ci)
    params = modal_params(cfg)
    log(f"filter workload {ci} H={cfg.H} d={cfg.d} L={cfg.L}")
    h = to_np64(_op(params, cfg.B, cfg.D, cfg.act).filter(cfg.L))
    torch.cuda.synchronize()
    ref = oracle.filter_taps(params, cfg.L)
    err = rel_err(h, ref)
    print(f"filter workload {ci}: rel err {err:.3e}")
    assert err <= 1e-4
    assert np.array_equal(h[:, 0], params.skip.astype(np.float64))


@pytest.mark.parametrize("H,d,L", [(3, 1, 1), (2, 5, 31), (2, 12, 33), (1, 33, 1000), (2, 64, 700),
                                   (5, 16, 4097)])
def test_filter_mode_counts_and_ragged_lengths(H, d, L):
    """Every mode-count padding (d -> next power of two) and ragged tap tiles,
    with poles close to the unit circle."""
    torch = require_gpu()
    rng = np.random.default_rng(H * 1000 + d * 10 + L)
    params = _rand_params(rng, H, d, 0.9, 0.9999)
    log(f"filter H={H} d={d} L={L}")
    h = to_np64(_op(params, 1, 64 * H, "f32").filter(L))
    torch.cuda.synchronize()
    ref = oracle.filter_taps(params, L)
    assert rel_err(h, ref) <= 1e-4
    assert np.array_equal(h[:, 0], params.skip.astype(np.float64))


# ------------------------------------------------------------------ tiny workload, full oracle


@pytest.mark.parametrize("chunk", [0, 64, 128, 192])
def test_workload1_prefill_and_decode(chunk):
    torch = require_gpu()
    cfg = get_config(1)
    params = modal_params(cfg)
    inp = prompt_inputs(cfg)
    dec = decode_inputs(cfg)
    op = _op(params, cfg.B, cfg.D, cfg.act)
    q, k, v = (to_dev(inp[n], cfg.act) for n in "qkv")
    log(f"workload 1 prefill chunk={chunk}")
    y, st = op.prefill(q, k, v, chunk=chunk)
    torch.cuda.synchronize()
    y_or, st_or = oracle.modal_scan(params, inp["q"], inp["k"], inp["v"])
    assert rel_err(to_np64(y), y_or) <= TOL["f32"]
    all_ch = np.arange(cfg.D)
    assert rel_err(state_for_channels(st, all_ch, cfg.P), st_or) <= TOL["f32"]

    dq, dk, dv = (to_dev(dec[n], cfg.act) for n in "qkv")
    ys = torch.empty((cfg.S, cfg.B, cfg.D), dtype=torch.float32, device="cuda")
    log("workload 1 decode")
    for s in range(cfg.S):
        op.decode_step(dq[s], dk[s], dv[s], st, y=ys[s])
    torch.cuda.synchronize()
    yd_or, st2_or = oracle.modal_scan(params, dec["q"], dec["k"], dec["v"], state=st_or,
                                      batch_axis=1, time_axis=0)
    assert rel_err(to_np64(ys).transpose(1, 0, 2), yd_or) <= TOL["f32"]
    assert rel_err(state_for_channels(st, all_ch, cfg.P), st2_or) <= TOL["f32"]


# ------------------------------------------------------------------ full-size workloads, sampled


@pytest.mark.parametrize("algo", ["auto", "scan"])
@pytest.mark.parametrize("ci", [2, 3, 4])
def test_workload_full_size_sampled(ci, algo):
    """Automatic (matrix-core sub-blocks for these shapes) and vector-scan prefill."""
    torch = require_gpu()
    cfg = get_config(ci)
    params = modal_params(cfg)
    tol = TOL[cfg.act]
    inp = prompt_inputs(cfg)
    op = _op(params, cfg.B, cfg.D, cfg.act)
    q, k, v = (to_dev(inp[n], cfg.act) for n in "qkv")
    plan = op.plan(cfg.L, algo=algo)
    # the automatic plan at these sizes is the matrix-core path the benchmark times
    assert plan["algo"] == ("mfma" if algo == "auto" else "scan")
    log(f"workload {ci} prefill {cfg.describe()} algo={algo} plan={plan}")
    y, st = op.prefill(q, k, v, algo=algo)
    torch.cuda.synchronize()
    del q, k, v
    chans = _sample_channels(cfg, 28, 100 + ci)
    batches = np.arange(cfg.B) if cfg.B <= 16 else np.sort(
        np.random.default_rng(200 + ci).choice(cfg.B, 8, replace=False))
    sub = lambda a: a if len(batches) == cfg.B else np.ascontiguousarray(a[batches])
    y_or, st_or = oracle.modal_scan(params, sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), channels=chans)
    del inp
    bt, ct = torch.as_tensor(batches, device="cuda"), torch.as_tensor(chans, device="cuda")
    y_gpu = to_np64(y.index_select(2, ct).index_select(0, bt))
    e_y = rel_err(y_gpu, y_or)
    st_gpu = state_for_channels(st, chans, cfg.P)[batches]
    e_s = rel_err(st_gpu, st_or)
    print(f"workload {ci} prefill ({algo}): y rel err {e_y:.3e}, state rel err {e_s:.3e}")
    record_margin(f"{cfg.name} prefill algo={plan['algo']}", "prefill y", e_y, tol)
    record_margin(f"{cfg.name} prefill algo={plan['algo']}", "prefill state", e_s, tol)
    assert e_y <= tol and e_s <= tol
    del y

    dec = decode_inputs(cfg)
    dq, dk, dv = (to_dev(dec[n], cfg.act) for n in "qkv")
    ys = torch.empty((cfg.S, cfg.B, cfg.D), dtype=op.tdtype, device="cuda")
    log(f"workload {ci} decode S={cfg.S}")
    for s in range(cfg.S):
        op.decode_step(dq[s], dk[s], dv[s], st, y=ys[s])
    torch.cuda.synchronize()
    yd_or, st2_or = oracle.modal_scan(params, np.ascontiguousarray(dec["q"][:, batches]),
                                      np.ascontiguousarray(dec["k"][:, batches]),
                                      np.ascontiguousarray(dec["v"][:, batches]), state=st_or,
                                      channels=chans, batch_axis=1, time_axis=0)
    yd_gpu = to_np64(ys.index_select(2, ct).index_select(1, bt))
    e_yd = rel_err(yd_gpu.transpose(1, 0, 2), yd_or)
    e_s2 = rel_err(state_for_channels(st, chans, cfg.P)[batches], st2_or)
    print(f"workload {ci} decode: y rel err {e_yd:.3e}, state rel err {e_s2:.3e}")
    record_margin(f"{cfg.name} decode S={cfg.S} (after {plan['algo']})", "decode y", e_yd, tol)
    record_margin(f"{cfg.name} decode S={cfg.S} (after {plan['algo']})", "decode state", e_s2, tol)
    assert e_yd <= tol and e_s2 <= tol


# ------------------------------------------------------------------ structure and edge cases


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [
    # (B, D, H, d, L, chunk, algo)
    (3, 36, 3, 5, 200, 64, "auto"),      # odd head dim 12, generic mode count, ragged last chunk
    (2, 16, 2, 1, 130, 64, "auto"),      # one mode
    (2, 128, 2, 64, 256, 128, "auto"),   # largest mode count
    (1, 64, 1, 8, 10, 0, "scan"),        # prompt shorter than one chunk
    (2, 256, 2, 16, 700, 64, "scan"),    # many chunks, ragged
    (1, 192, 3, 32, 320, 128, "scan"),   # three heads of 64 (wave-uniform heads), d = 32
    (2, 256, 2, 16, 700, 64, "mfma"),    # matrix-core sub-blocks, many chunks, ragged last sub-block
    (1, 192, 3, 32, 320, 128, "mfma"),   # 64-channel tiles, d = 32
    (2, 256, 2, 8, 300, 0, "mfma"),      # d = 8 (mode rows padded to 32), one chunk, ragged
    (1, 256, 4, 16, 130, 0, "mfma"),     # head dim 64 with d = 16 (64-channel tiles)
    (3, 128, 1, 16, 10, 0, "mfma"),      # prompt shorter than one sub-block
    (1, 128, 1, 32, 64, 0, "mfma"),      # exactly one sub-block
    (2, 512, 4, 16, 1000, 256, "mfma"),  # several chunks of several sub-blocks
])
def test_shapes_and_chunking(act, shape):
    torch = require_gpu()
    B, D, H, d, L, chunk, algo = shape
    seed = zlib.crc32(repr(shape).encode())  # stable across processes (str hashes are salted)
    rng = np.random.default_rng(seed)
    params = _rand_params(rng, H, d)
    q_, k_, v_ = (_rand_act(rng, (B, L, D), act) for _ in range(3))
    op = _op(params, B, D, act)
    log(f"shape {shape} act {act} seed {seed}")
    y, st = op.prefill(to_dev(q_, act), to_dev(k_, act), to_dev(v_, act), chunk=chunk, algo=algo)
    torch.cuda.synchronize()
    y_or, st_or = oracle.modal_scan(params, q_, k_, v_)
    assert rel_err(to_np64(y), y_or) <= TOL[act]
    assert rel_err(state_for_channels(st, np.arange(D), D // H), st_or) <= TOL[act]
    # a few decode steps on top
    qd, kd, vd = (_rand_act(rng, (4, B, D), act) for _ in range(3))
    ys = [op.decode_step(to_dev(qd[s], act), to_dev(kd[s], act), to_dev(vd[s], act), st) for s in range(4)]
    torch.cuda.synchronize()
    yd_or, _ = oracle.modal_scan(params, qd, kd, vd, state=st_or, batch_axis=1, time_axis=0)
    assert rel_err(np.stack([to_np64(t) for t in ys], 1), yd_or) <= TOL[act]


def test_empty_prompt_and_empty_batch():
    torch = require_gpu()
    rng = np.random.default_rng(1)
    params = _rand_params(rng, 2, 8)
    op = _op(params, 2, 32, "f32")
    x0 = torch.randn((2, 2, 8, 16, 2), device="cuda")
    out = torch.full_like(x0, 7.0)
    empty = torch.empty((2, 0, 32), device="cuda")
    log("empty prompt with state_in")
    op.prefill(empty, empty, empty, state_in=x0, state_out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, x0)
    log("empty prompt without state_in")
    op.prefill(empty, empty, empty, state_out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    op0 = _op(params, 0, 32, "f32")
    y0, _ = op0.prefill(torch.empty((0, 5, 32), device="cuda"), torch.empty((0, 5, 32), device="cuda"),
                        torch.empty((0, 5, 32), device="cuda"))
    assert y0.shape == (0, 5, 32)


@pytest.mark.parametrize("algo", ["scan", "mfma"])
@pytest.mark.parametrize("chunk", [0, 64])
def test_prompt_continuation_matrix_core(chunk, algo):
    """Continuation with a non-zero state_in on both in-chunk algorithms (head dim 128)."""
    torch = require_gpu()
    rng = np.random.default_rng(21 + chunk)
    B, D, H, d, L, cut = 2, 256, 2, 16, 330, 137
    params = _rand_params(rng, H, d, 0.8, 0.999)
    q_, k_, v_ = (_rand_act(rng, (B, L, D), "f32") for _ in range(3))
    q, k, v = (to_dev(a, "f32") for a in (q_, k_, v_))
    op = _op(params, B, D, "f32")
    log(f"continuation mfma/scan algo={algo} chunk={chunk}")
    head = [t[:, :cut].contiguous() for t in (q, k, v)]
    tail = [t[:, cut:].contiguous() for t in (q, k, v)]
    y1, st1 = op.prefill(*head, chunk=chunk, algo=algo)
    y2, st2 = op.prefill(*tail, state_in=st1, chunk=chunk, algo=algo)
    torch.cuda.synchronize()
    y_or, st_or = oracle.modal_scan(params, q_, k_, v_)
    assert rel_err(np.concatenate([to_np64(y1), to_np64(y2)], 1), y_or) <= TOL["f32"]
    assert rel_err(state_for_channels(st2, np.arange(D), D // H), st_or) <= TOL["f32"]


@pytest.mark.parametrize("chunk", [0, 64])
def test_prompt_continuation_with_state_in(chunk):
    """prefill(a) then prefill(b, state_in) equals prefill(a + b); also in place."""
    torch = require_gpu()
    cfg = get_config(1)
    params = modal_params(cfg)
    inp = prompt_inputs(cfg)
    op = _op(params, cfg.B, cfg.D, "f32")
    q, k, v = (to_dev(inp[n], "f32") for n in "qkv")
    cut = 100
    log(f"continuation chunk={chunk}")
    y_all, st_all = op.prefill(q, k, v, chunk=chunk)
    y1, st1 = op.prefill(q[:, :cut], k[:, :cut], v[:, :cut], chunk=chunk)
    y2, _ = op.prefill(q[:, cut:], k[:, cut:], v[:, cut:], state_in=st1, state_out=st1, chunk=chunk)
    torch.cuda.synchronize()
    y_or, st_or = oracle.modal_scan(params, inp["q"], inp["k"], inp["v"])
    assert rel_err(np.concatenate([to_np64(y1), to_np64(y2)], 1), y_or) <= TOL["f32"]
    assert rel_err(state_for_channels(st1, np.arange(cfg.D), cfg.P), st_or) <= TOL["f32"]
    # a non-zero state_in from the oracle continues exactly as the oracle does
    st_in = torch.from_numpy(state_to_gpu_layout(st_or, cfg.H, cfg.P)).cuda()
    y3, st3 = op.prefill(q[:, :60], k[:, :60], v[:, :60], state_in=st_in, chunk=chunk)
    torch.cuda.synchronize()
    y3_or, st3_or = oracle.modal_scan(params, inp["q"][:, :60], inp["k"][:, :60], inp["v"][:, :60],
                                      state=st_or)
    assert rel_err(to_np64(y3), y3_or) <= TOL["f32"]
    assert rel_err(state_for_channels(st3, np.arange(cfg.D), cfg.P), st3_or) <= TOL["f32"]


@pytest.mark.parametrize("algo", ["scan", "mfma"])
def test_fused_qkv_buffer_and_strided_output(algo):
    """q, k, v as thirds of one [B][L][3D] buffer; y written into a wider buffer."""
    torch = require_gpu()
    rng = np.random.default_rng(5)
    B, D, H, d, L = 2, 256, 2, 16, 300
    params = _rand_params(rng, H, d, 0.8, 0.999)
    qkv_np = _rand_act(rng, (B, L, 3 * D), "bf16")
    qkv = to_dev(qkv_np, "bf16")
    op = _op(params, B, D, "bf16")
    ybuf = torch.full((B, L, D + 64), 3.0, dtype=torch.bfloat16, device="cuda")
    log("fused qkv")
    op.prefill(qkv[:, :, :D], qkv[:, :, D:2 * D], qkv[:, :, 2 * D:], y=ybuf[:, :, :D], chunk=64, algo=algo)
    torch.cuda.synchronize()
    y_or, _ = oracle.modal_scan(params, np.ascontiguousarray(qkv_np[:, :, :D]),
                                np.ascontiguousarray(qkv_np[:, :, D:2 * D]),
                                np.ascontiguousarray(qkv_np[:, :, 2 * D:]))
    assert rel_err(to_np64(ybuf[:, :, :D]), y_or) <= TOL["bf16"]
    assert torch.all(ybuf[:, :, D:] == 3.0).item()


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("B,D,H,L,tile", [(2, 128, 2, 200, 64), (16, 2048, 16, 130, 128)])
def test_odd_row_stride_scalar_paths(act, B, D, H, L, tile):
    """An odd row stride forces the scalar (unvectorised) load paths: on a
    matrix-core plan cut into chunks, the state-only pass with element loads
    and the lane scan from its carries, at both channel tiles (a float32
    thread's two 4-channel halves sit half a tile apart)."""
    torch = require_gpu()
    rng = np.random.default_rng(6 + tile)
    d = 8
    params = _rand_params(rng, H, d)
    ld = D + 1
    big = [_rand_act(rng, (B, L, ld), act) for _ in range(3)]
    dev = [to_dev(a, act) for a in big]
    op = _op(params, B, D, act)
    plan = op.plan(L, chunk=64)
    assert plan["algo"] == "mfma" and plan["channel_tile"] == tile
    log(f"odd stride {act} tile {tile}")
    y, st = op.prefill(*(t[:, :, :D] for t in dev), chunk=64)
    torch.cuda.synchronize()
    y_or, st_or = oracle.modal_scan(params, *(np.ascontiguousarray(a[:, :, :D]) for a in big))
    assert rel_err(to_np64(y), y_or) <= TOL[act]
    assert rel_err(state_for_channels(st, np.arange(D), D // H), st_or) <= TOL[act]


@pytest.mark.parametrize("d,act", [(8, "f32"), (16, "f32"), (16, "bf16"), (32, "bf16"), (32, "f32")])
def test_matrix_core_128_channel_tiles(d, act):
    """Batch x heads large enough for 128-channel, 8-wave workgroups; whole
    prompt, and cut into 64-step chunks (state-only pass at that tile).
    float32 at d = 32 keeps 64-channel tiles: its three bfloat16 parts per
    operand do not fit a 128-channel tile in the LDS."""
    torch = require_gpu()
    rng = np.random.default_rng(40 + d)
    B, D, H, L = 16, 2048, 16, 200
    params = _rand_params(rng, H, d, 0.8, 0.999)
    q_, k_, v_ = (_rand_act(rng, (B, L, D), act) for _ in range(3))
    q, k, v = (to_dev(a, act) for a in (q_, k_, v_))
    op = _op(params, B, D, act)
    y_or, st_or = oracle.modal_scan(params, q_, k_, v_)
    for chunk in (0, 64):
        plan = op.plan(L, chunk=chunk)
        assert plan["algo"] == "mfma" and plan["channel_tile"] == (64 if (d, act) == (32, "f32") else 128)
        log(f"128-channel tiles d={d} {act} chunk={chunk} plan={plan}")
        y, st = op.prefill(q, k, v, chunk=chunk)
        torch.cuda.synchronize()
        e_y = rel_err(to_np64(y), y_or)
        e_s = rel_err(state_for_channels(st, np.arange(D), D // H), st_or)
        print(f"128-channel d={d} chunk={chunk}: y {e_y:.2e} state {e_s:.2e}")
        assert e_y <= TOL[act] and e_s <= TOL[act]


def test_long_prompt_single_batch_row_chunked():
    """One batch row of the 64k-token workload: too few channel tiles for the
    GPU, so the prompt is cut into chunks (state-only pass, carry scan, full
    pass).  Sampled channels against the oracle."""
    torch = require_gpu()
    cfg = get_config(4)
    params = modal_params(cfg)
    inp = prompt_inputs(cfg, batches=[1])
    op = _op(params, 1, cfg.D, cfg.act)
    plan = op.plan(cfg.L)
    assert plan["algo"] == "mfma" and plan["n_chunks"] > 1
    q, k, v = (to_dev(inp[n], cfg.act) for n in "qkv")
    log(f"single-row 64k prompt plan={plan}")
    y, st = op.prefill(q, k, v)
    torch.cuda.synchronize()
    del q, k, v
    chans = _sample_channels(cfg, 28, 404)
    y_or, st_or = oracle.modal_scan(params, inp["q"], inp["k"], inp["v"], channels=chans)
    del inp
    ct = torch.as_tensor(chans, device="cuda")
    e_y = rel_err(to_np64(y.index_select(2, ct)), y_or)
    e_s = rel_err(state_for_channels(st, chans, cfg.P), st_or)
    print(f"single-row 64k prompt: y rel err {e_y:.3e}, state rel err {e_s:.3e}")
    assert e_y <= TOL[cfg.act] and e_s <= TOL[cfg.act]


def test_impulse_response_matches_filter():
    torch = require_gpu()
    cfg = get_config(2)
    params = modal_params(cfg)
    B, D, L = 1, cfg.D, 1000
    q = torch.ones((B, L, D), dtype=torch.float32, device="cuda")
    k = torch.zeros_like(q)
    k[:, 0, :] = 1
    op = _op(params, B, D, "f32")
    log("impulse response")
    y, _ = op.prefill(q, k, q, chunk=128)
    h = op.filter(L)
    torch.cuda.synchronize()
    hy = to_np64(y[0]).T.reshape(cfg.H, cfg.P, L)
    ref = oracle.filter_taps(params, L)
    assert rel_err(hy, np.broadcast_to(ref[:, None, :], hy.shape)) <= 1e-4
    assert rel_err(to_np64(h), ref) <= 1e-4


def test_bitwise_determinism():
    torch = require_gpu()
    cfg = get_config(2)
    params = modal_params(cfg)
    inp = prompt_inputs(cfg, batches=[0, 1, 2, 3])
    op = _op(params, 4, cfg.D, cfg.act)
    q, k, v = (to_dev(inp[n], cfg.act) for n in "qkv")
    log("determinism")
    y1, s1 = op.prefill(q, k, v)
    y2, s2 = op.prefill(q, k, v)
    y3, s3 = op.prefill(q, k, v, algo="scan")
    y4, s4 = op.prefill(q, k, v, algo="scan")
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)
    assert torch.equal(y3, y4) and torch.equal(s3, s4)
    a1 = op.decode_step(q[:, 0], k[:, 0], v[:, 0], s1)
    a2 = op.decode_step(q[:, 0], k[:, 0], v[:, 0], s2)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(s1, s2)


# ------------------------------------------------------------------ limits and degenerate filters


@pytest.mark.parametrize("shape", [
    # (B, D, H, d, L, act): the largest batch the launch grids take, with the
    # largest mode count (lane scan) and the largest matrix-core mode count
    (65535, 16, 2, 64, 70, "f32"),
    (65535, 64, 1, 32, 70, "bf16"),
])
def test_maximum_batch_and_modes(shape):
    torch = require_gpu()
    B, D, H, d, L, act = shape
    rng = np.random.default_rng(B + d)
    params = _rand_params(rng, H, d, 0.5, 0.999)
    op = _op(params, B, D, act)
    log(f"maximum batch {shape} plan={op.plan(L)}")
    dt = np.float32
    gen = lambda: rng.standard_normal((B, L, D), dtype=dt)
    q_, k_, v_ = gen(), gen(), gen()
    if act == "bf16":
        from workloads import round_to_bf16_bits
        q_, k_, v_ = (round_to_bf16_bits(a) for a in (q_, k_, v_))
    y, st = op.prefill(*(to_dev(a, act) for a in (q_, k_, v_)))
    qd, kd, vd = (_rand_act(rng, (2, B, D), act) for _ in range(3))
    ys = [op.decode_step(to_dev(qd[s], act), to_dev(kd[s], act), to_dev(vd[s], act), st) for s in range(2)]
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4097, 33333, B - 1])
    sub = lambda a: np.ascontiguousarray(a[rows])
    y_or, st_or = oracle.modal_scan(params, sub(q_), sub(k_), sub(v_))
    rt = torch.as_tensor(rows, device="cuda")
    assert rel_err(to_np64(y.index_select(0, rt)), y_or) <= TOL[act]
    yd_or, st2_or = oracle.modal_scan(params, np.ascontiguousarray(qd[:, rows]), np.ascontiguousarray(kd[:, rows]),
                                      np.ascontiguousarray(vd[:, rows]), state=st_or, batch_axis=1, time_axis=0)
    yd = np.stack([to_np64(t.index_select(0, rt)) for t in ys], 1)
    assert rel_err(yd, yd_or) <= TOL[act]
    assert rel_err(state_for_channels(st.index_select(0, rt), np.arange(D), D // H), st2_or) <= TOL[act]


@pytest.mark.parametrize("algo", ["scan", "mfma"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_degenerate_poles(algo, act):
    """Poles at 0 (the filter stops after one tap past D), on the positive and
    negative real axis, next to the unit circle (|lambda| = 1 - 1e-5) and tiny
    (1e-3), one kind per head; whole prompt and chunked, then decode steps."""
    torch = require_gpu()
    rng = np.random.default_rng(77)
    B, D, H, d, L = 2, 320, 5, 8, 300
    r = np.zeros((H, d))
    th = np.zeros((H, d))
    r[1], th[1] = rng.uniform(0.5, 0.999, d), 0.0
    r[2], th[2] = rng.uniform(0.5, 0.999, d), np.pi
    r[3], th[3] = 1.0 - 1e-5, rng.uniform(0, np.pi, d)
    r[4], th[4] = 1e-3, rng.uniform(0, np.pi, d)
    poles = np.stack([r * np.cos(th), r * np.sin(th)], -1).astype(np.float32)
    res = (rng.standard_normal((H, d, 2)) / np.sqrt(2 * d)).astype(np.float32)
    params = ModalParams(poles, res, rng.standard_normal(H).astype(np.float32))
    q_, k_, v_ = (_rand_act(rng, (B, L, D), act) for _ in range(3))
    op = _op(params, B, D, act)
    y_or, st_or = oracle.modal_scan(params, q_, k_, v_)
    for chunk in (0, 64):
        log(f"degenerate poles algo={algo} act={act} chunk={chunk}")
        y, st = op.prefill(*(to_dev(a, act) for a in (q_, k_, v_)), chunk=chunk, algo=algo)
        torch.cuda.synchronize()
        assert rel_err(to_np64(y), y_or) <= TOL[act]
        assert rel_err(state_for_channels(st, np.arange(D), D // H), st_or) <= TOL[act]
    qd, kd, vd = (_rand_act(rng, (3, B, D), act) for _ in range(3))
    ys = [op.decode_step(to_dev(qd[s], act), to_dev(kd[s], act), to_dev(vd[s], act), st) for s in range(3)]
    torch.cuda.synchronize()
    yd_or, _ = oracle.modal_scan(params, qd, kd, vd, state=st_or, batch_axis=1, time_axis=0)
    assert rel_err(np.stack([to_np64(t) for t in ys], 1), yd_or) <= TOL[act]
    # the filter of the zero-pole head: D, then Re sum R, then zeros
    h = to_np64(op.filter(L))
    assert h[0, 0] == np.float32(params.skip[0])
    assert abs(h[0, 1] - float(res[0, :, 0].astype(np.float64).sum())) <= 1e-6
    assert np.all(h[0, 2:] == 0.0)


def test_state_checkpoint_roundtrip(tmp_path):
    """The modal state is the generation checkpoint: prefill L steps, save the
    state to a host file, restore it into fresh device memory, decode S steps;
    the outputs and final state match one prefill over all L + S steps."""
    torch = require_gpu()
    cfg = get_config(2)
    params = modal_params(cfg)
    B, L, S = 4, 300, 20
    rng = np.random.default_rng(91)
    q_, k_, v_ = (_rand_act(rng, (B, L + S, cfg.D), "bf16") for _ in range(3))
    op = _op(params, B, cfg.D, "bf16")
    q, k, v = (to_dev(a, "bf16") for a in (q_, k_, v_))
    log("checkpoint: prefill, save")
    _, st = op.prefill(*(t[:, :L].contiguous() for t in (q, k, v)))
    path = tmp_path / "state.npy"
    np.save(path, st.cpu().numpy())
    del st
    torch.cuda.synchronize()
    st2 = torch.from_numpy(np.load(path)).cuda()
    log("checkpoint: restore, decode")
    ys = [op.decode_step(q[:, L + s].contiguous(), k[:, L + s].contiguous(), v[:, L + s].contiguous(), st2)
          for s in range(S)]
    y_all, st_all = op.prefill(q, k, v)
    torch.cuda.synchronize()
    yd = np.stack([to_np64(t) for t in ys], 1)
    y_or, st_or = oracle.modal_scan(params, q_, k_, v_)
    assert rel_err(yd, y_or[:, L:]) <= TOL["bf16"]
    assert rel_err(yd, to_np64(y_all[:, L:])) <= TOL["bf16"]
    st_or_gpu = state_for_channels(st2, np.arange(cfg.D), cfg.P)
    assert rel_err(st_or_gpu, st_or) <= TOL["f32"]
    assert rel_err(state_for_channels(st_all, np.arange(cfg.D), cfg.P), st_or) <= TOL["f32"]
