"""Pins of the float64 oracle against facts fixed outside the oracle.

Each test checks the oracle against something it does not compute itself:
hand-derived worked examples, the direct (brute-force) causal convolution with
the closed-form filter, the one-mode geometric-series closed form, Horner
evaluation (numpy.polyval), FFT convolution (numpy.fft), and structural facts
(impulse response, composition, linearity, time shift, semiseparable rank,
stability bound).  Mistakes these catch include: a flipped sign of the
imaginary part in Re(R x), conjugated poles, update-before-read ordering
(h shifted by one tap), a dropped skip term D, a wrong channel-to-head map,
wrong strides, a wrong state layout or exponent in the final state.
"""

import os

import numpy as np
import pytest

from workloads import get_config, modal_params, prompt_inputs, decode_inputs
from workloads.generate import ModalParams

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples_d1.txt")


def _random_params(rng, H, d, r_lo=0.5, r_hi=0.99):
    r = rng.uniform(r_lo, r_hi, (H, d))
    th = rng.uniform(0, np.pi, (H, d))
    poles = np.stack([r * np.cos(th), r * np.sin(th)], -1).astype(np.float32)
    res = (rng.standard_normal((H, d, 2)) / np.sqrt(2 * d)).astype(np.float32)
    skip = rng.standard_normal(H).astype(np.float32)
    return ModalParams(poles, res, skip)


def _closed_form_h(params, T):
    """h[g][t] via numpy complex powers (np.power), independent of the oracle."""
    lam = params.poles[..., 0].astype(np.float64) + 1j * params.poles[..., 1]
    R = params.residues[..., 0].astype(np.float64) + 1j * params.residues[..., 1]
    t = np.arange(T - 1)
    pw = np.power(lam[:, :, None], t[None, None, :])          # [H][d][T-1]
    h = np.empty((params.H, T))
    h[:, 0] = params.skip
    h[:, 1:] = np.real(np.sum(R[:, :, None] * pw, axis=1))
    return h


def _direct_conv(params, q, k, v):
    """y = diag(q) T_h diag(k) v per channel with an explicit causal Toeplitz T_h."""
    B, T, D = q.shape
    P = D // params.H
    h = _closed_form_h(params, T)
    y = np.zeros((B, T, D))
    idx = np.arange(T)[:, None] - np.arange(T)[None, :]
    for g in range(params.H):
        Th = np.where(idx >= 0, h[g][np.clip(idx, 0, None)], 0.0)
        for c in range(g * P, (g + 1) * P):
            for b in range(B):
                u = k[b, :, c].astype(np.float64) * v[b, :, c]
                y[b, :, c] = q[b, :, c] * (Th @ u)
    return y


def _read_golden():
    blocks, cur = [], None
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "name":
            cur = {"name": vals[0]}
            blocks.append(cur)
        elif key == "lambda":
            cur["lambda"] = (float(vals[0]), float(vals[1]))
            cur["R"] = (float(vals[3]), float(vals[4]))
            cur["D"] = float(vals[6])
        else:
            cur[key] = np.array([float(x) for x in vals])
    return blocks


# ------------------------------------------------------------------ worked examples


@pytest.mark.parametrize("ex", _read_golden(), ids=lambda e: e["name"])
def test_hand_worked_examples(oracle_lib, ex):
    params = ModalParams(np.array([[ex["lambda"]]], np.float32), np.array([[ex["R"]]], np.float32),
                         np.array([ex["D"]], np.float32))
    T = ex["q"].size
    q, k, v = (ex[n].astype(np.float32).reshape(1, T, 1) for n in ("q", "k", "v"))
    y, st = oracle_lib.modal_scan(params, q, k, v)
    assert np.array_equal(y.ravel(), ex["y"])
    assert np.array_equal(st.ravel(), ex["x"])
    h = oracle_lib.filter_taps(params, T)
    assert np.array_equal(h.ravel(), ex["h"])


# ------------------------------------------------------------------ brute force


@pytest.mark.parametrize("d", [1, 3, 8])
def test_recurrence_equals_direct_convolution(oracle_lib, d):
    rng = np.random.default_rng(7 + d)
    B, D, H, T = 2, 8, 2, 160
    params = _random_params(rng, H, d)
    q, k, v = (rng.standard_normal((B, T, D)).astype(np.float32) for _ in range(3))
    y, _ = oracle_lib.modal_scan(params, q, k, v)
    ref = _direct_conv(params, q, k, v)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_bf16_inputs_and_strided_layout(oracle_lib):
    """bf16 bit patterns and a [S][B][D] (time-major) layout give the same numbers."""
    from workloads import bf16_bits_to_f32, round_to_bf16_bits
    rng = np.random.default_rng(3)
    B, D, H, T, d = 3, 12, 3, 40, 4
    params = _random_params(rng, H, d)
    raw = [round_to_bf16_bits(rng.standard_normal((B, T, D))) for _ in range(3)]
    f32 = [bf16_bits_to_f32(a) for a in raw]
    y_bits, st_bits = oracle_lib.modal_scan(params, *raw)
    ref = _direct_conv(params, *f32)
    assert np.max(np.abs(y_bits - ref)) <= 1e-12 * np.max(np.abs(ref))
    tm = [np.ascontiguousarray(a.transpose(1, 0, 2)) for a in raw]
    y_tm, st_tm = oracle_lib.modal_scan(params, *tm, batch_axis=1, time_axis=0)
    assert np.array_equal(y_tm, y_bits) and np.array_equal(st_tm, st_bits)


def test_channel_subset_matches_full(oracle_lib):
    rng = np.random.default_rng(11)
    B, D, H, T, d = 2, 16, 4, 50, 3
    params = _random_params(rng, H, d)
    q, k, v = (rng.standard_normal((B, T, D)).astype(np.float32) for _ in range(3))
    y, st = oracle_lib.modal_scan(params, q, k, v)
    sel = np.array([15, 0, 7, 8])
    ys, sts = oracle_lib.modal_scan(params, q, k, v, channels=sel)
    assert np.array_equal(ys, y[:, :, sel]) and np.array_equal(sts, st[:, sel])


# ------------------------------------------------------------------ closed forms


def test_one_mode_geometric_series(oracle_lib):
    """d = 1, q = 1, u = 1: x_t = (1 - lam^t)/(1 - lam), y_t = D + Re(R x_t)."""
    lam = np.float32(0.93) * np.exp(1j * 0.7)
    params = ModalParams(np.array([[[lam.real, lam.imag]]], np.float32),
                         np.array([[[0.6, -1.3]]], np.float32), np.array([0.25], np.float32))
    T = 300
    ones = np.ones((1, T, 1), np.float32)
    y, st = oracle_lib.modal_scan(params, ones, ones, ones)
    lam64 = complex(float(params.poles[0, 0, 0]), float(params.poles[0, 0, 1]))
    R = complex(float(params.residues[0, 0, 0]), float(params.residues[0, 0, 1]))
    t = np.arange(T)
    xt = (1 - lam64 ** t) / (1 - lam64)                 # state read at step t
    expect = 0.25 + np.real(R * xt)
    assert np.max(np.abs(y.ravel() - expect)) < 1e-12
    xT = (1 - lam64 ** T) / (1 - lam64)
    assert abs(complex(st[0, 0, 0, 0], st[0, 0, 0, 1]) - xT) < 1e-12


def test_final_state_is_horner_polynomial(oracle_lib):
    """x_L,n = sum_t lam_n^(L-1-t) u_t = polyval(u, lam_n)."""
    rng = np.random.default_rng(5)
    B, D, H, T, d = 2, 6, 2, 120, 5
    params = _random_params(rng, H, d)
    q, k, v = (rng.standard_normal((B, T, D)).astype(np.float32) for _ in range(3))
    _, st = oracle_lib.modal_scan(params, q, k, v)
    P = D // H
    for b in range(B):
        for c in range(D):
            u = k[b, :, c].astype(np.float64) * v[b, :, c]
            for n in range(d):
                lam = complex(*params.poles[c // P, n].astype(np.float64))
                want = np.polyval(u, lam)
                got = complex(*st[b, c, n])
                assert abs(got - want) <= 1e-12 * max(1.0, abs(want))


def test_fft_convolution_mid_size(oracle_lib):
    """L = 4096: the recurrence equals an FFT convolution with the materialised h."""
    cfg = get_config(2)
    params = modal_params(cfg)
    rng = np.random.default_rng(9)
    L, D = 4096, cfg.D
    chans = np.array([0, 130, 700, 2047])
    q = np.zeros((1, L, D), np.float32)
    k = np.zeros((1, L, D), np.float32)
    v = np.zeros((1, L, D), np.float32)
    for a in (q, k, v):
        a[0][:, chans] = rng.standard_normal((L, chans.size))
    y, _ = oracle_lib.modal_scan(params, q, k, v, channels=chans)
    h = oracle_lib.filter_taps(params, L)
    for i, c in enumerate(chans):
        u = k[0, :, c].astype(np.float64) * v[0, :, c]
        conv = np.fft.irfft(np.fft.rfft(h[c // cfg.P], 2 * L) * np.fft.rfft(u, 2 * L), 2 * L)[:L]
        ref = q[0, :, c] * conv
        assert np.max(np.abs(y[0, :, i] - ref)) <= 1e-10 * np.max(np.abs(ref))


# ------------------------------------------------------------------ structure


def test_impulse_response_is_filter(oracle_lib):
    rng = np.random.default_rng(2)
    H, d, T = 3, 6, 500
    params = _random_params(rng, H, d, 0.8, 0.999)
    D = H * 2
    q = np.ones((1, T, D), np.float32)
    k = np.zeros((1, T, D), np.float32)
    k[0, 0, :] = 1
    y, _ = oracle_lib.modal_scan(params, q, k, q)
    h = oracle_lib.filter_taps(params, T)
    for c in range(D):
        assert np.max(np.abs(y[0, :, c] - h[c // 2])) <= 1e-13 * np.max(np.abs(h))
    ref = _closed_form_h(params, T)
    assert np.max(np.abs(h - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_prefill_then_decode_equals_one_pass(oracle_lib):
    rng = np.random.default_rng(4)
    B, D, H, L, S, d = 2, 8, 2, 90, 30, 4
    params = _random_params(rng, H, d)
    q, k, v = (rng.standard_normal((B, L + S, D)).astype(np.float32) for _ in range(3))
    y_all, st_all = oracle_lib.modal_scan(params, q, k, v)
    y_p, st_p = oracle_lib.modal_scan(params, q[:, :L], k[:, :L], v[:, :L])
    st = st_p
    for s in range(S):
        sl = slice(L + s, L + s + 1)
        y_s, st = oracle_lib.modal_scan(params, q[:, sl], k[:, sl], v[:, sl], state=st)
        assert np.array_equal(y_s[:, 0], y_all[:, L + s])
    assert np.array_equal(y_p, y_all[:, :L])
    assert np.array_equal(st, st_all)


def test_linearity_and_time_shift(oracle_lib):
    rng = np.random.default_rng(6)
    B, D, H, T, d, sh = 1, 4, 2, 80, 3, 17
    params = _random_params(rng, H, d)
    q, k, v1, v2 = (rng.standard_normal((B, T, D)) for _ in range(4))
    ya, _ = oracle_lib.modal_scan(params, q, k, v1)
    yb, _ = oracle_lib.modal_scan(params, q, k, v2)
    yab, _ = oracle_lib.modal_scan(params, q, k, v1 + v2)
    assert np.max(np.abs(yab - ya - yb)) <= 1e-12 * np.max(np.abs(yab))
    pad = lambda a: np.concatenate([np.zeros((B, sh, D)), a[:, :T - sh]], axis=1)
    ys, _ = oracle_lib.modal_scan(params, pad(q), pad(k), pad(v1))
    assert np.all(ys[:, :sh] == 0)
    assert np.max(np.abs(ys[:, sh:] - ya[:, :T - sh])) <= 1e-12 * np.max(np.abs(ya))


def test_toeplitz_offdiagonal_rank(oracle_lib):
    """Off-diagonal blocks of the causal Toeplitz T_h have rank <= 2d (semiseparable)."""
    rng = np.random.default_rng(8)
    H, d, T = 1, 5, 200
    params = _random_params(rng, H, d, 0.7, 0.95)
    h = oracle_lib.filter_taps(params, T)[0]
    m = 100
    blk = np.array([[h[t - s] for s in range(m)] for t in range(m, T)])
    sv = np.linalg.svd(blk, compute_uv=False)
    assert np.sum(sv > 1e-10 * sv[0]) <= 2 * d
    assert sv[2 * d - 1] > 1e-10 * sv[0]  # the bound is reached with distinct poles


def test_stability_bounds(oracle_lib):
    for i in (1, 2, 3, 4):
        cfg = get_config(i)
        p = modal_params(cfg)
        mag = np.hypot(p.poles[..., 0].astype(np.float64), p.poles[..., 1])
        assert np.all(mag < 1.0) and np.all(mag >= cfg.r_lo * (1 - 1e-6))
    cfg = get_config(1)
    p = modal_params(cfg)
    inp = prompt_inputs(cfg)
    q, k, v = inp["q"], inp["k"], inp["v"]
    _, st = oracle_lib.modal_scan(p, q, k, v)
    umax = np.max(np.abs(k.astype(np.float64) * v), axis=1)   # [B][D]
    mag = np.hypot(p.poles[..., 0].astype(np.float64), p.poles[..., 1])
    for c in range(cfg.D):
        bound = umax[:, c, None] / (1 - mag[c // cfg.P])[None, :]
        got = np.hypot(st[:, c, :, 0], st[:, c, :, 1])
        assert np.all(got <= bound * (1 + 1e-12))
    h = oracle_lib.filter_taps(p, 4000)
    assert np.max(np.abs(h[:, -100:])) < 1e-6 * np.max(np.abs(h[:, 1:10]))


def test_workload1_full_run_is_finite(oracle_lib):
    cfg = get_config(1)
    p = modal_params(cfg)
    inp = prompt_inputs(cfg)
    dec = decode_inputs(cfg)
    y, st = oracle_lib.modal_scan(p, inp["q"], inp["k"], inp["v"])
    yd, st2 = oracle_lib.modal_scan(p, dec["q"], dec["k"], dec["v"], state=st,
                                    batch_axis=1, time_axis=0)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(yd)) and np.all(np.isfinite(st2))
    assert yd.shape == (cfg.B, cfg.S, cfg.D)


def test_stack_layer_matches_unrolled_definition(oracle_lib):
    """The projected layer equals rms -> in_proj -> brute-force Hyena -> out_proj."""
    rng = np.random.default_rng(12)
    D, H, d, B, L = 8, 2, 3, 2, 24
    params = _random_params(rng, H, d)
    w_in = rng.standard_normal((3 * D, D)) * 0.3
    w_out = rng.standard_normal((D, D)) * 0.3
    x = rng.standard_normal((B, L, D))
    out, _, _, _ = oracle_lib.stack_layer(params, w_in, w_out, x)
    s = 1 / np.sqrt((x ** 2).mean(-1, keepdims=True) + 1e-6)
    qkv = np.einsum("btk,nk->btn", x, w_in) * s
    y = _direct_conv(params, qkv[..., :D], qkv[..., D:2 * D], qkv[..., 2 * D:])
    ref = np.einsum("btk,nk->btn", y, w_out)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_stack_layer_generated_steps_match_unrolled_definition(oracle_lib):
    """The generated-step leg of the projected layer: S steps fed one at a time
    after an L-token prompt equal the unrolled definition over one sequence of
    L + S tokens (rms -> in_proj -> brute-force causal convolution with the
    closed-form filter -> out_proj), and the final state equals the Vandermonde
    sum over all L + S inputs.  B != S and D != 3D, so a transposed [S][B][D]
    output, a state not carried from the prompt, or steps projected without the
    normalisation all change the result."""
    rng = np.random.default_rng(13)
    D, H, d, B, L, S = 8, 2, 3, 2, 20, 5
    params = _random_params(rng, H, d, 0.6, 0.97)
    w_in = rng.standard_normal((3 * D, D)) * 0.3
    w_out = rng.standard_normal((D, D)) * 0.3
    x_all = rng.standard_normal((B, L + S, D)) * rng.uniform(0.5, 2.0, (B, L + S, 1))
    x_prompt = np.ascontiguousarray(x_all[:, :L])
    x_steps = np.ascontiguousarray(x_all[:, L:].transpose(1, 0, 2))          # [S][B][D]
    out_p, out_s, st_p, st_f = oracle_lib.stack_layer(params, w_in, w_out, x_prompt, x_steps)
    s = 1 / np.sqrt((x_all ** 2).mean(-1, keepdims=True) + 1e-6)
    qkv = np.einsum("btk,nk->btn", x_all, w_in) * s
    q, k, v = qkv[..., :D], qkv[..., D:2 * D], qkv[..., 2 * D:]
    ref = np.einsum("btk,nk->btn", _direct_conv(params, q, k, v), w_out)   # [B][L+S][D]
    scale = np.max(np.abs(ref))
    assert out_s.shape == (S, B, D)
    assert np.max(np.abs(out_p - ref[:, :L])) <= 1e-12 * scale
    assert np.max(np.abs(out_s - ref[:, L:].transpose(1, 0, 2))) <= 1e-12 * scale
    # states: x_n after T inputs = sum_t lambda_n^(T-1-t) u_t, evaluated directly
    lam = params.poles[..., 0].astype(np.float64) + 1j * params.poles[..., 1]
    u = k * v
    for T, st in ((L, st_p), (L + S, st_f)):
        expo = (T - 1 - np.arange(T))[None, :]
        for c in range(D):
            g = c // (D // H)
            ref_st = np.einsum("bt,nt->bn", u[:, :T, c], lam[g][:, None] ** expo)
            got = st[:, c, :, 0] + 1j * st[:, c, :, 1]
            assert np.max(np.abs(got - ref_st)) <= 1e-12 * np.max(np.abs(ref_st)), (T, c)


def test_rms_and_dense_special_cases():
    """Pins of the projected stack's two helpers against closed forms, not their
    own formulas: a constant row has RMS |c|; a one-hot row of width n has RMS
    |v|/sqrt(n); RMS scales with |a|; x W^T with W = identity returns x, with a
    permutation permutes columns, and a unit row e_i picks column i of W (a
    transposed W fails)."""
    import oracle
    c = np.full((1, 64), -3.0)
    assert oracle.rms_inv(c, 0.0)[0] == 1.0 / 3.0
    assert abs(oracle.rms_inv(c, 1e-6)[0] - 1.0 / np.sqrt(9.0 + 1e-6)) <= 1e-15
    onehot = np.zeros((1, 100))
    onehot[0, 17] = 5.0
    assert abs(oracle.rms_inv(onehot, 0.0)[0] - np.sqrt(100.0) / 5.0) <= 1e-14
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 40))
    assert np.allclose(oracle.rms_inv(-4.0 * x, 0.0), oracle.rms_inv(x, 0.0) / 4.0, rtol=1e-14, atol=0)
    w = rng.standard_normal((7, 40))
    assert np.array_equal(oracle.dense(x, np.eye(40)), x)
    perm = rng.permutation(40)
    assert np.array_equal(oracle.dense(x, np.eye(40)[perm]), x[:, perm])
    e = np.zeros((1, 40))
    e[0, 11] = 1.0
    assert np.array_equal(oracle.dense(e, w)[0], w[:, 11])
    assert oracle.dense(x, w).shape == (3, 7)


def test_fir_conv_full_window_equals_modal_recurrence(oracle_lib):
    """The explicit-filter form over every past step is the modal recurrence:
    float64 inputs (no cache rounding) and the float64 taps of the closed form."""
    import oracle
    rng = np.random.default_rng(21)
    B, T, D, H, d = 2, 300, 8, 2, 5
    params = _random_params(rng, H, d, 0.8, 0.999)
    q, k, v = (rng.standard_normal((B, T, D)) for _ in range(3))
    h = oracle_lib.filter_taps(params, T)
    y_fir = oracle.fir_conv(h, q, k, v, "f64")
    y_rec, _ = oracle_lib.modal_scan(params, q, k, v)
    assert np.max(np.abs(y_fir - y_rec)) <= 1e-11 * np.max(np.abs(y_rec))
    # decode-only outputs and a channel subset with explicit heads agree with the full run
    sub = np.array([1, 6])
    y_sub = oracle.fir_conv(h, q[:, :, sub], k[:, :, sub], v[:, :, sub], "f64", t_from=250,
                            heads=sub // (D // H))
    assert np.max(np.abs(y_sub - y_fir[:, 250:, sub])) <= 1e-14 * np.max(np.abs(y_rec))


def test_fir_conv_truncated_window_closed_forms():
    """W = 1 reduces to q h[0] u; an impulse u = e_0 with q = 1 returns the
    first W taps and zeros after them."""
    import oracle
    rng = np.random.default_rng(22)
    B, T, D, H = 1, 40, 4, 2
    h = rng.standard_normal((H, T))
    q, k, v = (rng.standard_normal((B, T, D)) for _ in range(3))
    heads = np.arange(D) // (D // H)
    y1 = oracle.fir_conv(h, q, k, v, "f64", window=1)
    assert np.allclose(y1, q * h[heads, 0][None, None, :] * k * v, rtol=1e-15, atol=0)
    kk = np.zeros((B, T, D))
    kk[:, 0, :] = 1.0
    for W in (1, 7, T):
        y = oracle.fir_conv(h, np.ones((B, T, D)), kk, np.ones((B, T, D)), "f64", window=W)
        expect = np.where(np.arange(T)[:, None] < W, h[heads].T[:T], 0.0)
        assert np.array_equal(y[0], expect), W


def test_fir_cache_rounding_to_bfloat16():
    """The cache keeps u in the activation dtype: (1 + 2^-7)^2 = 1 + 2^-6 + 2^-14
    rounds to 1 + 2^-6 in bfloat16 (ties-to-even elsewhere), exactly in float32."""
    import oracle
    one_p = np.uint16(0x3F81)  # 1 + 2^-7 in bfloat16
    k = np.full((1, 1, 2), one_p, dtype=np.uint16)
    h = np.array([[3.0]])
    y_bf = oracle.fir_conv(h, np.full((1, 1, 2), np.uint16(0x3F80)), k, k, "bf16")
    assert np.all(y_bf == 3.0 * (1 + 2 ** -6))
    k32 = np.full((1, 1, 2), 1 + 2 ** -7, dtype=np.float32)
    y32 = oracle.fir_conv(h, np.ones((1, 1, 2), np.float32), k32, k32, "f32")
    assert np.all(y32 == 3.0 * (1 + 2 ** -6 + 2 ** -14))
    # ties to even: 1 + 2^-8 (exactly halfway between 1 and 1 + 2^-7) rounds down to 1,
    # 1 + 3 * 2^-8 rounds up to 1 + 2^-6
    assert oracle.round_to_act(np.array([1 + 2 ** -8]), "bf16")[0] == 1.0
    assert oracle.round_to_act(np.array([1 + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6


def test_distill_gradient_matches_finite_differences(oracle_lib):
    """The analytic gradient of the filter discrepancy against central
    differences of the loss (each parameter perturbed in float64)."""
    import oracle
    rng = np.random.default_rng(31)
    H, d, L = 2, 3, 60
    params = _random_params(rng, H, d, 0.6, 0.95)
    target = rng.standard_normal((H, L)) * 0.3
    loss, g_poles, g_res, g_skip = oracle.distill_loss_grad(params, target, L)
    assert np.all(loss > 0)

    def loss_at(p):
        return oracle.distill_loss_grad(p, target, L)[0]

    from workloads import ModalParams
    step = 1e-6
    for name, arr, g in (("poles", params.poles, g_poles), ("residues", params.residues, g_res)):
        for idx in [(0, 0, 0), (0, 2, 1), (1, 1, 0), (1, 2, 1)]:
            plus, minus = arr.astype(np.float64).copy(), arr.astype(np.float64).copy()
            plus[idx] += step
            minus[idx] -= step
            mk = lambda a: ModalParams(a, params.residues, params.skip) if name == "poles" else \
                ModalParams(params.poles, a, params.skip)
            fd = (loss_at(mk(plus))[idx[0]] - loss_at(mk(minus))[idx[0]]) / (2 * step)
            assert abs(fd - g[idx]) <= 1e-5 * max(1.0, abs(fd)), (name, idx, fd, g[idx])
    sp, sm = params.skip.astype(np.float64).copy(), params.skip.astype(np.float64).copy()
    sp[1] += step
    sm[1] -= step
    fd = (loss_at(ModalParams(params.poles, params.residues, sp))[1] -
          loss_at(ModalParams(params.poles, params.residues, sm))[1]) / (2 * step)
    assert abs(fd - g_skip[1]) <= 1e-6 * max(1.0, abs(fd))


def test_distill_loss_and_gradient_hand_computed():
    """A one-mode, three-tap case worked by hand: lambda = 0.5 + 0.5i,
    R = 1 + 2i, D = 1 give hhat = [D, Re R, Re(R lambda)] = [1, 1, -0.5];
    against the target [0.25, 0, 1] the residual is e = [0.75, 1, -1.5] and
    J = 0.5625 + 1 + 2.25 = 3.8125.  By hand:
      dJ/dD = 2 e0 = 1.5;
      hhat[1] = Re R,  hhat[2] = Re R Re l - Im R Im l, so
      dJ/dRe R = 2 (e1 + e2 Re l) = 0.5,   dJ/dIm R = 2 e2 (-Im l) = 1.5,
      dJ/dRe l = 2 e2 Re R = -3,           dJ/dIm l = 2 e2 (-Im R) = 6.
    Every value is a binary fraction, so float64 reproduces it exactly."""
    import oracle
    params = ModalParams(np.array([[[0.5, 0.5]]], np.float32), np.array([[[1.0, 2.0]]], np.float32),
                         np.array([1.0], np.float32))
    target = np.array([[0.25, 0.0, 1.0]])
    loss, g_poles, g_res, g_skip = oracle.distill_loss_grad(params, target, 3)
    assert loss[0] == 3.8125
    assert g_skip[0] == 1.5
    assert np.array_equal(g_res[0, 0], [0.5, 1.5])
    assert np.array_equal(g_poles[0, 0], [-3.0, 6.0])
    # two taps: lambda no longer enters, its gradient is exactly zero
    loss2, g_poles2, g_res2, _ = oracle.distill_loss_grad(params, target[:, :2], 2)
    assert loss2[0] == 0.5625 + 1.0
    assert np.array_equal(g_poles2[0, 0], [0.0, 0.0]) and np.array_equal(g_res2[0, 0], [2.0, 0.0])


def test_distill_zero_at_generating_parameters_and_hankel_rank(oracle_lib):
    """A filter generated by an order-d modal system: the objective and its
    gradient vanish at the generating parameters, and its Hankel matrix has
    rank 2d (d complex modes, real part taken)."""
    import oracle
    rng = np.random.default_rng(32)
    H, d, L = 2, 4, 400
    params = _random_params(rng, H, d, 0.7, 0.97)
    target = oracle_lib.filter_taps(params, L)
    loss, g_poles, g_res, g_skip = oracle.distill_loss_grad(params, target, L)
    assert np.all(loss == 0.0)
    assert np.all(g_poles == 0.0) and np.all(g_res == 0.0) and np.all(g_skip == 0.0)
    sv = oracle.hankel_singular_values(target[0], 60)
    assert sv[2 * d - 1] > 1e-8 * sv[0]
    assert np.all(sv[2 * d:] <= 1e-10 * sv[0])


def _modal_system(rng, H, d, r_lo, r_hi, th_lo=0.05, th_hi=np.pi - 0.05):
    r = rng.uniform(r_lo, r_hi, (H, d))
    lam = r * np.exp(1j * rng.uniform(th_lo, th_hi, (H, d)))
    R = (rng.standard_normal((H, d)) + 1j * rng.standard_normal((H, d))) / np.sqrt(2 * d)
    return lam, R, rng.standard_normal(H)


def test_modal_fit_recovers_generating_parameters(oracle_lib):
    """A filter generated by d distinct modes (float64 taps) is reproduced by
    the matrix-pencil fit: the fitted poles are the generating poles (as a set,
    upper half-plane), the residues match pole by pole, the skip is h[0].
    A fit with more modes than the filter has puts zero residue on the rest."""
    import oracle
    rng = np.random.default_rng(41)
    for H, d, L, lo, hi in ((3, 8, 400, 0.6, 0.97), (2, 16, 2048, 0.8, 0.999), (2, 1, 40, 0.5, 0.9)):
        lam, R, D = _modal_system(rng, H, d, lo, hi)
        p = ModalParams(np.stack([lam.real, lam.imag], -1), np.stack([R.real, R.imag], -1), D)
        h = oracle_lib.filter_taps(p, L)
        P, Rf, S = oracle.modal_fit_init(h, d)
        assert np.array_equal(S, D)
        for g in range(H):
            got = P[g, :, 0] + 1j * P[g, :, 1]
            order = [int(np.argmin(np.abs(got - z))) for z in lam[g]]
            assert sorted(order) == list(range(d))
            assert np.max(np.abs(got[order] - lam[g])) <= 1e-8
            Rg = Rf[g, :, 0] + 1j * Rf[g, :, 1]
            assert np.max(np.abs(Rg[order] - R[g])) <= 1e-6 * np.max(np.abs(R[g]))
        # one more mode than the filter holds: the extra one carries (almost) nothing
        P2, R2, S2 = oracle.modal_fit_init(h, d + 1)
        h2 = oracle_lib.filter_taps(ModalParams(P2, R2, S2), L)
        assert np.max(np.abs(h2 - h)) <= 1e-9 * np.max(np.abs(h))


def test_modal_fit_keeps_the_strong_modes():
    """Modal truncation: d strong modes plus d modes with residues 1e-7 times
    smaller, fitted with d modes -- the fit finds the strong poles and leaves
    an error of the order of the weak modes."""
    import oracle
    rng = np.random.default_rng(42)
    H, d, L = 2, 4, 600
    lam, R, D = _modal_system(rng, H, 2 * d, 0.7, 0.95)
    R[:, d:] *= 1e-7
    p = ModalParams(np.stack([lam.real, lam.imag], -1), np.stack([R.real, R.imag], -1), D)
    import oracle as o
    h = o.filter_taps(p, L)
    P, Rf, S = oracle.modal_fit_init(h, d)
    h_fit = o.filter_taps(ModalParams(P, Rf, S), L)
    assert np.max(np.abs(h_fit - h)) <= 1e-5 * np.max(np.abs(h))
    for g in range(H):
        got = P[g, :, 0] + 1j * P[g, :, 1]
        assert max(np.min(np.abs(got - z)) for z in lam[g, :d]) <= 1e-4
