"""The seeded input generator: determinism, rounding and block independence."""

import numpy as np

from workloads import (bf16_bits_to_f32, decode_inputs, dense_weights, get_config,
                       modal_params, prompt_inputs, round_to_bf16_bits)
from workloads.generate import BLOCK_ROWS, _rng


def test_bf16_round_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7                      # bf16 spacing in [1, 2)
    cases = {
        one: 0x3F80,
        one + ulp / 2: 0x3F80,           # tie -> even (1.0)
        one + 3 * ulp / 2: 0x3F82,       # tie -> even (1 + 2 ulp)
        one + ulp / 2 + 2.0 ** -30: 0x3F81,  # just above the tie
        -2.0: 0xC000,
        0.0: 0x0000,
        3.0e38: 0x7F62,                  # large normal
    }
    for x, bits in cases.items():
        assert int(round_to_bf16_bits(np.array([x]))[0]) == bits, x
    x = np.random.default_rng(0).standard_normal(10000)
    b = bf16_bits_to_f32(round_to_bf16_bits(x)).astype(np.float64)
    assert np.all(np.abs(b - x) <= np.abs(x) * 2.0 ** -8 * (1 + 1e-12))


def test_f32_widening_is_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    f = bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    back = (f[finite].view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(back, bits[finite])


def test_generation_is_deterministic_and_blocked():
    cfg = get_config(1)
    a = prompt_inputs(cfg)
    b = prompt_inputs(cfg)
    for n in "qkv":
        assert np.array_equal(a[n], b[n])
    # block 0 of k, batch row 0 is its own stream
    x = _rng(cfg.seed, 2, 0, 0).standard_normal((min(BLOCK_ROWS, cfg.L), cfg.D)).astype(np.float32)
    assert np.array_equal(a["k"][0, :BLOCK_ROWS], x)
    assert not np.array_equal(a["q"], a["k"])


def test_row_subset_matches_full_draw():
    cfg = get_config(2)
    sub = prompt_inputs(cfg, names=("v",), batches=[3])["v"]
    full_row = prompt_inputs(cfg, names=("v",), batches=[0, 3])["v"][1]
    assert np.array_equal(sub[0], full_row)
    d1 = decode_inputs(cfg, names=("q",), steps=[5, 6])["q"]
    d2 = decode_inputs(cfg, names=("q",), steps=[6])["q"]
    assert np.array_equal(d1[1], d2[0])


def test_params_distribution_and_rounding():
    for i in (1, 2, 3, 4, 5):
        cfg = get_config(i)
        p = modal_params(cfg)
        assert p.poles.dtype == np.float32 and p.poles.shape == (cfg.H, cfg.d, 2)
        th = np.arctan2(p.poles[..., 1], p.poles[..., 0])
        assert np.all(th >= 0) and np.all(th <= np.pi)
        r = np.hypot(p.poles[..., 0].astype(np.float64), p.poles[..., 1])
        assert np.all(r < 1) and np.all(r >= cfg.r_lo * (1 - 1e-6))
    cfg = get_config(5)
    p0, p1 = modal_params(cfg, 0), modal_params(cfg, 1)
    assert not np.array_equal(p0.poles, p1.poles)
    w_in, w_out = dense_weights(cfg, 0)
    assert w_in.shape == (3 * cfg.D, cfg.D) and w_out.shape == (cfg.D, cfg.D)
    sd = bf16_bits_to_f32(w_in).std()
    assert abs(sd - cfg.w_std) < 0.01 * cfg.w_std
