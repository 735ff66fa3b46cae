"""GPU parity of the explicit-filter (non-distilled) decode baseline against the
oracle's explicit convolution, on the same seeded inputs and the same float32
taps (computed by the oracle, rounded to float32).  The cache keeps u in the
activation dtype on both sides."""

import numpy as np
import pytest

import oracle
from _gpu_common import TOL, log, rel_err, require_gpu, to_dev, to_np64
from distilled_modal_ssm_amd import binding as hb
from workloads import decode_inputs, get_config, modal_params, prompt_inputs

pytestmark = pytest.mark.gpu


def _rand(rng, shape, act):
    from workloads import round_to_bf16_bits
    x = rng.standard_normal(shape)
    return round_to_bf16_bits(x) if act == "bf16" else x.astype(np.float32)


def _params(rng, H, d):
    from workloads import ModalParams
    r = rng.uniform(0.8, 0.999, (H, d))
    th = rng.uniform(0, np.pi, (H, d))
    poles = np.stack([r * np.cos(th), r * np.sin(th)], -1).astype(np.float32)
    res = (rng.standard_normal((H, d, 2)) / np.sqrt(2 * d)).astype(np.float32)
    return ModalParams(poles, res, rng.standard_normal(H).astype(np.float32))


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("window", [0, 1, 17, 64])
def test_fir_decode_small(act, window):
    torch = require_gpu()
    B, D, H, d, L, S = 2, 64, 4, 8, 100, 40
    rng = np.random.default_rng(100 + window + (act == "bf16"))
    params = _params(rng, H, d)
    q, k, v = (_rand(rng, (B, L + S, D), act) for _ in range(3))
    h32 = oracle.filter_taps(params, L + S).astype(np.float32)
    op = hb.ModalHyena(params.poles, params.residues, params.skip, B, D, act)
    fir = hb.FirHyena(op, L + S)
    log(f"fir small act={act} window={window}")
    Q, K, V = (to_dev(a, act) for a in (q, k, v))
    fir.fill(K[:, :L].contiguous(), V[:, :L].contiguous())
    h = torch.from_numpy(h32).cuda()
    ys = [fir.step(h, L + s, Q[:, L + s].contiguous(), K[:, L + s].contiguous(), V[:, L + s].contiguous(),
                   window=window) for s in range(S)]
    torch.cuda.synchronize()
    y_gpu = np.stack([to_np64(t) for t in ys], 1)
    y_or = oracle.fir_conv(h32.astype(np.float64), q, k, v, act, window=window, t_from=L)
    assert rel_err(y_gpu, y_or) <= TOL[act]


@pytest.mark.parametrize("window", [0, 17])
def test_fir_decode_f32_block_split(window):
    """float32 with D a multiple of the 512-channel block: a lane's two 4-channel
    halves sit 256 channels apart, here in different heads (head dim 128)."""
    torch = require_gpu()
    B, D, H, d, L, S = 2, 1024, 8, 8, 100, 10
    rng = np.random.default_rng(300 + window)
    params = _params(rng, H, d)
    q, k, v = (_rand(rng, (B, L + S, D), "f32") for _ in range(3))
    h32 = oracle.filter_taps(params, L + S).astype(np.float32)
    op = hb.ModalHyena(params.poles, params.residues, params.skip, B, D, "f32")
    fir = hb.FirHyena(op, L + S)
    log(f"fir f32 block split window={window}")
    Q, K, V = (to_dev(a, "f32") for a in (q, k, v))
    fir.fill(K[:, :L].contiguous(), V[:, :L].contiguous())
    h = torch.from_numpy(h32).cuda()
    ys = [fir.step(h, L + s, Q[:, L + s].contiguous(), K[:, L + s].contiguous(), V[:, L + s].contiguous(),
                   window=window) for s in range(S)]
    torch.cuda.synchronize()
    y_gpu = np.stack([to_np64(t) for t in ys], 1)
    y_or = oracle.fir_conv(h32.astype(np.float64), q, k, v, "f32", window=window, t_from=L)
    assert rel_err(y_gpu, y_or) <= TOL["f32"]


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_fir_non_temporal_loads(act):
    """Both cache-load forms at a small size (the library picks non-temporal
    loads only for windows beyond 256 MB): each against the oracle, and the two
    bit for bit, since only the load hint differs."""
    torch = require_gpu()
    B, D, H, d, L, S = 2, 1024, 8, 8, 100, 6  # D a multiple of 512 for the float32 block split
    rng = np.random.default_rng(500 + (act == "bf16"))
    params = _params(rng, H, d)
    q, k, v = (_rand(rng, (B, L + S, D), act) for _ in range(3))
    h32 = oracle.filter_taps(params, L + S).astype(np.float32)
    op = hb.ModalHyena(params.poles, params.residues, params.skip, B, D, act)
    Q, K, V = (to_dev(a, act) for a in (q, k, v))
    h = torch.from_numpy(h32).cuda()
    y_or = oracle.fir_conv(h32.astype(np.float64), q, k, v, act, window=0, t_from=L)
    outs = {}
    for loads in (hb.HM_FIR_LOADS_PLAIN, hb.HM_FIR_LOADS_NONTEMPORAL):
        log(f"fir act={act} loads={loads}")
        fir = hb.FirHyena(op, L + S)
        fir.fill(K[:, :L].contiguous(), V[:, :L].contiguous())
        ys = [fir.step(h, L + s, Q[:, L + s].contiguous(), K[:, L + s].contiguous(), V[:, L + s].contiguous(),
                       loads=loads) for s in range(S)]
        torch.cuda.synchronize()
        outs[loads] = np.stack([to_np64(t) for t in ys], 1)
        assert rel_err(outs[loads], y_or) <= TOL[act]
    assert np.array_equal(outs[hb.HM_FIR_LOADS_PLAIN], outs[hb.HM_FIR_LOADS_NONTEMPORAL])


def test_fir_full_window_matches_modal_decode():
    """Over every past step, the explicit filter and the distilled recurrence are
    the same operator: the two GPU decode paths agree (float32 activations)."""
    torch = require_gpu()
    B, D, H, d, L, S = 2, 128, 2, 16, 300, 20
    rng = np.random.default_rng(7)
    params = _params(rng, H, d)
    q, k, v = (_rand(rng, (B, L + S, D), "f32") for _ in range(3))
    op = hb.ModalHyena(params.poles, params.residues, params.skip, B, D, "f32")
    fir = hb.FirHyena(op, L + S)
    Q, K, V = (to_dev(a, "f32") for a in (q, k, v))
    y_p, st = op.prefill(Q[:, :L].contiguous(), K[:, :L].contiguous(), V[:, :L].contiguous())
    fir.fill(K[:, :L].contiguous(), V[:, :L].contiguous())
    h = op.filter(L + S)
    y_m, y_f = [], []
    for s in range(S):
        qs, ks, vs = (X[:, L + s].contiguous() for X in (Q, K, V))
        y_m.append(op.decode_step(qs, ks, vs, st))
        y_f.append(fir.step(h, L + s, qs, ks, vs))
    torch.cuda.synchronize()
    a = np.stack([to_np64(t) for t in y_m], 1)
    b = np.stack([to_np64(t) for t in y_f], 1)
    assert rel_err(b, a) <= 1e-4


@pytest.mark.parametrize("window", [0, 256])
def test_fir_width2048_full_size_sampled(window):
    """The width-2048 bf16 workload at full size: prompt rows cached, all 512
    generated steps through the explicit filter, sampled channels checked."""
    torch = require_gpu()
    cfg = get_config(2)
    params = modal_params(cfg)
    inp, dec = prompt_inputs(cfg), decode_inputs(cfg)
    op = hb.ModalHyena(params.poles, params.residues, params.skip, cfg.B, cfg.D, cfg.act)
    fir = hb.FirHyena(op, cfg.L + cfg.S)
    K, V = to_dev(inp["k"], "bf16"), to_dev(inp["v"], "bf16")
    fir.fill(K, V)
    del K, V
    h32 = oracle.filter_taps(params, cfg.L + cfg.S).astype(np.float32)
    h = torch.from_numpy(h32).cuda()
    dq, dk, dv = (to_dev(dec[n], "bf16") for n in "qkv")
    ys = torch.empty((cfg.S, cfg.B, cfg.D), dtype=torch.bfloat16, device="cuda")
    log(f"fir width2048 window={window}")
    for s in range(cfg.S):
        fir.step(h, cfg.L + s, dq[s], dk[s], dv[s], window=window, y=ys[s])
    torch.cuda.synchronize()
    chans = np.array([0, 5, 127, 128, 1000, 2047])
    full = {n: np.concatenate([inp[n][:, :, chans], dec[n][:, :, chans].transpose(1, 0, 2)], 1) for n in "qkv"}
    y_or = oracle.fir_conv(h32.astype(np.float64), full["q"], full["k"], full["v"], "bf16", window=window,
                           t_from=cfg.L, heads=chans // cfg.P)
    y_gpu = to_np64(ys[:, :, torch.as_tensor(chans, device="cuda")]).transpose(1, 0, 2)
    err = rel_err(y_gpu, y_or)
    print(f"fir width2048 window={window}: rel err {err:.2e}")
    assert err <= TOL["bf16"]
