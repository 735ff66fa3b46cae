"""GPU parity of the FFT prefill (Hyena's own evaluation of the long
convolution) against the oracle's modal recurrence: the same convolution,
which the FFT path evaluates with float32 taps and float32 transforms."""

import numpy as np
import pytest

import oracle
from _gpu_common import TOL, log, rel_err, require_gpu, to_dev, to_np64
from distilled_modal_ssm_amd import binding as hb
from workloads import get_config, modal_params, prompt_inputs

pytestmark = pytest.mark.gpu


def _rand(rng, shape, act):
    from workloads import round_to_bf16_bits
    x = rng.standard_normal(shape)
    return round_to_bf16_bits(x) if act == "bf16" else x.astype(np.float32)


def _params(rng, H, d, r_lo, r_hi):
    from workloads import ModalParams
    r = rng.uniform(r_lo, r_hi, (H, d))
    th = rng.uniform(0, np.pi, (H, d))
    poles = np.stack([r * np.cos(th), r * np.sin(th)], -1).astype(np.float32)
    res = (rng.standard_normal((H, d, 2)) / np.sqrt(2 * d)).astype(np.float32)
    return ModalParams(poles, res, rng.standard_normal(H).astype(np.float32))


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("B,D,H,d,L", [
    (1, 2, 1, 1, 1), (2, 8, 2, 3, 3), (3, 64, 4, 8, 257), (1, 32, 2, 16, 2048), (2, 16, 1, 32, 4096),
    # three passes over HBM: every (NA, NB) split from N = 16384 to 262144; pair
    # blocks ragged (24 and 17 pairs per row) and straddling heads
    (2, 64, 4, 8, 4097), (1, 48, 3, 5, 9000), (1, 32, 2, 16, 20000), (1, 34, 1, 4, 40000),
    (1, 16, 2, 8, 131072)])
def test_fft_prefill_shapes(act, B, D, H, d, L):
    torch = require_gpu()
    rng = np.random.default_rng(B * 1000 + L + d)
    params = _params(rng, H, d, 0.9, 0.999)
    q, k, v = (_rand(rng, (B, L, D), act) for _ in range(3))
    op = hb.ModalHyena(params.poles, params.residues, params.skip, B, D, act)
    log(f"fft prefill B={B} D={D} H={H} d={d} L={L} act={act}")
    y = op.fft_prefill(*(to_dev(a, act) for a in (q, k, v)))
    torch.cuda.synchronize()
    y_or, _ = oracle.modal_scan(params, q, k, v)
    err = rel_err(to_np64(y), y_or)
    print(f"fft L={L} act={act}: rel err {err:.2e}")
    assert err <= TOL[act]


@pytest.mark.parametrize("ci", [2, 3, 4])
def test_fft_prefill_workload_sampled(ci):
    """Full-size width-2048, batch-256 and 64k prompts (the last through the
    three-pass transforms); sampled channels and rows."""
    torch = require_gpu()
    cfg = get_config(ci)
    params = modal_params(cfg)
    inp = prompt_inputs(cfg)
    op = hb.ModalHyena(params.poles, params.residues, params.skip, cfg.B, cfg.D, cfg.act)
    log(f"fft prefill workload {ci}")
    y = op.fft_prefill(*(to_dev(inp[n], cfg.act) for n in "qkv"))
    torch.cuda.synchronize()
    chans = np.unique([0, 1, 127, 128, 777, 2046, 2047, cfg.D - 1])
    rows = np.arange(cfg.B) if cfg.B <= 16 else np.array([0, 17, 200, 255])
    sub = {n: np.ascontiguousarray(inp[n][rows]) for n in "qkv"}
    y_or, _ = oracle.modal_scan(params, sub["q"], sub["k"], sub["v"], channels=chans)
    y_gpu = to_np64(y.index_select(2, torch.as_tensor(chans, device="cuda"))
                    .index_select(0, torch.as_tensor(rows, device="cuda")))
    err = rel_err(y_gpu, y_or)
    print(f"fft workload {ci}: rel err {err:.2e}")
    assert err <= TOL[cfg.act]
