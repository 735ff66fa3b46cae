"""The allocation-free prefill (hyena_modal_prefill_noalloc) against the
workspace form it shares its kernels with, through the C ABI.

Two calls in a row on one GPU share the library's scratch array: the first
a chunked matrix-core plan continuing a prompt from a given state (tables and
chunk carries in the scratch), the second a smaller chunked lane-scan plan.
Each must equal hyena_modal_prefill_ex with a caller-owned workspace bit for
bit (same kernels, same plan) and the float64 oracle within the activation
dtype's tolerance.  Then the first shape again, after the smaller call has
overwritten the scratch.
"""

import numpy as np
import pytest

import oracle
from _gpu_common import TOL, log, rel_err, require_gpu, state_for_channels, state_to_gpu_layout, to_dev, to_np64
from distilled_modal_ssm_amd import ModalHyena
from distilled_modal_ssm_amd import binding as hb
from workloads.generate import ModalParams

pytestmark = pytest.mark.gpu

CASES = [
    # (B, D, H, d, L, act, chunk, algo, with state_in)
    (2, 512, 4, 16, 1000, "bf16", 256, "mfma", True),
    (1, 256, 2, 8, 300, "f32", 64, "scan", False),
    (2, 512, 4, 16, 1000, "bf16", 256, "mfma", True),
]


def _params(rng, H, d):
    r = rng.uniform(0.6, 0.99, (H, d))
    th = rng.uniform(0, np.pi, (H, d))
    poles = np.stack([r * np.cos(th), r * np.sin(th)], -1).astype(np.float32)
    res = (rng.standard_normal((H, d, 2)) / np.sqrt(2 * d)).astype(np.float32)
    return ModalParams(poles, res, rng.standard_normal(H).astype(np.float32))


def _act(rng, shape, act):
    from workloads import round_to_bf16_bits
    x = rng.standard_normal(shape)
    return round_to_bf16_bits(x) if act == "bf16" else x.astype(np.float32)


def _run_case(torch, i, case):
    B, D, H, d, L, act, chunk, algo, with_state = case
    rng = np.random.default_rng(700 + B * 10 + d)
    params = _params(rng, H, d)
    q_, k_, v_ = (_act(rng, (B, L, D), act) for _ in range(3))
    st0 = rng.standard_normal((B, D, d, 2)) if with_state else None
    op = ModalHyena(params.poles, params.residues, params.skip, B, D, act)
    q, k, v = (to_dev(a, act) for a in (q_, k_, v_))
    st_in = torch.from_numpy(state_to_gpu_layout(st0, H, D // H)).cuda() if with_state else None
    y_ref, st_ref = torch.empty_like(q), op.new_state()
    y_na, st_na = torch.empty_like(q), op.new_state()
    y_na.fill_(7.0)
    st_na.fill_(7.0)
    n = hb.hyena_modal_prefill_workspace(op.desc, L, chunk=chunk, algo=algo)
    assert 0 < n <= hb.HM_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    log(f"no-alloc call {i}: {case}, workspace {n} B")
    hb.hyena_modal_prefill(op.desc, L, q, k, v, D, y_ref, D, st_in, st_ref, ws, n, chunk=chunk, algo=algo)
    hb.hyena_modal_prefill_noalloc(op.desc, L, q, k, v, D, y_na, D, st_in, st_na, chunk=chunk, algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ref), f"call {i}: y differs from the workspace form"
    assert torch.equal(st_na, st_ref), f"call {i}: state differs from the workspace form"
    y_or, st_or = oracle.modal_scan(params, q_, k_, v_, state=st0)
    assert rel_err(to_np64(y_na), y_or) <= TOL[act]
    assert rel_err(state_for_channels(st_na, np.arange(D), D // H), st_or) <= TOL[act]


def test_noalloc_prefill_matches_workspace_form_on_consecutive_calls():
    torch = require_gpu()
    hb.load()
    for i, case in enumerate(CASES):
        _run_case(torch, i, case)
