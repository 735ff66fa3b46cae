"""Library calls captured in HIP graphs (torch's graph API over the library's
launches on the capturing stream), as the benchmark replays them.

Every graph is replayed several times, with eager work of the program and
host synchronisations between the replays, and every replay is compared bit
for bit with the same calls made eagerly: the kernels are deterministic (no
atomics, fixed summation order), so a captured launch must reproduce them
exactly."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

from _gpu_common import log, require_gpu, to_dev
from distilled_modal_ssm_amd import ModalHyena
from distilled_modal_ssm_amd import binding as hb
from workloads import dense_weights, get_config, modal_params, prompt_inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _busy(torch, ref):
    """Unrelated eager work between replays (fills, a reduction, a copy)."""
    scratch = torch.empty(1 << 22, device="cuda")
    scratch.fill_(3.0)
    s = scratch.sum()
    ref.clone()
    torch.cuda.synchronize()
    return float(s)


def _inputs(torch, cfg, B, L, S, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    dt = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    mk = lambda *shape: torch.randn(*shape, generator=g, device="cuda").to(dt)
    return [mk(B, L, cfg.D) for _ in range(3)], [mk(S, B, cfg.D) for _ in range(3)]


@pytest.mark.parametrize("ci", [2, 4])
def test_decode_graph_replays(ci):
    """S decode steps in one graph (the benchmark's form), from a prefilled state."""
    torch = require_gpu()
    cfg = get_config(ci)
    params = modal_params(cfg)
    B, L, S = cfg.B, 200, 24
    (q, k, v), (dq, dk, dv) = _inputs(torch, cfg, B, L, S, 10 + ci)
    op = ModalHyena(params.poles, params.residues, params.skip, B, cfg.D, cfg.act)
    log(f"decode graph workload {ci}: prefill")
    _, st0 = op.prefill(q, k, v)
    st_e = st0.clone()
    ys_e = torch.empty((S, B, cfg.D), dtype=op.tdtype, device="cuda")
    for s in range(S):
        op.decode_step(dq[s], dk[s], dv[s], st_e, y=ys_e[s])
    torch.cuda.synchronize()

    st_g = st0.clone()
    ys_g = torch.full_like(ys_e, 5.0)
    graph = torch.cuda.CUDAGraph()
    log(f"decode graph workload {ci}: capture")
    with torch.cuda.graph(graph):
        for s in range(S):
            op.decode_step(dq[s], dk[s], dv[s], st_g, y=ys_g[s])
    for r in range(REPLAYS):
        st_g.copy_(st0)
        ys_g.fill_(5.0)
        _busy(torch, st0)
        log(f"decode graph workload {ci}: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys_g, ys_e), f"replay {r}: outputs"
        assert torch.equal(st_g, st_e), f"replay {r}: state"


def test_prefill_graph_replays_chunked():
    """A chunked matrix-core prefill (tables, state-only pass, carry scan, full
    pass) with a state_in, captured once."""
    torch = require_gpu()
    cfg = dataclasses.replace(get_config(2), B=2)
    params = modal_params(cfg)
    L = 330
    (q, k, v), _ = _inputs(torch, cfg, cfg.B, L, 1, 31)
    op = ModalHyena(params.poles, params.residues, params.skip, cfg.B, cfg.D, cfg.act)
    plan = op.plan(L, chunk=64)
    assert plan["algo"] == "mfma" and plan["n_chunks"] == 6
    x0 = torch.randn(op.new_state().shape, device="cuda") * 0.1
    log("prefill graph: eager")
    y_e, st_e = op.prefill(q, k, v, state_in=x0, chunk=64)
    torch.cuda.synchronize()
    y_g = torch.empty_like(y_e)
    st_g = torch.empty_like(st_e)
    op.workspace(L, chunk=64)  # allocate outside the capture
    graph = torch.cuda.CUDAGraph()
    log("prefill graph: capture")
    with torch.cuda.graph(graph):
        op.prefill(q, k, v, y=y_g, state_in=x0, state_out=st_g, chunk=64)
    for r in range(REPLAYS):
        y_g.fill_(-1.0)
        st_g.fill_(-1.0)
        _busy(torch, y_e)
        log(f"prefill graph: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {r}: y"
        assert torch.equal(st_g, st_e), f"replay {r}: state"


def test_stack_token_graph_replays():
    """One generated token through a two-layer projected stack (per layer the
    gate with the RMS-fused in_proj, then out_proj with the next layer's
    prepare), captured once and replayed token after token, as the benchmark
    does."""
    torch = require_gpu()
    from distilled_modal_ssm_amd.stack import HyenaStack
    cfg = dataclasses.replace(get_config(5), layers=2, B=4, L=128)
    layers = [(modal_params(cfg, l), *dense_weights(cfg, l)) for l in range(cfg.layers)]
    st = HyenaStack(layers, cfg.B, cfg.L)
    X = torch.randn(cfg.B, cfg.L, cfg.D, device="cuda").to(torch.bfloat16)
    log("stack graph: prefill")
    out = st.prefill(X)
    st.start_generation(out)
    torch.cuda.synchronize()
    # the generation state: every layer's state buffer and, on the deferred
    # path, its u_prev and rho
    gen = list(st.states) + (list(st.u_prev) + list(st.rho) if st.deferred else [])
    x_start = st.xd.clone()
    s_start = [s.clone() for s in gen]
    tokens = 4
    ref = []
    for _ in range(tokens):
        ref.append(st.decode_step().clone())
    s_ref = [s.clone() for s in gen]
    torch.cuda.synchronize()

    st.xd.copy_(x_start)
    for s, s0 in zip(gen, s_start):
        s.copy_(s0)
    graph = torch.cuda.CUDAGraph()
    log("stack graph: capture")
    with torch.cuda.graph(graph):
        st.decode_step()
    for r in range(REPLAYS):
        st.xd.copy_(x_start)
        for s, s0 in zip(gen, s_start):
            s.copy_(s0)
        for t in range(tokens):
            _busy(torch, x_start)
            log(f"stack graph: pass {r} token {t}")
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(st.xd, ref[t]), f"pass {r} token {t}"
        for s, s1 in zip(gen, s_ref):
            assert torch.equal(s, s1), f"pass {r}: generation state"


def test_fir_graph_replays():
    """Explicit-filter decode steps (cache append + two passes each) in one graph."""
    torch = require_gpu()
    cfg = dataclasses.replace(get_config(2), B=4)
    params = modal_params(cfg)
    L, S = 300, 16
    (q, k, v), (dq, dk, dv) = _inputs(torch, cfg, cfg.B, L, S, 41)
    op = ModalHyena(params.poles, params.residues, params.skip, cfg.B, cfg.D, cfg.act)
    h = op.filter(L + S)
    for window in (0, 64):
        fir = hb.FirHyena(op, L + S)
        fir.fill(k, v)
        y_e = torch.empty((S, cfg.B, cfg.D), dtype=op.tdtype, device="cuda")
        log(f"fir graph window {window}: eager")
        for s in range(S):
            fir.step(h, L + s, dq[s], dk[s], dv[s], window=window, y=y_e[s])
        torch.cuda.synchronize()
        y_g = torch.empty_like(y_e)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for s in range(S):
                fir.step(h, L + s, dq[s], dk[s], dv[s], window=window, y=y_g[s])
        for r in range(REPLAYS):
            y_g.fill_(9.0)
            fir.cache[:, L:].fill_(7.0)  # the rows the steps append: rebuilt by every replay
            _busy(torch, y_e)
            log(f"fir graph window {window}: replay {r}")
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_g, y_e), f"window {window} replay {r}"


def test_distill_graph_replays():
    """Adam iterations (objective, gradient, update) captured once.  The bias
    corrections are taken at capture, so each replay restarts from the
    captured iteration's parameters and moments."""
    torch = require_gpu()
    from distilled_modal_ssm_amd.distill import ModalDistiller
    cfg = get_config(2)
    params = modal_params(cfg)
    target = ModalHyena(params.poles, params.residues, params.skip, 1, cfg.H, "f32").filter(512)
    n = 20
    eager = ModalDistiller(target, 8)
    hist_e = eager.fit(n, lr=1e-2)
    torch.cuda.synchronize()

    dist = ModalDistiller(target, 8)
    names = ("poles", "residues", "skip", "m", "v")
    start = {a: getattr(dist, a).clone() for a in names}
    hist_g = torch.empty_like(hist_e)
    graph = torch.cuda.CUDAGraph()
    log("distill graph: capture")
    with torch.cuda.graph(graph):
        for i in range(n):
            dist.step(1e-2, loss=hist_g[i])
    for r in range(REPLAYS):
        for a in names:
            getattr(dist, a).copy_(start[a])
        hist_g.fill_(-1.0)
        _busy(torch, hist_e)
        log(f"distill graph: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(hist_g, hist_e), f"replay {r}: losses"
        for a in ("poles", "residues", "skip"):
            assert torch.equal(getattr(dist, a), getattr(eager, a)), f"replay {r}: {a}"
