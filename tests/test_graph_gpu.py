"""The forward step captured in a HIP graph.

A caller that replays moe_forward from a graph (a serving loop, the
benchmark's graph figure) must get exactly what eager calls give: every call
launches kernels only, on buffers the caller allocated, and the bias is
read and updated in place.  Each case runs a few forward steps eagerly, then
captures the same steps in one graph and replays it three times from the
same starting bias, with eager torch work, junk in the outputs and host
synchronisations between replays; every replay must leave the eager run's
output, bias and routing tables bit for bit.
"""
import pytest
import torch

from sparse_mixture_experts_04_amd import _lib as L
from sparse_mixture_experts_04_amd import synth
from sparse_mixture_experts_04_amd.configs import MoEConfig

from parity_util import log

pytestmark = pytest.mark.gpu

DEV = "cuda"
STEPS = 4

CASES = [
    # 1.5 rows per routed expert: the 32-row decode GEMM
    MoEConfig("graph_decode", T=64, d=512, F=256, act="bf16", bias_range=0.05),
    # 96 rows per routed expert: the large-batch GEMM
    MoEConfig("graph_big", T=4096, d=512, F=256, act="bf16", bias_range=0.05),
    # 192 rows per routed expert: 256-row tiles, shared experts' down fused
    # with the combine
    MoEConfig("graph_big256", T=8192, d=512, F=256, act="bf16", bias_range=0.05),
    # MXFP4 routed weights, 64-row shared-expert GEMM with K slices
    MoEConfig("graph_fp4", T=64, d=512, F=256, act="bf16", bias_range=0.05, fp4_weights=True),
    # capacity-limited dispatch
    MoEConfig("graph_cap", T=300, d=256, F=128, act="bf16", bias_range=0.05,
              capacity_factor=1.0),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_graph_replays_match_eager(cfg):
    log(f"[graph] {cfg.describe()} fp4={cfg.fp4_weights} cap={cfg.capacity_factor}")
    inp = synth.make_inputs(cfg, device=DEV)
    desc = L.make_desc(cfg.T, cfg.d, cfg.F, synth.act_dtype(cfg), gate_norm=cfg.gate_norm,
                       gate_scale=cfg.gate_scale, capacity_factor=cfg.capacity_factor,
                       fp4_weights=cfg.fp4_weights)
    keep = None
    if cfg.fp4_weights:
        w, keep = L.fp4_weights(inp)
    else:
        w = L.weights_from(inp)
    T, E, k, S = cfg.T, cfg.E, cfg.k, cfg.S
    y = torch.empty((T, cfg.d), dtype=synth.act_dtype(cfg), device=DEV)
    routing = {"topk_idx": torch.empty((T, k), dtype=torch.int32, device=DEV),
               "gates": torch.empty((T, k + S), dtype=torch.float32, device=DEV),
               "counts": torch.empty(E, dtype=torch.int32, device=DEV),
               "pair_pos": torch.empty(T * k, dtype=torch.int32, device=DEV)}
    ws = L.alloc_workspace(desc, L.CALL_FORWARD, DEV)
    bias0 = inp["bias"].clone()
    bias = bias0.clone()

    def step():
        L.forward(desc, inp["x"], w, bias, cfg.gamma, y, routing, ws=ws)

    for _ in range(STEPS):
        step()
    torch.cuda.synchronize()
    eager = {"y": y.clone(), "bias": bias.clone(), **{n: t.clone() for n, t in routing.items()}}
    assert not torch.equal(eager["bias"], bias0)   # the steps moved the bias

    bias.copy_(bias0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(STEPS):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        bias.copy_(bias0)
        y.fill_(float("nan"))
        for t in routing.values():
            t.fill_(-3)
        junk = (torch.randn(1 << 16, device=DEV) ** 2).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {"y": y, "bias": bias, **routing}
        for n, ref in eager.items():
            assert torch.equal(got[n], ref), f"replay {rep}: {n} differs"
        assert torch.isfinite(junk)
    del keep


@pytest.mark.parametrize("cfg", CASES[:3], ids=lambda c: c.name)
def test_forward_marked_matches_forward(cfg):
    """moe_forward_marked (the benchmark's timed entry point) gives bit for
    bit what moe_forward gives, and its seven events come in launch order."""
    log(f"[marked] {cfg.describe()} fp4={cfg.fp4_weights}")
    inp = synth.make_inputs(cfg, device=DEV)
    desc = L.make_desc(cfg.T, cfg.d, cfg.F, synth.act_dtype(cfg),
                       fp4_weights=cfg.fp4_weights)
    keep = None
    if cfg.fp4_weights:
        w, keep = L.fp4_weights(inp)
    else:
        w = L.weights_from(inp)
    outs = []
    for marked in (False, True):
        y = torch.empty((cfg.T, cfg.d), dtype=synth.act_dtype(cfg), device=DEV)
        routing = {"topk_idx": torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV),
                   "counts": torch.empty(cfg.E, dtype=torch.int32, device=DEV)}
        bias = inp["bias"].clone()
        ev = None
        if marked:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
            for e in ev:
                e.record()
            torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        start.record()
        L.forward(desc, inp["x"], w, bias, cfg.gamma, y, routing, events=ev)
        torch.cuda.synchronize()
        outs.append((y, bias, routing))
        if marked:
            spans = [start.elapsed_time(ev[0])] + [ev[i].elapsed_time(ev[i + 1]) for i in range(6)]
            assert all(t >= 0.0 for t in spans), spans
    (y0, b0, r0), (y1, b1, r1) = outs
    assert torch.equal(y0, y1) and torch.equal(b0, b1)
    for n in r0:
        assert torch.equal(r0[n], r1[n]), n
    del keep
