"""Router planes prepared once per weights (moe_router_prepare).

The planes are the exact three-way bf16 split of w_router: their sum is
w_router bit for bit, each plane is the nearest bf16 of what the planes
above it leave, and the padding rows are zero.  A forward pass given the
prepared planes must give the same routing, gates, bias and output, bit for
bit, as one that splits w_router itself.
"""
import pytest
import torch

from sparse_mixture_experts_04_amd import _lib as L
from sparse_mixture_experts_04_amd import synth
from sparse_mixture_experts_04_amd.configs import MoEConfig

from parity_util import log

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    MoEConfig("planes_f32", T=128, d=512, F=128, act="f32", bias_range=0.1),
    MoEConfig("planes_big", T=4096, d=512, F=256, act="bf16", bias_range=0.05),
    MoEConfig("planes_decode", T=64, d=1024, F=256, act="bf16", bias_range=0.05),
    MoEConfig("planes_fp4", T=64, d=512, F=256, act="bf16", bias_range=0.05, fp4_weights=True),
    MoEConfig("planes_e64", T=300, d=256, F=128, E=64, S=0, act="bf16", bias_range=0.05),
]


def _desc(cfg):
    return L.make_desc(cfg.T, cfg.d, cfg.F, synth.act_dtype(cfg), E=cfg.E, S=cfg.S, k=cfg.k,
                       gate_norm=cfg.gate_norm, gate_scale=cfg.gate_scale,
                       capacity_factor=cfg.capacity_factor, fp4_weights=cfg.fp4_weights)


def test_planes_are_the_exact_split():
    cfg = MoEConfig("planes_split", T=1, d=768, F=128, act="bf16")
    w = synth.make_router(cfg, device=DEV)
    # values that stress the split: large, tiny, negative, exact bf16 values
    w[0, :4] = torch.tensor([1.0, -3.0e5, 1.0e-20, 0.1], device=DEV)
    planes = L.router_planes(_desc(cfg), w)
    rows = cfg.E + cfg.S
    assert planes.shape == (3, 320, cfg.d)
    p = planes.to(torch.float64)
    total = p[0, :rows] + p[1, :rows] + p[2, :rows]
    assert torch.equal(total, w.to(torch.float64))
    # each plane is the nearest bf16 of the remainder the planes above leave
    r0 = w
    assert torch.equal(planes[0, :rows], r0.to(torch.bfloat16))
    r1 = r0 - planes[0, :rows].to(torch.float32)
    assert torch.equal(planes[1, :rows], r1.to(torch.bfloat16))
    r2 = r1 - planes[1, :rows].to(torch.float32)
    assert torch.equal(planes[2, :rows], r2.to(torch.bfloat16))
    assert not planes[:, rows:].to(torch.float32).any()


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_with_prepared_planes_matches(cfg):
    log(f"[planes] {cfg.describe()} fp4={cfg.fp4_weights}")
    inp = synth.make_inputs(cfg, device=DEV)
    desc = _desc(cfg)
    keep = None
    if cfg.fp4_weights:
        w, keep = L.fp4_weights(inp)
    else:
        w = L.weights_from(inp)
    planes = L.router_planes(desc, inp["w_router"])
    wp = L.with_router_planes(w, planes)
    T, E, k, S = cfg.T, cfg.E, cfg.k, cfg.S
    ws = L.alloc_workspace(desc, L.CALL_FORWARD, DEV)
    out = []
    for weights in (w, wp):
        y = torch.full((T, cfg.d), float("nan"), dtype=synth.act_dtype(cfg), device=DEV)
        routing = {"topk_idx": torch.full((T, k), -1, dtype=torch.int32, device=DEV),
                   "gates": torch.full((T, k + S), float("nan"), dtype=torch.float32,
                                       device=DEV),
                   "margin": torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)}
        bias = inp["bias"].clone()
        ws.fill_(0xAB)  # junk where the split would go: the prepared planes are read instead
        L.forward(desc, inp["x"], weights, bias, 1e-3, y, routing, ws=ws)
        torch.cuda.synchronize()
        out.append((y, routing, bias))
    (y0, r0, b0), (y1, r1, b1) = out
    assert torch.equal(y0.view(torch.int16) if y0.dtype == torch.bfloat16 else y0.view(torch.int32),
                       y1.view(torch.int16) if y1.dtype == torch.bfloat16 else y1.view(torch.int32))
    for key in r0:
        assert torch.equal(r0[key], r1[key]), key
    assert torch.equal(b0, b1)
    assert (r0["topk_idx"] >= 0).all() and not torch.isnan(r0["gates"]).any()
    del keep
