"""GPU parity of the FP4 (MXFP4) routed-expert weights against the oracle.

Quantization must match the oracle's codes and scale bytes exactly; the
layer with FP4 routed weights is compared with the oracle layer computed on
the dequantized weights (the quantization is a defined transform, so the
same output tolerance as the bf16 layer applies).
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_04_amd import _lib as L
from sparse_mixture_experts_04_amd import configs, synth
from sparse_mixture_experts_04_amd.configs import MoEConfig

from parity_util import (check_bias, check_dispatch, check_routing, desc_for, log, np64, npi,
                         rel_l2, run_forward, run_stages)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16(a):
    return torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16)


def _special_block_rows():
    # rows of 32 hitting the rounding ties, saturation, signed zeros, zeros
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.0, -0.25, -5.0, -0.0, 0.3, 4.5]
    r0 = ties + [0.0] * (32 - len(ties))
    r1 = [0.0] * 32                                   # all zero -> X = -127
    r2 = [v * 2.0 ** -30 for v in r0]                 # tiny block
    r3 = [v * 2.0 ** 40 for v in r0]                  # huge block
    r4 = [-0.0] * 32
    return np.array([r0, r1, r2, r3, r4], dtype=np.float32)


@pytest.mark.parametrize("shape", [(3, 64, 512), (2, 130, 96), (1, 5, 32)])
def test_quantize_bit_exact(shape):
    E, N, K = shape
    rng = np.random.default_rng(E * 1000 + N)
    w = rng.normal(size=(E, N, K)).astype(np.float32) * np.exp2(
        rng.integers(-12, 12, size=(E, N, 1))).astype(np.float32)
    if N * K >= 5 * 32:
        w.reshape(-1, 32)[:5] = _special_block_rows()
    wb = _bf16(w)
    codes, scales = L.quantize_mxfp4(wb.to(DEV))
    torch.cuda.synchronize()
    c_ref, x_ref = O.mxfp4_quantize(wb.float().numpy())
    p_ref, s_ref = O.mxfp4_pack(c_ref, x_ref)
    assert np.array_equal(codes.cpu().numpy(), p_ref)
    assert np.array_equal(scales.cpu().numpy(), s_ref)


def _fp4_oracle_weights(inp):
    """Host fp64 weights with the routed experts replaced by their MXFP4
    dequantization (the oracle's own quantization of the same bf16)."""
    w = {}
    for n in ("w_gate", "w_up", "w_down"):
        c, X = O.mxfp4_quantize(inp[n].float().cpu().numpy())
        w[n] = O.mxfp4_dequantize(c, X)
    for n in ("ws_gate", "ws_up", "ws_down"):
        w[n] = inp[n].float().cpu().numpy().astype(np.float64)
    return w


SMALL = {
    "fp4_small": MoEConfig("fp4_small", T=64, d=512, F=256, act="bf16", bias_range=0.05,
                           fp4_weights=True),
    "fp4_ragged": MoEConfig("fp4_ragged", T=37, d=768, F=384, act="bf16", bias_range=0.05,
                            fp4_weights=True),
    "fp4_cap": MoEConfig("fp4_cap", T=300, d=256, F=128, act="bf16", bias_range=0.05,
                         fp4_weights=True, capacity_factor=1.0),
    # shared experts' K slices: 4 uneven ones for down (6 K steps), 1 and 2
    # at the largest decode batch, none without shared experts
    "fp4_uneven": MoEConfig("fp4_uneven", T=64, d=512, F=384, act="bf16", bias_range=0.05,
                            fp4_weights=True),
    "fp4_t2047": MoEConfig("fp4_t2047", T=2047, d=256, F=256, act="bf16", bias_range=0.05,
                           fp4_weights=True),
    "fp4_e64_s0": MoEConfig("fp4_e64_s0", T=100, d=256, F=128, E=64, S=0, act="bf16",
                            bias_range=0.05, fp4_weights=True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_fp4_layer_full_parity(name):
    cfg = SMALL[name]
    log(f"[fp4 parity] {name}: {cfg.describe()}")
    inp = {k: v.to(DEV) for k, v in synth.make_inputs(cfg, device="cpu").items()}
    desc = desc_for(cfg)
    wq, keep = L.fp4_weights(inp)
    b, bias_new = run_stages(desc, inp, cfg.gamma, weights=wq)
    x64, wr64, b64 = np64(inp["x"]), np64(inp["w_router"]), np64(inp["bias"])
    topk = npi(b.topk)
    _, g_ref, st = check_routing(x64, wr64, b64, topk, np64(b.gates))
    cap = O.capacity(cfg.capacity_factor, cfg.k, cfg.T, cfg.E)
    dp = check_dispatch(topk, b, E=cfg.E, cap=cap)
    check_bias(npi(b.counts), cfg.gamma, inp["bias"], bias_new, cfg.T)
    hw = _fp4_oracle_weights(inp)
    yr_ref, ys_ref = O.expert_ffn(x64, hw, dp["offsets"], dp["sorted_pair"], cfg.k)
    n = int(dp["offsets"][-1])
    e_yr = rel_l2(np64(b.y_routed)[:n], yr_ref[:n])
    e_ys = rel_l2(np64(b.y_shared), ys_ref)
    y_ref = O.combine(yr_ref, ys_ref, g_ref, dp["pair_pos"], cfg.k)
    e_y = rel_l2(np64(b.y), y_ref)
    log(f"  routing {st}; rel L2 y_routed {e_yr:.2e} y_shared {e_ys:.2e} y {e_y:.2e}")
    assert e_yr <= 2e-2 and e_ys <= 2e-2 and e_y <= 2e-2
    # the shared experts' hidden rows (K-sliced with fp32 partials when the
    # shared tiles are few) against the oracle's SwiGLU
    T, k = cfg.T, cfg.k
    for s_ in range(cfg.S):
        h_ref = O.swiglu_hidden(x64, hw["ws_gate"][s_], hw["ws_up"][s_])
        e_h = rel_l2(np64(b.h)[k * T + s_ * T:k * T + (s_ + 1) * T], h_ref)
        assert e_h <= 1e-2, (s_, e_h)
    # the fused entry point gives the same bits
    bf, _ = run_forward(desc, inp, cfg.gamma, weights=wq)
    for nm in ("topk", "counts", "offsets", "pair_pos", "y"):
        assert torch.equal(getattr(b, nm), getattr(bf, nm)), nm
    del keep


def test_fp4_decode_workload_sampled():
    cfg = configs.get("Cfp4")
    log(f"[fp4 workload] {cfg.describe()}")
    inp = synth.make_inputs(cfg, device=DEV)
    desc = desc_for(cfg)
    wq, keep = L.fp4_weights(inp)
    b, bias_new = run_forward(desc, inp, cfg.gamma, weights=wq)
    x64, wr64, b64 = np64(inp["x"]), np64(inp["w_router"]), np64(inp["bias"])
    topk = npi(b.topk)
    _, g_ref, st = check_routing(x64, wr64, b64, topk, np64(b.gates))
    dp = check_dispatch(topk, b)
    check_bias(npi(b.counts), cfg.gamma, inp["bias"], bias_new, cfg.T)
    toks = [0, 63]

    def get(e):
        if e < cfg.E:
            out = []
            for n in ("w_gate", "w_up", "w_down"):
                c, X = O.mxfp4_quantize(inp[n][e].float().cpu().numpy())
                out.append(O.mxfp4_dequantize(c, X))
            return tuple(out)
        s = e - cfg.E
        return tuple(np64(inp[n][s]) for n in ("ws_gate", "ws_up", "ws_down"))

    y_ref = O.output_rows(toks, x64, topk, g_ref, get, pair_pos=dp["pair_pos"])
    e = rel_l2(np64(b.y)[toks], y_ref)
    log(f"  routing {st}; sampled {len(toks)} tokens: rel L2 {e:.2e}")
    assert e <= 2e-2
    del keep, inp
    torch.cuda.empty_cache()
