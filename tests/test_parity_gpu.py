"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Full parity (every output element) on shapes the oracle finishes in
seconds and at the full sizes of the prefill, decode and large-batch
workloads; the skewed workload's 100 bias steps at full size in lock-step,
with its outputs checked at three of them; the native-shape and capacity
workloads on sampled tokens.
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_04_amd import configs, synth
from sparse_mixture_experts_04_amd.configs import MoEConfig

from parity_util import (Buffers, cap_for, check_bias, check_dispatch,
                         check_forward_matches_stages, check_routing, desc_for, device_weights,
                         expert_getter, fused_combine, host_weights, log, np64, npi,
                         per_expert_rel_l2, rel_l2, run_forward, run_stages)

pytestmark = pytest.mark.gpu

DEV = "cuda"

SMALL = {
    "A": configs.get("A"),                                                   # fp32, T=128
    "A_ragged": MoEConfig("A_ragged", T=77, d=512, F=128, act="f32", bias_range=0.1,
                          wd_std_from_F=True),
    "bf16_small": MoEConfig("bf16_small", T=300, d=512, F=256, act="bf16", bias_range=0.05),
    "bf16_tall": MoEConfig("bf16_tall", T=1500, d=256, F=128, act="bf16", bias_range=0.05),
    "bf16_one": MoEConfig("bf16_one", T=1, d=768, F=384, act="bf16", bias_range=0.05),
    # 48 to 160 rows per routed expert on average: the 128-row tiles
    "bf16_mt128": MoEConfig("bf16_mt128", T=2200, d=512, F=256, act="bf16", bias_range=0.05),
    # 164 rows per routed expert: the 256-row tiles
    "bf16_mt256": MoEConfig("bf16_mt256", T=7000, d=256, F=128, act="bf16", bias_range=0.05),
    # gates by logsumexp over log-sigmoids, scaled ("Under The Hood: Inkling")
    "bf16_lse": MoEConfig("bf16_lse", T=300, d=512, F=256, act="bf16", bias_range=0.05,
                          gate_norm="logsumexp", gate_scale=6.5),
    "bf16_lse_big": MoEConfig("bf16_lse_big", T=2500, d=768, F=384, act="bf16",
                              bias_range=0.05, gate_norm="logsumexp", gate_scale=6.5),
    # per-expert capacity ("Inkling, Dissected" 02d): overflow pairs dropped
    "bf16_cap": MoEConfig("bf16_cap", T=2200, d=512, F=256, act="bf16", bias_range=0.05,
                          capacity_factor=1.0),
    "bf16_cap_skew": MoEConfig("bf16_cap_skew", T=1500, d=256, F=128, act="bf16",
                               bias_range=0.0, skew_kappa=8.0, capacity_factor=1.25),
    "f32_cap": MoEConfig("f32_cap", T=128, d=512, F=128, act="f32", bias_range=0.1,
                         wd_std_from_F=True, capacity_factor=0.75),
    # other expert counts: 64 or 128 routed experts, 0 to 2 shared
    "e64_s0": MoEConfig("e64_s0", T=256, d=256, F=128, E=64, S=0, act="bf16",
                        bias_range=0.05),
    "e128_s1_big": MoEConfig("e128_s1_big", T=2048, d=256, F=256, E=128, S=1, act="bf16",
                             bias_range=0.05),
    # 192 rows per routed expert and one shared expert: the 256-row tiles and
    # the forward's fused shared-expert down + combine over a single expert
    "e128_s1_mt256": MoEConfig("e128_s1_mt256", T=4096, d=256, F=256, E=128, S=1,
                               act="bf16", bias_range=0.05),
    # the fused combine with capacity-dropped pairs
    "bf16_cap_mt256": MoEConfig("bf16_cap_mt256", T=7000, d=256, F=128, act="bf16",
                                bias_range=0.05, capacity_factor=1.0),
    "e64_s2_f32_cap": MoEConfig("e64_s2_f32_cap", T=200, d=256, F=128, E=64, S=2, act="f32",
                                bias_range=0.1, wd_std_from_F=True, capacity_factor=1.0),
    "e128_s0_lse_cap": MoEConfig("e128_s0_lse_cap", T=1200, d=512, F=128, E=128, S=0,
                                 act="bf16", bias_range=0.05, gate_norm="logsumexp",
                                 gate_scale=2.5, capacity_factor=1.25),
    # either side of the one-workgroup dispatch (at most 4096 pairs; in the
    # forward it also writes the tile plan and applies the bias update),
    # under a capacity that drops pairs
    "bf16_dispatch_4092": MoEConfig("bf16_dispatch_4092", T=682, d=256, F=128, act="bf16",
                                    bias_range=0.05, capacity_factor=1.0),
    "bf16_dispatch_4098": MoEConfig("bf16_dispatch_4098", T=683, d=256, F=128, act="bf16",
                                    bias_range=0.05, capacity_factor=1.0),
}


def to_dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def out_tol(cfg):
    return 1e-4 if cfg.act == "f32" else 2e-2


@pytest.mark.parametrize("name", list(SMALL))
def test_full_parity_stagewise(name):
    cfg = SMALL[name]
    log(f"[full parity] {name}: {cfg.describe()}")
    inp = to_dev(synth.make_inputs(cfg, device="cpu"))
    desc = desc_for(cfg)
    b, bias_new = run_stages(desc, inp, cfg.gamma)

    x64, wr64, b64 = np64(inp["x"]), np64(inp["w_router"]), np64(inp["bias"])
    topk = npi(b.topk)
    r, g_ref, st = check_routing(x64, wr64, b64, topk, np64(b.gates),
                                 gate_norm=cfg.gate_norm, gate_scale=cfg.gate_scale)
    log(f"  routing {st}")
    dp = check_dispatch(topk, b, E=cfg.E, cap=cap_for(cfg))
    if cfg.capacity_factor:
        m = O.load_metrics(dp["counts"], dp["kept"], cfg.k, cfg.T)
        log(f"  capacity {cap_for(cfg)}: MaxVio {m['max_vio']:.2f}, dropped {m['drop_rate']:.3f}")
    check_bias(npi(b.counts), cfg.gamma, inp["bias"], bias_new, cfg.T)

    hw = host_weights(inp)
    T, k = cfg.T, cfg.k
    # gate/up stage (h) against the oracle's SwiGLU hidden rows
    h = np64(b.h)
    h_ref = np.zeros_like(h)
    for e in range(cfg.E):
        lo, hi = dp["offsets"][e], dp["offsets"][e + 1]
        if hi > lo:
            rows = dp["sorted_pair"][lo:hi] // k
            h_ref[lo:hi] = O.swiglu_hidden(x64[rows], hw["w_gate"][e], hw["w_up"][e])
    for s in range(cfg.S):
        h_ref[k * T + s * T: k * T + (s + 1) * T] = O.swiglu_hidden(x64, hw["ws_gate"][s],
                                                                      hw["ws_up"][s])
    tol = out_tol(cfg)
    e_h = rel_l2(h, h_ref)
    # expert outputs
    yr_ref, ys_ref = O.expert_ffn(x64, hw, dp["offsets"], dp["sorted_pair"], k)
    e_yr, e_ys = rel_l2(np64(b.y_routed), yr_ref), rel_l2(np64(b.y_shared), ys_ref)
    # combine alone, on the GPU's expert outputs and gates
    y_comb = O.combine(np64(b.y_routed), np64(b.y_shared), np64(b.gates), dp["pair_pos"], k)
    e_comb = rel_l2(np64(b.y), y_comb)
    # end to end (oracle arithmetic for the GPU's selection)
    y_ref = O.combine(yr_ref, ys_ref, g_ref, dp["pair_pos"], k)
    e_y = rel_l2(np64(b.y), y_ref)
    log(f"  rel L2: h {e_h:.2e} y_routed {e_yr:.2e} y_shared {e_ys:.2e} "
        f"combine {e_comb:.2e} y {e_y:.2e} (tol {tol})")
    assert e_h <= tol and e_yr <= tol and e_ys <= tol
    assert e_comb <= (1e-6 if cfg.act == "f32" else 4e-3)
    assert e_y <= tol

    # the fused entry point: the same routing and bias bit for bit; y bit
    # for bit, or within the oracle tolerance where it fuses the shared
    # experts' down GEMM with the combine
    bf, bias_f = run_forward(desc, inp, cfg.gamma)
    check_forward_matches_stages(cfg, b, bias_new, bf, bias_f)
    if fused_combine(cfg):
        e_yf = rel_l2(np64(bf.y), y_ref)
        log(f"  forward y rel L2 {e_yf:.2e}")
        assert e_yf <= tol


def test_empty_batch():
    cfg = SMALL["bf16_small"]
    inp = to_dev(synth.make_inputs(MoEConfig("empty", T=0, d=512, F=256, act="bf16")))
    desc = desc_for(cfg, T=0)
    b, bias = run_forward(desc, inp, 1e-3)
    assert torch.equal(bias, inp["bias"])          # every load equals the ideal 0
    assert int(b.offsets[-1].item()) == 0 and int(b.counts.abs().sum().item()) == 0


def test_determinism_bitwise():
    cfg = SMALL["bf16_tall"]
    inp = to_dev(synth.make_inputs(cfg, device="cpu"))
    desc = desc_for(cfg)
    b1, bias1 = run_forward(desc, inp, cfg.gamma)
    b2, bias2 = run_forward(desc, inp, cfg.gamma)
    for n in ("topk", "gates", "margin", "counts", "offsets", "sorted_pair", "pair_pos", "y"):
        assert torch.equal(getattr(b1, n), getattr(b2, n)), n
    assert torch.equal(bias1, bias2)


def check_full_size_output(cfg, inp, b, dp, g_ref, y_forward=None):
    """Every output of a full-size workload against the oracle fed the GPU's
    selection: each routed expert's rows of y_routed (per-expert relative
    L2, so an error confined to one tile of one expert shows), each shared
    expert's y_shared per 256-column slice, combine on the GPU's own expert
    outputs, and y end to end over every token; with y_forward (moe_forward's
    y on the same inputs), that y end to end too."""
    k, T, S = cfg.k, cfg.T, cfg.S
    x64 = np64(inp["x"])
    W = device_weights(inp)
    yr_ref, ys_ref = O.expert_ffn(x64, W, dp["offsets"], dp["sorted_pair"], k)
    yr = np64(b.y_routed)
    e_exp, at = per_expert_rel_l2(yr, yr_ref, dp["offsets"])
    ys = np64(b.y_shared)
    e_sl = max((rel_l2(ys[s_, :, c:c + 256], ys_ref[s_, :, c:c + 256])
                for s_ in range(S) for c in range(0, cfg.d, 256)), default=0.0)
    y_comb = O.combine(yr, ys, np64(b.gates), dp["pair_pos"], k)
    del yr, ys
    y = np64(b.y)
    e_comb = rel_l2(y, y_comb)
    y_ref = O.combine(yr_ref, ys_ref, g_ref, dp["pair_pos"], k)
    del yr_ref, ys_ref
    e_y = rel_l2(y, y_ref)
    tok = np.linalg.norm(y - y_ref, axis=1) / np.linalg.norm(y_ref, axis=1)
    log(f"  every token: y rel L2 {e_y:.2e} (worst token {tok.max():.2e}); worst expert "
        f"{at} {e_exp:.2e}; worst shared 256-column slice {e_sl:.2e}; combine {e_comb:.2e}; "
        f"weight upcasts {sum(w.upcast_s for w in W.values()):.1f} s")
    tol = out_tol(cfg)
    assert e_exp <= tol and e_sl <= tol and e_y <= tol
    assert e_comb <= 4e-3
    if y_forward is not None:
        e_yf = rel_l2(np64(y_forward), y_ref)
        log(f"  forward y rel L2 {e_yf:.2e}")
        assert e_yf <= tol


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["B", "C", "D", "I", "Ecap"])
def test_workload_parity_every_token(name):
    """Workloads B (prefill chunk), C (decode), D (large batch), I (the
    native shape with logsumexp gates) and Ecap (skewed routing under
    capacity 1.25, its first batch) at their own sizes: routing, dispatch
    and bias in full, and every output element against the oracle (D: the
    whole 11.5 TFLOP layer in float64); moe_forward run twice gives the same
    bits."""
    cfg = configs.get(name)
    log(f"[workload parity, every token] {name}: {cfg.describe()}")
    inp = synth.make_inputs(cfg, device=DEV)
    desc = desc_for(cfg)
    b, bias_new = run_stages(desc, inp, cfg.gamma)
    x64, wr64, b64 = np64(inp["x"]), np64(inp["w_router"]), np64(inp["bias"])
    topk = npi(b.topk)
    r, g_ref, st = check_routing(x64, wr64, b64, topk, np64(b.gates),
                                 gate_norm=cfg.gate_norm, gate_scale=cfg.gate_scale)
    log(f"  routing {st}")
    assert 0 <= st["exempt_differ"] <= st["exempt"]
    dp = check_dispatch(topk, b, cap=cap_for(cfg))
    check_bias(npi(b.counts), cfg.gamma, inp["bias"], bias_new, cfg.T)
    del x64, r
    # the fused entry point: the stage calls' routing and bias bit for bit,
    # and its own y against the oracle over every token
    bf, bias_f = run_forward(desc, inp, cfg.gamma)
    check_forward_matches_stages(cfg, b, bias_new, bf, bias_f)
    check_full_size_output(cfg, inp, b, dp, g_ref, y_forward=bf.y)
    b2, _ = run_forward(desc, inp, cfg.gamma)
    assert torch.equal(bf.y, b2.y) and torch.equal(bf.sorted_pair, b2.sorted_pair)
    del inp, b, bf, b2
    torch.cuda.empty_cache()


def combine_rel_l2_chunked(b, k, chunk=2048):
    """Relative L2 of the GPU's y against the oracle's combine of the GPU's
    own expert outputs and gates, over every token, taken in token chunks
    (only the chunk's expert rows are brought to the host)."""
    T = b.y.shape[0]
    num = den = 0.0
    pp_all = b.pair_pos.view(T, k)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        pp = npi(pp_all[t0:t1]).reshape(-1)
        live = np.nonzero(pp >= 0)[0]
        rows = np.unique(pp[live])
        yr = np64(b.y_routed[torch.tensor(rows, device=b.y.device)])
        remap = np.full(pp.shape, -1, dtype=np.int64)
        remap[live] = np.searchsorted(rows, pp[live])
        ref = O.combine(yr, np64(b.y_shared[:, t0:t1]), np64(b.gates[t0:t1]), remap, k)
        got = np64(b.y[t0:t1])
        num += float(np.sum((got - ref) ** 2))
        den += float(np.sum(ref ** 2))
    return (num / den) ** 0.5


def check_skewed_step_outputs(cfg, inp, b, dp, g_ref, step, x64, y_forward=None):
    """At one step of the skewed workload: every row of four experts (the
    hottest, the second hottest, the median and the lightest non-empty one)
    against the oracle's SwiGLU of the same tokens; every row of each shared
    expert on one 256-column slice of y_shared; combine over every token on
    the GPU's expert outputs; and y end to end on the tokens owning the
    hottest expert's first, tile-boundary, middle and last rows."""
    k, E = cfg.k, cfg.E
    counts = dp["counts"]
    order = np.argsort(-counts, kind="stable")
    nz = order[counts[order] > 0]
    picks = [int(nz[0]), int(nz[1]), int(nz[len(nz) // 2]), int(nz[-1])]
    W = device_weights(inp)
    worst = 0.0
    for e in picks:
        lo, hi = int(dp["offsets"][e]), int(dp["offsets"][e + 1])
        rows = dp["sorted_pair"][lo:hi] // k
        ref = O.swiglu(x64[rows], W["w_gate"][e], W["w_up"][e], W["w_down"][e])
        err = rel_l2(np64(b.y_routed[lo:hi]), ref)
        log(f"    expert {e}: {hi - lo} rows, rel L2 {err:.2e}")
        worst = max(worst, err)
    c0 = (step * 256 * 13) % cfg.d
    e_sh = 0.0
    for s_ in range(cfg.S):
        hs = O.swiglu_hidden(x64, W["ws_gate"][s_], W["ws_up"][s_])
        ref = hs @ W["ws_down"][s_][c0:c0 + 256].T
        e_sh = max(e_sh, rel_l2(np64(b.y_shared[s_, :, c0:c0 + 256]), ref))
        del hs
    e_comb = combine_rel_l2_chunked(b, k)
    hot = picks[0]
    lo, hi = int(dp["offsets"][hot]), int(dp["offsets"][hot + 1])
    at = sorted({lo, lo + 255, lo + 256, (lo + hi) // 2, hi - 1} & set(range(lo, hi)))
    toks = sorted({int(dp["sorted_pair"][i]) // k for i in at})
    y_ref = O.output_rows(toks, x64, npi(b.topk), g_ref, expert_getter(inp, E),
                          pair_pos=dp["pair_pos"])
    e_y = rel_l2(np64(b.y)[toks], y_ref)
    e_yf = 0.0 if y_forward is None else rel_l2(np64(y_forward)[toks], y_ref)
    log(f"  step {step}: experts {picks} worst rel L2 {worst:.2e}; shared columns "
        f"{c0}..{c0 + 255} {e_sh:.2e}; combine (every token) {e_comb:.2e}; y on "
        f"{len(toks)} tokens of expert {hot} {e_y:.2e} (forward {e_yf:.2e})")
    assert worst <= 2e-2 and e_sh <= 2e-2 and e_y <= 2e-2 and e_yf <= 2e-2
    assert e_comb <= 4e-3


@pytest.mark.timeout(900)
def test_skewed_workload_100_steps_lockstep():
    """Workload E at its own size (T=16384, d=7168, F=2048, skewed router):
    all 100 bias steps on fresh tokens, each step against the oracle fed the
    bias the GPU routed with ("Inkling, Dissected", 02e: the bias moves after
    each batch; 02g runs 100 such steps): selection outside near-ties, gates,
    counts, offsets, the permutation and the new bias bit for bit.  At steps
    0, 49 and 99 every output is checked as well (check_full_size_output:
    every expert's rows, every shared slice, combine and y on every token,
    for the stage calls and for moe_forward), after the hottest experts'
    tile-boundary rows (check_skewed_step_outputs).  Near-tie counts are
    logged per step and in total."""
    cfg = configs.get("E")
    log(f"[skewed lock-step, 100 steps] {cfg.describe()}")
    inp = synth.make_inputs(cfg, device=DEV)
    desc = desc_for(cfg)
    wr64 = np64(inp["w_router"])
    bias = inp["bias"].clone()
    exempt = differ = 0
    for step in range(cfg.steps):
        inp["x"] = synth.make_x(cfg, DEV, step)
        inp["bias"] = bias.clone()
        full = step in (0, 49, 99)
        bf = None
        if full:
            b, bias = run_stages(desc, inp, cfg.gamma)
            # moe_forward on the same inputs (its fused shared down + combine)
            bf, bias_f = run_forward(desc, inp, cfg.gamma)
            check_forward_matches_stages(cfg, b, bias, bf, bias_f)
        else:
            b, bias = run_forward(desc, inp, cfg.gamma)
        x64 = np64(inp["x"])
        topk = npi(b.topk)
        _, g_ref, st = check_routing(x64, wr64, np64(inp["bias"]), topk, np64(b.gates))
        dp = check_dispatch(topk, b)
        check_bias(npi(b.counts), cfg.gamma, inp["bias"], bias, cfg.T)
        exempt += st["exempt"]
        differ += st["exempt_differ"]
        c = dp["counts"]
        log(f"  step {step}: max/mean load {c.max() / c.mean():.2f}, near-ties {st['exempt']} "
            f"(differ {st['exempt_differ']}), gate rel {st['gate_max_rel']:.1e}")
        if full:
            check_skewed_step_outputs(cfg, inp, b, dp, g_ref, step, x64,
                                      y_forward=bf.y)
            check_full_size_output(cfg, inp, b, dp, g_ref, y_forward=bf.y)
        del b, bf, x64
    log(f"  100 steps: near-tie tokens {exempt}, of which {differ} picked the other set")
    assert 0 <= differ <= exempt
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [256, 2048])
def test_dispatch_marks_out_of_range_ids_dropped(T):
    """Expert ids outside [0, E) handed to moe_dispatch join no expert: the
    valid pairs are grouped exactly as the oracle groups them, the invalid
    ones get pair_pos = -1 and no load, and combine leaves them out."""
    from sparse_mixture_experts_04_amd import _lib as L
    cfg = MoEConfig(f"bad_ids_{T}", T=T, d=256, F=128, act="bf16")
    E, k, S = cfg.E, cfg.k, cfg.S
    rng = np.random.default_rng(T)
    topk = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int64)
    bad = rng.random((T, k)) < 0.1
    topk[bad] = rng.choice([-1, -7, E, E + 5, 1 << 20], size=int(bad.sum()))
    desc = desc_for(cfg)
    b = Buffers(desc, DEV)
    b.topk.copy_(torch.tensor(topk, dtype=torch.int32))
    b.pair_pos.fill_(12345)
    L.dispatch(desc, b.topk, b.counts, b.offsets, b.sorted_pair, b.pair_pos)
    # the oracle's grouping with every invalid id sent to one extra bin past
    # the last expert (it sorts after every valid pair)
    mapped = np.where((topk >= 0) & (topk < E), topk, E)
    dp = O.dispatch(mapped, n_routed=E + 1)
    n_valid = int(dp["offsets"][E])
    pp_ref = np.where(mapped.ravel() < E, dp["pair_pos"], -1)
    torch.cuda.synchronize()
    assert np.array_equal(npi(b.counts), dp["counts"][:E])
    assert np.array_equal(npi(b.offsets), dp["offsets"][:E + 1])
    assert np.array_equal(npi(b.sorted_pair)[:n_valid], dp["sorted_pair"][:n_valid])
    assert np.array_equal(npi(b.pair_pos), pp_ref)
    act = synth.act_dtype(cfg)
    b.y_routed = synth.normal((T * k, cfg.d), 1.0, DEV, cfg.name, "y_routed", 0, act)
    b.y_shared = synth.normal((S, T, cfg.d), 1.0, DEV, cfg.name, "y_shared", 0, act)
    b.gates = torch.rand((T, k + S), device=DEV)
    L.combine(desc, b.y_routed, b.y_shared, b.gates, b.pair_pos, b.y)
    torch.cuda.synchronize()
    ref = O.combine(np64(b.y_routed), np64(b.y_shared), np64(b.gates), pp_ref, k)
    assert rel_l2(np64(b.y), ref) <= 4e-3


@pytest.mark.parametrize("cf", [0.0, 1.25])
def test_skewed_bias_trajectory_100_steps(cf):
    """The skewed router's 100 bias steps at a size the oracle runs in
    seconds (T=2048, d=512, 256 routed + 2 shared experts, kappa = 8), with
    and without capacity: every step against the oracle fed the GPU's bias,
    then the GPU's whole bias trajectory against the oracle's own."""
    cfg = MoEConfig(f"E_small_{cf}", T=2048, d=512, F=128, act="bf16", bias_range=0.0,
                    skew_kappa=8.0, steps=100, capacity_factor=cf)
    log(f"[skewed 100 steps] {cfg.describe()} cf={cf}")
    T, E, k = cfg.T, cfg.E, cfg.k
    desc = desc_for(cfg)
    wr = synth.make_router(cfg)
    wr64 = wr.numpy().astype(np.float64)
    xs = [synth.make_x(cfg, "cpu", i) for i in range(cfg.steps)]
    cap = cap_for(cfg)
    b = Buffers(desc, DEV)
    from sparse_mixture_experts_04_amd import _lib as L
    w_dev = wr.to(DEV)
    bias = torch.zeros(E, dtype=torch.float32, device=DEV)
    flips, traj = 0, []
    for i in range(cfg.steps):
        x = xs[i].to(DEV)
        b_in = bias.clone()
        L.router(desc, x, w_dev, bias, b.topk, b.gates, b.margin)
        L.dispatch(desc, b.topk, b.counts, b.offsets, b.sorted_pair, b.pair_pos)
        L.bias_update(desc, b.counts, cfg.gamma, bias)
        torch.cuda.synchronize()
        topk = npi(b.topk)
        _, _, st = check_routing(np64(xs[i]), wr64, np64(b_in), topk, np64(b.gates))
        flips += st["exempt_differ"]
        check_dispatch(topk, b, E=E, cap=cap)
        check_bias(npi(b.counts), cfg.gamma, b_in, bias, T)
        traj.append(b_in.cpu().numpy())
    ob = np.zeros(E, np.float32)
    first_diff = None
    for i in range(cfg.steps):
        if first_diff is None and not np.array_equal(ob.view(np.uint32), traj[i].view(np.uint32)):
            first_diff = i
        r = O.route(np64(xs[i]), wr64, ob, n_routed=E, k=k)
        dp = O.dispatch(r["topk_idx"], n_routed=E, cap=cap)
        ob = O.bias_update(dp["counts"], cfg.gamma, ob, T, k)
    log(f"  near-tie flips {flips}; first step where the trajectories differ: {first_diff}")
    if flips == 0:
        assert first_diff is None


@pytest.mark.parametrize("T", [1200, 3000, 7000])
def test_expert_ffn_tile_boundaries(T):
    # Hand-picked per-expert row counts around every tile size the GEMMs use
    # (32-row tiles at T=1200, 128-row tiles at T=3000, 256-row tiles at
    # T=7000, each with its balanced tails): 0, 1, 31..33, 63..65, 127..129,
    # 255..257, 383, 384, 511..513, the rest spread over the other experts.
    # sorted_pair is a seeded permutation of the pair ids, so rows gather
    # arbitrary tokens.
    cfg = MoEConfig(f"tiles{T}", T=T, d=512 if T < 5000 else 256, F=256 if T < 5000 else 128,
                    act="bf16")
    inp = to_dev(synth.make_inputs(cfg, device="cpu"))
    E, k = cfg.E, cfg.k
    special = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 384,
               511, 512, 513]
    counts = np.zeros(E, dtype=np.int64)
    counts[:len(special)] = special
    left = k * T - counts.sum()
    assert left >= 0
    rest = np.arange(len(special), E)
    counts[rest] = left // len(rest)
    counts[rest[: left % len(rest)]] += 1
    assert counts.sum() == k * T
    rng = np.random.default_rng(T)
    sorted_pair = rng.permutation(k * T)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    desc = desc_for(cfg)
    d_off = torch.tensor(offsets, dtype=torch.int32, device=DEV)
    d_sp = torch.tensor(sorted_pair, dtype=torch.int32, device=DEV)
    b = Buffers(desc, DEV)
    from sparse_mixture_experts_04_amd import _lib as L
    L.expert_ffn(desc, inp["x"], L.weights_from(inp), d_off, d_sp, b.y_routed, b.y_shared)
    torch.cuda.synchronize()
    yr_ref, ys_ref = O.expert_ffn(np64(inp["x"]), host_weights(inp), offsets, sorted_pair, k)
    yr = np64(b.y_routed)
    for e in range(len(special)):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            err = rel_l2(yr[lo:hi], yr_ref[lo:hi])
            assert err <= 2e-2, (e, counts[e], err)
    e_all, e_sh = rel_l2(yr, yr_ref), rel_l2(np64(b.y_shared), ys_ref)
    log(f"  T={T}: y_routed {e_all:.2e} y_shared {e_sh:.2e}")
    assert e_all <= 2e-2 and e_sh <= 2e-2


def test_expert_ffn_ep_share_sampled():
    """The expert GEMMs at one GPU's share of 8-way expert parallelism: 32
    routed experts (ids 96..127) holding 3072 rows each, i.e. the 98,304
    (token, expert) pairs that 8 GPUs of 16,384 tokens send to one GPU, and
    the shared experts on the GPU's own 16,384 tokens, at d=7168, F=2048.
    Sampled rows against the oracle's SwiGLU of the same rows."""
    cfg = configs.get("D")
    inp = synth.make_inputs(cfg, device=DEV)
    E, k, T = cfg.E, cfg.k, cfg.T
    P = k * T
    counts = np.zeros(E, dtype=np.int64)
    counts[96:128] = P // 32
    offsets = np.concatenate([[0], np.cumsum(counts)])
    rng = np.random.default_rng(8)
    sorted_pair = rng.permutation(P)
    desc = desc_for(cfg)
    b = Buffers(desc, DEV)
    from sparse_mixture_experts_04_amd import _lib as L
    L.expert_ffn(desc, inp["x"], L.weights_from(inp),
                 torch.tensor(offsets, dtype=torch.int32, device=DEV),
                 torch.tensor(sorted_pair, dtype=torch.int32, device=DEV), b.y_routed, b.y_shared)
    torch.cuda.synchronize()
    get = expert_getter(inp)
    worst = 0.0
    for e in (96, 111, 127):
        lo = int(offsets[e])
        rows = [0, 1, 31, 32, 255, 256, 1535, 1536, 3071]
        toks = sorted_pair[lo + np.array(rows)] // k
        wg, wu, wd = get(e)
        ref = O.swiglu(np64(inp["x"][torch.tensor(toks, device=DEV)]), wg, wu, wd)
        got = np64(b.y_routed[lo + torch.tensor(rows, device=DEV)])
        for i in range(len(rows)):
            worst = max(worst, rel_l2(got[i], ref[i]))
    for s_ in range(cfg.S):
        toks = [0, 1, 8191, 16383]
        wg, wu, wd = get(E + s_)
        ref = O.swiglu(np64(inp["x"][torch.tensor(toks, device=DEV)]), wg, wu, wd)
        got = np64(b.y_shared[s_][torch.tensor(toks, device=DEV)])
        for i in range(len(toks)):
            worst = max(worst, rel_l2(got[i], ref[i]))
    log(f"  EP share: worst sampled row rel L2 {worst:.2e}")
    assert worst <= 2e-2
    del inp, b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1000, 4096])
def test_identical_tokens_with_an_exact_tie(T):
    """Every token the same, and the 6th choice's routing vector copied into
    a lower-numbered expert, so the two keys are exactly equal for every
    token: the lower id must win everywhere ("Inkling, Dissected", 02b,
    with ties to the lower index), six experts then hold T rows each and the
    other 250 none (T = 1000 runs the 32-row GEMM, T = 4096 the large one),
    the bias moves down for the six and up for the rest, and the outputs
    match the oracle's."""
    cfg = MoEConfig(f"same_{T}", T=T, d=512, F=256, act="bf16", bias_range=0.0)
    log(f"[identical tokens] {cfg.describe()}")
    inp = synth.make_inputs(cfg, device="cpu")
    inp["x"][:] = inp["x"][0]
    x0 = inp["x"][0].double().numpy()
    z = np64(inp["w_router"][: cfg.E]) @ x0
    order = np.argsort(-z, kind="stable")
    j6 = int(order[5])
    i_low = int(min(e for e in range(cfg.E) if e not in set(order[:6].tolist())))
    assert i_low < j6
    inp["w_router"][i_low] = inp["w_router"][j6]
    inp = to_dev(inp)
    desc = desc_for(cfg)
    b, bias_new = run_stages(desc, inp, cfg.gamma)

    topk = npi(b.topk)
    want = np.array(list(order[:5]) + [i_low])
    assert np.array_equal(topk, np.broadcast_to(want, topk.shape)), topk[:2]
    x64, wr64, b64 = np64(inp["x"]), np64(inp["w_router"]), np64(inp["bias"])
    r, g_ref, _ = check_routing(x64, wr64, b64, topk, np64(b.gates))
    assert np.array_equal(r["topk_idx"], topk)        # the oracle breaks the tie the same way
    dp = check_dispatch(topk, b, E=cfg.E)
    assert sorted(np.nonzero(dp["counts"])[0].tolist()) == sorted(want.tolist())
    assert set(dp["counts"][want].tolist()) == {T}
    check_bias(npi(b.counts), cfg.gamma, inp["bias"], bias_new, cfg.T)
    hw = host_weights(inp)
    yr_ref, ys_ref = O.expert_ffn(x64, hw, dp["offsets"], dp["sorted_pair"], cfg.k)
    y_ref = O.combine(yr_ref, ys_ref, g_ref, dp["pair_pos"], cfg.k)
    e_y = rel_l2(np64(b.y), y_ref)
    log(f"  tie {i_low} over {j6}; rel L2 y {e_y:.2e}")
    assert e_y <= out_tol(cfg)
    y = np64(b.y)
    assert np.array_equal(y, np.broadcast_to(y[0], y.shape))   # identical rows out


def test_twenty_way_exact_tie():
    """The 6th choice's routing vector copied into 19 other experts outside
    the top 5, every token the same: 20 experts share the 6th key exactly,
    more candidates than the selection hands to the exact pass in its record,
    so that pass lists them again from the keys.  The lowest of the 20 ids
    must win ("Inkling, Dissected", 02b, ties to the lower index), as in the
    oracle, and the outputs match."""
    cfg = MoEConfig("same20", T=600, d=512, F=256, act="bf16", bias_range=0.0)
    log(f"[20-way tie] {cfg.describe()}")
    inp = synth.make_inputs(cfg, device="cpu")
    inp["x"][:] = inp["x"][0]
    x0 = inp["x"][0].double().numpy()
    z = np64(inp["w_router"][: cfg.E]) @ x0
    order = np.argsort(-z, kind="stable")
    j6 = int(order[5])
    top5 = set(order[:5].tolist())
    others = [e for e in range(cfg.E) if e not in top5 and e != j6][:19]
    for e in others:
        inp["w_router"][e] = inp["w_router"][j6]
    tied = sorted(others + [j6])
    inp = to_dev(inp)
    desc = desc_for(cfg)
    b, bias_new = run_forward(desc, inp, cfg.gamma)
    topk = npi(b.topk)
    want = np.array(list(order[:5]) + [tied[0]])
    assert np.array_equal(topk, np.broadcast_to(want, topk.shape)), topk[:2]
    x64, wr64, b64 = np64(inp["x"]), np64(inp["w_router"]), np64(inp["bias"])
    r, g_ref, _ = check_routing(x64, wr64, b64, topk, np64(b.gates))
    assert np.array_equal(r["topk_idx"], topk)
    dp = check_dispatch(topk, b, E=cfg.E)
    check_bias(npi(b.counts), cfg.gamma, inp["bias"], bias_new, cfg.T)
    hw = host_weights(inp)
    yr_ref, ys_ref = O.expert_ffn(x64, hw, dp["offsets"], dp["sorted_pair"], cfg.k)
    y_ref = O.combine(yr_ref, ys_ref, g_ref, dp["pair_pos"], cfg.k)
    e_y = rel_l2(np64(b.y), y_ref)
    log(f"  20 tied experts from {tied[0]}; rel L2 y {e_y:.2e}")
    assert e_y <= out_tol(cfg)


def test_binding_rejects_short_routing_tables():
    """The expert calls read offsets[0..E] and sorted_pair[0..T*k-1]; the
    binding refuses tables of any other length before anything launches."""
    from sparse_mixture_experts_04_amd import _lib as L
    cfg = MoEConfig("short_tables", T=64, d=256, F=128, act="bf16")
    inp = synth.make_inputs(cfg, device=DEV)
    desc = desc_for(cfg)
    b = Buffers(desc, DEV)
    w = L.weights_from(inp)
    short_off = b.offsets[:-1]
    short_sp = b.sorted_pair[:-1]
    with pytest.raises(ValueError, match="offsets"):
        L.expert_gate_up(desc, inp["x"], w, short_off, b.sorted_pair, b.h)
    with pytest.raises(ValueError, match="sorted_pair"):
        L.expert_gate_up(desc, inp["x"], w, b.offsets, short_sp, b.h)
    with pytest.raises(ValueError, match="offsets"):
        L.expert_down(desc, w, short_off, b.h, b.y_routed, b.y_shared)
    with pytest.raises(ValueError, match="sorted_pair"):
        L.expert_ffn(desc, inp["x"], w, b.offsets, short_sp, b.y_routed, b.y_shared)


def test_layer_past_2_31_elements():
    """T = 65536 at the layer's width (d = 7168, F = 2048): the expert-sorted
    outputs Y [6T, d] hold 2.8e9 elements, so every sorted row from
    2^31 / d on is addressed past 2^31 elements (and past 4 GiB).  Routing,
    dispatch and the bias are checked in full; the output on the first and
    last token and on the tokens that own sorted rows at and past that
    boundary."""
    cfg = MoEConfig("past_2_31", T=65536, d=7168, F=2048, act="bf16")
    log(f"[past 2^31] {cfg.describe()}")
    inp = synth.make_inputs(cfg, device=DEV)
    desc = desc_for(cfg)
    b, bias_new = run_forward(desc, inp, cfg.gamma)
    x64, wr64, b64 = np64(inp["x"]), np64(inp["w_router"]), np64(inp["bias"])
    topk = npi(b.topk)
    r, g_ref, st = check_routing(x64, wr64, b64, topk, np64(b.gates))
    log(f"  routing {st}")
    dp = check_dispatch(topk, b)
    check_bias(npi(b.counts), cfg.gamma, inp["bias"], bias_new, cfg.T)
    sp = dp["sorted_pair"]
    edge = (1 << 31) // cfg.d  # first sorted row whose elements lie past 2^31
    assert cfg.k * cfg.T > edge + 2
    rows = [edge, edge + 1, (edge + len(sp)) // 2, len(sp) - 1]
    toks = sorted({0, cfg.T - 1} | {int(sp[i]) // cfg.k for i in rows})
    y_ref = O.output_rows(toks, x64, topk, g_ref, expert_getter(inp), pair_pos=dp["pair_pos"])
    e = rel_l2(np64(b.y[toks]), y_ref)
    log(f"  sampled {len(toks)} tokens: rel L2 {e:.2e}")
    assert e <= 2e-2
    del inp, b
    torch.cuda.empty_cache()
