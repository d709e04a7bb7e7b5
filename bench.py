"""Benchmark of the MoE-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one ``moe_forward`` call (router, dispatch, expert SwiGLU GEMMs,
combine, bias update) over one batch already resident in HBM:

* headline workload: T=16384 tokens, d=7168, F=2048, 256 routed + 2 shared
  experts, top-6, bf16 weights and activations, fp32 router;
* decode workload (reported alongside): the same layer at T=64, with bf16
  weights and with the routed experts' weights in FP4 (MXFP4);
* skewed workload (reported alongside): the headline shape with a skewed
  router, 100 consecutive batches (fresh tokens each) and the balancing
  bias updating after every batch; again with a hard per-expert capacity
  of 1.25x the ideal load (drop rate per batch);
* native-shape workload (reported alongside): hidden 6144, expert width
  3072, gates by logsumexp over log-sigmoids times a route scale, at the
  headline batch size;
* Router Balance Lab (reported alongside): 64 experts, d = 32, 2048
  Zipf-lumpy tokens per step, capacity 1.25x, 100 routing steps at bias
  steps 0, 0.01 and 0.05, with MaxVio, drop rate and layer quality.

Prints one JSON line.  ``value`` is tokens/s of the headline workload;
``roofline`` is for its dominant kernel, the grouped gate/up GEMM (matrix
cores), timed with HIP events on the stream it runs on; ``decode`` carries
the T=64 numbers against HBM bandwidth; ``cpu_baseline`` times the CPU
oracle on a bounded sample of the headline workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % bf16 MFMA peak (T=16384) / % HBM BW (T=64 decode)"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

# Steps of the timed sequences re-run after the timing for a parity check
# against the oracle (in the CPU-baseline leg): workload, the bias the step
# routed with (host), and which batch of tokens (None: the workload's x).
PROBES = []


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="D", help="headline workload (D)")
    ap.add_argument("--decode-workload", default="C")
    ap.add_argument("--fp4-decode-workload", default="Cfp4")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--skewed-workload", default="E")
    ap.add_argument("--skewed-steps", type=int, default=100)
    ap.add_argument("--capacity-workload", default="Ecap")
    ap.add_argument("--no-skewed", action="store_true")
    ap.add_argument("--native-workload", default="I")
    ap.add_argument("--no-native", action="store_true")
    ap.add_argument("--prefill-workload", default="B")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-ep-share", action="store_true")
    ap.add_argument("--no-library-gemm", action="store_true")
    ap.add_argument("--lab-workload", default="Lab")
    ap.add_argument("--no-lab", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=1024)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device-to-device copy of this size (for scaling "
                         "hardware byte counters)")
    return ap.parse_args()


def expert_flops(cfg):
    # per (token, expert) pair: gate and up GEMMs 2*(2*d*F), down 2*d*F
    pairs = (cfg.k + cfg.S) * cfg.T
    return 4.0 * cfg.d * cfg.F * pairs, 2.0 * cfg.d * cfg.F * pairs


def setup(cfg, torch, L, synth):
    inp = synth.make_inputs(cfg, device="cuda")
    desc = L.make_desc(cfg.T, cfg.d, cfg.F, synth.act_dtype(cfg), gate_norm=cfg.gate_norm,
                       gate_scale=cfg.gate_scale, capacity_factor=cfg.capacity_factor,
                       fp4_weights=cfg.fp4_weights)
    if cfg.fp4_weights:         # quantized once, outside the timed region
        w, q = L.fp4_weights(inp)
        inp.update({"fp4_" + k: v for k, v in q.items()})   # keep them alive
    else:
        w = L.weights_from(inp)
    # the router's bf16 planes of w_router, prepared once per weights like
    # the quantization (moe_router_prepare), outside the timed region
    inp["_router_planes"] = L.router_planes(desc, inp["w_router"])
    w = L.with_router_planes(w, inp["_router_planes"])
    y = torch.empty((cfg.T, cfg.d), dtype=synth.act_dtype(cfg), device="cuda")
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    ws = L.alloc_workspace(desc, L.CALL_FORWARD, "cuda")
    torch.cuda.synchronize()
    return inp, desc, w, y, counts, ws


def spread(ms):
    """p10, median and p90 of per-step times."""
    v = sorted(ms)
    return [round(v[len(v) // 10], 4), round(v[len(v) // 2], 4), round(v[(9 * len(v)) // 10], 4)]


def capture_steps(step, indices, torch):
    """One HIP graph of the calls step(i) for i in `indices` (a forward
    through the C ABI on preallocated buffers: kernels only, no memset, copy
    or sync).  Every kernel has run eagerly before, so nothing initialises
    during capture."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in indices:
            step(i)
    torch.cuda.synchronize()
    return g


def time_forward(cfg, steps, warmup, torch, L, synth, replay=False, group=5, marked=False,
                 fresh_bias=False):
    """Times `steps` back-to-back forwards after `warmup` untimed ones.  By
    default the bias is updated in place by every step, so later steps route
    differently (at T=64 they touch more experts).  With `fresh_bias`, every
    step instead routes with the workload's own initial bias and updates a
    copy of its own (one preallocated buffer per step), which times the
    workload exactly as stated, bias update included.  With `replay`, the
    same sequence is then run again from the initial bias (the path is
    deterministic, so it routes step for step as the timed run did): once in
    groups of `group` timed steps between event pairs, for the spread of the
    per-step time, and once untimed with each step's expert loads copied
    out, so that per-step figures (bytes streamed) refer to the very steps
    that were timed.  The last step's loads stay in `counts` either way.
    With `marked`, the timed steps call moe_forward_marked, whose events
    between the stages give every step's stage and GEMM-kernel times
    (averaged into inp["_marks_ms"]).  inp["_probe_bias"] is left holding
    (on the host) the bias the last timed step routed with, so that step can
    be re-run for a parity check."""
    inp, desc, w, y, counts, ws = setup(cfg, torch, L, synth)
    bias0 = inp["bias"].clone()
    bias = bias0.clone()
    routing = {"counts": counts}
    n_all = warmup + steps
    fresh = [bias0.clone() for _ in range(n_all)] if fresh_bias else None

    def step(events=None, i=0):
        b = fresh[i] if fresh_bias else bias
        L.forward(desc, inp["x"], w, b, cfg.gamma, y, routing, ws=ws, events=events)

    def restart():
        # back to the initial bias state before a replayed sequence
        if fresh_bias:
            for f in fresh:
                f.copy_(bias0)
        else:
            bias.copy_(bias0)

    marks = [None] * steps
    if marked:
        marks = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
        for m in marks:
            for e in m:
                e.record()          # the raw handles exist once an event was recorded
    for i in range(warmup):
        step(i=i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        step(marks[i], i=warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    if marked:
        # marks: router, dispatch, tile plan, gate/up GEMM, down GEMM, combine, bias
        acc = {n: 0.0 for n in ("router", "dispatch", "gate_up", "down", "combine",
                                "bias_update", "gate_up_gemm", "down_gemm")}
        for i, m in enumerate(marks):
            start = ev0 if i == 0 else marks[i - 1][6]
            acc["router"] += start.elapsed_time(m[0])
            acc["dispatch"] += m[0].elapsed_time(m[1])
            acc["gate_up"] += m[1].elapsed_time(m[3])
            acc["gate_up_gemm"] += m[2].elapsed_time(m[3])
            acc["down"] += m[3].elapsed_time(m[4])
            acc["down_gemm"] += m[3].elapsed_time(m[4])
            acc["combine"] += m[4].elapsed_time(m[5])
            acc["bias_update"] += m[5].elapsed_time(m[6])
        inp["_marks_ms"] = {n: v / steps for n, v in acc.items()}
    wall = time.perf_counter() - t0
    ms_events = ev0.elapsed_time(ev1) / steps
    # the bias the last timed step routed with (an untimed replay)
    restart()
    for i in range(n_all - 1):
        step(i=i)
    inp["_probe_bias"] = (fresh[n_all - 1] if fresh_bias else bias).cpu().numpy().copy()
    torch.cuda.synchronize()
    if replay:
        ngroups = max(1, steps // group)
        restart()
        for i in range(warmup):
            step(i=i)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(ngroups)]
        for gi, (a, b) in enumerate(evs):
            a.record()
            for j in range(group):
                step(i=min(n_all - 1, warmup + gi * group + j))
            b.record()
        torch.cuda.synchronize()
        inp["_spread"] = spread([a.elapsed_time(b) / group for a, b in evs])
        restart()
        for i in range(warmup):
            step(i=i)
        loads = torch.empty((steps, cfg.E), dtype=counts.dtype, device=counts.device)
        for i in range(steps):
            step(i=warmup + i)
            loads[i].copy_(counts)
        torch.cuda.synchronize()
        inp["_loads"] = loads.cpu()
        # the timed steps once more, replayed from one HIP graph
        restart()
        for i in range(warmup):
            step(i=i)
        start = [f.clone() for f in fresh] if fresh_bias else bias.clone()
        graph = capture_steps(lambda i: step(i=i), range(warmup, n_all), torch)
        if fresh_bias:
            for f, s0 in zip(fresh, start):
                f.copy_(s0)
        else:
            bias.copy_(start)
        torch.cuda.synchronize()
        ev0.record()
        graph.replay()
        ev1.record()
        torch.cuda.synchronize()
        inp["_graph_ms"] = ev0.elapsed_time(ev1) / steps
        del graph
    return inp, desc, w, ws, counts, wall * 1e3 / steps, ms_events


def time_stages(cfg, inp, desc, w, steps, torch, L, synth):
    """The same path through the per-stage entry points, with HIP events on
    torch's current stream (the stream every call launches on).  The expert
    GEMM stages use the marked entry points, which also record events
    between their kernel launches.  Returns average ms per stage and per
    GEMM kernel, and the routing counts of the last step."""
    dev = "cuda"
    T, k, S, E = cfg.T, cfg.k, cfg.S, cfg.E
    act = synth.act_dtype(cfg)
    i32, f32 = torch.int32, torch.float32
    topk = torch.empty((T, k), dtype=i32, device=dev)
    gates = torch.empty((T, k + S), dtype=f32, device=dev)
    counts = torch.empty(E, dtype=i32, device=dev)
    offsets = torch.empty(E + 1, dtype=i32, device=dev)
    sp = torch.empty(T * k, dtype=i32, device=dev)
    pp = torch.empty(T * k, dtype=i32, device=dev)
    h = torch.empty(((k + S) * T, cfg.F), dtype=act, device=dev)
    yr = torch.empty((T * k, cfg.d), dtype=act, device=dev)
    ys = torch.empty((S, T, cfg.d), dtype=act, device=dev)
    y = torch.empty((T, cfg.d), dtype=act, device=dev)
    bias = inp["bias"].clone()
    wsr = L.alloc_workspace(desc, L.CALL_ROUTER, dev)
    wsd = L.alloc_workspace(desc, L.CALL_DISPATCH, dev)
    wsg = L.alloc_workspace(desc, L.CALL_GATE_UP, dev)
    wsn = L.alloc_workspace(desc, L.CALL_DOWN, dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    rec = []
    for _ in range(steps + 1):
        r = {n: ev() for n in ("t0", "router", "dispatch", "gu_plan", "gu_gemm",
                               "dn_plan", "dn_gemm", "combine", "bias")}
        for e in r.values():
            e.record()          # raw handles exist once an event was recorded
        rec.append(r)
    torch.cuda.synchronize()
    for r in rec:
        r["t0"].record()
        L.router(desc, inp["x"], inp["w_router"], bias, topk, gates, ws=wsr)
        r["router"].record()
        L.dispatch(desc, topk, counts, offsets, sp, pp, ws=wsd)
        r["dispatch"].record()
        L.expert_gate_up_marked(desc, inp["x"], w, offsets, sp, h,
                                [r["gu_plan"], r["gu_gemm"]], ws=wsg)
        L.expert_down_marked(desc, w, offsets, h, yr, ys,
                             [r["dn_plan"], r["dn_gemm"]], ws=wsn)
        L.combine(desc, yr, ys, gates, pp, y)
        r["combine"].record()
        L.bias_update(desc, counts, cfg.gamma, bias)
        r["bias"].record()
    torch.cuda.synchronize()
    rec = rec[1:]            # the first pass warms up
    span = lambda a, b: sum(r[a].elapsed_time(r[b]) for r in rec) / len(rec)
    stages = {"router": span("t0", "router"), "dispatch": span("router", "dispatch"),
              "gate_up": span("dispatch", "gu_gemm"), "down": span("gu_gemm", "dn_gemm"),
              "combine": span("dn_gemm", "combine"), "bias_update": span("combine", "bias")}
    kernels = {"gate_up_gemm": span("gu_plan", "gu_gemm"), "down_gemm": span("dn_plan", "dn_gemm")}
    return stages, kernels, counts.cpu()


def traffic_for(kernel_file, profile):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "sparse_mixture_experts_04_amd", "csrc", kernel_file)
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if rec.get("source_sha256") != digest:
        return None
    return rec.get("bytes_per_launch")


def load_profile(counts, mean_load):
    """Routed-load profile of one batch: the five largest loads and the
    smallest over the mean, and the slope of log load against log rank over
    ranks 1-64 (a Zipf profile of exponent a has slope -a)."""
    import numpy as np
    v = np.sort(np.asarray(counts, dtype=np.float64))[::-1]
    r = np.arange(1, 65)
    head = v[:64]
    ok = head > 0
    slope = float(np.polyfit(np.log(r[ok]), np.log(head[ok]), 1)[0]) if ok.sum() > 1 else None
    return {"top5_over_mean": [round(float(x) / mean_load, 3) for x in v[:5]],
            "min_over_mean": round(float(v[-1]) / mean_load, 3),
            "loglog_slope_ranks_1_64": None if slope is None else round(slope, 3)}


def time_skewed(cfg, steps, torch, L, synth):
    """Consecutive batches of the skewed workload: fresh tokens every batch
    (generated outside the timed region), the bias carried from batch to
    batch.  Returns per-batch times and the routing load statistics."""
    import statistics
    inp, desc, w, y, counts, ws = setup(cfg, torch, L, synth)
    bias = inp["bias"].clone()
    routing = {"counts": counts}
    mean_load = cfg.T * cfg.k / cfg.E
    cap = None
    if cfg.capacity_factor > 0:     # rows an expert keeps: ceil(cf * k*T / E)
        import math
        import numpy as np
        cap = math.ceil(float(np.float32(cfg.capacity_factor)) * float(cfg.k * cfg.T) / cfg.E)
    ms, maxmean, dropped = [], [], []
    profile = None
    probe_bias = None
    for s in range(steps + 1):          # batch 0 also warms up
        x = synth.make_x(cfg, device="cuda", step=s)
        if s == 1:
            probe_bias = bias.cpu().numpy().copy()   # the first timed batch's bias
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        L.forward(desc, x, w, bias, cfg.gamma, y, routing, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        if s > 0:
            ms.append(e0.elapsed_time(e1))
        maxmean.append(counts.max().item() / mean_load)
        if s == 0:
            profile = load_profile(counts.cpu().numpy(), mean_load)
        if cap is not None:
            dropped.append((counts - cap).clamp(min=0).sum().item() / (cfg.k * cfg.T))
    f_gu, f_dn = expert_flops(cfg)
    med = statistics.median(ms)
    del inp, w, ws, y
    torch.cuda.empty_cache()
    return {"workload": f"skewed MoE layer, {cfg.describe()}, router offset kappa="
                        f"{cfg.skew_kappa}, {steps} consecutive batches, bias step "
                        f"{cfg.gamma}" + (f", capacity {cfg.capacity_factor} x ideal load"
                                          if cap is not None else ", dropless"),
            "ms_per_step_median": round(med, 4),
            "ms_per_step_p10_p90": [round(sorted(ms)[len(ms) // 10], 4),
                                    round(sorted(ms)[(9 * len(ms)) // 10], 4)],
            "tokens_s": round(cfg.T / (med / 1e3), 1),
            "mfma_frac": round((f_gu + f_dn) / (med / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "max_over_mean_load": {"first": round(maxmean[0], 3),
                                   "middle": round(maxmean[len(maxmean) // 2], 3),
                                   "last": round(maxmean[-1], 3)},
            "bias_range": [round(bias.min().item(), 5), round(bias.max().item(), 5)],
            "load_profile_first_batch": profile,
            "per_step": {"ms": [round(v, 4) for v in ms],
                         "max_over_mean_load": [round(v, 3) for v in maxmean[1:]],
                         "note": "timed batches 1..N (batch 0 warms up)"},
            "_probe": {"bias": probe_bias, "x_step": 1},
            **({"capacity_rows": cap,
                "drop_rate_per_step": [round(v, 4) for v in dropped[1:]],
              "drop_rate": {"first": round(dropped[0], 4),
                              "middle": round(dropped[len(dropped) // 2], 4),
                              "last": round(dropped[-1], 4),
                              "mean": round(sum(dropped) / len(dropped), 4)}}
               if cap is not None else {})}


def lab_measures(lab, x, torch):
    """The Router Balance Lab's measures ("Inkling, Dissected", 02g) of the
    lab's last step on tokens x, as float64 device scalars (no host sync):

    * MaxVio: the hottest expert's demand over the ideal load k*T/E, minus 1;
    * drop rate: the fraction of the k*T expert slots dropped at capacity;
    * layer quality: the gate-weighted affinity of the surviving pairs (the
      router's own gates, a dropped pair adding nothing) over that of the
      unbiased, uncapacitated top-k with its own gates, summed over the batch.

    Bookkeeping around the step, taken by this harness from the step's
    outputs; the affinities are recomputed here in float64."""
    T, E, k = lab.cfg.T, lab.cfg.E, lab.cfg.k
    slots = float(k * T)
    max_vio = lab.counts.max().to(torch.float64) * (E / slots) - 1.0
    kept = (lab.pair_pos >= 0).view(T, k)
    drop_rate = 1.0 - kept.sum().to(torch.float64) / slots
    s = torch.sigmoid(x.to(torch.float64) @ lab.w_router.to(torch.float64).T)
    sel = torch.gather(s, 1, lab.topk.long())
    captured = (lab.gates.to(torch.float64) * sel * kept).sum()
    best = torch.topk(s, k, dim=1).values
    unbiased = (best * best / best.sum(dim=1, keepdim=True)).sum()
    return torch.stack([max_vio, drop_rate, captured / unbiased])


def balance_lab(cfg, torch, gammas=(0.0, 0.01, 0.05)):
    """The Router Balance Lab ("Inkling, Dissected", 02g) on the GPU: for
    each bias step gamma, the bias starts at zero and runs the workload's
    steps over fresh batches; the lab's measures (MaxVio, drop rate, layer
    quality) are averaged over the run.  A step is moe_router ->
    moe_dispatch (capacity) -> moe_bias_update; its time is measured
    separately, without the measures, with HIP events."""
    from sparse_mixture_experts_04_amd import synth
    from sparse_mixture_experts_04_amd.lab import BalanceLab
    w = synth.make_lab_router(cfg).to("cuda")
    xs = [synth.make_lab_x(cfg, i, device="cuda") for i in range(cfg.steps)]
    runs = {}
    for g in gammas:
        lab = BalanceLab(cfg, w, g, "cuda")
        meas = []
        for x in xs:
            lab.step(x)
            meas.append(lab_measures(lab, x, torch))
        meas = torch.stack(meas).cpu()
        mean, last = meas.mean(dim=0).tolist(), meas[-1].tolist()
        runs[f"gamma={g}"] = {"max_vio": round(mean[0], 4), "drop_rate": round(mean[1], 5),
                              "quality": round(mean[2], 5),
                              "last_step": [round(v, 5) for v in last]}
    lab = BalanceLab(cfg, w, cfg.gamma, "cuda")
    for x in xs[:5]:
        lab.step(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for x in xs:
        lab.step(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / len(xs)
    # the same steps replayed from one HIP graph (the step is launch-bound)
    graph = lab.capture(xs)
    lab.reset()
    graph.replay()
    lab.reset()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / len(xs)
    del graph
    return {"workload": f"Router Balance Lab, {cfg.describe()}, frozen router, "
                        f"Zipf-lumpy tokens (head/tail {cfg.lab_head_tail:g}), capacity "
                        f"{cfg.capacity_factor} x ideal, {cfg.steps} steps, routing only",
            "measures_mean_over_steps": runs,
            "ms_per_step": round(ms, 4), "tokens_s": round(cfg.T / (ms / 1e3), 1),
            "ms_per_step_hip_graph": round(ms_graph, 4),
            "tokens_s_hip_graph": round(cfg.T / (ms_graph / 1e3), 1)}


def ep_share(cfg, inp, w, torch, L, synth, steps):
    """The expert GEMMs at one GPU's share of 8-way expert parallelism over
    8 x T tokens: 32 routed experts (ids 96..127) with k*T/32 rows each,
    gathered from the local token buffer by a seeded permutation (the rows an
    all-to-all would deliver), and the shared experts on the T local tokens.
    One moe_expert_ffn call (tile plan, gate/up + SwiGLU, down)."""
    E, k, T, S = cfg.E, cfg.k, cfg.T, cfg.S
    P = k * T
    counts = torch.zeros(E, dtype=torch.int64)
    counts[96:128] = P // 32
    offsets = torch.zeros(E + 1, dtype=torch.int32)
    offsets[1:] = torch.cumsum(counts, 0).to(torch.int32)
    offsets = offsets.cuda()
    g = torch.Generator(device="cpu")
    g.manual_seed(8)
    sorted_pair = torch.randperm(P, generator=g).to(torch.int32).cuda()
    act = synth.act_dtype(cfg)
    y_routed = torch.empty((P, cfg.d), dtype=act, device="cuda")
    y_shared = torch.empty((S, T, cfg.d), dtype=act, device="cuda")
    desc = L.make_desc(T, cfg.d, cfg.F, act)
    ws = L.alloc_workspace(desc, L.CALL_EXPERT_FFN, "cuda")

    def call():
        L.expert_ffn(desc, inp["x"], w, offsets, sorted_pair, y_routed, y_shared, ws=ws)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 6.0 * cfg.d * cfg.F * (P + S * T)
    del y_routed, y_shared, ws
    torch.cuda.empty_cache()
    return {"workload": f"expert GEMMs at one GPU's share of 8-way expert parallelism: 32 "
                        f"routed experts x {P // 32} rows + {S} shared experts x {T} rows, "
                        f"d={cfg.d}, F={cfg.F}, bf16",
            "ms_per_call": round(ms, 4),
            "tflops": round(flops / (ms / 1e3) / 1e12, 1),
            "mfma_frac": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def library_gemm(cfg, torch, reps=5):
    """Reference point for the gate/up GEMM's roofline fraction: the vendor
    library (hipBLASLt through torch.matmul / torch.bmm, bf16) on plain GEMMs
    of the same FLOPs on this GPU, random operands, not part of the layer.
    dense: all T*(k+S) rows against one [d, 2F] weight; batched: the routed
    rows split evenly over the E experts (T*k/E each, no gather, every tile
    full) against each expert's own [d, 2F] weight."""
    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    bf = torch.bfloat16
    out = {"what": "hipBLASLt (torch.matmul / torch.bmm) bf16 GEMMs of the gate/up GEMM's "
                   "shape, random operands; context for the roofline fraction"}
    M, N, K = cfg.T * (cfg.k + cfg.S), 2 * cfg.F, cfg.d
    a = torch.randn((M, K), generator=g, device="cuda").to(bf)
    b = torch.randn((K, N), generator=g, device="cuda").to(bf)
    ms = timed(lambda: torch.matmul(a, b))
    tf = 2.0 * M * N * K / (ms / 1e3) / 1e12
    out["dense"] = {"shape": [M, N, K], "ms": round(ms, 4), "tflops": round(tf, 1),
                    "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    del a, b
    rows = cfg.T * cfg.k // cfg.E
    a = torch.randn((cfg.E, rows, K), generator=g, device="cuda").to(bf)
    w = torch.randn((cfg.E, K, N), generator=g, device="cuda").to(bf)   # contiguous operand
    ms = timed(lambda: torch.bmm(a, w))
    tf = 2.0 * cfg.E * rows * N * K / (ms / 1e3) / 1e12
    out["batched_uniform"] = {"experts": cfg.E, "rows_each": rows, "shape": [rows, N, K],
                              "ms": round(ms, 4), "tflops": round(tf, 1),
                              "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    del a, w
    torch.cuda.empty_cache()
    return out


def decode_bytes(cfg, counts):
    n_active = int((counts > 0).sum())
    esz = 2 if cfg.act == "bf16" else 4
    per_expert = 3 * cfg.F * cfg.d * esz
    routed = 3 * cfg.F * cfg.d * (0.5 + 1 / 32) if cfg.fp4_weights else per_expert
    router = (cfg.E + cfg.S) * cfg.d * 4
    xy = 2 * cfg.T * cfg.d * esz
    return int(n_active * routed + cfg.S * per_expert + router + xy), n_active


class _Upcast:
    """An expert stack on the device seen by the oracle as float64 host
    matrices, converted on access; the conversion time is summed apart from
    the oracle's arithmetic."""

    def __init__(self, t):
        self.t = t
        self.seconds = 0.0
        self.n = 0

    def __len__(self):
        return self.t.shape[0]

    def __getitem__(self, e):
        import numpy as np
        t0 = time.perf_counter()
        m = self.t[e].float().cpu().numpy().astype(np.float64)
        self.seconds += time.perf_counter() - t0
        self.n += 1
        return m


def _oracle_weights(inp):
    return {n: _Upcast(inp[n]) for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up",
                                         "ws_down")}


def _sample_tokens(T, n, seed=0):
    import numpy as np
    if n >= T:
        return list(range(T))
    rng = np.random.default_rng(seed)
    return sorted({0, T - 1} | set(rng.choice(T, size=n - 2, replace=False).tolist()))


def probe_parity(probe, main_cfg, main_inp, torch, L, synth, configs, O, nsample):
    """Re-runs one step of a timed sequence (same tokens, same bias, so the
    same bits as the timed run) and checks it against the oracle: near-tie
    tokens (oracle 6th/7th key margin below 1e-6) counted and how many of
    them picked the other set, selection elsewhere, the gates' largest
    relative error, and the output's relative L2 on sampled tokens."""
    import numpy as np
    cfg = configs.get(probe["workload"])
    inp = main_inp if cfg.name == main_cfg.name else synth.make_inputs(cfg, device="cuda")
    if probe["x_step"] is not None:
        inp = dict(inp)
        inp["x"] = synth.make_x(cfg, device="cuda", step=probe["x_step"])
    desc = L.make_desc(cfg.T, cfg.d, cfg.F, synth.act_dtype(cfg), gate_norm=cfg.gate_norm,
                       gate_scale=cfg.gate_scale, capacity_factor=cfg.capacity_factor,
                       fp4_weights=cfg.fp4_weights)
    keep = None
    if cfg.fp4_weights:
        w, keep = L.fp4_weights(inp)
    else:
        w = L.weights_from(inp)
    T, k, S = cfg.T, cfg.k, cfg.S
    i32 = torch.int32
    topk = torch.empty((T, k), dtype=i32, device="cuda")
    gates = torch.empty((T, k + S), dtype=torch.float32, device="cuda")
    pair_pos = torch.empty(T * k, dtype=i32, device="cuda")
    y = torch.empty((T, cfg.d), dtype=synth.act_dtype(cfg), device="cuda")
    bias = torch.tensor(probe["bias"], device="cuda")
    L.forward(desc, inp["x"], w, bias, cfg.gamma, y,
              {"topk_idx": topk, "gates": gates, "pair_pos": pair_pos})
    torch.cuda.synchronize()
    del keep
    x64 = inp["x"].float().cpu().numpy().astype(np.float64)
    wr64 = inp["w_router"].cpu().numpy().astype(np.float64)
    b64 = probe["bias"].astype(np.float64)
    t0 = time.perf_counter()
    r = O.route(x64, wr64, b64, n_routed=cfg.E, k=k, gate_norm=cfg.gate_norm,
                gate_scale=cfg.gate_scale)
    tg = topk.cpu().numpy().astype(np.int64)
    exempt = r["margin"] < 1e-6
    differ = np.any(tg != r["topk_idx"], axis=1)
    shared = list(range(cfg.E, cfg.E + S))
    if cfg.gate_norm == "ratio":
        g_ref, _ = O.joint_gates(r["s"], tg, shared, cfg.gate_scale)
    else:
        g_ref, _ = O.joint_gates_logsumexp(r["z"], tg, shared, cfg.gate_scale)
    g = gates.cpu().numpy().astype(np.float64)
    gate_rel = float(np.max(np.abs(g - g_ref) / g_ref)) if g.size else 0.0
    out = {"step": probe["what"], "tokens": T,
           "near_ties": {"exempt": int(exempt.sum()), "exempt_differ": int((differ & exempt).sum())},
           "selection_mismatch_outside_near_ties": int((differ & ~exempt).sum()),
           "gate_max_rel_err": float(f"{gate_rel:.3e}")}
    if nsample > 0:
        out.update(_probe_output(cfg, inp, x64, tg, g_ref, pair_pos, y, nsample, O))
    out["oracle_s"] = round(time.perf_counter() - t0, 1)
    if cfg.name != main_cfg.name:
        del inp
    torch.cuda.empty_cache()
    return out


def _probe_output(cfg, inp, x64, tg, g_ref, pair_pos, y, nsample, O):
    """Relative L2 of the GPU's y on sampled tokens against the oracle's
    output rows for the GPU's selection."""
    import numpy as np
    k, S = cfg.k, cfg.S
    toks = _sample_tokens(cfg.T, nsample)
    W = _oracle_weights(inp)

    def expert(e):
        if e < cfg.E:
            return W["w_gate"][e], W["w_up"][e], W["w_down"][e]
        return W["ws_gate"][e - cfg.E], W["ws_up"][e - cfg.E], W["ws_down"][e - cfg.E]

    y_ref = O.output_rows(toks, x64, tg, g_ref, expert, k=k, n_routed=cfg.E, n_shared=S,
                          pair_pos=pair_pos.cpu().numpy().astype(np.int64))
    got = y[toks].float().cpu().numpy().astype(np.float64)
    rel = float(np.linalg.norm(got - y_ref) / np.linalg.norm(y_ref))
    return {"output_rel_l2_sampled": float(f"{rel:.3e}"), "sampled_tokens": len(toks)}


def cpu_baseline(cfg, inp, ntok, torch, L, synth, configs):
    """The oracle, as it stands, on the first ``ntok`` tokens of the batch
    (with the batch's initial bias), timed on the host cores.  The oracle
    converts each expert's bf16 weights to float64 when it first uses them;
    that conversion is timed apart from the arithmetic, and the full batch's
    time is estimated from both (every expert is touched at T=16384).  In
    the same leg, every timed workload's re-run step is checked against the
    oracle (probe_parity)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as O

    x = inp["x"][:ntok].float().cpu().numpy()
    wr = inp["w_router"].cpu().numpy()
    bias = inp["bias"].cpu().numpy()
    weights = _oracle_weights(inp)
    t0 = time.perf_counter()
    out = O.moe_forward(x, wr, weights, bias, cfg.gamma, k=cfg.k)
    dt = time.perf_counter() - t0
    assert out["y"].shape == (ntok, cfg.d)
    up_s = sum(w.seconds for w in weights.values())
    n_mats = sum(w.n for w in weights.values())
    arith_s = dt - up_s
    # full batch: all (E + S) experts' 3 matrices converted once, arithmetic x T/ntok
    full_s = up_s / max(1, n_mats) * 3 * (cfg.E + cfg.S) + arith_s * cfg.T / ntok
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info
                   if i.get("user_api") == "blas"})
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                       None)
    except OSError:
        pass
    # the sample's arithmetic: router plus 8 SwiGLU experts per token (6 routed, 2 shared)
    flop = ntok * (2.0 * cfg.d * (cfg.E + cfg.S) + (cfg.k + cfg.S) * 6.0 * cfg.d * cfg.F)
    n_routed = len(set(out["router"]["topk_idx"].ravel().tolist()))
    res = {"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "seconds": round(dt, 2), "cpu": cpu, "blas": blas,
           "weight_upcast_s": round(up_s, 2), "arithmetic_s": round(arith_s, 2),
           "arithmetic_tokens_s": round(ntok / arith_s, 1),
           "arithmetic_gflop_s": round(flop / arith_s / 1e9, 1),
           "full_batch_estimate": {"seconds": round(full_s, 1),
                                   "tokens_s": round(cfg.T / full_s, 1),
                                   "how": "weight conversion of all experts at the sample's "
                                          "per-matrix rate + the sample's arithmetic x T/ntok"},
           "sample": (f"first {ntok} tokens of the T={cfg.T} batch: full oracle forward "
                      f"(fp64 router, dispatch, {n_routed} routed + {cfg.S} shared SwiGLU "
                      f"experts, combine, bias update), the experts' bf16 weights converted "
                      f"to fp64 as the oracle uses them")}
    parity = {}
    for pr in PROBES:
        key = pr["key"]
        try:
            parity[key] = probe_parity(pr, cfg, inp, torch, L, synth, configs, O,
                                       pr["nsample"])
        except Exception as e:  # noqa: BLE001 - reported, not hidden
            parity[key] = {"error": f"{type(e).__name__}: {e}"}
    res["parity_vs_oracle"] = parity
    return res


def section(result, key, fn):
    """Run one reported-alongside measurement; an exception is recorded in
    the JSON line under the section's key (and printed to stderr) instead of
    losing the line."""
    import traceback
    try:
        result[key] = fn()
    except Exception as e:  # noqa: BLE001 - reported, not hidden
        traceback.print_exc(file=sys.stderr)
        result[key] = {"error": f"{type(e).__name__}: {e}"}


def decode_run(dc, args, torch, L, synth, fresh_bias):
    """One timed decode sequence and its figures against HBM bandwidth."""
    steps = max(args.steps, 20)
    inp, desc, w, ws, counts, ms, _ = time_forward(dc, steps, args.warmup, torch, L, synth,
                                                   replay=True, fresh_bias=fresh_bias)
    stages = None
    if not dc.fp4_weights and fresh_bias:
        stages, _, _ = time_stages(dc, inp, desc, w, 10, torch, L, synth)
    # bytes of each timed step (its own active experts), averaged
    per_step = [decode_bytes(dc, c) for c in inp.pop("_loads")]
    nbytes = int(round(sum(b for b, _ in per_step) / len(per_step)))
    actives = [n for _, n in per_step]
    n_active = round(sum(actives) / len(actives), 1)
    gbs = nbytes / (ms / 1e3) / 1e9
    out = {"tokens_s": round(dc.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
           "ms_per_step_p10_p50_p90": inp.pop("_spread"),
           "ms_per_step_hip_graph": round(inp.pop("_graph_ms"), 4)}
    if stages is not None:
        out["stage_ms"] = {k: round(v, 4) for k, v in stages.items()}
    out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes,
                       "active_experts": n_active,
                       "active_experts_first_last": [actives[0], actives[-1]],
                       "scope": "whole moe_forward step; bytes averaged over the timed steps"}
    # output sampled on every token at the stated bias; FP4 layers are
    # checked for routing here (their outputs in the GPU tests: the oracle's
    # quantization takes ~1 s per matrix)
    PROBES.append({"workload": dc.name, "bias": inp.pop("_probe_bias"), "x_step": None,
                   "nsample": 0 if dc.fp4_weights else (dc.T if fresh_bias else 8),
                   "key": dc.name + ("" if fresh_bias else " (bias drifting)"),
                   "what": "the last timed step" + (", bias as stated" if fresh_bias
                                                    else ", bias after the earlier steps")})
    del inp, ws
    torch.cuda.empty_cache()
    return out


def decode(dc, args, torch, L, synth):
    """A decode workload (bf16 or FP4 routed weights) against HBM bandwidth:
    timed as stated (every step routes with the workload's bias, here 0, and
    applies its own bias update), and, beside it, as a sequence whose bias
    drifts from step to step (at T=64 a drifting bias spreads the tokens
    over more experts, so those steps stream more bytes)."""
    weights = ("routed experts' weights MXFP4 (E2M1, power-of-two scale per 32), shared "
               "experts bf16" if dc.fp4_weights else "bf16 weights")
    out = {"workload": f"decode MoE layer, {dc.describe()}, {weights}, fp32 router, every "
                       f"step from the stated bias"}
    out.update(decode_run(dc, args, torch, L, synth, fresh_bias=True))
    drift = decode_run(dc, args, torch, L, synth, fresh_bias=False)
    out["bias_drifting"] = {"what": f"consecutive steps, the bias moving by {dc.gamma} per "
                                    f"step from the stated one", **drift}
    return out


def prefill(pc, args, torch, L, synth):
    """The prefill-chunk workload against both rooflines: with ~96 rows per
    routed expert every expert's weights are streamed once per step (about
    125 FLOP per byte, under the bf16 ridge, so HBM bounds it) while the
    matrix cores run 96-row tiles."""
    inp, _, _, ws, counts, ms, _ = time_forward(pc, max(5, min(args.steps, 20)), args.warmup,
                                                torch, L, synth)
    f_gu, f_dn = expert_flops(pc)
    nbytes, n_active = decode_bytes(pc, counts.cpu())
    PROBES.append({"workload": pc.name, "bias": inp.pop("_probe_bias"), "x_step": None,
                   "nsample": 64, "key": pc.name, "what": "the last timed step"})
    del inp, ws
    torch.cuda.empty_cache()
    return {"workload": f"prefill-chunk MoE layer, {pc.describe()}, fp32 router",
            "tokens_s": round(pc.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
            "mfma_frac": round((f_gu + f_dn) / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "hbm_frac": round(nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes": nbytes, "active_experts": n_active}


def native(nc, args, torch, L, synth):
    """The layer at the native shape with logsumexp gates."""
    inp, _, _, ws, _, ms, _ = time_forward(nc, max(5, min(args.steps, 10)), args.warmup,
                                           torch, L, synth)
    f_gu, f_dn = expert_flops(nc)
    PROBES.append({"workload": nc.name, "bias": inp.pop("_probe_bias"), "x_step": None,
                   "nsample": 8, "key": nc.name, "what": "the last timed step"})
    del inp, ws
    torch.cuda.empty_cache()
    return {"workload": f"MoE layer at the native shape, {nc.describe()}, gates "
                        f"{nc.gate_norm} x {nc.gate_scale}, fp32 router",
            "tokens_s": round(nc.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
            "mfma_frac": round((f_gu + f_dn) / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_mixture_experts_04_amd import _lib as L
    from sparse_mixture_experts_04_amd import configs, synth

    cfg = configs.get(args.workload)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    inp, desc, w, ws, counts, ms_wall, ms_ev = time_forward(cfg, args.steps, args.warmup,
                                                            torch, L, synth, replay=True,
                                                            marked=True)
    # stage and GEMM-kernel times of the timed steps themselves (events that
    # moe_forward_marked records between its launches on the same stream)
    mk = inp.pop("_marks_ms")
    stages = {n: mk[n] for n in ("router", "dispatch", "gate_up", "down", "combine",
                                 "bias_update")}
    kernels = {"gate_up_gemm": mk["gate_up_gemm"], "down_gemm": mk["down_gemm"]}
    f_gu, f_dn = expert_flops(cfg)
    ms = ms_wall
    tokens_s = cfg.T / (ms / 1e3)
    # dominant kernel: the grouped gate/up GEMM (+ SwiGLU) over every row
    rows = cfg.T * (cfg.k + cfg.S)
    gu_tflops = f_gu / (kernels["gate_up_gemm"] / 1e3) / 1e12
    result = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1/d) weights, N(0,1) tokens)",
        "config": {"workload": f"large-batch MoE layer, {cfg.describe()}, fp32 router",
                   "T": cfg.T, "d": cfg.d, "F": cfg.F, "experts": f"{cfg.E}+{cfg.S}",
                   "top_k": cfg.k},
        "layer_tflops": round((f_gu + f_dn) / (ms / 1e3) / 1e12, 1),
        "layer_mfma_frac": round((f_gu + f_dn) / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "ms_per_step_events": round(ms_ev, 4),
        "ms_per_step_p10_p50_p90": inp.pop("_spread"),   # over groups of 5 of the timed steps
        "ms_per_step_hip_graph": round(inp.pop("_graph_ms"), 4),
        "stage_ms": {k: round(v, 4) for k, v in stages.items()},
        "stage_note": ("256-row tiles: 'down' is the routed experts' down GEMM; 'combine' is "
                       "the shared experts' down GEMM fused with the combine"
                       if cfg.T * cfg.k // cfg.E >= 160 and cfg.S > 0 else None),
        "kernel_ms": {k: round(v, 4) for k, v in kernels.items()},
        "roofline": {"kernel": "ffn_big_kernel<gate/up> (grouped gate/up GEMM + SwiGLU over "
                               "every routed and shared row)",
                     "bound": "mfma", "achieved": round(gu_tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tflops / PEAK_BF16_TFLOPS, 4),
                     "flop_per_launch": f_gu, "rows": rows,
                     "ms_per_launch": round(kernels["gate_up_gemm"], 4),
                     "traffic": traffic_for("ffn_big.hip", "ffn_big_gate_up_D_traffic.json")},
    }
    max_load = counts.max().item()
    result["max_over_mean_load"] = round(max_load / (cfg.T * cfg.k / cfg.E), 3)
    PROBES.insert(0, {"workload": cfg.name, "bias": inp.pop("_probe_bias"), "x_step": None,
                      "nsample": 8, "key": cfg.name, "what": "the last timed step"})
    del ws
    torch.cuda.empty_cache()
    if not args.no_ep_share:
        section(result, "ep_share",
                lambda: ep_share(cfg, inp, w, torch, L, synth, max(3, min(args.steps, 10))))
    if not args.no_library_gemm:
        section(result, "library_gemm", lambda: library_gemm(cfg, torch))
    if not args.no_decode:
        section(result, "decode", lambda: decode(configs.get(args.decode_workload), args,
                                                 torch, L, synth))
        section(result, "decode_fp4", lambda: decode(configs.get(args.fp4_decode_workload),
                                                     args, torch, L, synth))
    if not args.no_prefill:
        section(result, "prefill", lambda: prefill(configs.get(args.prefill_workload), args,
                                                   torch, L, synth))
    if not args.no_native:
        section(result, "native", lambda: native(configs.get(args.native_workload), args,
                                                 torch, L, synth))
    if not args.no_skewed:
        for key, name in (("skewed", args.skewed_workload), ("capacity", args.capacity_workload)):
            section(result, key, lambda: time_skewed(configs.get(name), args.skewed_steps,
                                                     torch, L, synth))
            probe = result[key].pop("_probe", None)
            if probe is not None:
                PROBES.append({"workload": name, "bias": probe["bias"],
                               "x_step": probe["x_step"], "nsample": 8, "key": name,
                               "what": "the first timed batch"})
    if not args.no_lab:
        section(result, "balance_lab", lambda: balance_lab(configs.get(args.lab_workload), torch))
    if not args.no_cpu_baseline:
        section(result, "cpu_baseline",
                lambda: cpu_baseline(cfg, inp, args.cpu_sample_tokens, torch, L, synth,
                                     configs))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
