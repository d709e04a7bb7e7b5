"""Reference oracle for the MoE feed-forward layer (TEST INFRASTRUCTURE ONLY).

This is a plain, slow CPU implementation of the layer, written from the
pages' description of the method.  It exists to check the HIP path; only the
test suite, the package's smoke check and the benchmark's CPU-baseline leg
may import or call it.  It shares no code with the HIP path: its only inputs
are host arrays (NumPy or anything ``np.asarray`` accepts).

Precision: every floating-point step runs in float64 on the exact input
values (fp32 and bf16 inputs convert to float64 exactly), except the
balancing-bias update, which keeps the bias as a float32 state so that its
value is bit-comparable.

Sources (page title, section):

* "Inkling, Dissected", chapter 02 "Anatomy of one MoE layer": 256 routed
  experts of which each token uses 6, 2 shared experts every token uses, and
  one joint normalisation over the 8 contributors.
* "Inkling, Dissected", 02b "Sigmoid, not softmax": the router equation
  (independent sigmoids, top-6 by s + b, gates from raw s over
  kept-and-shared) and its NumPy sketch of one token's forward.
* "Inkling, Dissected", 02c "A routing decision, by hand": a 4-expert top-2
  worked example (used as a golden test).
* "Inkling, Dissected", 02e "The aux-loss-free bias": the balancing rule
  b_i <- b_i + gamma * sign(Lbar - L_i), with L_i the tokens that selected
  expert i this batch and Lbar the total selections divided by the number
  of routed experts.
* "Under The Hood: Inkling from Thinking Machines", "MoE: the expert
  configuration" (each expert is a SwiGLU FFN; shared experts have the same
  width) and "The routing strategy: sigmoid + shared expert sink" (top-6 over
  routed experts only; shared scores join the normalisation, written there
  as log-sigmoid followed by logsumexp over the joint set of 8, and the
  weights are then scaled by route_scale times a learned global scale) and
  "Quantization: BF16 vs NVFP4" (FP4 weights with small-block scales, on
  the routed experts only; the gates, the shared experts and the router
  stay in high precision).

Readings where the pages leave a step open:

* the top-k list is in rank order: descending s + b, exact ties to the lower
  expert index;
* sign(0) = 0, and Lbar is compared exactly as sign(k*T - E*L_i);
* the bias updates after the forward that used it;
* SwiGLU expert: y = W_down (silu(W_gate x) * (W_up x)), silu(u) = u*sigmoid(u),
  no bias terms, weights stored [out, in];
* loads count routed selections only;
* the Router Balance Lab's layer quality weights each surviving expert by
  its gate times its affinity, against the unbiased, uncapacitated top-k
  (``layer_quality``).

Every function here is pinned by ``tests/test_oracle.py``; none is left
unpinned.
"""
import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(z):
    """s = 1 / (1 + exp(-z)), float64 ("Inkling, Dissected", 02b)."""
    z = _f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def router_logits(x, w_router):
    """z[t, i] = x_t . w_i for every routed and shared expert (02b).

    ``w_router`` is [n_routed + n_shared, d], one routing vector per row.
    """
    return _f64(x) @ _f64(w_router).T


def select_topk(key, k):
    """Top-k expert ids of each row of ``key`` in rank order.

    Rank order is descending key; among exactly equal keys the lower expert
    index ranks first (a stable sort of the negated keys).  Also returns the
    margin key_(k) - key_(k+1) between the last kept and the first dropped
    expert (+inf when every expert is kept).
    """
    key = _f64(key)
    order = np.argsort(-key, axis=1, kind="stable")
    top = order[:, :k]
    ks = np.take_along_axis(key, order, axis=1)
    if key.shape[1] > k:
        margin = ks[:, k - 1] - ks[:, k]
    else:
        margin = np.full(key.shape[0], np.inf)
    return top.astype(np.int64), margin


def _joint_idx(top, shared_ids, T):
    shared = np.broadcast_to(np.asarray(shared_ids, dtype=np.int64),
                             (T, len(shared_ids)))
    return np.concatenate([top, shared], axis=1)


def joint_gates(s, top, shared_ids, scale=1.0):
    """g over the kept routed experts followed by the shared experts.

    g_i = s_i / sum_{j in kept U shared} s_j, summed in slot order (02b; the
    shared-expert sink of the Hugging Face write-up), times ``scale`` (1 for
    the layer of "Inkling, Dissected").  ``s`` holds raw affinities: the
    balancing bias never enters the gates.
    """
    s = _f64(s)
    T = s.shape[0]
    idx = _joint_idx(top, shared_ids, T)
    sel = np.take_along_axis(s, idx, axis=1)
    denom = np.zeros(T)
    for j in range(sel.shape[1]):
        denom = denom + sel[:, j]
    return sel / denom[:, None] * scale, idx


def logsigmoid(z):
    """log(sigmoid(z)) = min(z, 0) - log(1 + exp(-|z|)), float64."""
    z = _f64(z)
    return np.minimum(z, 0.0) - np.log1p(np.exp(-np.abs(z)))


def joint_gates_logsumexp(z, top, shared_ids, scale=1.0):
    """Gates in the form of "Under The Hood: Inkling", the routing strategy:
    the logits of the kept routed experts and of the shared experts go
    through log-sigmoid, are normalised by their logsumexp over that joint
    set, and the weights are multiplied by ``scale`` (route_scale times the
    learned global scale).

    g_i = exp(ls_i - lse), ls = logsigmoid(z[kept U shared]),
    lse = m + log(sum_j exp(ls_j - m)), m = max_j ls_j (sum in slot order).
    """
    z = _f64(z)
    T = z.shape[0]
    idx = _joint_idx(top, shared_ids, T)
    ls = logsigmoid(np.take_along_axis(z, idx, axis=1))
    m = ls.max(axis=1)
    acc = np.zeros(T)
    for j in range(ls.shape[1]):
        acc = acc + np.exp(ls[:, j] - m)
    lse = m + np.log(acc)
    return np.exp(ls - lse[:, None]) * scale, idx


def route(x, w_router, bias, n_routed=256, k=6, gate_norm="ratio", gate_scale=1.0):
    """Router of one batch: sigmoid affinities, biased top-k, joint gates.

    ``gate_norm`` is "ratio" (``joint_gates``) or "logsumexp"
    (``joint_gates_logsumexp``); both scale the gates by ``gate_scale``.
    Returns a dict with ``z`` [T, n_routed+n_shared], ``s`` (affinities),
    ``key`` = s[:, :n_routed] + b, ``topk_idx`` [T, k] in rank order,
    ``margin`` [T], ``gates`` [T, k + n_shared] (routed slots first, then the
    shared experts in id order) and ``idx`` [T, k + n_shared].
    """
    z = router_logits(x, w_router)
    s = sigmoid(z)
    n_total = s.shape[1]
    key = s[:, :n_routed] + _f64(bias)[None, :]
    top, margin = select_topk(key, k)
    shared = list(range(n_routed, n_total))
    if gate_norm == "ratio":
        gates, idx = joint_gates(s, top, shared, gate_scale)
    elif gate_norm == "logsumexp":
        gates, idx = joint_gates_logsumexp(z, top, shared, gate_scale)
    else:
        raise ValueError(gate_norm)
    return {"z": z, "s": s, "key": key, "topk_idx": top, "margin": margin,
            "gates": gates, "idx": idx}


def capacity(capacity_factor, k, T, n_routed):
    """Pairs an expert keeps per batch ("Inkling, Dissected", 02d: a hard
    capacity per expert; the lab of 02g sets it at 1.25x the ideal load):
    C = ceil(cf * k*T / E), with cf taken as the float32 the descriptor
    holds and the product and quotient in float64.  None (no limit) for
    cf = 0.
    """
    cf = float(np.float32(capacity_factor))
    if cf == 0.0:
        return None
    return int(np.ceil(cf * float(k * T) / float(n_routed)))


def dispatch(topk_idx, n_routed=256, cap=None):
    """Expert-contiguous grouping of the (token, slot) pairs.

    A pair is numbered p = t*k + j (token t, slot j).  Returns
    ``counts`` [n_routed] (the loads L_i, the demand), ``kept``
    [n_routed] (min(L_i, cap)), ``offsets`` [n_routed+1] (exclusive prefix
    sum of kept), ``sorted_pair`` [sum kept] (the kept pair numbers grouped
    by expert; within one expert in ascending p, hence ascending token) and
    ``pair_pos`` [T*k], each pair's row in that order or -1 when the pair
    was dropped ("Inkling, Dissected", 02d: overflow beyond an expert's
    capacity is dropped).  Without ``cap`` nothing is dropped and pair_pos
    is the inverse permutation.  Which pairs overflow is this module's
    reading: an expert keeps its first ``cap`` pairs in ascending token
    order.
    """
    flat = np.asarray(topk_idx, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=n_routed)
    order = np.argsort(flat, kind="stable")          # grouped, ascending p
    start = np.concatenate([[0], np.cumsum(counts)])
    rank = np.empty_like(order)
    rank[order] = np.arange(flat.size) - start[flat[order]]   # rank inside its expert
    kept = counts if cap is None else np.minimum(counts, cap)
    offsets = np.concatenate([[0], np.cumsum(kept)])
    keep = rank < (kept[flat])
    sorted_pair = order[keep[order]]
    pair_pos = np.full(flat.size, -1, dtype=np.int64)
    pair_pos[keep] = offsets[flat[keep]] + rank[keep]
    return {"counts": counts.astype(np.int64), "kept": kept.astype(np.int64),
            "offsets": offsets.astype(np.int64),
            "sorted_pair": sorted_pair.astype(np.int64),
            "pair_pos": pair_pos.astype(np.int64)}


def load_metrics(counts, kept, k, T):
    """Router Balance Lab measures ("Inkling, Dissected", 02g): MaxVio, the
    hottest expert's demand over the ideal load k*T/E, minus 1; and the drop
    rate, the fraction of the k*T expert slots dropped at capacity."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.size
    max_vio = float(counts.max()) * E / (k * T) - 1.0
    drop_rate = float(k * T - np.asarray(kept).sum()) / (k * T)
    return {"max_vio": max_vio, "drop_rate": drop_rate}


def layer_quality(s, topk_idx, pair_pos, k=6):
    """Router Balance Lab's layer quality ("Inkling, Dissected", 02g): how
    much of the tokens' affinity the gate-weighted experts still deliver
    after capacity drops, relative to a router with neither bias nor
    capacity limit.

    This module's reading: a token's mixture over a set of routed experts
    weights expert j by g_j = s_j / sum of s over the set (the gates of
    02b); the mixture captures sum of g_j * s_j over the pairs that
    survived capacity (a dropped pair contributes nothing, and the other
    gates are not renormalised).  The reference router takes the top-k by
    s alone (no bias, nothing dropped).  Quality = captured / oracle, both
    summed over the batch.  ``s`` holds the routed experts' affinities
    [T, n_routed]; ``pair_pos`` is dispatch's (-1 for a dropped pair).
    """
    s = _f64(s)
    T = s.shape[0]
    top = np.asarray(topk_idx, dtype=np.int64).reshape(T, k)
    kept = np.asarray(pair_pos, dtype=np.int64).reshape(T, k) >= 0
    g, _ = joint_gates(s, top, [])
    sel = np.take_along_axis(s, top, axis=1)
    captured = float(np.sum(np.where(kept, g * sel, 0.0)))
    top0, _ = select_topk(s, k)
    g0, _ = joint_gates(s, top0, [])
    best = float(np.sum(g0 * np.take_along_axis(s, top0, axis=1)))
    return captured / best


def balance_lab(x_of_step, w_router, bias, gamma, capacity_factor, steps, k=6):
    """The Router Balance Lab's loop ("Inkling, Dissected", 02g): a frozen
    router, one fresh batch per step, hard capacity, and the selection-only
    bias of 02e updated from each step's demand.  ``x_of_step(i)`` returns
    step i's tokens.  Returns one record per step: the bias the step routed
    with, the counts, MaxVio, drop rate and layer quality.  No shared
    experts (w_router has one row per routed expert); gates by ratio.
    """
    b = np.asarray(bias, dtype=np.float32).copy()
    E = b.size
    out = []
    for i in range(steps):
        x = _f64(x_of_step(i))
        T = x.shape[0]
        r = route(x, w_router, b, n_routed=E, k=k)
        dp = dispatch(r["topk_idx"], n_routed=E, cap=capacity(capacity_factor, k, T, E))
        rec = {"bias": b, "topk_idx": r["topk_idx"], "margin": r["margin"],
               "counts": dp["counts"]}
        rec.update(load_metrics(dp["counts"], dp["kept"], k, T))
        rec["quality"] = layer_quality(r["s"], r["topk_idx"], dp["pair_pos"], k)
        out.append(rec)
        b = bias_update(dp["counts"], gamma, b, T, k)
    return out


# ------------------------------------------------- FP4 expert weights

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # magnitudes of codes 0..7
MX_BLOCK = 32


def mxfp4_quantize(w):
    """FP4 (E2M1) codes with one power-of-two scale per 32 consecutive
    values of the last axis: the OCP microscaling format MXFP4, which the
    MI355X converts in hardware.  It stands in for the NVFP4 of "Under The
    Hood: Inkling", "Quantization: BF16 vs NVFP4" (FP4 values, small blocks,
    per-block scales), whose 16-value blocks with FP8 scales are Blackwell's
    format.

    For a block with largest magnitude a: X = floor(log2 a) - 2 (2 is the
    largest E2M1 exponent), clamped to [-127, 127], and X = -127 when a = 0.
    Each value v becomes the E2M1 magnitude nearest to |v| / 2^X (ties to
    the even code, magnitudes above 6 saturate to 6) with v's sign bit as
    bit 3 of the code.  Returns (codes uint8 [..., K], X int64 [..., K/32]).
    """
    w = _f64(w)
    K = w.shape[-1]
    assert K % MX_BLOCK == 0
    blocks = w.reshape(w.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(amax)                      # amax = m * 2^e, m in [0.5, 1)
    X = np.where(amax > 0, e.astype(np.int64) - 1 - 2, -127)
    X = np.clip(X, -127, 127)
    m = np.abs(blocks) * np.exp2(-X)[..., None].astype(np.float64)
    # the two grid magnitudes around m, then the nearer one; on a tie the
    # even code; above the top of the grid, the top
    hi = np.clip(np.searchsorted(E2M1_VALUES, m), 1, 7)     # E2M1[hi-1] < m <= E2M1[hi]
    lo = hi - 1
    d_lo = m - E2M1_VALUES[lo]
    d_hi = E2M1_VALUES[hi] - m
    mag = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    mag = np.where(m >= E2M1_VALUES[7], 7, mag)
    codes = mag + 8 * np.signbit(blocks)
    return codes.reshape(w.shape).astype(np.uint8), X.astype(np.int64)


def mxfp4_dequantize(codes, X):
    """Values of MXFP4 codes: (-1)^bit3 * E2M1[code & 7] * 2^X, float64."""
    codes = np.asarray(codes)
    K = codes.shape[-1]
    mag = E2M1_VALUES[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    blocks = mag.reshape(codes.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    return (blocks * np.exp2(np.asarray(X, dtype=np.float64))[..., None]).reshape(codes.shape)


def mxfp4_pack(codes, X):
    """Byte layout of one expert stack [E, N, K] of MXFP4 weights (K a
    multiple of 128): code bytes [E, K/128, N, 64], i.e. for each 128-value
    K tile the 64 bytes of every row n, rows consecutive, with value 2i of the
    tile in the low nibble of byte i; and scale bytes X + 127 laid out
    [E, K/128, N, 4], i.e. for each K tile the scales of its 4 blocks of 32
    values for every row n, rows consecutive.  The layout is the library's
    storage format, not the pages' (they fix only values, block size and
    scales)."""
    codes = np.asarray(codes, dtype=np.uint8)
    E, N, K = codes.shape
    if K % 128:
        raise ValueError("the code layout tiles K by 128 values")
    nib = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)   # [E, N, K/2]
    packed = np.ascontiguousarray(nib.reshape(E, N, K // 128, 64).transpose(0, 2, 1, 3))
    scales = (np.asarray(X) + 127).astype(np.uint8)                      # [E, N, K/32]
    scales = np.ascontiguousarray(scales.reshape(E, N, K // 128, 4).transpose(0, 2, 1, 3))
    return packed, scales


def silu(u):
    """silu(u) = u * sigmoid(u)."""
    return _f64(u) * sigmoid(u)


def swiglu_hidden(X, w_gate, w_up):
    """The SwiGLU hidden activations silu(X Wg^T) * (X Wu^T)."""
    X = _f64(X)
    return silu(X @ _f64(w_gate).T) * (X @ _f64(w_up).T)


def swiglu(X, w_gate, w_up, w_down):
    """One SwiGLU expert on the rows of X: (silu(X Wg^T) * (X Wu^T)) Wd^T.

    ("Under The Hood: Inkling", "MoE: the expert configuration": each expert
    is a SwiGLU FFN.)  Weights are [out, in].
    """
    return swiglu_hidden(X, w_gate, w_up) @ _f64(w_down).T


def expert_ffn(x, weights, offsets, sorted_pair, k=6):
    """Every routed expert on its rows, and every shared expert on all rows.

    ``weights`` maps ``w_gate``, ``w_up`` [E, F, d], ``w_down`` [E, d, F] and
    ``ws_gate``, ``ws_up``, ``ws_down`` (same with leading S) to arrays.
    Returns ``y_routed`` [T*k, d] in sorted-pair order (rows past the kept
    pairs stay zero) and ``y_shared`` [S, T, d].
    """
    x = _f64(x)
    T, d = x.shape
    offsets = np.asarray(offsets)
    sorted_pair = np.asarray(sorted_pair)
    E = len(offsets) - 1
    y_routed = np.zeros((T * k, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = sorted_pair[lo:hi] // k
        y_routed[lo:hi] = swiglu(x[rows], weights["w_gate"][e],
                                 weights["w_up"][e], weights["w_down"][e])
    S = len(weights["ws_gate"])
    y_shared = np.stack([swiglu(x, weights["ws_gate"][s], weights["ws_up"][s],
                                weights["ws_down"][s]) for s in range(S)]) \
        if S else np.zeros((0, T, d))
    return y_routed, y_shared


def combine(y_routed, y_shared, gates, pair_pos, k=6):
    """y_t = sum_j g[t,j] Y[pair_pos[t*k+j]] + sum_s g[t,k+s] Y_s[s,t].

    Routed slots in rank order, then the shared experts in id order (02b:
    the gate-weighted sum over the 8 contributors).  A slot dropped at its
    expert's capacity (pair_pos -1, 02d) contributes nothing; the other
    gates keep their values.
    """
    gates = _f64(gates)
    T = gates.shape[0]
    pp = np.asarray(pair_pos).reshape(T, k)
    y = np.zeros((T, np.shape(y_routed)[1]))
    yr = _f64(y_routed)
    for j in range(k):
        live = pp[:, j] >= 0          # dropped pairs (pair_pos -1) add nothing
        y[live] = y[live] + gates[live, j:j + 1] * yr[pp[live, j]]
    for s in range(len(y_shared)):
        y = y + gates[:, k + s:k + s + 1] * _f64(y_shared[s])
    return y


def bias_update(counts, gamma, bias, T, k=6):
    """b_i <- b_i + gamma * sign(Lbar - L_i), float32 state.

    ("Inkling, Dissected", 02e.)  Lbar = k*T / E, so the sign is taken
    exactly as sign(k*T - E*L_i); sign(0) = 0.  The step is one float32
    addition of float32(gamma) times the sign.
    """
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.size
    sgn = np.sign(k * T - E * counts).astype(np.float32)
    b = np.asarray(bias, dtype=np.float32)
    return (b + np.float32(gamma) * sgn).astype(np.float32)


def moe_forward(x, w_router, weights, bias, gamma, k=6, gate_norm="ratio", gate_scale=1.0,
                capacity_factor=0.0):
    """The whole layer for one batch, followed by the bias update.

    Returns the router dict, the dispatch dict, ``y_routed``, ``y_shared``,
    ``y`` [T, d] and the next bias ``bias_next`` (float32).  The bias
    update counts the demand (every selection), dropped or not.
    """
    x = _f64(x)
    T = x.shape[0]
    E = np.shape(bias)[0]
    r = route(x, w_router, bias, n_routed=E, k=k, gate_norm=gate_norm, gate_scale=gate_scale)
    dp = dispatch(r["topk_idx"], n_routed=E, cap=capacity(capacity_factor, k, T, E))
    y_routed, y_shared = expert_ffn(x, weights, dp["offsets"], dp["sorted_pair"], k)
    y = combine(y_routed, y_shared, r["gates"], dp["pair_pos"], k)
    b_next = bias_update(dp["counts"], gamma, bias, T, k)
    return {"router": r, "dispatch": dp, "y_routed": y_routed,
            "y_shared": y_shared, "y": y, "bias_next": b_next}


def moe_layer_per_token(x_t, experts, w_router, bias, k=6):
    """One token through the layer of "Inkling, Dissected" 02b, spelled out
    with plain per-expert loops and none of the batch helpers above:
    affinity of every expert, the k routed experts with the largest biased
    score picked one at a time (the lower id first on exact ties), one
    normalisation over them and the shared experts, the weighted sum of
    their outputs.  ``experts`` is a list of callables, routed experts
    first and the shared experts last.  Used on small inputs to cross-check
    the grouped ``route`` + ``expert_ffn`` + ``combine``.
    """
    x_t = _f64(x_t)
    w = _f64(w_router)
    n_routed = len(bias)
    affinity = []
    for e in range(w.shape[0]):
        z = float(np.dot(w[e], x_t))
        affinity.append(1.0 / (1.0 + np.exp(-z)) if z >= 0 else np.exp(z) / (1.0 + np.exp(z)))
    left = list(range(n_routed))
    picked = []
    while len(picked) < k:
        best = left[0]
        for e in left[1:]:
            if affinity[e] + float(bias[e]) > affinity[best] + float(bias[best]):
                best = e
        picked.append(best)
        left.remove(best)
    contributors = picked + list(range(n_routed, w.shape[0]))
    total = 0.0
    for e in contributors:
        total += affinity[e]
    y = np.zeros_like(x_t)
    for e in contributors:
        y = y + (affinity[e] / total) * experts[e](x_t)
    return y


def output_rows(tokens, x, topk_idx, gates, expert_weights, k=6, n_routed=256,
                n_shared=2, pair_pos=None):
    """y_t for a few tokens, given their routing (for large workloads).

    ``expert_weights(e)`` returns (w_gate, w_up, w_down) of expert e (shared
    experts are ids n_routed..n_routed+n_shared-1).  Experts are visited in id
    order and each expert's weights are fetched once, so the cost is one
    weight conversion per distinct expert.  Contributions are added per
    token in slot order, as ``combine`` does; with ``pair_pos`` given, routed
    slots dropped at capacity (-1) are left out.
    """
    tokens = list(tokens)
    x = _f64(x)
    topk_idx = np.asarray(topk_idx)
    gates = _f64(gates)
    need = {}
    for t in tokens:
        for j, e in enumerate(list(topk_idx[t]) + list(range(n_routed, n_routed + n_shared))):
            if j < k and pair_pos is not None and pair_pos[t * k + j] < 0:
                continue
            need.setdefault(int(e), []).append((t, j))
    contrib = {}
    for e in sorted(need):
        wg, wu, wd = expert_weights(e)
        rows = [t for t, _ in need[e]]
        ye = swiglu(x[rows], wg, wu, wd)
        for (t, j), yrow in zip(need[e], ye):
            contrib[(t, j)] = yrow
    out = np.zeros((len(tokens), x.shape[1]))
    for n, t in enumerate(tokens):
        for j in range(k + n_shared):
            if (t, j) in contrib:
                out[n] = out[n] + gates[t, j] * contrib[(t, j)]
    return out
