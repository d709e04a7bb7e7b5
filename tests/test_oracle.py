"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values
the pages print, closed forms, brute-force enumeration, invariants, or a
special case that reduces to a library routine.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit, log_expit, logsumexp

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- sigmoid

def test_sigmoid_matches_library_and_closed_forms():
    z = np.linspace(-40.0, 40.0, 2001)
    assert np.array_equal(O.sigmoid(np.zeros(3)), np.full(3, 0.5))
    np.testing.assert_allclose(O.sigmoid(z), expit(z), rtol=1e-15, atol=0)
    # sigma(-z) = 1 - sigma(z)
    np.testing.assert_allclose(O.sigmoid(-z), 1.0 - O.sigmoid(z), rtol=0, atol=2e-16)
    assert O.sigmoid(np.array([math.log(3.0)]))[0] == pytest.approx(0.75, abs=1e-16)


# ------------------------------------------------- worked example (02c)

def test_worked_example_page_02c():
    g = _golden("p1_02c_worked_example.json")
    k = g["k"]
    s = O.sigmoid(np.array([g["logits"]]))
    np.testing.assert_allclose(s[0], g["affinity_printed"], atol=5e-4)

    top, _ = O.select_topk(s, k)
    assert list(top[0]) == g["unbiased"]["top"]
    gates, _ = O.joint_gates(s, top, [])
    np.testing.assert_allclose(gates[0], g["unbiased"]["gates_printed"], atol=1.5e-3)

    b = np.array(g["bias"])
    key = s + b[None, :]
    np.testing.assert_allclose(key[0], g["biased"]["scores_printed"], atol=1.5e-3)
    top_b, _ = O.select_topk(key, k)
    assert list(top_b[0]) == g["biased"]["top"]
    # the new pair's gates use the affinities without the bias
    gates_b, _ = O.joint_gates(s, top_b, [])
    np.testing.assert_allclose(gates_b[0], g["biased"]["gates_printed"], atol=1.5e-3)

    sn = g["strong_need"]
    key = np.array([sn["affinity"]]) + np.array([sn["bias"]])
    top_s, _ = O.select_topk(key, k)
    assert sn["must_keep"] in top_s[0]


# ------------------------------------------------ top-k by brute force

def _brute_force_topk(key, k):
    """The unique k-subset A with: for all a in A, o not in A,
    key_a > key_o or (key_a == key_o and a < o); listed in rank order."""
    n = len(key)
    found = []
    for A in itertools.combinations(range(n), k):
        rest = [o for o in range(n) if o not in A]
        if all(key[a] > key[o] or (key[a] == key[o] and a < o) for a in A for o in rest):
            found.append(A)
    assert len(found) == 1
    A = list(found[0])
    # rank order: bubble the chosen ids by (key desc, id asc) with plain loops
    for i in range(len(A)):
        for j in range(len(A) - 1 - i):
            a, c = A[j], A[j + 1]
            if key[c] > key[a] or (key[c] == key[a] and c < a):
                A[j], A[j + 1] = c, a
    return A


@pytest.mark.parametrize("k", [6, 3])
def test_topk_brute_force_8_expert_toys(k):
    rng = np.random.default_rng(1234 + k)
    for trial in range(300):
        if trial % 3 == 0:
            # coarse grid: exact ties are frequent
            key = rng.integers(0, 4, size=8) / 4.0
        else:
            s = expit(rng.normal(size=8))
            b = rng.uniform(-0.05, 0.05, size=8)
            key = s + b
        top, margin = O.select_topk(key[None, :], k)
        assert list(top[0]) == _brute_force_topk(list(key), k)
        ks = sorted(key, reverse=True)
        assert margin[0] == ks[k - 1] - ks[k]


def test_uniform_scores_reduce_to_index_order():
    # W_r = 0 gives s = 0.5 for every expert; with b = 0 the top-6 are 0..5
    # and each of the 8 gates is exactly 1/8.
    T, d = 5, 16
    r = O.route(np.ones((T, d)), np.zeros((258, d)), np.zeros(256))
    assert np.array_equal(r["topk_idx"], np.tile(np.arange(6), (T, 1)))
    assert np.array_equal(r["gates"], np.full((T, 8), 0.125))
    assert np.array_equal(r["idx"][:, 6:], np.tile([256, 257], (T, 1)))


# ---------------------------------------------------------------- gates

def _rand_router(T=64, d=32, E=256, S=2, seed=0, bias_range=0.05):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, d))
    w = rng.normal(size=(E + S, d)) / math.sqrt(d)
    b = rng.uniform(-bias_range, bias_range, size=E)
    return x, w, b


def test_gate_invariants_and_contributor_count():
    x, w, b = _rand_router(seed=1)
    r = O.route(x, w, b)
    g = r["gates"]
    assert g.shape == (64, 8)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(g > 0) and np.all(g < 1)
    for t in range(64):
        routed = r["idx"][t, :6]
        assert len(set(routed)) == 6 and np.all(routed < 256) and np.all(routed >= 0)
        assert list(r["idx"][t, 6:]) == [256, 257]


def test_logsigmoid_against_library_and_closed_forms():
    z = np.concatenate([np.linspace(-800, 800, 4001), [-1e-300, 0.0, 1e-300]])
    np.testing.assert_allclose(O.logsigmoid(z), log_expit(z), rtol=1e-15, atol=1e-300)
    assert O.logsigmoid(0.0) == pytest.approx(-np.log(2.0), rel=1e-16)
    # far left: log sigmoid(z) = z - log1p(exp(z)) -> z; far right: -exp(-z)
    assert O.logsigmoid(-700.0) == -700.0
    assert O.logsigmoid(40.0) == pytest.approx(-np.exp(-40.0), rel=1e-15)


def test_logsumexp_gates_against_ratio_and_scale():
    # the two normalisations agree in exact arithmetic; the scale multiplies
    x, w, b = _rand_router(seed=7)
    r = O.route(x, w, b)
    shared = [256, 257]
    g_ratio, idx = O.joint_gates(r["s"], r["topk_idx"], shared)
    g_lse, idx2 = O.joint_gates_logsumexp(r["z"], r["topk_idx"], shared)
    assert np.array_equal(idx, idx2)
    np.testing.assert_allclose(g_lse, g_ratio, rtol=1e-13, atol=0)
    np.testing.assert_allclose(g_lse.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    g_lse8, _ = O.joint_gates_logsumexp(r["z"], r["topk_idx"], shared, scale=6.5)
    np.testing.assert_allclose(g_lse8, 6.5 * g_lse, rtol=1e-15, atol=0)
    g_ratio8, _ = O.joint_gates(r["s"], r["topk_idx"], shared, scale=6.5)
    np.testing.assert_allclose(g_ratio8, 6.5 * g_ratio, rtol=1e-15, atol=0)
    # route() picks the form; the selection is the same
    r2 = O.route(x, w, b, gate_norm="logsumexp", gate_scale=6.5)
    assert np.array_equal(r2["topk_idx"], r["topk_idx"])
    np.testing.assert_allclose(r2["gates"], g_lse8, rtol=0, atol=0)
    with pytest.raises(ValueError):
        O.route(x, w, b, gate_norm="softmax")


def test_logsumexp_gates_hand_example():
    # one token, 2 routed of 3 plus one shared expert: z = [0, ln 3, -ln 3 | 0]
    # keeps experts 1 and 0 (s = 3/4, 1/2), shared s = 1/2; sum = 7/4
    z = np.array([[0.0, np.log(3.0), -np.log(3.0), 0.0]])
    top = np.array([[1, 0]])
    g, idx = O.joint_gates_logsumexp(z, top, [3], scale=8.0)
    assert list(idx[0]) == [1, 0, 3]
    np.testing.assert_allclose(g[0], 8.0 * np.array([3 / 7, 2 / 7, 2 / 7]), rtol=1e-15)
    # extreme logits stay finite (log domain)
    zx = np.array([[-900.0, 900.0, 0.0, -900.0]])
    gx, _ = O.joint_gates_logsumexp(zx, np.array([[1, 2]]), [3])
    assert np.all(np.isfinite(gx)) and gx[0, 0] == pytest.approx(2.0 / 3.0, rel=1e-15)


def test_gates_match_log_domain_normalisation():
    # Hugging Face write-up: log-sigmoid -> logsumexp over the joint set of 8
    # equals the ratio of sigmoids (before its extra route scaling).
    x, w, b = _rand_router(seed=2)
    r = O.route(x, w, b)
    zsel = np.take_along_axis(r["z"], r["idx"], axis=1)
    ls = log_expit(zsel)
    g_log = np.exp(ls - logsumexp(ls, axis=1, keepdims=True))
    np.testing.assert_allclose(r["gates"], g_log, rtol=1e-12, atol=0)


def test_bias_steers_selection_only():
    x, w, b = _rand_router(seed=3)
    r_b = O.route(x, w, b)
    r_0 = O.route(x, w, np.zeros(256))
    same = np.all(np.sort(r_b["topk_idx"], 1) == np.sort(r_0["topk_idx"], 1), axis=1)
    assert same.sum() > 0
    # same chosen set => identical gates (as a multiset over the same experts)
    for t in np.nonzero(same)[0]:
        gb = dict(zip(r_b["idx"][t], r_b["gates"][t]))
        g0 = dict(zip(r_0["idx"][t], r_0["gates"][t]))
        for e in gb:
            assert gb[e] == pytest.approx(g0[e], rel=1e-15, abs=0)
    # gates are computed from raw sigmoids of the router logits
    s_sel = np.take_along_axis(expit(x @ w.T), r_b["idx"], 1)
    np.testing.assert_allclose(r_b["gates"], s_sel / s_sel.sum(1, keepdims=True),
                               rtol=1e-14)


def test_bias_only_flips_near_ties():
    # If i is in the unbiased top-6 and s_i - s_(7) > 2 max|b|, i stays kept.
    for seed in range(20):
        x, w, b = _rand_router(T=128, seed=100 + seed, bias_range=0.02)
        r_b = O.route(x, w, b)
        s = r_b["s"][:, :256]
        top0, _ = O.select_topk(s, 6)
        s7 = np.sort(s, axis=1)[:, -7]
        bound = 2 * np.abs(b).max()
        for t in range(128):
            for i in top0[t]:
                if s[t, i] - s7[t] > bound:
                    assert i in r_b["topk_idx"][t]


# ------------------------------------------------------------- dispatch

def test_dispatch_matches_explicit_loops():
    rng = np.random.default_rng(5)
    E, k, T = 16, 3, 37
    top = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    dp = O.dispatch(top, n_routed=E)
    counts = [0] * E
    for t in range(T):
        for j in range(k):
            counts[top[t, j]] += 1
    expect_sorted = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if top[t, j] == e:
                    expect_sorted.append(t * k + j)
    assert list(dp["counts"]) == counts
    assert list(dp["offsets"]) == [sum(counts[:e]) for e in range(E + 1)]
    assert list(dp["sorted_pair"]) == expect_sorted
    for pos, p in enumerate(expect_sorted):
        assert dp["pair_pos"][p] == pos


def test_dispatch_invariants_large():
    x, w, b = _rand_router(T=512, seed=6)
    r = O.route(x, w, b)
    dp = O.dispatch(r["topk_idx"])
    assert dp["counts"].sum() == 512 * 6
    sp = dp["sorted_pair"]
    assert np.array_equal(np.sort(sp), np.arange(512 * 6))
    assert np.array_equal(dp["pair_pos"][sp], np.arange(512 * 6))
    flat = r["topk_idx"].ravel()
    for e in range(256):
        seg = sp[dp["offsets"][e]:dp["offsets"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)


def test_capacity_dispatch_matches_explicit_loops():
    # walk the pairs in ascending pair number; each expert keeps its first
    # `cap` pairs ("Inkling, Dissected" 02d; drop order: ascending token)
    rng = np.random.default_rng(11)
    E, k, T = 8, 3, 41
    top = np.stack([rng.choice(E, size=k, replace=False, p=np.r_[0.4, [0.6 / 7] * 7])
                    for _ in range(T)])
    for cap in (1, 5, 12, 1000):
        dp = O.dispatch(top, n_routed=E, cap=cap)
        seen = [0] * E
        kept_pairs = {e: [] for e in range(E)}
        dropped = []
        for p in range(T * k):
            e = top[p // k, p % k]
            if seen[e] < cap:
                kept_pairs[e].append(p)
            else:
                dropped.append(p)
            seen[e] += 1
        assert list(dp["counts"]) == seen
        assert list(dp["kept"]) == [min(c, cap) for c in seen]
        expect_sorted = [p for e in range(E) for p in kept_pairs[e]]
        assert list(dp["sorted_pair"]) == expect_sorted
        assert list(dp["offsets"]) == [sum(min(c, cap) for c in seen[:e]) for e in range(E + 1)]
        for pos, p in enumerate(expect_sorted):
            assert dp["pair_pos"][p] == pos
        for p in dropped:
            assert dp["pair_pos"][p] == -1
    # a capacity at or above every load changes nothing
    full = O.dispatch(top, n_routed=E)
    big = O.dispatch(top, n_routed=E, cap=int(full["counts"].max()))
    for key in ("counts", "offsets", "sorted_pair", "pair_pos"):
        assert np.array_equal(full[key], big[key])


def test_capacity_value_and_load_metrics():
    # C = ceil(cf * k*T / E), cf rounded to float32 first
    assert O.capacity(1.25, 6, 2048, 64) == 240
    assert O.capacity(1.0, 6, 2048, 64) == 192
    assert O.capacity(1.25, 6, 16384, 256) == 480
    assert O.capacity(0.0, 6, 2048, 64) is None
    assert O.capacity(1.1, 6, 100, 256) == 3           # 1.1f * 600 / 256 = 2.578...
    assert O.capacity(1.0, 6, 1, 256) == 1             # 6/256 rounds up to one row
    # MaxVio: hottest demand over the ideal load, minus 1; drop rate over k*T slots
    E, k, T = 4, 2, 8                                   # ideal load 4
    m = O.load_metrics([4, 4, 4, 4], [4, 4, 4, 4], k, T)
    assert m == {"max_vio": 0.0, "drop_rate": 0.0}
    m = O.load_metrics([8, 4, 2, 2], [5, 4, 2, 2], k, T)
    assert m["max_vio"] == 1.0 and m["drop_rate"] == 3 / 16


def test_layer_quality_hand_example():
    """02g's quality: gate-weighted affinity of the surviving pairs over the
    unbiased, uncapacitated top-k's, summed over the batch.  One token with
    s = (0.8, 0.6, 0.2), k = 2: the unbiased pick {0, 1} captures
    (0.64 + 0.36) / 1.4 = 1/1.4."""
    s = np.array([[0.8, 0.6, 0.2]])
    ref = 1.0 / 1.4
    # bias swapped expert 1 for 2, nothing dropped: (0.64 + 0.04) / 1.0
    assert abs(O.layer_quality(s, [[0, 2]], [0, 1], k=2) - 0.68 / ref) < 1e-15
    # expert 2's pair dropped: its share is lost, expert 0's gate stays 0.8
    assert abs(O.layer_quality(s, [[0, 2]], [0, -1], k=2) - 0.64 / ref) < 1e-15
    # unbiased pick with expert 0 dropped: only 0.6 * 0.6 / 1.4 survives
    assert abs(O.layer_quality(s, [[0, 1]], [-1, 0], k=2) - 0.36) < 1e-15
    # slot order does not matter
    assert abs(O.layer_quality(s, [[2, 0]], [1, 0], k=2) - 0.68 / ref) < 1e-15
    # a batch is a ratio of sums, not a mean of ratios: a second token with
    # equal affinities 0.5 captures 0.5 whatever it picks
    s2 = np.array([[0.8, 0.6, 0.2], [0.5, 0.5, 0.5]])
    q = O.layer_quality(s2, [[0, 2], [1, 2]], [0, 1, 2, 3], k=2)
    assert abs(q - (0.68 + 0.5) / (ref + 0.5)) < 1e-15


def test_layer_quality_limits():
    rng = np.random.default_rng(5)
    s = rng.uniform(0.05, 0.95, size=(300, 64))
    top, _ = O.select_topk(s, 6)
    # unbiased and nothing dropped: exactly the oracle
    assert O.layer_quality(s, top, np.arange(300 * 6), k=6) == 1.0
    # everything dropped: nothing captured
    assert O.layer_quality(s, top, np.full(300 * 6, -1), k=6) == 0.0
    # dropping pairs of the unbiased selection only loses what they carried
    pp = np.arange(300 * 6)
    pp[::7] = -1
    q = O.layer_quality(s, top, pp, k=6)
    assert 0.8 < q < 0.9


def test_balance_lab_two_step_toy():
    """Four experts, k = 2, four identical tokens, capacity 1.0 x ideal
    (C = 2): step 0 piles every token on experts 0 and 1 (MaxVio 1, half
    the slots dropped, tokens 2 and 3 lose both pairs); the bias then moves
    by gamma = 0.3 against the load and step 1 picks experts 2 and 0."""
    E, k, T = 4, 2, 4
    z = np.array([2.0, 1.9, 0.0, -1.0])
    x = np.tile(z, (T, 1))
    w = np.eye(E)
    recs = O.balance_lab(lambda i: x, w, np.zeros(E, np.float32), 0.3, 1.0, 2, k=k)
    sg = [1.0 / (1.0 + math.exp(-v)) for v in z]
    # step 0
    r0 = recs[0]
    assert np.array_equal(r0["counts"], [4, 4, 0, 0])
    assert r0["max_vio"] == 1.0 and r0["drop_rate"] == 0.5
    assert np.array_equal(r0["topk_idx"], np.tile([0, 1], (T, 1)))
    assert abs(r0["quality"] - 0.5) < 1e-15
    # step 1: keys s - 0.3, s - 0.3, s + 0.3, s + 0.3
    r1 = recs[1]
    assert np.array_equal(r1["bias"], np.float32([-0.3, -0.3, 0.3, 0.3]))
    assert np.array_equal(r1["topk_idx"], np.tile([2, 0], (T, 1)))
    assert np.array_equal(r1["counts"], [4, 0, 4, 0])
    assert r1["max_vio"] == 1.0 and r1["drop_rate"] == 0.5
    got = (sg[2] ** 2 + sg[0] ** 2) / (sg[2] + sg[0])
    best = (sg[0] ** 2 + sg[1] ** 2) / (sg[0] + sg[1])
    assert abs(r1["quality"] - 2 * got / (4 * best)) < 1e-14
    # without a bias step the trajectory stands still
    still = O.balance_lab(lambda i: x, w, np.zeros(E, np.float32), 0.0, 1.0, 3, k=k)
    assert all(np.array_equal(r["counts"], [4, 4, 0, 0]) for r in still)
    assert all(not r["bias"].any() for r in still)


def test_combine_skips_dropped_slots():
    rng = np.random.default_rng(12)
    T, k, d = 5, 3, 4
    yr = rng.normal(size=(T * k, d))
    ys = rng.normal(size=(2, T, d))
    g = rng.uniform(0.1, 1.0, size=(T, k + 2))
    pp = rng.permutation(T * k)
    pp[[1, 7, 8]] = -1
    y = O.combine(yr, ys, g, pp, k)
    for t in range(T):
        want = np.zeros(d)
        for j in range(k):
            if pp[t * k + j] >= 0:
                want = want + g[t, j] * yr[pp[t * k + j]]
        want = want + g[t, k] * ys[0, t] + g[t, k + 1] * ys[1, t]
        np.testing.assert_allclose(y[t], want, rtol=1e-15, atol=1e-15)


# ---------------------------------------------- expert FFN + combine

def _torch_swiglu(x, wg, wu, wd):
    x, wg, wu, wd = (torch.as_tensor(np.asarray(a, np.float64)) for a in (x, wg, wu, wd))
    return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T) @ wd.T).numpy()


def _rand_weights(E, S, d, F, seed):
    rng = np.random.default_rng(seed)
    return {"w_gate": rng.normal(size=(E, F, d)) / math.sqrt(d),
            "w_up": rng.normal(size=(E, F, d)) / math.sqrt(d),
            "w_down": rng.normal(size=(E, d, F)) / math.sqrt(F),
            "ws_gate": rng.normal(size=(S, F, d)) / math.sqrt(d),
            "ws_up": rng.normal(size=(S, F, d)) / math.sqrt(d),
            "ws_down": rng.normal(size=(S, d, F)) / math.sqrt(F)}


def test_identical_experts_reduce_to_dense_swiglu():
    # With one weight set shared by all 258 experts, sum(g) = 1 makes the
    # layer a plain dense SwiGLU MLP whatever the routing.
    T, d, F = 48, 32, 16
    x, w, b = _rand_router(T=T, d=d, seed=7)
    one = _rand_weights(1, 1, d, F, seed=8)
    weights = {"w_gate": np.repeat(one["w_gate"], 256, 0),
               "w_up": np.repeat(one["w_up"], 256, 0),
               "w_down": np.repeat(one["w_down"], 256, 0),
               "ws_gate": np.repeat(one["w_gate"], 2, 0),
               "ws_up": np.repeat(one["w_up"], 2, 0),
               "ws_down": np.repeat(one["w_down"], 2, 0)}
    out = O.moe_forward(x, w, weights, b, 1e-3)
    dense = _torch_swiglu(x, one["w_gate"][0], one["w_up"][0], one["w_down"][0])
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-13)


def test_single_active_expert_isolates_gate_slot():
    # Zero every down projection except expert e*: y_t is then g_t[slot of e*]
    # times that expert's SwiGLU output for tokens routed to e*, else 0.
    T, d, F, E = 64, 16, 8, 256
    x, w, b = _rand_router(T=T, d=d, seed=9)
    weights = _rand_weights(E, 2, d, F, seed=10)
    r = O.route(x, w, b)
    e_star = int(np.bincount(r["topk_idx"].ravel(), minlength=E).argmax())
    weights["w_down"] = np.zeros_like(weights["w_down"])
    weights["w_down"][e_star] = _rand_weights(1, 1, d, F, seed=11)["w_down"][0]
    weights["ws_down"] = np.zeros_like(weights["ws_down"])
    out = O.moe_forward(x, w, weights, b, 1e-3)
    ye = _torch_swiglu(x, weights["w_gate"][e_star], weights["w_up"][e_star],
                       weights["w_down"][e_star])
    s = expit(x @ w.T)
    for t in range(T):
        if e_star in r["topk_idx"][t]:
            sel = list(r["topk_idx"][t]) + [256, 257]
            g = s[t, e_star] / s[t, sel].sum()
            np.testing.assert_allclose(out["y"][t], g * ye[t], rtol=1e-12, atol=1e-14)
        else:
            assert np.all(out["y"][t] == 0)


def test_down_projection_linearity():
    T, d, F = 40, 16, 8
    x, w, b = _rand_router(T=T, d=d, seed=12)
    weights = _rand_weights(256, 2, d, F, seed=13)
    y1 = O.moe_forward(x, w, weights, b, 1e-3)["y"]
    w2 = dict(weights)
    w2["w_down"] = weights["w_down"] * 2.0
    w2["ws_down"] = weights["ws_down"] * 2.0
    y2 = O.moe_forward(x, w, w2, b, 1e-3)["y"]
    assert np.array_equal(y2, 2.0 * y1)


def test_grouped_matches_per_token_loops():
    T, d, F = 24, 16, 8
    x, w, b = _rand_router(T=T, d=d, seed=14)
    weights = _rand_weights(256, 2, d, F, seed=15)
    out = O.moe_forward(x, w, weights, b, 1e-3)
    experts = []
    for e in range(256):
        experts.append(lambda v, e=e: _torch_swiglu(v[None], weights["w_gate"][e],
                                                    weights["w_up"][e],
                                                    weights["w_down"][e])[0])
    for s_ in range(2):
        experts.append(lambda v, s_=s_: _torch_swiglu(v[None], weights["ws_gate"][s_],
                                                      weights["ws_up"][s_],
                                                      weights["ws_down"][s_])[0])
    for t in range(T):
        yt = O.moe_layer_per_token(x[t], experts, w, b)
        np.testing.assert_allclose(out["y"][t], yt, rtol=1e-12, atol=1e-14)
    # sampled-row helper agrees as well
    get = lambda e: ((weights["w_gate"][e], weights["w_up"][e], weights["w_down"][e])
                     if e < 256 else (weights["ws_gate"][e - 256], weights["ws_up"][e - 256],
                                      weights["ws_down"][e - 256]))
    rows = O.output_rows([0, 5, 23], x, out["router"]["topk_idx"],
                         out["router"]["gates"], get)
    np.testing.assert_allclose(rows, out["y"][[0, 5, 23]], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------- bias update

def test_bias_accumulates_page_02e():
    g = _golden("p1_02e_bias_accumulates.json")
    T, k, E = 128, 6, 256            # ideal load = 3
    counts = np.full(E, 3)
    counts[0] = 10                   # overloaded
    counts[1], counts[2], counts[3] = 1, 0, 1   # underloaded (total kept at k*T)
    assert counts.sum() == k * T
    b = np.zeros(E, np.float32)
    for _ in range(g["batches"]):
        b = O.bias_update(counts, g["gamma"], b, T, k)
    assert b.dtype == np.float32
    assert b[0] == pytest.approx(g["expected_overloaded"], abs=1e-6)
    assert b[1] == pytest.approx(-g["expected_overloaded"], abs=1e-6)
    assert np.all(b[counts == 3] == 0.0)      # sign(0) = 0: untouched


def test_bias_update_single_step_exact():
    T, k = 64, 6                      # ideal load 1.5 is never hit exactly
    counts = np.array([0, 1, 2, 3] * 64)
    b0 = np.linspace(-0.1, 0.1, 256).astype(np.float32)
    b1 = O.bias_update(counts, 1e-3, b0, T, k)
    step = np.float32(1e-3)
    expect = np.where(counts < 1.5, b0 + step, b0 - step).astype(np.float32)
    assert np.array_equal(b1, expect)


# ---------------------------------------------- FP4 (MXFP4) expert weights

def _e2m1_from_bits(code):
    # sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is subnormal
    sgn = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    return sgn * (m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))


def test_mxfp4_value_table_from_bit_definition():
    codes = np.arange(16, dtype=np.uint8).reshape(1, 16).repeat(2, axis=1)   # K = 32
    for X in (-127, -3, 0, 5, 127):
        got = O.mxfp4_dequantize(codes, np.array([[X]]))[0]
        want = [_e2m1_from_bits(c) * 2.0 ** X for c in codes[0]]
        assert np.array_equal(got, want)


def test_mxfp4_scale_exponent_and_ties():
    # a block whose largest magnitude lies in [4, 8) keeps scale 2^0, so the
    # values below land on the grid as given; ties go to the even code
    vals = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -5.0, 0.3, 6.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -0.0, -4.0, 0.5, 6.0]
    w = np.zeros((1, 32))
    w[0, :len(vals)] = vals
    c, X = O.mxfp4_quantize(w)
    assert X[0, 0] == 0
    d = O.mxfp4_dequantize(c, X)[0, :len(vals)]
    assert np.array_equal(d, want) and np.signbit(d[8])
    # X = floor(log2 amax) - 2: amax 3.9 -> -1, 4.0 -> 0, 1e-3 -> -12; zeros -> -127
    for amax, xw in ((3.9, -1), (4.0, 0), (7.99, 0), (8.0, 1), (1e-3, -12), (0.0, -127)):
        w = np.zeros((1, 32))
        w[0, 5] = amax
        assert O.mxfp4_quantize(w)[1][0, 0] == xw, amax
    # the exponent clamps at the top of the E8M0 range
    w = np.zeros((1, 32)); w[0, 0] = 2.0 ** 200
    assert O.mxfp4_quantize(w)[1][0, 0] == 127


def test_mxfp4_error_bound_and_round_trip():
    rng = np.random.default_rng(21)
    w = rng.normal(size=(64, 256)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))
    c, X = O.mxfp4_quantize(w)
    d = O.mxfp4_dequantize(c, X)
    scale = np.repeat(np.exp2(X.astype(float)), 32, axis=1)
    m = np.abs(w) / scale
    # nearest grid point: half the local spacing, at most 1 below 6; saturation above 6
    bound = np.where(m > 6.0, m - 6.0, np.where(m > 4, 1.0, np.where(m > 2, 0.5, 0.25))) * scale
    assert np.all(np.abs(w - d) <= bound + 0.0)
    # values already on the grid come back exactly
    c2, X2 = O.mxfp4_quantize(d)
    assert np.array_equal(O.mxfp4_dequantize(c2, X2), d)


def test_mxfp4_pack_layout():
    # E=1, N=3, K=256: code of row n, value k is (3n + k) mod 16
    n_, k_ = np.meshgrid(np.arange(3), np.arange(256), indexing="ij")
    codes = ((3 * n_ + k_) % 16).astype(np.uint8).reshape(1, 3, 256)
    X = np.zeros((1, 3, 8), dtype=np.int64)
    X[0, 1, :] = [3, -4, 0, 1, 2, 5, -127, 127]
    packed, scales = O.mxfp4_pack(codes, X)
    assert packed.shape == (1, 2, 3, 64)              # [E, K/128, N, 64]
    assert packed[0, 0, 0, 0] == 0x10                 # row 0, values 0, 1
    assert packed[0, 0, 0, 7] == 0xFE                 # row 0, values 14, 15
    assert packed[0, 1, 2, 0] == 0x76                 # row 2, values 128, 129: 6, 7
    assert packed[0, 1, 1, 63] == 0x21                # row 1, values 254, 255: 1, 2
    flat = packed.reshape(-1)                         # K tile 1 starts after 3 rows of tile 0
    assert flat[3 * 64] == packed[0, 1, 0, 0] == 0x10  # row 0, values 128, 129: 0, 1
    assert scales.shape == (1, 2, 3, 4)               # [E, K/128, N, 4]
    assert list(scales[0, 0, 1]) == [130, 123, 127, 128]   # row 1, blocks 0..3
    assert list(scales[0, 1, 1]) == [129, 132, 0, 254]     # row 1, blocks 4..7
    assert list(scales[0, 1, 0]) == [127] * 4
    assert scales.reshape(-1)[12 + 4] == 129          # tile 1 starts after 3 rows x 4 bytes
    with pytest.raises(ValueError):
        O.mxfp4_pack(codes[:, :, :192], X[:, :, :6])
