"""Pins for the CPU oracle: hand-derived trees, closed forms, brute force,
exact rationals, the CART special case and invariants.

None of the expected values below come from the oracle itself or from the GPU
path: they are hand-derived (tests/golden), exact rational arithmetic over row
sets, a textbook CART written out here, or sklearn.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle


def _params(d):
    return oracle.make_params(**d)


def _frac(pair):
    return Fraction(pair[0], pair[1])


def _traverse(tree, row):
    v = 0
    while not (tree[v]["flags"] & oracle.LEAF):
        f = int(tree[v]["feature"])
        v = int(tree[v]["left"]) if int(row[f]) <= int(tree[v]["threshold_bin"]) else int(tree[v]["right"])
    return v


def _node_rows(tree, bins):
    """Row set of every node, by routing each row down the tree (not via the oracle's partition)."""
    n_nodes = len(tree)
    rows = {v: [] for v in range(n_nodes)}
    for i in range(bins.shape[0]):
        v = 0
        rows[0].append(i)
        while not (tree[v]["flags"] & oracle.LEAF):
            f = int(tree[v]["feature"])
            v = int(tree[v]["left"]) if int(bins[i, f]) <= int(tree[v]["threshold_bin"]) else int(tree[v]["right"])
            rows[v].append(i)
    return rows


def _run_golden(path):
    with open(path) as fh:
        gd = json.load(fh)
    inp = gd["inputs"]
    bins = np.array(inp["bins"], dtype=np.uint8)
    label = np.array(inp["label"], dtype=np.float32)
    p = _params(inp["params"])
    r = oracle.train(bins, inp["n_bins"], label, p, 1, base_score=inp["base_score"], dump_tree=0)
    return gd, r


@pytest.mark.parametrize("name", ["example_a.json", "example_d.json"])
def test_hand_trees_node_by_node(golden_dir, name):
    gd, r = _run_golden(os.path.join(golden_dir, name))
    exp = gd["expected"]
    tree = r["nodes"][0]
    assert int(r["n_nodes"][0]) == len(exp["nodes"])
    assert int(r["scale"][0]) == exp["scale"]
    for v, e in enumerate(exp["nodes"]):
        nd = tree[v]
        assert int(nd["feature"]) == e["feature"]
        assert int(nd["threshold_bin"]) == e["threshold_bin"]
        assert int(nd["left"]) == e["left"]
        assert int(nd["right"]) == e["right"]
        assert bool(nd["flags"] & oracle.LEAF) == e["leaf"]
        if e["leaf"]:
            want = _frac(e["leaf_value_exact"])
            got = float(nd["leaf_value"])
            # one IEEE division of exact operands: the correctly rounded value
            assert got == float(want)
            if e.get("leaf_value_negative_zero"):
                assert got == 0.0 and math.copysign(1.0, got) < 0
        else:
            want = _frac(e["gain_exact"])
            assert abs(Fraction(float(nd["gain"])) - want) <= abs(want) * Fraction(1, 2**50)
    if "root_gain_fp64_hex" in exp:
        assert float(tree[0]["gain"]).hex() == exp["root_gain_fp64_hex"]
    for i, pe in enumerate(exp["pred_exact"]):
        assert r["pred"][i] == float(_frac(pe))
    for i in exp.get("pred_positive_zero_rows", []):
        assert math.copysign(1.0, r["pred"][i]) > 0


def test_tie_rules(golden_dir):
    with open(os.path.join(golden_dir, "ties.json")) as fh:
        gd = json.load(fh)
    for case in gd["cases"]:
        bins = np.array(case["bins"], dtype=np.uint8)
        label = np.array(case["label"], dtype=np.float32)
        r = oracle.train(bins, case["n_bins"], label, _params(case["params"]), 1)
        root = r["nodes"][0][0]
        assert int(root["feature"]) == case["expected_root"]["feature"], case["name"]
        assert int(root["threshold_bin"]) == case["expected_root"]["threshold_bin"], case["name"]


def _round_half_even(x: Fraction) -> int:
    return round(x)  # Fraction.__round__ rounds half to even


def test_gradient_grid_closed_form():
    # n = 5 -> L = 3; max |g| = 0.75 = 0.75 * 2^0 -> e = 0 -> S = 49
    pred = np.array([0.1, 0.2, -0.3, 0.75, 0.0])
    label = np.zeros(5, dtype=np.float32)
    k, S, _ = oracle.gradient_grid(pred, label)
    assert S == 49
    for i in range(5):
        assert int(k[i]) == _round_half_even(Fraction(float(pred[i])) * 2**49)
    # a half-way case: g0 = 1 + 2^-52 (e = 1), n = 2 (L = 1) -> S = 50,
    # g0 * 2^50 = 2^50 + 2^-2 -> 2^50; g1 = 3 * 2^-51 -> 3/2 * 1 -> ties to 2
    pred = np.array([1.0 + 2.0**-52, 3.0 * 2.0**-51])
    label = np.zeros(2, dtype=np.float32)
    k, S, _ = oracle.gradient_grid(pred, label)
    assert S == 50
    assert int(k[0]) == 2**50
    assert int(k[1]) == 2  # 1.5 rounds half to even
    pred = np.array([1.0 + 2.0**-52, 5.0 * 2.0**-51])
    k, S, _ = oracle.gradient_grid(pred, label)
    assert int(k[1]) == 2  # 2.5 rounds half to even
    # all-zero gradients -> S = 0, k = 0
    k, S, _ = oracle.gradient_grid(np.ones(3), np.ones(3, dtype=np.float32))
    assert S == 0 and not k.any()


@pytest.mark.parametrize("n", [1, 2, 3, 1000, 4097])
def test_gradient_grid_bound(n):
    rng = np.random.default_rng(n)
    pred = rng.normal(size=n) * 10.0
    label = rng.normal(size=n).astype(np.float32)
    k, S, g = oracle.gradient_grid(pred, label)
    L = math.ceil(math.log2(n)) if n > 1 else 0
    assert oracle.ceil_log2(n) == L
    assert np.abs(k).max() <= 2 ** (52 - L)
    # the grid is within half a step of g, and the total stays below 2^52
    assert np.all(np.abs(np.ldexp(k.astype(np.float64), -S) - g) <= 2.0 ** (-S - 1))
    assert abs(int(np.sum(k, dtype=object))) <= 2**52
    # the largest element uses the top of the range (M >= 2^(e-1))
    assert np.abs(k).max() >= 2 ** (52 - L - 1) - 1


def _tiny_cases():
    out = []
    for seed, (n, nbins, D, lam, gam, msl, mcw) in enumerate([
        (40, [3, 5, 2], 3, 1.0, 0.0, 1, 0.0),
        (64, [4, 4, 4, 4], 3, 0.0, 0.0, 1, 0.0),
        (57, [7, 2, 3], 4, 2.5, 0.5, 3, 0.0),
        (80, [5, 6], 3, 1.0, 0.0, 2, 2.0),
        (33, [2, 2, 2, 2, 2], 4, 1.0, 0.25, 1, 1.0),
    ]):
        out.append(dict(seed=100 + seed, n=n, n_bins=nbins, params=dict(
            max_depth=D, reg_lambda=lam, gamma=gam, min_samples_leaf=msl, min_child_weight=mcw,
            learning_rate=0.5)))
    return out


@pytest.mark.parametrize("case", _tiny_cases(), ids=lambda c: "seed%d" % c["seed"])
def test_histograms_bruteforce_and_invariants(case):
    bins, label, nb = datagen.make_random(case["n"], case["n_bins"], case["seed"], label_kind=1)
    p = _params(case["params"])
    r = oracle.train(bins, nb, label, p, 2, dump_tree=1)
    tree = r["nodes"][1][: r["n_nodes"][1]]
    k = r["dump_k"]
    rows = _node_rows(tree, bins)
    off = oracle.bin_offsets(nb)
    for v, nd in enumerate(tree):
        rv = rows[v]
        assert int(nd["count"]) == len(rv)
        assert int(nd["gsum_q"]) == sum(int(k[i]) for i in rv)
        if int(nd["depth"]) >= p.max_depth:
            continue
        cnt = r["dump_cnt"][v]
        gq = r["dump_gq"][v]
        for f in range(bins.shape[1]):
            for c in range(int(nb[f])):
                sel = [i for i in rv if int(bins[i, f]) == c]
                assert int(cnt[off[f] + c]) == len(sel)
                assert int(gq[off[f] + c]) == sum(int(k[i]) for i in sel)
            assert int(cnt[off[f]:off[f + 1]].sum()) == len(rv)
            assert int(gq[off[f]:off[f + 1]].sum()) == int(nd["gsum_q"])
        if not (nd["flags"] & oracle.LEAF) and int(tree[nd["left"]]["depth"]) < p.max_depth:
            lc, rc = int(nd["left"]), int(nd["right"])
            assert np.array_equal(cnt, r["dump_cnt"][lc] + r["dump_cnt"][rc])
            assert np.array_equal(gq, r["dump_gq"][lc] + r["dump_gq"][rc])
    # every row ends in exactly one leaf, and that leaf is the one it routes to
    for i in range(bins.shape[0]):
        assert int(r["dump_leaf_of_row"][i]) == _traverse(tree, bins[i])


def _exact_gain(GL, HL, GR, HR, GP, HP, lam, gam):
    def s(G, H):
        return G * G / (H + lam)
    return Fraction(1, 2) * (s(GL, HL) + s(GR, HR) - s(GP, HP)) - gam


@pytest.mark.parametrize("case", _tiny_cases(), ids=lambda c: "seed%d" % c["seed"])
def test_split_choice_against_exact_rationals(case):
    """Brute force over every (feature, bin), splitting the rows directly."""
    bins, label, nb = datagen.make_random(case["n"], case["n_bins"], case["seed"], label_kind=1)
    p = _params(case["params"])
    r = oracle.train(bins, nb, label, p, 1, dump_tree=0)
    tree = r["nodes"][0][: r["n_nodes"][0]]
    S = int(r["scale"][0])
    # labels are multiples of 1/8 below 8 in magnitude and pred = 0, so the grid is exact
    g = [Fraction(-float(x)) for x in label]
    assert all(Fraction(int(kk), 2**S) == gi for kk, gi in zip(r["dump_k"], g))
    lam, gam = Fraction(p.reg_lambda), Fraction(p.gamma)
    rows = _node_rows(tree, bins)
    for v, nd in enumerate(tree):
        if int(nd["depth"]) >= p.max_depth:
            continue
        rv = rows[v]
        GP, HP = sum(g[i] for i in rv), Fraction(len(rv))
        cands = []
        for f in range(bins.shape[1]):
            for t in range(int(nb[f]) - 1):
                L = [i for i in rv if int(bins[i, f]) <= t]
                R = [i for i in rv if int(bins[i, f]) > t]
                if len(L) < p.min_samples_leaf or len(R) < p.min_samples_leaf:
                    continue
                if len(L) < p.min_child_weight or len(R) < p.min_child_weight:
                    continue
                if not L or not R:
                    continue
                GL = sum(g[i] for i in L)
                cands.append((_exact_gain(GL, Fraction(len(L)), GP - GL, Fraction(len(R)), GP, HP,
                                          lam, gam), f, t, len(L)))
        tol = Fraction(1, 2**40) * (1 + abs(GP * GP))
        best = max((c[0] for c in cands), default=None)
        if nd["flags"] & oracle.LEAF:
            assert best is None or best <= tol, (v, best)
            continue
        f, t = int(nd["feature"]), int(nd["threshold_bin"])
        chosen = [c for c in cands if c[1] == f and c[2] == t]
        assert chosen, "chosen split is not a valid candidate"
        assert chosen[0][0] > -tol
        assert best - chosen[0][0] <= tol
        assert abs(Fraction(float(nd["gain"])) - chosen[0][0]) <= tol
        # among candidates whose exact gain is clearly below the best, none may win;
        # among exact ties with the same partition, the smallest (feature, bin) wins
        near = [c for c in cands if best - c[0] <= tol]
        same_part = [c for c in near if c[0] == chosen[0][0] and c[3] == chosen[0][3]]
        assert (f, t) <= min((c[1], c[2]) for c in same_part)


def _cart_fit(X, y, rows, depth_left):
    """P2-style greedy CART on SSE with exact rationals: thresholds from observed
    values, first best while folding, none for degenerate splits."""
    ys = [y[i] for i in rows]
    mean = sum(ys, Fraction(0)) / len(ys)
    if depth_left == 0:
        return ("leaf", mean)
    best = None

    def sse(idx):
        if not idx:
            return Fraction(0)
        m = sum((y[i] for i in idx), Fraction(0)) / len(idx)
        return sum(((y[i] - m) ** 2 for i in idx), Fraction(0))

    for f in range(X.shape[1]):
        for thr in sorted(set(int(X[i, f]) for i in rows)):
            L = [i for i in rows if int(X[i, f]) <= thr]
            R = [i for i in rows if int(X[i, f]) > thr]
            if not L or not R:
                continue
            sc = sse(L) + sse(R)
            if best is None or sc < best[0]:
                best = (sc, f, thr, L, R)
    if best is None:
        return ("leaf", mean)
    _, f, thr, L, R = best
    return ("split", f, thr, _cart_fit(X, y, L, depth_left - 1), _cart_fit(X, y, R, depth_left - 1))


def _cart_to_bfs(root):
    out, queue = [], [root]
    while queue:
        nxt = []
        for nd in queue:
            if nd[0] == "leaf":
                out.append(("leaf", nd[1]))
            else:
                out.append(("split", nd[1], nd[2]))
                nxt.extend([nd[3], nd[4]])
        queue = nxt
    return out


@pytest.mark.parametrize("seed", [7, 8, 9])
def test_cart_special_case(seed):
    """lambda = 0, gamma = 0, base 0, eta = 1, one tree: gain is half the SSE
    reduction and the leaf is the mean label, i.e. greedy CART on bins."""
    rng = np.random.default_rng(seed)
    n, F, D = 48, 3, 3
    bins = rng.integers(0, 12, size=(n, F)).astype(np.uint8)
    label = (rng.integers(-2**12, 2**12, size=n) / 2.0**8).astype(np.float32)
    y = [Fraction(float(v)) for v in label]
    cart = _cart_to_bfs(_cart_fit(bins, y, list(range(n)), D))
    p = oracle.make_params(D, reg_lambda=0.0, gamma=0.0, min_samples_leaf=1, learning_rate=1.0)
    r = oracle.train(bins, [12] * F, label, p, 1)
    tree = r["nodes"][0][: r["n_nodes"][0]]
    assert len(tree) == len(cart)
    for nd, c in zip(tree, cart):
        if c[0] == "leaf":
            assert nd["flags"] & oracle.LEAF
            assert float(nd["leaf_value"]) == float(c[1])
        else:
            assert (int(nd["feature"]), int(nd["threshold_bin"])) == (c[1], c[2])


def test_cart_special_case_sklearn():
    sk = pytest.importorskip("sklearn.tree")
    rng = np.random.default_rng(3)
    n, F, D = 200, 4, 4
    bins = rng.integers(0, 50, size=(n, F)).astype(np.uint8)
    label = (rng.normal(size=n) * 64).round().astype(np.float32) / np.float32(16)
    p = oracle.make_params(D, reg_lambda=0.0, gamma=0.0, min_samples_leaf=1, learning_rate=1.0)
    r = oracle.train(bins, [50] * F, label, p, 1, dump_tree=0)
    m = sk.DecisionTreeRegressor(max_depth=D, random_state=0).fit(bins.astype(np.float64), label)
    # same partition of rows into leaves, same leaf means
    ours = r["dump_leaf_of_row"]
    theirs = m.apply(bins.astype(np.float64))
    pairs = set(zip(ours.tolist(), theirs.tolist()))
    assert len(pairs) == len(set(ours.tolist())) == len(set(theirs.tolist()))
    np.testing.assert_allclose(r["pred"], m.predict(bins.astype(np.float64)), rtol=0, atol=1e-6)


@pytest.mark.parametrize("case", _tiny_cases(), ids=lambda c: "seed%d" % c["seed"])
def test_leaf_weights_closed_form(case):
    bins, label, nb = datagen.make_random(case["n"], case["n_bins"], case["seed"], label_kind=1)
    p = _params(case["params"])
    r = oracle.train(bins, nb, label, p, 1, dump_tree=0)
    tree = r["nodes"][0][: r["n_nodes"][0]]
    leaf = r["dump_leaf_of_row"]
    for v, nd in enumerate(tree):
        if not (nd["flags"] & oracle.LEAF):
            continue
        idx = np.nonzero(leaf == v)[0]
        # first tree, base 0: w = -sum(g)/(n + lambda) = sum(label)/(n + lambda),
        # the label sum is exact (multiples of 1/8), so the FP64 division matches
        s = float(sum(Fraction(float(label[i])) for i in idx))
        assert float(nd["leaf_value"]) == s / (len(idx) + p.reg_lambda) or (
            s == 0.0 and float(nd["leaf_value"]) == 0.0)


@pytest.mark.parametrize("k", [1])
def test_multi_round_predictions_by_traversal(k):
    bins, label, nb = datagen.make_workload(k)
    wl = dict(datagen.WORKLOADS[k])
    p = oracle.make_params(**wl)
    T = wl["n_trees"]
    r = oracle.train(bins, nb, label, p, T, keep_pred_per_tree=True)
    pred = np.zeros(bins.shape[0])
    for t in range(T):
        tree = r["nodes"][t][: r["n_nodes"][t]]
        for i in range(bins.shape[0]):
            w = float(tree[_traverse(tree, bins[i])]["leaf_value"])
            pred[i] = pred[i] + (p.learning_rate * w)
        assert np.array_equal(pred, r["pred_per_tree"][t])
    assert np.array_equal(pred, r["pred"])
    # the training loss falls from tree to tree
    mse = [float(np.mean((r["pred_per_tree"][t] - label) ** 2)) for t in range(T)]
    assert all(b < a for a, b in zip(mse, mse[1:]))


def test_determinism():
    bins, label, nb = datagen.make_random(3000, [16, 3, 64, 2], 11, label_kind=2)
    p = oracle.make_params(4, reg_lambda=1.0, gamma=0.1, min_samples_leaf=5, learning_rate=0.3)
    a = oracle.train(bins, nb, label, p, 4)
    b = oracle.train(bins, nb, label, p, 4)
    assert a["nodes"].tobytes() == b["nodes"].tobytes()
    assert a["pred"].tobytes() == b["pred"].tobytes()


def test_sharded_histograms_sum_to_whole():
    """Integer histograms of row shards add up bit-exactly to the whole."""
    bins, label, nb = datagen.make_random(5000, [8, 32, 2], 5)
    k, S, _ = oracle.gradient_grid(np.zeros(5000), label)
    rows = np.arange(5000, dtype=np.int32)
    whole = oracle.node_histogram(bins, nb, rows, k, S)
    parts = [oracle.node_histogram(bins, nb, sh, k, S) for sh in np.array_split(rows, 7)]
    assert np.array_equal(whole[0], sum(pp[0] for pp in parts))
    assert np.array_equal(whole[1], sum(pp[1] for pp in parts))


@pytest.mark.parametrize("bad", [
    dict(min_samples_leaf=0), dict(min_child_weight=-1.0), dict(reg_lambda=-0.5),
    dict(gamma=-1e-9), dict(reg_lambda=float("inf")), dict(gamma=float("nan")),
    dict(learning_rate=float("inf")), dict(max_depth=-1),
])
def test_parameter_rules(bad):
    kw = dict(max_depth=3)
    kw.update(bad)
    assert oracle.validate_params(**kw) != 0
    assert oracle.validate_params(max_depth=3) == 0


@pytest.mark.parametrize("case", _tiny_cases(), ids=lambda c: "seed%d" % c["seed"])
def test_structure_invariants(case):
    bins, label, nb = datagen.make_random(case["n"], case["n_bins"], case["seed"], label_kind=0)
    p = _params(case["params"])
    r = oracle.train(bins, nb, label, p, 3)
    for t in range(3):
        tree = r["nodes"][t][: r["n_nodes"][t]]
        depth_prev = 0
        expect_child = 1
        for v, nd in enumerate(tree):
            assert int(nd["depth"]) >= depth_prev
            depth_prev = int(nd["depth"])
            assert int(nd["depth"]) <= p.max_depth
            if nd["flags"] & oracle.LEAF:
                assert (int(nd["feature"]), int(nd["left"]), int(nd["right"])) == (-1, -1, -1)
                continue
            # breadth-first: children are appended in parent order, left then right
            assert int(nd["left"]) == expect_child and int(nd["right"]) == expect_child + 1
            expect_child += 2
            assert float(nd["gain"]) > 0.0
            L, R = tree[int(nd["left"])], tree[int(nd["right"])]
            assert int(L["count"]) + int(R["count"]) == int(nd["count"])
            for c in (L, R):
                assert int(c["count"]) >= p.min_samples_leaf
                assert int(c["count"]) >= p.min_child_weight
                assert int(c["depth"]) == int(nd["depth"]) + 1


def test_depth_zero_is_single_leaf():
    bins, label, nb = datagen.make_random(100, [4, 4], 1)
    p = oracle.make_params(0, learning_rate=1.0)
    r = oracle.train(bins, nb, label, p, 1)
    assert int(r["n_nodes"][0]) == 1
    root = r["nodes"][0][0]
    assert root["flags"] & oracle.LEAF
    s = float(sum(Fraction(float(x)) for x in label))
    assert abs(float(root["leaf_value"]) - s / 101.0) <= 1e-12 * (1 + abs(s))


# ---------------------------------------------------------------- binning --
# The binning reading (the Training Core page's "Quantized" state): a value's
# bin is the number of its feature's upper bounds strictly below it.

def test_binning_hand_example():
    """Bounds 1 < 2 < 3 (four bins), worked by hand: a value equal to a bound
    stays in the lower bin, -inf goes to bin 0 and +inf to bin 3, NaN to bin 0
    (and is counted).  The unused fourth entry holds -100: counting it would
    move every value up one bin."""
    x = np.array([-np.inf, 0.5, 1.0, 1.5, 2.0, 2.5, 3.0, 3.5, np.inf, np.nan], dtype=np.float32)
    upper = np.array([1.0, 2.0, 3.0, -100.0], dtype=np.float32)
    out, n_nan = oracle.bin_features(x.reshape(-1, 1), [4], upper)
    assert out[:, 0].tolist() == [0, 0, 0, 1, 1, 2, 2, 3, 3, 0]
    assert n_nan == 1


def test_binning_matches_searchsorted():
    """numpy.searchsorted(bounds, x, side='left') is the count of bounds
    strictly below x: the same definition, computed by a library routine.
    Values include every bound exactly, its float32 neighbours and +-inf."""
    rng = np.random.default_rng(11)
    nbins = [1, 2, 3, 17, 64, 255, 256, 5]
    off = oracle.bin_offsets(nbins)
    upper = np.full(int(off[-1]), 7.0, dtype=np.float32)
    bounds = []
    for f, nb in enumerate(nbins):
        b = np.unique(rng.normal(0, 2, size=3 * nb).astype(np.float32))[: nb - 1]
        assert b.shape[0] == nb - 1
        upper[off[f]: off[f] + nb - 1] = b
        bounds.append(b)
    n = 3000
    raw = rng.normal(0, 2.5, size=(n, len(nbins))).astype(np.float32)
    for f, b in enumerate(bounds):
        if b.shape[0] == 0:
            continue
        pick = rng.integers(0, b.shape[0], size=600)
        raw[:200, f] = b[pick[:200]]
        raw[200:400, f] = np.nextafter(b[pick[200:400]], np.float32(np.inf))
        raw[400:600, f] = np.nextafter(b[pick[400:600]], np.float32(-np.inf))
    raw[600, :] = np.inf
    raw[601, :] = -np.inf
    out, n_nan = oracle.bin_features(raw, nbins, upper)
    assert n_nan == 0
    for f, b in enumerate(bounds):
        want = np.searchsorted(b, raw[:, f], side="left")
        assert np.array_equal(out[:, f].astype(np.int64), want), f
    assert out[601].tolist() == [0] * len(nbins)
    assert out[600].tolist() == [nb - 1 for nb in nbins]


def test_binning_degenerate_and_bad_bounds():
    """One bin (no bounds) puts every value in bin 0; bounds that are NaN,
    equal or decreasing are rejected."""
    raw = np.array([[-1e30], [0.0], [1e30]], dtype=np.float32)
    out, n_nan = oracle.bin_features(raw, [1], np.array([5.0], dtype=np.float32))
    assert out[:, 0].tolist() == [0, 0, 0] and n_nan == 0
    for bad in ([2.0, 1.0, 0.0], [1.0, 1.0, 0.0], [np.nan, 1.0, 0.0], [0.0, np.nan, 0.0]):
        out, rc = oracle.bin_features(raw, [3], np.array(bad, dtype=np.float32))
        assert out is None and rc == -1, bad


def test_partition_order_hand_case():
    """Stable partition (Training Core, section 3 routing and section 6 step 5;
    "stable" as the pages' partition is described): rows with bin <= t go
    left, and each side keeps the order in which the rows were given.  The
    expected lists are worked out by hand below, for an input order that is
    not sorted (so a partition that sorted its output, or reversed one side,
    would fail) and for the ascending order the root starts from (each side
    then stays ascending)."""
    # row id:  0  1  2  3  4  5  6  7
    col = [3, 0, 2, 1, 3, 0, 1, 2]
    bins = np.array([[c, 7 - c] for c in col], dtype=np.uint8)
    # given order 5, 0, 3, 2, 4, 1 -> bins of feature 0: 0, 3, 1, 2, 3, 0
    left, right = oracle.partition(bins, [5, 0, 3, 2, 4, 1], 0, 1)
    assert left.tolist() == [5, 3, 1]
    assert right.tolist() == [0, 2, 4]
    # ascending ids, t = 1: left = ids with bin <= 1, right = the rest, both ascending
    left, right = oracle.partition(bins, list(range(8)), 0, 1)
    assert left.tolist() == [1, 3, 5, 6]
    assert right.tolist() == [0, 2, 4, 7]
    # feature 1 (bins 7 - col): t = 5 sends bins <= 5, i.e. col >= 2, left
    left, right = oracle.partition(bins, list(range(8)), 1, 5)
    assert left.tolist() == [0, 2, 4, 7]
    assert right.tolist() == [1, 3, 5, 6]
    # t at the top bin: everything left, nothing right; order unchanged
    left, right = oracle.partition(bins, [7, 6, 5], 0, 255)
    assert left.tolist() == [7, 6, 5] and right.tolist() == []


def test_partition_order_in_training_is_ascending():
    """Inside train(), every leaf's row list is a stable partition of the
    ascending root, so the rows of each leaf come out ascending.  The oracle
    reports the leaf of every row; rebuilding the leaves' row lists by
    repeated stable partition with the tree's own splits (feature, threshold
    from the node array) must give each leaf exactly those rows, in
    ascending order."""
    bins, label, nb = datagen.make_random(500, [9, 4, 16, 2], seed=77)
    p = oracle.make_params(max_depth=4)
    r = oracle.train(bins, nb, label, p, 1, dump_tree=0, dump_hist=False)
    tree = r["nodes"][0][: r["n_nodes"][0]]
    lists = {0: list(range(bins.shape[0]))}
    for v in range(len(tree)):
        nd = tree[v]
        if nd["flags"] & oracle.LEAF:
            continue
        left, right = oracle.partition(bins, lists[v], int(nd["feature"]), int(nd["threshold_bin"]))
        assert left.tolist() == sorted(left.tolist()) and right.tolist() == sorted(right.tolist())
        lists[int(nd["left"])], lists[int(nd["right"])] = left.tolist(), right.tolist()
    leaf_of = r["dump_leaf_of_row"]
    for v in range(len(tree)):
        if tree[v]["flags"] & oracle.LEAF:
            assert lists[v] == np.nonzero(leaf_of == v)[0].tolist()


def _oracle_tree(nodes):
    """Oracle node array from (feature, threshold_bin, left, right, leaf_value) tuples
    (a leaf has left = -1)."""
    arr = np.zeros(len(nodes), dtype=oracle.NODE_DTYPE)
    for v, (f, t, l, r, w) in enumerate(nodes):
        arr[v]["feature"], arr[v]["threshold_bin"], arr[v]["left"], arr[v]["right"] = f, t, l, r
        arr[v]["leaf_value"] = w
        arr[v]["flags"] = oracle.LEAF if l < 0 else 0
    return arr


def test_predict_hand_ensemble():
    """Forward pass of "Gradient boosted trees (spec model)": routing bin <= t to
    the left, initial prediction plus learning rate times each tree's output.
    Worked by hand: base 0.25, eta 0.5; tree 1 splits feature 0 at bin 0 into
    leaves 1.0 | 2.0; tree 2 splits feature 1 at bin 1 into leaves -1.0 | 3.0;
    tree 3 is a single leaf 0.5.  All values are dyadic, so every partial sum
    is exact."""
    t1 = _oracle_tree([(0, 0, 1, 2, 0.0), (-1, -1, -1, -1, 1.0), (-1, -1, -1, -1, 2.0)])
    t2 = _oracle_tree([(1, 1, 1, 2, 0.0), (-1, -1, -1, -1, -1.0), (-1, -1, -1, -1, 3.0)])
    t3 = _oracle_tree([(-1, -1, -1, -1, 0.5), (-1, -1, -1, -1, 0.0), (-1, -1, -1, -1, 0.0)])
    trees = np.stack([t1, t2, t3])
    bins = np.array([[0, 0], [0, 2], [1, 1], [1, 3], [3, 0]], dtype=np.uint8)
    out = oracle.predict(bins, trees, [3, 3, 1], base_score=0.25, learning_rate=0.5)
    # row: base + 0.5 * (tree1 + tree2 + tree3)
    want = [0.25 + 0.5 * (1.0 - 1.0 + 0.5), 0.25 + 0.5 * (1.0 + 3.0 + 0.5),
            0.25 + 0.5 * (2.0 - 1.0 + 0.5), 0.25 + 0.5 * (2.0 + 3.0 + 0.5),
            0.25 + 0.5 * (2.0 - 1.0 + 0.5)]
    assert out.tolist() == want
    # no trees: the initial prediction
    assert oracle.predict(bins, trees[:0], [], base_score=0.25).tolist() == [0.25] * 5


def test_predict_hand_tree_d(golden_dir):
    """The hand-derived tree of example D predicts its own hand-derived values."""
    with open(os.path.join(golden_dir, "example_d.json")) as fh:
        gd = json.load(fh)
    nodes = []
    for e in gd["expected"]["nodes"]:
        w = float(_frac(e["leaf_value_exact"])) if e["leaf"] else 0.0
        if e.get("leaf_value_negative_zero"):
            w = -0.0
        nodes.append((e["feature"], e["threshold_bin"], e["left"], e["right"], w))
    tree = _oracle_tree(nodes)
    bins = np.array(gd["inputs"]["bins"], dtype=np.uint8)
    out = oracle.predict(bins, tree, [len(nodes)], base_score=0.0, learning_rate=1.0)
    assert out.tolist() == [float(_frac(p)) for p in gd["expected"]["pred_exact"]]
    for i in gd["expected"]["pred_positive_zero_rows"]:
        assert math.copysign(1.0, out[i]) > 0


@pytest.mark.parametrize("k", [1, 3])
def test_predict_equals_training_predictions(k):
    """Two independent routes to the same numbers: training adds each leaf's
    eta*w to the rows its partitioned row list holds; the forward pass routes
    every row through the trees.  They must agree bit for bit, tree by tree."""
    bins, label, nb = datagen.make_workload(k)
    wl = dict(datagen.WORKLOADS[k])
    p = oracle.make_params(**wl)
    T = 3
    r = oracle.train(bins, nb, label, p, T, keep_pred_per_tree=True)
    for t in range(1, T + 1):
        out = oracle.predict(bins, r["nodes"][:t], r["n_nodes"][:t], 0.0, p.learning_rate)
        assert np.array_equal(out, r["pred_per_tree"][t - 1])


def test_predict_rejects_bad_trees():
    t = _oracle_tree([(0, 0, 1, 2, 0.0), (-1, -1, -1, -1, 1.0), (-1, -1, -1, -1, 2.0)])
    bins = np.array([[0], [1]], dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.predict(bins, t, [2])          # row 1 goes to a child past the node count
    bad = t.copy()
    bad[0]["feature"] = 5                     # no such feature
    with pytest.raises(ValueError):
        oracle.predict(bins, bad, [3])
    loop = _oracle_tree([(0, 0, 0, 0, 0.0)])  # a node that is its own child
    with pytest.raises(ValueError):
        oracle.predict(bins, loop, [1])


# ------------------------------------------------------------ logistic objective

def _ulps(a: float, b: float) -> int:
    import struct
    ia = struct.unpack("<q", struct.pack("<d", a))[0]
    ib = struct.unpack("<q", struct.pack("<d", b))[0]
    return abs(ia - ib)


def test_exp_neg_against_math_exp():
    """orc_exp_neg (Cody-Waite reduction + degree-13 Taylor series) stays
    within 2 ulp of the C library's exp over [-700, 0] (a dense sweep, a
    geometric sweep down to 1e-300 and the ends of the reduction interval)
    and near multiples of ln 2; e^0 = 1 exactly; arguments below -700 give 0."""
    xs = np.concatenate([-np.linspace(0.0, 700.0, 200_001), -np.geomspace(1e-300, 700.0, 20_001),
                         [-0.0, -1e-310, -0.34657359027997264, -0.6931471805599453, -709.0 + 9.0]])
    worst = max(_ulps(oracle.exp_neg(float(x)), math.exp(float(x))) for x in xs)
    assert worst <= 2, worst
    assert oracle.exp_neg(0.0) == 1.0 and oracle.exp_neg(-0.0) == 1.0
    for k in range(0, 1000, 37):
        x = -k * math.log(2.0)
        for dx in (0.0, 1e-9, -1e-9):
            y = min(x + dx, 0.0)
            assert _ulps(oracle.exp_neg(y), math.exp(y)) <= 2
    assert oracle.exp_neg(-700.5) == 0.0 and oracle.exp_neg(-1e308) == 0.0


def test_logistic_gradient_and_hessian():
    """g = sigmoid(p) - y and h = sigmoid(p) (1 - sigmoid(p)) against 50-digit
    decimal arithmetic: h within 4 ulp; g, a difference of rounded values,
    within 4 ulp of the larger of sigmoid(p) and y (the subtraction itself is
    exact or one rounding); exact values at p = 0; h is even in p bit for bit;
    g(p, y) + g(-p, 1 - y) = 0 up to one rounding of 1."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    assert oracle.logistic_gh(0.0, 0.0) == (0.5, 0.25)
    assert oracle.logistic_gh(0.0, 1.0) == (-0.5, 0.25)
    rng = np.random.default_rng(3)
    ps = np.concatenate([rng.normal(0.0, 3.0, 2000), rng.uniform(-40.0, 40.0, 500),
                         [1e-12, -1e-12, 36.0, -36.0, 699.0, -699.0, 701.0, -701.0, 1e4]])
    # beyond |p| = 700 e^-|p| is taken as 0: sigmoid is 0 or 1 and h = 0
    assert oracle.logistic_gh(-701.0, 0.0) == (0.0, 0.0)
    assert oracle.logistic_gh(701.0, 1.0) == (0.0, 0.0)
    for p in ps:
        if abs(p) > 700.0:
            continue
        for y in (0.0, 1.0, 0.25):
            g, h = oracle.logistic_gh(float(p), y)
            s = 1 / (1 + (-Decimal(float(p))).exp())
            gx = float(s - Decimal(y))
            hx = float(s * (1 - s))
            assert abs(g - gx) <= 4 * 2.0 ** -53 * max(float(s), y), (p, y, g, gx)
            assert _ulps(h, hx) <= 4 or abs(h - hx) <= 2.0 ** -1000, (p, y, h, hx)
            assert oracle.logistic_gh(-float(p), y)[1] == h
            g2, _ = oracle.logistic_gh(-float(p), 1.0 - y)
            assert abs(g + g2) <= 2.0 ** -52


def test_logistic_grid_bounds():
    """Both grids keep every value within 31 bits and every sum over all rows
    exact (|sum| <= 2^52), with the largest magnitude using at least 29 bits
    (or the 52 - ceil(log2 n) bits the squared-error grid allows)."""
    rng = np.random.default_rng(4)
    for n in (1, 7, 1000, 70_000):
        pred = rng.normal(0.0, 2.0, n)
        label = (rng.uniform(size=n) < 0.4).astype(np.float32)
        kg, kh, Sg, Sh = oracle.logistic_grid(pred, label)
        L = oracle.ceil_log2(n)
        for k, S in ((kg, Sg), (kh, Sh)):
            m = int(np.abs(k).max())
            assert m < 2 ** 31 and m * n <= 2 ** 52
            assert m >= min(2 ** 29, 2 ** (51 - L)) or m == 0
        assert (kh >= 0).all()


def test_logistic_hand_tree():
    """Worked by hand at base 0: sigmoid(0) = 1/2, so g = 1/2 - y and h = 1/4 for
    every row.  Four rows, one feature with bins 0..3, labels 0, 0, 1, 1,
    lambda 1: G_P = 0, H_P = 1.  t = 0: (1/2)^2/(1/4 + 1) + (1/2)^2/(3/4 + 1) =
    1/5 + 1/7, gain 6/35; t = 1: 1/(1/2 + 1) twice, gain 2/3; t = 2: 6/35.  The
    root splits at t = 1 with leaves -1/(1/2 + 1) = -2/3 and 2/3.  The grids:
    max |g| = 1/2 gives S = 30 (the 30-bit cap; 52 - 0 - 2 = 50 otherwise) and
    max h = 1/4 gives Sh = 31, so kg = -+2^29 and kh = 2^29 exactly.
    With min_child_weight 0.6 every child's H is below 0.6 (counts would all
    pass), so the root stays a leaf with weight -0/(1 + 1) = -0.0."""
    bins = np.array([[0], [1], [2], [3]], dtype=np.uint8)
    label = np.array([0, 0, 1, 1], dtype=np.float32)
    p = oracle.make_params(1, reg_lambda=1.0, learning_rate=1.0, objective=oracle.LOGISTIC)
    r = oracle.train(bins, [4], label, p, 1, dump_tree=0)
    tree = r["nodes"][0][: r["n_nodes"][0]]
    assert r["scale"][0] == 30 and r["scale_h"][0] == 31
    assert r["dump_k"].tolist() == [2 ** 29, 2 ** 29, -(2 ** 29), -(2 ** 29)]
    assert r["dump_kh"].tolist() == [2 ** 29] * 4
    assert len(tree) == 3
    assert (int(tree[0]["feature"]), int(tree[0]["threshold_bin"])) == (0, 1)
    assert float(tree[0]["gain"]) == 0.5 * (2.0 / 3.0 + 2.0 / 3.0)
    assert float(tree[1]["leaf_value"]) == -1.0 / 1.5 and float(tree[2]["leaf_value"]) == 1.0 / 1.5
    assert int(tree[0]["hsum_q"]) == 2 ** 31 and int(tree[1]["hsum_q"]) == 2 ** 30
    assert r["pred"].tolist() == [-1.0 / 1.5, -1.0 / 1.5, 1.0 / 1.5, 1.0 / 1.5]
    p.min_child_weight = 0.6
    r = oracle.train(bins, [4], label, p, 1)
    root = r["nodes"][0][0]
    assert r["n_nodes"][0] == 1 and root["flags"] & oracle.LEAF
    assert float(root["leaf_value"]) == 0.0 and math.copysign(1.0, float(root["leaf_value"])) < 0


@pytest.mark.parametrize("seed", [21, 22, 23, 24])
def test_logistic_split_choice_against_exact_rationals(seed):
    """Brute force for the logistic objective: the grid values (kg, kh) taken as
    exact rationals, every (feature, bin) of every node scored from the rows
    directly -- H from the Hessians, min_child_weight on H -- and the oracle's
    chosen split must be the exact best (up to the FP64 rounding of the gain),
    with leaf weights -G/(H + lambda) of the rows they hold."""
    nb = [5, 3, 7]
    bins, _, nb = datagen.make_random(60, nb, seed)
    rng = np.random.default_rng(seed)
    label = (rng.uniform(size=60) < 0.5).astype(np.float32)
    base = float(rng.normal(0.0, 1.0))
    p = oracle.make_params(3, reg_lambda=0.5, gamma=0.01, min_child_weight=1.5, min_samples_leaf=2,
                           learning_rate=0.5, objective=oracle.LOGISTIC)
    pred0 = np.full(60, base) + rng.normal(0.0, 0.5, 60)
    r = oracle.train(bins, nb, label, p, 1, pred0=pred0, dump_tree=0)
    kg, kh, Sg, Sh = oracle.logistic_grid(pred0, label)
    assert np.array_equal(kg, r["dump_k"]) and np.array_equal(kh, r["dump_kh"])
    g = [Fraction(int(x), 2 ** Sg) for x in kg]
    h = [Fraction(int(x), 2 ** Sh) for x in kh]
    tree = r["nodes"][0][: r["n_nodes"][0]]
    lam, gam = Fraction(p.reg_lambda), Fraction(p.gamma)
    rows = _node_rows(tree, bins)
    for v, nd in enumerate(tree):
        rv = rows[v]
        GP, HP = sum(g[i] for i in rv), sum(h[i] for i in rv)
        if nd["flags"] & oracle.LEAF:
            assert float(nd["leaf_value"]) == float(-GP / (HP + lam)) or (
                GP == 0 and float(nd["leaf_value"]) == 0.0)
        if int(nd["depth"]) >= p.max_depth:
            continue
        cands = []
        for f in range(bins.shape[1]):
            for t in range(int(nb[f]) - 1):
                L = [i for i in rv if int(bins[i, f]) <= t]
                R = [i for i in rv if int(bins[i, f]) > t]
                if len(L) < p.min_samples_leaf or len(R) < p.min_samples_leaf:
                    continue
                HL = sum(h[i] for i in L)
                HR = HP - HL
                if HL < Fraction(p.min_child_weight) or HR < Fraction(p.min_child_weight):
                    continue
                if not (HL > 0 and HR > 0):
                    continue
                GL = sum(g[i] for i in L)
                cands.append((_exact_gain(GL, HL, GP - GL, HR, GP, HP, lam, gam), f, t))
        tol = Fraction(1, 2 ** 40) * (1 + abs(GP * GP))
        best = max((c[0] for c in cands), default=None)
        if nd["flags"] & oracle.LEAF:
            assert best is None or best <= tol, (v, best)
            continue
        chosen = [c for c in cands if (c[1], c[2]) == (int(nd["feature"]), int(nd["threshold_bin"]))]
        assert chosen and best - chosen[0][0] <= tol
        assert abs(Fraction(float(nd["gain"])) - chosen[0][0]) <= tol


def test_logistic_training_lowers_the_loss():
    bins, _, nb = datagen.make_random(4000, [16, 8, 32, 2], 31)
    label = ((bins[:, 0].astype(np.int32) + bins[:, 2] // 2) > 20).astype(np.float32)
    p = oracle.make_params(4, learning_rate=0.5, objective=oracle.LOGISTIC)
    r = oracle.train(bins, nb, label, p, 5, keep_pred_per_tree=True)

    def logloss(pr):
        s = 1.0 / (1.0 + np.exp(-pr))
        return float(-np.mean(label * np.log(s) + (1 - label) * np.log(1 - s)))
    losses = [math.log(2.0)] + [logloss(r["pred_per_tree"][t]) for t in range(5)]
    assert all(b < a for a, b in zip(losses, losses[1:])), losses
    # the training predictions are the forward pass of the trees
    out = oracle.predict(bins, r["nodes"], r["n_nodes"], 0.0, p.learning_rate)
    assert np.array_equal(out, r["pred"])


# ------------------------------------------------------------------ bin bounds

FLT_MIN = float(np.finfo(np.float32).tiny)


def test_bounds_equal_width_hand():
    """lo = 0, hi = 10, four bins: bounds 2.5, 5, 7.5 (exact); NaN and +-inf
    are left out of the range; the entry after the bounds is +inf."""
    col = np.array([3.0, 0.0, np.nan, 10.0, np.inf, -np.inf, 7.0], dtype=np.float32)
    u = oracle.feature_bounds(col[:, None], [4], oracle.BOUNDS_EQUAL_WIDTH)
    assert u.tolist() == [2.5, 5.0, 7.5, math.inf]
    # two features side by side, each with its own range and bin count
    raw = np.stack([col, np.array([-4, -2, 0, 2, 4, 6, 8], dtype=np.float32)], axis=1)
    u = oracle.feature_bounds(raw, [4, 3], oracle.BOUNDS_EQUAL_WIDTH)
    assert u.tolist() == [2.5, 5.0, 7.5, math.inf, 0.0, 4.0, math.inf]
    # the extremes land in the first and last bins
    b, _ = oracle.bin_features(raw, [4, 3], u)
    assert b[1, 0] == 0 and b[3, 0] == 3 and b[0, 1] == 0 and b[6, 1] == 2


def test_bounds_degenerate_features():
    """A constant feature and a feature with no finite value: the bounds climb
    from the value (or 0) by next_up, so every value of the constant feature
    falls in bin 0 and the bounds still strictly increase."""
    raw = np.array([[5.0, np.nan], [5.0, np.inf], [5.0, np.nan]], dtype=np.float32)
    for method in (oracle.BOUNDS_EQUAL_WIDTH, oracle.BOUNDS_QUANTILE):
        u = oracle.feature_bounds(raw, [4, 3], method)
        a = u[:3]
        assert a[0] == 5.0 and a[1] == np.nextafter(np.float32(5.0), np.float32(np.inf))
        assert (np.diff(a) > 0).all()
        b, _ = oracle.bin_features(raw, [4, 3], u)
        assert (b[:, 0] == 0).all()
    u = oracle.feature_bounds(raw, [4, 3], oracle.BOUNDS_EQUAL_WIDTH)
    assert u[4] == 0.0 and u[5] == FLT_MIN  # no finite value: lo = hi = 0


def test_bounds_next_up_rules():
    """next_up skips the subnormals: -FLT_MIN -> 0 -> FLT_MIN."""
    raw = np.full((4, 1), -FLT_MIN, dtype=np.float32)
    u = oracle.feature_bounds(raw, [4], oracle.BOUNDS_QUANTILE)
    assert u[:3].tolist() == [-FLT_MIN, 0.0, FLT_MIN]
    raw = np.full((4, 1), np.float32(np.finfo(np.float32).max))
    u = oracle.feature_bounds(raw, [3], oracle.BOUNDS_QUANTILE)
    assert u[:2].tolist() == [float(np.finfo(np.float32).max), math.inf]


def test_bounds_quantile_hand():
    """Values 1 .. 100, four bins: bound k is the ceil(k 100/4)-th smallest
    value: 25, 50, 75; binning then puts exactly 25 values in each bin."""
    col = np.arange(100, 0, -1, dtype=np.float32)
    u = oracle.feature_bounds(col[:, None], [4], oracle.BOUNDS_QUANTILE)
    assert u[:3].tolist() == [25.0, 50.0, 75.0]
    b, _ = oracle.bin_features(col[:, None], [4], u)
    assert np.bincount(b[:, 0], minlength=4).tolist() == [25, 25, 25, 25]


@pytest.mark.parametrize("B", [4, 64, 256])
def test_bounds_quantile_is_the_inverted_cdf(B):
    """Without ties, bound k is numpy's inverted-CDF quantile at k/B of the
    finite values (B a power of two, so k/B and k m/B are exact), and at least
    a fraction k/B of them lies at or below it, less than k/B below it."""
    rng = np.random.default_rng(B)
    col = rng.standard_t(3, size=20000).astype(np.float32)
    col[::97] = np.nan
    col[5] = np.inf
    col[6] = -np.inf
    u = oracle.feature_bounds(col[:, None], [B], oracle.BOUNDS_QUANTILE)[: B - 1]
    v = col[np.isfinite(col)].astype(np.float64)
    q = np.quantile(v, np.arange(1, B) / B, method="inverted_cdf")
    assert np.array_equal(u.astype(np.float64), q)
    for k in range(1, B):
        assert (v <= u[k - 1]).mean() >= k / B > (v < u[k - 1]).mean()


def test_bounds_quantile_sample_rows():
    """Above 32768 rows the quantiles come from rows 0, s, 2s, ... with
    s = ceil(n / 32768): the bounds equal those of that sample given alone."""
    n = 100_001
    s = -(-n // oracle.QUANTILE_SAMPLE)
    rng = np.random.default_rng(7)
    raw = rng.exponential(size=(n, 3)).astype(np.float32)
    raw[:, 2] = np.round(raw[:, 2] * 4)  # heavy ties
    full = oracle.feature_bounds(raw, [16, 256, 64], oracle.BOUNDS_QUANTILE)
    samp = oracle.feature_bounds(raw[::s], [16, 256, 64], oracle.BOUNDS_QUANTILE)
    assert raw[::s].shape[0] <= oracle.QUANTILE_SAMPLE
    assert np.array_equal(full, samp)
    off = 0
    for B in (16, 256, 64):
        assert (np.diff(full[off: off + B - 1]) > 0).all()
        off += B
    b, nan = oracle.bin_features(raw, [16, 256, 64], full)
    assert nan == 0


def test_bounds_equal_width_ignores_row_order():
    rng = np.random.default_rng(8)
    raw = rng.normal(size=(5000, 4)).astype(np.float32) * np.float32(1e3)
    u1 = oracle.feature_bounds(raw, [7, 64, 255, 2], oracle.BOUNDS_EQUAL_WIDTH)
    u2 = oracle.feature_bounds(raw[rng.permutation(5000)], [7, 64, 255, 2], oracle.BOUNDS_EQUAL_WIDTH)
    assert np.array_equal(u1, u2)
    # every bin of a 255-bin feature spans (hi - lo)/255 up to rounding
    lo, hi = raw[:, 2].min(), raw[:, 2].max()
    w = np.diff(np.concatenate([[lo], u1[7 + 64: 7 + 64 + 254], [hi]]).astype(np.float64))
    assert np.allclose(w, (float(hi) - float(lo)) / 255, rtol=1e-4)


def test_bounds_signed_zero():
    """-0 and +0 are one value for the bounds: a quantile at a run of zeros of
    both signs is +0, and so is an equal-width end at zero."""
    col = np.array([-0.0, 0.0, -0.0, 1.0, -1.0, 0.0, -0.0, 2.0], dtype=np.float32)
    u = oracle.feature_bounds(col[:, None], [4], oracle.BOUNDS_QUANTILE)
    # sorted: -1, 0 x 5, 1, 2; ranks 1, 3, 5 are zeros; the chain lifts the repeats
    assert u[0] == 0.0 and math.copysign(1.0, float(u[0])) > 0
    assert u[1] == FLT_MIN and u[2] == np.nextafter(np.float32(FLT_MIN), np.float32(1))
    col = np.array([-0.0, 4.0, 1.0], dtype=np.float32)
    u = oracle.feature_bounds(col[:, None], [4], oracle.BOUNDS_EQUAL_WIDTH)
    assert u[:3].tolist() == [1.0, 2.0, 3.0]
