"""Parity of every HIP entry point with the CPU oracle, element by element, on
seeded inputs (bit-exact for histograms, splits, partitions, tree structure;
leaf values and predictions bit-exact too, inside the 1e-9 relative bar).

Each test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import datagen
import histogram_split_finding_amd as g
import oracle
from gpu_util import (DEV, compare_tree, hist_from_device, i32, min_split_count, nodes_tensor,
                      orc_has_hist, packed_rows, say, to_dev)

pytestmark = pytest.mark.gpu


def _ws(n, lst, tb):
    return g.new_workspace(g.gbdt_workspace_bytes(n, lst, tb))


# ------------------------------------------------------------------ gradients --

# (3,000,017 rows: several grid-stride steps of four rows per thread, ragged end)
@pytest.mark.parametrize("n,seed,scale", [(1, 1, 1.0), (2, 2, 3.0), (4097, 3, 10.0), (100003, 4, 1e-3),
                                          (1 << 20, 5, 100.0), (3000017, 6, 2.0)])
def test_gradients(n, seed, scale):
    say("gradients n=%d seed=%d" % (n, seed))
    rng = np.random.default_rng(seed)
    pred = rng.normal(size=n) * scale
    label = rng.normal(size=n).astype(np.float32)
    k, S, _ = oracle.gradient_grid(pred, label)
    q = torch.zeros(n, dtype=torch.int64, device=DEV)
    sc = torch.zeros(1, dtype=torch.int32, device=DEV)
    gs = torch.zeros(1, dtype=torch.int64, device=DEV)
    ws = _ws(n, 1, 1)
    g.gbdt_compute_gradients(to_dev(pred), to_dev(label), q, sc, gs, ws)
    assert g.gbdt_read_error(ws) == 0
    assert int(sc.item()) == S
    assert np.array_equal(q.cpu().numpy(), k)
    assert int(gs.item()) == int(k.sum())


def test_gradients_all_zero_and_nonfinite():
    say("gradients zero / non-finite")
    n = 1000
    pred = np.full(n, 2.0)
    label = np.full(n, 2.0, dtype=np.float32)
    q = torch.full((n,), 7, dtype=torch.int64, device=DEV)
    sc = torch.full((1,), 9, dtype=torch.int32, device=DEV)
    gs = torch.zeros(1, dtype=torch.int64, device=DEV)
    ws = _ws(n, 1, 1)
    g.gbdt_compute_gradients(to_dev(pred), to_dev(label), q, sc, gs, ws)
    assert g.gbdt_read_error(ws) == 0
    assert int(sc.item()) == 0 and not q.any().item() and int(gs.item()) == 0
    label[17] = np.nan
    g.gbdt_compute_gradients(to_dev(pred), to_dev(label), q, sc, gs, ws)
    assert g.gbdt_read_error(ws) == -3


# ----------------------------------------------------------------- histograms --

HIST_CASES = [
    # (name, n, n_bins, segment sizes, seed)
    ("mixed_bins", 60000, [2, 7, 256, 64, 2, 2, 33, 1, 255, 16, 3], [1, 5, 1023, 1024, 1025, 4000, 20000], 11),
    ("wide_blocks", 30000, [256] * 70 + [2] * 5, [3000, 1, 12000, 9000], 12),
    ("one_big_node", 300000, [32] * 8, [300000], 13),
    ("many_small", 20000, [256] * 10 + [2] * 44, [37] * 300 + [1100] * 5, 14),
]


@pytest.mark.parametrize("case", HIST_CASES, ids=[c[0] for c in HIST_CASES])
@pytest.mark.parametrize("use_skip", [True, False])
@pytest.mark.parametrize("pack_bits", [True, False])
def test_build_histograms(case, use_skip, pack_bits):
    name, n, nbins, segs, seed = case
    say("build_histograms %s skip=%s bits=%s" % (name, use_skip, pack_bits))
    bins, label, nb = datagen.make_random(n, nbins, seed, bin_kind=1)
    rng = np.random.default_rng(seed)
    pred = rng.normal(size=n)
    k, S, _ = oracle.gradient_grid(pred, label)
    perm = rng.permutation(n).astype(np.int32)
    ft = g.FeatureTable(nb, DEV, pack_bits=pack_bits)
    # skip bins from the whole matrix (the pack step's census)
    rb_full = packed_rows(bins, ft)
    if not use_skip:
        ft.skip_bin.fill_(-1)
    del rb_full
    src = packed_rows(bins[perm], ft, q=k[perm])
    total = sum(segs)
    assert total <= n
    nodes, begin = [], 0
    for s in segs:
        nodes.append(dict(begin=begin, count=s))
        begin += s
    ids = list(range(len(segs)))
    TB = ft.total_bins
    hist_g = torch.full((len(segs) * TB,), 123, dtype=torch.int64, device=DEV)
    hist_c = torch.full((len(segs) * TB,), 77, dtype=torch.int32, device=DEV)
    ws = _ws(n, len(segs), TB)
    g.gbdt_build_histograms(src.rows(identity_rid=True), ft.struct(use_skip), nodes_tensor(nodes),
                            i32(ids), i32([len(ids)]), len(ids), total, hist_g, hist_c, ws)
    assert g.gbdt_read_error(ws) == 0
    b0 = 0
    for j, s in enumerate(segs):
        cnt, gq = oracle.node_histogram(bins, nb, perm[b0:b0 + s], k, S)
        dc, dg = hist_from_device(hist_g, hist_c, j, TB)
        assert np.array_equal(dc, cnt), (name, j)
        assert np.array_equal(dg, gq), (name, j)
        b0 += s


def test_build_histograms_empty_list_and_empty_node():
    say("build_histograms empty")
    bins, label, nb = datagen.make_random(100, [4, 4], 3)
    k, S, _ = oracle.gradient_grid(np.zeros(100), label)
    ft = g.FeatureTable(nb, DEV)
    src = packed_rows(bins, ft, q=k)
    TB = ft.total_bins
    hist_g = torch.full((2 * TB,), 5, dtype=torch.int64, device=DEV)
    hist_c = torch.full((2 * TB,), 5, dtype=torch.int32, device=DEV)
    ws = _ws(100, 2, TB)
    nodes = nodes_tensor([dict(begin=0, count=0), dict(begin=0, count=100)])
    g.gbdt_build_histograms(src.rows(True), ft.struct(), nodes, i32([0, 1]), i32([0]), 2, 100, hist_g,
                            hist_c, ws)
    torch.cuda.synchronize()
    assert (hist_g == 5).all().item()  # nothing listed, nothing written
    g.gbdt_build_histograms(src.rows(True), ft.struct(), nodes, i32([0, 1]), i32([2]), 2, 100, hist_g,
                            hist_c, ws)
    assert g.gbdt_read_error(ws) == 0
    dc, dg = hist_from_device(hist_g, hist_c, 0, TB)
    assert not dc.any() and not dg.any()  # an empty node gets a zero histogram
    cnt, gq = oracle.node_histogram(bins, nb, np.arange(100, dtype=np.int32), k, S)
    dc, dg = hist_from_device(hist_g, hist_c, 1, TB)
    assert np.array_equal(dc, cnt) and np.array_equal(dg, gq)


def test_build_histograms_rejects_bad_bins_and_q():
    say("build_histograms device checks")
    bins, label, nb = datagen.make_random(500, [4, 4], 3)
    ft = g.FeatureTable(nb, DEV)
    rb = g.RowBuffer(ft, 500, DEV)
    ws = _ws(500, 1, ft.total_bins)
    bad = bins.copy()
    bad[10, 1] = 9
    g.gbdt_pack_matrix(to_dev(bad), rb, ft, ws)
    assert g.gbdt_read_error(ws) == -3
    src = packed_rows(bins, ft, q=np.full(500, 1 << 50, dtype=np.int64))
    hist_g = torch.zeros(ft.total_bins, dtype=torch.int64, device=DEV)
    hist_c = torch.zeros(ft.total_bins, dtype=torch.int32, device=DEV)
    g.gbdt_build_histograms(src.rows(True), ft.struct(), nodes_tensor([dict(begin=0, count=500)]), i32([0]),
                            i32([1]), 1, 500, hist_g, hist_c, ws)
    assert g.gbdt_read_error(ws) == -4


# --------------------------------------------------------------- subtraction --

def test_subtract_histograms():
    say("subtract")
    rng = np.random.default_rng(5)
    TB, slots = 3001, 9
    small_g = rng.integers(-2**40, 2**40, size=(slots, TB))
    small_c = rng.integers(0, 1000, size=(slots, TB)).astype(np.uint32)
    hg = small_g.copy()
    hc = small_c.copy()
    pairs = np.zeros(3, dtype=g.PAIR_DTYPE)
    for j, (p, s, l) in enumerate([(0, 1, 2), (3, 5, 4), (6, 7, 8)]):
        hg[p] = small_g[s] + rng.integers(-2**40, 2**40, size=TB)
        hc[p] = small_c[s] + rng.integers(0, 1000, size=TB).astype(np.uint32)
        pairs[j] = (p, s, l, 0)
    dg = to_dev(hg.reshape(-1))
    dc = to_dev(hc.reshape(-1).view(np.int32))
    ws = _ws(1, 1, 1)
    g.gbdt_subtract_histograms(dg, dc, TB, to_dev(pairs.view(np.uint8)), i32([3]), 4, ws)
    assert g.gbdt_read_error(ws) == 0
    og = dg.cpu().numpy().reshape(slots, TB)
    oc = dc.cpu().numpy().view(np.uint32).reshape(slots, TB)
    for p, s, l in [(0, 1, 2), (3, 5, 4), (6, 7, 8)]:
        assert np.array_equal(og[l], hg[p] - hg[s])
        assert np.array_equal(oc[l], hc[p] - hc[s])
        assert np.array_equal(og[p], hg[p]) and np.array_equal(og[s], hg[s])


# ------------------------------------------------------------------ split find --

FIND_CASES = [
    ("plain", 5000, [256, 2, 17, 64, 2], dict(max_depth=4), 21),
    ("lambda0_gamma", 3000, [8] * 12, dict(max_depth=4, reg_lambda=0.0, gamma=0.3), 22),
    ("msl_mcw", 4000, [32, 5, 2, 256], dict(max_depth=4, min_samples_leaf=50, min_child_weight=120.5), 23),
    ("ties_dup_columns", 2000, [16, 16, 16], dict(max_depth=4), 24),
    ("wide", 20000, [256] * 40, dict(max_depth=4, reg_lambda=2.5), 25),
    ("unsplittable", 50, [4, 4], dict(max_depth=4, min_samples_leaf=40), 26),
]


@pytest.mark.parametrize("case", FIND_CASES, ids=[c[0] for c in FIND_CASES])
def test_find_best_splits(case):
    name, n, nbins, pk, seed = case
    say("find_best_splits %s" % name)
    bins, label, nb = datagen.make_random(n, nbins, seed, bin_kind=1, label_kind=2)
    if name == "ties_dup_columns":
        bins[:, 1] = bins[:, 0]
    p = oracle.make_params(**pk)
    gp = g.make_params(**pk)
    rng = np.random.default_rng(seed)
    k, S, _ = oracle.gradient_grid(rng.normal(size=n) * 0.1, label)
    # nodes: random row subsets of several sizes
    subsets = [np.arange(n, dtype=np.int32)]
    for frac in (0.5, 0.1, 0.013):
        m = max(1, int(n * frac))
        subsets.append(np.sort(rng.choice(n, size=m, replace=False)).astype(np.int32))
    ft = g.FeatureTable(nb, DEV)
    TB = ft.total_bins
    hg = np.zeros((len(subsets), TB), dtype=np.int64)
    hc = np.zeros((len(subsets), TB), dtype=np.uint32)
    nodes, expect = [], []
    for j, rows in enumerate(subsets):
        cnt, gq = oracle.node_histogram(bins, nb, rows, k, S)
        hg[j], hc[j] = gq, cnt
        gs = int(k[rows].sum())
        nodes.append(dict(begin=0, count=len(rows), gsum=gs))
        expect.append(oracle.best_split(cnt, gq, nb, gs, len(rows), S, p))
    splits = torch.zeros(len(subsets) * g.SPLIT_DTYPE.itemsize, dtype=torch.uint8, device=DEV)
    ws = _ws(n, len(subsets), TB)
    g.gbdt_find_best_splits(to_dev(hg.reshape(-1)), to_dev(hc.reshape(-1).view(np.int32)), ft.struct(),
                            nodes_tensor(nodes), i32(range(len(subsets))), i32([len(subsets)]),
                            len(subsets), gp, i32([S]), splits, ws)
    got = g.splits_to_host(splits)
    for j, e in enumerate(expect):
        a = got[j]
        assert int(a["valid"]) == int(e["valid"]), (name, j)
        if e["valid"]:
            assert (int(a["feature"]), int(a["threshold_bin"])) == (int(e["feature"]), int(e["threshold_bin"])), (name, j)
            assert float(a["gain"]) == float(e["gain"]), (name, j, float(a["gain"]), float(e["gain"]))
            assert int(a["n_left"]) == int(e["n_left"]) and int(a["g_left"]) == int(e["gq_left"])


# ------------------------------------------------------------------ partition --

@pytest.mark.parametrize("n,nbins,seed", [(50000, [2, 256, 13, 64, 2, 2, 9], 31), (20011, [256] * 70, 32),
                                          (3, [4], 33), (30000, [256] * 10 + [2] * 44, 34),
                                          (9000, [2] * 40 + [1] * 3, 35), (7001, [2] * 150 + [5] * 3, 36)])
@pytest.mark.parametrize("pack_bits", [True, False])
def test_partition_rows(n, nbins, seed, pack_bits):
    say("partition n=%d F=%d bits=%s" % (n, len(nbins), pack_bits))
    bins, label, nb = datagen.make_random(n, nbins, seed, bin_kind=1)
    rng = np.random.default_rng(seed)
    k = rng.integers(-2**30, 2**30, size=n)
    perm = rng.permutation(n).astype(np.int32)
    ft = g.FeatureTable(nb, DEV, pack_bits=pack_bits)
    src = packed_rows(bins[perm], ft, q=k[perm], rid=perm)
    dst = packed_rows(np.zeros_like(bins), ft, q=np.full(n, -5, dtype=np.int64), rid=np.full(n, -9, dtype=np.int32))
    # segments: a few nodes, some listed (split), some not
    cuts = sorted(set([0, n] + [int(x) for x in rng.choice(np.arange(1, n), size=min(6, max(n - 1, 0)), replace=False)]))
    nodes, splits, listed = [], [], []
    for j in range(len(cuts) - 1):
        b, e = cuts[j], cuts[j + 1]
        f = int(rng.integers(0, len(nbins)))
        t = int(rng.integers(0, nb[f]))
        left, right = oracle.partition(bins, perm[b:e], f, t)
        nodes.append(dict(begin=b, count=e - b))
        splits.append((1.0, f, t, 0, len(left), 1))
        if j % 3 != 1:
            listed.append(j)
    sp = np.array(splits, dtype=g.SPLIT_DTYPE)
    ws = _ws(n, len(nodes), ft.total_bins)
    g.gbdt_partition_rows(src.rows(), dst.rows(), nodes_tensor(nodes), to_dev(sp.view(np.uint8)),
                          i32(listed), i32([len(listed)]), len(nodes), n, ws)
    assert g.gbdt_read_error(ws) == 0
    drid = dst.rid.cpu().numpy()
    dq = dst.q.cpu().numpy()
    dbins = dst.blocked_to_rowmajor().cpu().numpy()
    for j in range(len(nodes)):
        b, e = cuts[j], cuts[j + 1]
        if j in listed:
            f, t = int(sp[j]["feature"]), int(sp[j]["threshold_bin"])
            left, right = oracle.partition(bins, perm[b:e], f, t)
            assert np.array_equal(drid[b:e], np.concatenate([left, right]))
            assert np.array_equal(dq[b:e], k[drid[b:e]])
            assert np.array_equal(dbins[b:e], bins[drid[b:e]])
        else:
            assert (drid[b:e] == -9).all() and (dq[b:e] == -5).all()


def test_partition_count_mismatch_is_reported():
    say("partition mismatch")
    n = 5000
    bins, label, nb = datagen.make_random(n, [8, 8], 4)
    ft = g.FeatureTable(nb, DEV)
    src = packed_rows(bins, ft, q=np.zeros(n, dtype=np.int64))
    dst = packed_rows(bins, ft, q=np.zeros(n, dtype=np.int64), rid=np.zeros(n, dtype=np.int32))
    left, _ = oracle.partition(bins, np.arange(n, dtype=np.int32), 0, 3)
    sp = np.array([(1.0, 0, 3, 0, len(left) + 1, 1)], dtype=g.SPLIT_DTYPE)
    ws = _ws(n, 1, ft.total_bins)
    g.gbdt_partition_rows(src.rows(True), dst.rows(), nodes_tensor([dict(begin=0, count=n)]),
                          to_dev(sp.view(np.uint8)), i32([0]), i32([1]), 1, n, ws)
    assert g.gbdt_read_error(ws) == -7


# --------------------------------------------------------- prediction update --

def _random_tree(rng, F, nb, depth, p_leaf=0.25):
    """A flat breadth-first tree with random splits (children appended in order)."""
    nodes = [dict(depth=0)]
    v = 0
    while v < len(nodes):
        nd = nodes[v]
        if nd["depth"] < depth and (v == 0 or rng.random() > p_leaf):
            f = int(rng.integers(0, F))
            nd.update(feature=f, threshold_bin=int(rng.integers(0, nb[f])), left=len(nodes),
                      right=len(nodes) + 1, flags=0)
            nodes.append(dict(depth=nd["depth"] + 1))
            nodes.append(dict(depth=nd["depth"] + 1))
        else:
            nd.update(feature=-1, threshold_bin=-1, left=-1, right=-1, flags=1,
                      leaf_value=float(rng.normal()))
        v += 1
    return nodes


def _route(nodes, bins):
    leaf = np.zeros(bins.shape[0], dtype=np.int64)
    active = np.ones(bins.shape[0], dtype=bool)
    while active.any():
        idx = np.nonzero(active)[0]
        for v in np.unique(leaf[idx]):
            nd = nodes[v]
            sel = idx[leaf[idx] == v]
            if nd["flags"] & 1:
                active[sel] = False
                continue
            go_left = bins[sel, nd["feature"]] <= nd["threshold_bin"]
            leaf[sel] = np.where(go_left, nd["left"], nd["right"])
    return leaf


# (the last case: three byte blocks of 24 bytes and two bit words, read
# with wide loads per block and the bit words placed after five blocks' room)
@pytest.mark.parametrize("n,nbins,depth,seed", [(70001, [2, 64, 256, 7, 33], 7, 8), (5000, [256] * 70, 5, 9),
                                                (1, [4], 3, 10), (40000, [256] * 10 + [2] * 44, 8, 11),
                                                (3000, [2] * 37, 6, 12), (20000, [256] * 70 + [2] * 60, 6, 13)])
@pytest.mark.parametrize("pack_bits", [True, False])
def test_update_predictions(n, nbins, depth, seed, pack_bits):
    """Step 7 by routing every row through the finished tree."""
    say("update_predictions n=%d bits=%s" % (n, pack_bits))
    rng = np.random.default_rng(seed)
    bins, label, nb = datagen.make_random(n, nbins, seed, bin_kind=1)
    nodes = _random_tree(rng, len(nbins), nb, depth)
    pred = rng.normal(size=n)
    eta = 0.3
    leaf = _route(nodes, bins)
    w = np.array([nd.get("leaf_value", 0.0) for nd in nodes])
    expect = pred + eta * w[leaf]
    ft = g.FeatureTable(nb, DEV, pack_bits=pack_bits)
    X = packed_rows(bins, ft)
    dpred = to_dev(pred)
    ws = _ws(n, 1, 1)
    g.gbdt_update_predictions(dpred, X.matrix(), nodes_tensor(nodes), i32([len(nodes)]), len(nodes), eta, ws)
    assert g.gbdt_read_error(ws) == 0
    assert np.array_equal(dpred.cpu().numpy(), expect)


def test_update_predictions_rejects_bad_tree():
    say("update_predictions bad tree")
    bins, label, nb = datagen.make_random(1000, [4, 4], 3)
    ft = g.FeatureTable(nb, DEV)
    X = packed_rows(bins, ft)
    # node 1 points back to node 0: a cycle the walk must refuse
    nodes = [dict(feature=0, threshold_bin=1, left=1, right=2, flags=0),
             dict(feature=1, threshold_bin=1, left=0, right=2, flags=0),
             dict(flags=1, leaf_value=1.0)]
    pred = np.zeros(1000)
    dpred = to_dev(pred)
    ws = _ws(1000, 1, 1)
    g.gbdt_update_predictions(dpred, X.matrix(), nodes_tensor(nodes), i32([3]), 3, 1.0, ws)
    assert g.gbdt_read_error(ws) == -7
    out = dpred.cpu().numpy()
    right = bins[:, 0] > 1
    assert np.array_equal(out[right], np.ones(right.sum()))  # rows that reach the leaf
    assert not out[~right].any()                              # rows that hit the bad node


def test_update_predictions_rejects_bad_threshold():
    """A split node whose threshold_bin is negative stops the walk there like
    any node that fails the table's check: GBDT_E_INTERNAL, and the rows that
    reach it keep their predictions."""
    say("update_predictions bad threshold")
    bins, label, nb = datagen.make_random(1000, [4, 4], 5)
    ft = g.FeatureTable(nb, DEV)
    X = packed_rows(bins, ft)
    nodes = [dict(feature=0, threshold_bin=1, left=1, right=2, flags=0),
             dict(feature=1, threshold_bin=-1, left=3, right=4, flags=0),
             dict(flags=1, leaf_value=2.0),
             dict(flags=1, leaf_value=3.0),
             dict(flags=1, leaf_value=4.0)]
    dpred = to_dev(np.zeros(1000))
    ws = _ws(1000, 1, 1)
    g.gbdt_update_predictions(dpred, X.matrix(), nodes_tensor(nodes), i32([5]), 5, 1.0, ws)
    assert g.gbdt_read_error(ws) == -7
    out = dpred.cpu().numpy()
    right = bins[:, 0] > 1
    assert np.array_equal(out[right], np.full(right.sum(), 2.0))  # node 2, a leaf
    assert not out[~right].any()                                  # node 1 fails the check


# ------------------------------------------------------------ whole tree path --

TRAIN_CASES = [
    ("rand_d3", 3000, [8, 16, 2, 32], dict(max_depth=3, learning_rate=0.5), 4, 41),
    ("rand_d5_msl", 20000, [256, 2, 2, 64, 7, 256], dict(max_depth=5, min_samples_leaf=30, gamma=0.05), 3, 42),
    ("rand_d6_lambda0", 9000, [16] * 9, dict(max_depth=6, reg_lambda=0.0, min_child_weight=3.0), 3, 43),
    ("wide_d4", 12000, [256] * 70, dict(max_depth=4, reg_lambda=2.0), 2, 44),
    # three byte blocks and two bit words: the update's wide loads per block
    ("wide_bits_d5", 8000, [256] * 70 + [2] * 60, dict(max_depth=5), 2, 51),
    ("deep_tiny", 700, [4, 4, 3], dict(max_depth=9), 3, 45),
    ("depth0", 100, [4, 4], dict(max_depth=0), 2, 46),
    # depth 1 moves no rows; depth 2 builds its last level from the root's
    # unmoved rows (filtered) and partitions nothing
    ("depth1", 3000, [256, 2, 9], dict(max_depth=1), 3, 49),
    ("depth2", 5000, [256, 2, 9, 64], dict(max_depth=2, learning_rate=0.5), 3, 50),
    ("single_row", 1, [4, 4], dict(max_depth=3), 2, 47),
    # n >= 2^22: int32 q (ceil(log2 n) >= 22) and 4096-row partition tiles, with
    # a 3-dword byte block and a bit block
    ("q32_bits_n4M", (1 << 22) + 1233, [256, 2, 64, 2, 13, 256, 7, 2, 33, 2, 200, 2, 9, 5],
     dict(max_depth=4, learning_rate=0.5), 2, 48),
]


def _train_both(bins, label, nb, pk, T, dump_tree):
    p = oracle.make_params(**pk)
    r = oracle.train(bins, nb, label, p, T, dump_tree=dump_tree, keep_pred_per_tree=True)
    ds = g.Dataset(bins, label, nb, DEV)
    bst = g.Booster(ds, g.make_params(**pk))
    preds = []
    for _ in range(T):
        bst.trees.append(bst.grow_tree())
        preds.append(bst.pred.cpu().numpy().copy())
    bst.check()
    return r, bst, preds


@pytest.mark.parametrize("case", TRAIN_CASES, ids=[c[0] for c in TRAIN_CASES])
def test_grow_tree_matches_oracle(case):
    name, n, nbins, pk, T, seed = case
    say("grow_tree %s" % name)
    bins, label, nb = datagen.make_random(n, nbins, seed, bin_kind=1, label_kind=2)
    r, bst, preds = _train_both(bins, label, nb, pk, T, dump_tree=T - 1)
    trees = bst.host_trees()
    p = oracle.make_params(**pk)
    for t in range(T):
        compare_tree(trees[t], r["nodes"][t][: r["n_nodes"][t]])
        assert np.array_equal(preds[t], r["pred_per_tree"][t]), (name, t)
    # histograms of the last tree: every node the driver built or derived
    tree = r["nodes"][T - 1][: r["n_nodes"][T - 1]]
    TB = bst.ds.ft.total_bins
    for v in sorted(orc_has_hist(tree, p.max_depth, min_split_count(p))):
        dc, dg = hist_from_device(bst.hist_g, bst.hist_cnt, v, TB)
        assert np.array_equal(dc, r["dump_cnt"][v]), (name, v)
        assert np.array_equal(dg, r["dump_gq"][v]), (name, v)


def test_workload1_all_trees():
    say("workload 1, every tree")
    bins, label, nb = datagen.make_workload(1)
    wl = dict(datagen.WORKLOADS[1])
    r, bst, preds = _train_both(bins, label, nb, wl, wl["n_trees"], dump_tree=0)
    trees = bst.host_trees()
    for t in range(wl["n_trees"]):
        compare_tree(trees[t], r["nodes"][t][: r["n_nodes"][t]])
        assert np.array_equal(preds[t], r["pred_per_tree"][t])


def test_repeat_runs_are_bit_identical():
    say("determinism")
    bins, label, nb = datagen.make_random(30000, [256, 2, 64, 16] * 3, 51, bin_kind=1, label_kind=2)
    pk = dict(max_depth=6, learning_rate=0.3)
    outs = []
    for _ in range(2):
        ds = g.Dataset(bins, label, nb, DEV)
        bst = g.Booster(ds, g.make_params(**pk)).train(3)
        bst.check()
        outs.append((b"".join(t.tobytes() for t in bst.host_trees()), bst.pred.cpu().numpy().tobytes()))
    assert outs[0] == outs[1]


def test_skip_bins_and_bit_layout_do_not_change_bits():
    say("skip bins on/off, bit block on/off")
    bins, label, nb = datagen.make_random(25000, [256, 2, 2, 64, 8, 1, 2], 52, bin_kind=1, label_kind=2)
    pk = dict(max_depth=5)
    res = []
    for use_skip, pack_bits in ((True, True), (False, True), (True, False), (False, False)):
        ds = g.Dataset(bins, label, nb, DEV, use_skip_bins=use_skip, pack_bits=pack_bits)
        bst = g.Booster(ds, g.make_params(**pk)).train(2)
        bst.check()
        res.append((b"".join(t.tobytes() for t in bst.host_trees()), bst.pred.cpu().numpy().tobytes()))
    assert res[0] == res[1] == res[2] == res[3]


# ---------------------------------------------------------------- binning --

def _bin_inputs(n, nbins, seed):
    """Raw float32 [n][F] and per-feature strictly increasing bounds; values
    include every bound exactly, its float32 neighbours and +-inf."""
    rng = np.random.default_rng(seed)
    off = oracle.bin_offsets(nbins)
    upper = np.full(int(off[-1]), 1e9, dtype=np.float32)
    raw = rng.normal(0, 2.5, size=(n, len(nbins))).astype(np.float32)
    for f, nb in enumerate(nbins):
        b = np.unique(rng.normal(0, 2, size=3 * nb + 8).astype(np.float32))[: nb - 1]
        upper[off[f]: off[f] + nb - 1] = b
        if nb > 1:
            m = n // 4
            pick = rng.integers(0, nb - 1, size=3 * m)
            rows = rng.permutation(n)[: 3 * m]
            raw[rows[:m], f] = b[pick[:m]]
            raw[rows[m:2 * m], f] = np.nextafter(b[pick[m:2 * m]], np.float32(np.inf))
            raw[rows[2 * m:], f] = np.nextafter(b[pick[2 * m:]], np.float32(-np.inf))
    if n > 2:
        raw[n // 2, :] = np.inf
        raw[n // 3, :] = -np.inf
    return raw, upper


BIN_CASES = [
    # n * F = 7007: whole 16-value chunks and a ragged tail; bins from 1 to 256
    ("ragged_mixed", 1001, [4, 1, 2, 256, 17, 3, 64], 51),
    # the 28 x 64-bin feature shape over several grid strides of chunks
    ("f28_b64", 200003, [64] * 28, 52),
    # 25,600 bins: the bounds do not fit LDS and are read from global memory
    ("global_bounds", 3001, [256] * 100, 53),
    ("one_feature", 37, [255], 54),
    # 60 x 256 bins: the largest bound table that still fits LDS (62 KiB)
    ("lds_wide_table", 2001, [256] * 60, 57),
    ("one_row", 1, [9, 2, 200], 55),
]


@pytest.mark.parametrize("case", BIN_CASES, ids=[c[0] for c in BIN_CASES])
def test_bin_features_matches_oracle(case):
    name, n, nbins, seed = case
    say("bin_features %s n=%d F=%d" % (name, n, len(nbins)))
    raw, upper = _bin_inputs(n, nbins, seed)
    want, n_nan = oracle.bin_features(raw, nbins, upper)
    assert n_nan == 0
    ft = g.FeatureTable(nbins, DEV, pack_bits=False)
    out = torch.full((n, len(nbins)), 0xEE, dtype=torch.uint8, device=DEV)
    ws = _ws(n, 1, 1)
    g.gbdt_bin_features(to_dev(raw), ft, to_dev(upper), out, ws)
    assert g.gbdt_read_error(ws) == 0
    assert np.array_equal(out.cpu().numpy(), want)


def test_bin_features_extreme_bounds():
    say("bin_features bounds spanning the float range, and close together")
    # feature 0: bounds -3e38, 0, 3e38 (their span overflows); feature 1: two
    # bounds one float32 step apart; feature 2: equal-width bounds
    one_ulp = np.nextafter(np.float32(1.0), np.float32(2.0))
    upper = np.array([-3e38, 0.0, 3e38, 0.0,
                      1.0, one_ulp, 0.0,
                      -1.0, -0.5, 0.0, 0.5, 1.0, 0.0], dtype=np.float32)
    nbins = [4, 3, 6]
    rng = np.random.default_rng(58)
    n = 4000
    raw = np.empty((n, 3), dtype=np.float32)
    raw[:, 0] = rng.choice(np.array([-np.inf, -3.4e38, -3e38, -1.0, 0.0, 1.0, 3e38, 3.4e38, np.inf],
                                    dtype=np.float32), size=n)
    raw[:, 1] = rng.choice(np.array([0.5, 1.0, one_ulp, np.nextafter(one_ulp, np.float32(2.0)), 2.0],
                                    dtype=np.float32), size=n)
    raw[:, 2] = rng.uniform(-1.5, 1.5, size=n).astype(np.float32)
    raw[::7, 2] = rng.choice(upper[7:12], size=raw[::7, 2].shape[0])
    want, n_nan = oracle.bin_features(raw, nbins, upper)
    assert n_nan == 0
    ft = g.FeatureTable(nbins, DEV, pack_bits=False)
    out = torch.zeros((n, 3), dtype=torch.uint8, device=DEV)
    ws = _ws(n, 1, 1)
    g.gbdt_bin_features(to_dev(raw), ft, to_dev(upper), out, ws)
    assert g.gbdt_read_error(ws) == 0
    assert np.array_equal(out.cpu().numpy(), want)


def test_bin_features_nan_and_bad_bounds():
    say("bin_features NaN values and bad bounds")
    nbins = [8, 3]
    raw, upper = _bin_inputs(500, nbins, 56)
    raw[7, 0] = np.nan
    raw[499, 1] = np.nan
    want, n_nan = oracle.bin_features(raw, nbins, upper)
    assert n_nan == 2
    ft = g.FeatureTable(nbins, DEV, pack_bits=False)
    out = torch.zeros((500, 2), dtype=torch.uint8, device=DEV)
    ws = _ws(500, 1, 1)
    g.gbdt_bin_features(to_dev(raw), ft, to_dev(upper), out, ws)
    assert g.gbdt_read_error(ws) == -3
    assert np.array_equal(out.cpu().numpy(), want)  # NaN -> bin 0, the rest as usual
    bad = upper.copy()
    bad[2] = bad[1]  # feature 0: two equal bounds
    assert oracle.bin_features(raw, nbins, bad)[0] is None
    ws2 = _ws(500, 1, 1)
    raw_ok = np.nan_to_num(raw, nan=0.0)
    g.gbdt_bin_features(to_dev(raw_ok), ft, to_dev(bad), out, ws2)
    assert g.gbdt_read_error(ws2) == -3


def test_bin_features_empty_and_misaligned():
    say("bin_features empty input and a misaligned pointer")
    ft = g.FeatureTable([4, 4], DEV, pack_bits=False)
    upper = to_dev(np.array([0, 1, 2, 0, 0, 1, 2, 0], dtype=np.float32))
    ws = _ws(1, 1, 1)
    out = torch.full((0, 2), 7, dtype=torch.uint8, device=DEV)
    g.gbdt_bin_features(torch.zeros((0, 2), dtype=torch.float32, device=DEV), ft, upper, out, ws)
    assert g.gbdt_read_error(ws) == 0
    big = torch.zeros(2 * 64 + 1, dtype=torch.float32, device=DEV)
    raw = big[1:].view(64, 2)  # 4-byte offset: not 16-byte aligned
    out = torch.zeros((64, 2), dtype=torch.uint8, device=DEV)
    with pytest.raises(g.GbdtError):
        g.gbdt_bin_features(raw, ft, upper, out, ws)
