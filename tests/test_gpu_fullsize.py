"""Parity at the five workloads' full sizes, in the launch configuration the
bench times (Dataset + Booster + gbdt_grow_tree).

Workloads 1-3: every node of the first trees and every prediction against
the oracle, run here, bit for bit.  Workloads 4-5 (10M x 100, 50M x 28):
the first two trees node by node, every histogram the GPU builds or derives,
the fixed-point gradients and every prediction against the oracle's outputs
stored by tests/golden/make_fullsize_golden.py (the oracle takes minutes
per tree there); and a second test in which the oracle computes sampled
outputs one by one while properties that hold at any size are checked on
everything: per-node row counts and gradient sums by routing every row
through the GPU tree, leaf weights from those sums, and the prediction
update.
"""
import gzip
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import datagen
import histogram_split_finding_amd as g
import oracle
from gpu_util import DEV, compare_tree, hist_from_device, min_split_count, orc_has_hist, say

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

pytestmark = pytest.mark.gpu


def _train_gpu(k, T):
    bins, label, nb = datagen.make_workload(k)
    wl = dict(datagen.WORKLOADS[k])
    ds = g.Dataset(bins, label, nb, DEV)
    bst = g.Booster(ds, g.make_params(**wl))
    preds = [bst.pred.cpu().numpy().copy()]
    for _ in range(T):
        bst.trees.append(bst.grow_tree())
        preds.append(bst.pred.cpu().numpy().copy())
    bst.check()
    return bins, label, nb, wl, bst, preds


@pytest.mark.parametrize("k,T", [(1, 5), (2, 4), (3, 3)])
def test_small_workloads_every_node(k, T):
    say("full-size workload %d: %d trees against the oracle" % (k, T))
    bins, label, nb, wl, bst, preds = _train_gpu(k, T)
    r = oracle.train(bins, nb, label, oracle.make_params(**wl), T, keep_pred_per_tree=True)
    trees = bst.host_trees()
    for t in range(T):
        compare_tree(trees[t], r["nodes"][t][: r["n_nodes"][t]])
        assert np.array_equal(preds[t + 1], r["pred_per_tree"][t]), (k, t)


def _route(tree, bins):
    """Node of every row at every depth (rows routed from the root)."""
    n = bins.shape[0]
    at = np.zeros(n, dtype=np.int32)
    per_depth = [at.copy()]
    feat = tree["feature"]
    thr = tree["threshold_bin"]
    left = tree["left"]
    right = tree["right"]
    leaf = (tree["flags"] & 1).astype(bool)
    while True:
        internal = ~leaf[at]
        if not internal.any():
            break
        idx = np.nonzero(internal)[0]
        v = at[idx]
        b = bins[idx, feat[v]]
        at = at.copy()
        at[idx] = np.where(b <= thr[v], left[v], right[v])
        per_depth.append(at)
    return per_depth


def _exact_group_sums(groups, k, n_groups):
    """int64 sums of k per group, exact (two float64 bincounts of 24-bit parts)."""
    lo = (k & ((1 << 24) - 1)).astype(np.float64)
    hi = (k >> 24).astype(np.float64)
    s_lo = np.bincount(groups, weights=lo, minlength=n_groups)
    s_hi = np.bincount(groups, weights=hi, minlength=n_groups)
    return s_hi.astype(np.int64) * (1 << 24) + s_lo.astype(np.int64)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("k,T", [(4, 2), (5, 2)])
def test_large_workloads_sampled_and_properties(k, T):
    say("full-size workload %d: %d trees, sampled oracle outputs + properties" % (k, T))
    bins, label, nb, wl, bst, preds = _train_gpu(k, T)
    p = oracle.make_params(**wl)
    t = T - 1
    tree = bst.host_trees()[t]
    n = bins.shape[0]
    # gradient grid of the last tree
    kq, S, _ = oracle.gradient_grid(preds[t], label)
    # (the driver keeps q as int32 when ceil(log2 n) >= 22: exact, |q| <= 2^30)
    dq = bst.q.view(torch.int32)[:n] if oracle.ceil_log2(n) >= 22 else bst.q
    assert np.array_equal(dq.cpu().numpy().astype(np.int64), kq)
    # row counts, gradient sums and leaf weights of every node, by routing
    depth_nodes = _route(tree, bins)
    nn = len(tree)
    count = np.zeros(nn, dtype=np.int64)
    gsum = np.zeros(nn, dtype=np.int64)
    seen = np.zeros(nn, dtype=bool)
    for at in depth_nodes:
        c = np.bincount(at, minlength=nn)
        s = _exact_group_sums(at, kq, nn)
        nodes_here = np.unique(at)
        count[nodes_here] = c[nodes_here]
        gsum[nodes_here] = s[nodes_here]
        seen[nodes_here] = True
    assert seen.all(), "every node holds rows"
    assert np.array_equal(tree["count"].astype(np.int64), count)
    assert np.array_equal(tree["gsum"], gsum)
    lam = float(p.reg_lambda)
    for v in range(nn):
        if tree[v]["flags"] & 1:
            G = np.ldexp(np.float64(gsum[v]), -S)
            w = -G / (np.float64(count[v]) + lam)
            assert float(tree[v]["leaf_value"]) == float(w), v
    # prediction update: pred + (eta * w(leaf of the row))
    leaf_of = depth_nodes[-1]
    w_all = tree["leaf_value"]
    expect = preds[t] + (p.learning_rate * w_all[leaf_of])
    assert np.array_equal(preds[t + 1], expect)
    # sampled oracle histograms and splits: the root and nodes down the tree
    TB = bst.ds.ft.total_bins
    ms = min_split_count(p)
    sample = [0]
    for d in (1, p.max_depth // 2, p.max_depth - 1):
        cand = [v for v in range(1, nn) if tree[v]["depth"] == d and tree[v]["count"] >= ms]
        if cand:
            sample.append(cand[len(cand) // 2])
    for v in sample:
        rows = np.nonzero(depth_nodes[int(tree[v]["depth"])] == v)[0].astype(np.int32)
        cnt, gq = oracle.node_histogram(bins, nb, rows, kq, S)
        dc, dg = hist_from_device(bst.hist_g, bst.hist_cnt, v, TB)
        assert np.array_equal(dc, cnt), ("hist cnt", k, v)
        assert np.array_equal(dg, gq), ("hist G", k, v)
        sp = oracle.best_split(cnt, gq, nb, int(gsum[v]), len(rows), S, p)
        nd = tree[v]
        if sp["valid"]:
            assert (int(nd["feature"]), int(nd["threshold_bin"])) == (int(sp["feature"]), int(sp["threshold_bin"])), v
            assert float(nd["gain"]) == float(sp["gain"]), v
        else:
            assert nd["flags"] & 1, v
        say("  node %d (depth %d, %d rows) matches the oracle" % (v, int(nd["depth"]), len(rows)))


def test_binning_full_size_sampled():
    """Binning at the 50M x 28 x 64-bin shape, in the launch configuration the
    bench times: 63 equal-width bounds per feature over [-3, 3] on standard
    normal values; 4096 sampled rows (and the first and last) against the
    oracle, which bins each row on its own."""
    n, F, B = 50_000_000, 28, 64
    say("binning full size %d x %d, %d bins" % (n, F, B))
    gen = torch.Generator(device=DEV)
    gen.manual_seed(61)
    raw = torch.randn((n, F), generator=gen, dtype=torch.float32, device=DEV)
    nbins = [B] * F
    k = np.arange(1, B, dtype=np.float64)
    one = np.concatenate([(-3.0 + 6.0 * k / B).astype(np.float32), np.zeros(1, dtype=np.float32)])
    upper = np.tile(one, F)
    ft = g.FeatureTable(nbins, DEV, pack_bits=False)
    out = torch.empty((n, F), dtype=torch.uint8, device=DEV)
    ws = g.new_workspace(g.gbdt_workspace_bytes(n, 1, 1))
    g.gbdt_bin_features(raw, ft, torch.from_numpy(upper).to(DEV), out, ws)
    assert g.gbdt_read_error(ws) == 0
    rng = np.random.default_rng(62)
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, size=4096)]))
    idx = torch.from_numpy(rows).to(DEV)
    want, n_nan = oracle.bin_features(raw[idx].cpu().numpy(), nbins, upper)
    assert n_nan == 0
    assert np.array_equal(out[idx].cpu().numpy(), want)
    # property over every value: bins are in range and ordered like the values
    # within a feature (checked on a 1M-row slice against a sort)
    assert int(out.max().item()) <= B - 1
    col = raw[:1_000_000, 5]
    b = out[:1_000_000, 5].to(torch.int32)
    order = torch.argsort(col)
    assert bool((b[order][1:] >= b[order][:-1]).all().item())


def _sha(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("k", [4, 5])
def test_large_workloads_whole_trees_match_oracle(k):
    """The first two trees of the 10M x 100 and 50M x 28 workloads against the
    oracle's stored outputs: every node (structure and fixed-point sums exact,
    leaf values and gains bit for bit), the gradients of each tree, the
    histogram of every node the GPU builds directly or derives by
    subtraction, and every prediction after each tree."""
    with gzip.open(os.path.join(GOLDEN, "fullsize_w%d.json.gz" % k), "rt") as fh:
        gold = json.load(fh)
    say("full-size workload %d: %d trees against the oracle's stored outputs" % (k, len(gold["trees"])))
    bins, label, nb = datagen.make_workload(k)
    assert datagen.fingerprint(bins) == gold["bins_fnv1a64"]
    assert datagen.fingerprint(label) == gold["label_fnv1a64"]
    wl = dict(datagen.WORKLOADS[k])
    ds = g.Dataset(bins, label, nb, DEV)
    bst = g.Booster(ds, g.make_params(**wl))
    p = oracle.make_params(**wl)
    ms = min_split_count(p)
    n, TB, D = bins.shape[0], ds.ft.total_bins, int(p.max_depth)
    del bins, label
    q32 = oracle.ceil_log2(n) >= 22
    rows = gold["sample_rows"]
    for t, gt in enumerate(gold["trees"]):
        nodes, nn = bst.grow_tree()
        torch.cuda.synchronize()
        tree = g.nodes_to_host(nodes, int(nn.item()))
        assert len(tree) == gt["n_nodes"], (t, len(tree), gt["n_nodes"])
        for f in ("feature", "threshold_bin", "left", "right", "flags", "depth", "count"):
            want = np.asarray(gt[f], dtype=np.int64)
            bad = np.nonzero(tree[f].astype(np.int64) != want)[0]
            assert bad.size == 0, (t, f, bad[:8].tolist())
        assert np.array_equal(tree["gsum"], np.asarray(gt["gsum_q"], dtype=np.int64)), (t, "gsum")
        for f in ("leaf_value", "gain"):
            bits = np.asarray(gt[f + "_bits"], dtype=np.uint64)
            bad = np.nonzero(tree[f].view(np.uint64) != bits)[0]
            assert bad.size == 0, (t, f, bad[:8].tolist())
        dq = bst.q.view(torch.int32)[:n] if q32 else bst.q[:n]
        assert _sha(dq.cpu().numpy().astype(np.int64)) == gt["q_sha256"], (t, "gradients")
        hg = bst.hist_g.view(-1, TB).cpu().numpy()
        hc = bst.hist_cnt.view(-1, TB).cpu().numpy().view(np.uint32)
        built = sorted(orc_has_hist(tree, D, ms))
        hs = gt["hist_sha256"]
        bad = [v for v in built if _sha(hc[v], hg[v])[:len(hs[str(v)])] != hs[str(v)]]
        assert not bad, (t, "histograms", bad[:8])
        pred = bst.pred.cpu().numpy()
        assert np.array_equal(pred[rows].view(np.uint64), np.asarray(gt["pred_sample_bits"], dtype=np.uint64))
        assert _sha(pred) == gt["pred_sha256"], (t, "predictions")
        say("  tree %d: %d nodes, %d histograms, %d predictions match" % (t, len(tree), len(built), n))
    bst.check()
