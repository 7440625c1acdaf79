"""The nibble block: features of 3 to 16 bins stored as 4-bit cells, eight to
a word (the ExaBoost PR's two-cells-per-byte packing, here for the columns
that fit 16 bins), read by the histogram, the partition, the prediction
update and the ensemble prediction.

Every layout must give the oracle's trees and predictions bit for bit, and
the same bits as the layout without the nibble block; the first tree's
histograms are compared with the oracle's for every node the GPU builds or
derives.
"""
import numpy as np
import pytest

import datagen
import histogram_split_finding_amd as g
import oracle
from gpu_util import DEV, compare_tree, hist_from_device, min_split_count, orc_has_hist, say

pytestmark = pytest.mark.gpu

SHAPES = [
    # mixed: bytes, nibbles (3..16 bins) and bits
    dict(n=6000, n_bins=[5, 2, 16, 3, 256, 9, 12, 2, 4, 33], depth=5, T=3, seed=81),
    # numerai-like: every feature a nibble of about 5 bins, several words
    dict(n=9001, n_bins=[5] * 37 + [7, 3, 16], depth=6, T=2, seed=82),
    # one nibble word, no byte block, no bits
    dict(n=3000, n_bins=[3, 4, 5, 6, 7, 8], depth=4, T=3, seed=83),
]


def _train(bins, label, nb, pk, T, pack_nibbles):
    ds = g.Dataset(bins, label, nb, DEV, pack_nibbles=pack_nibbles)
    bst = g.Booster(ds, g.make_params(**pk))
    return ds, bst


@pytest.mark.parametrize("case", SHAPES)
def test_nibble_layout_trees_match_oracle(case):
    say("nibbles: %s" % case)
    bins, label, nb = datagen.make_random(case["n"], case["n_bins"], case["seed"], bin_kind=1, label_kind=2)
    pk = dict(max_depth=case["depth"], min_samples_leaf=2, learning_rate=0.4)
    T = case["T"]
    ds, bst = _train(bins, label, nb, pk, T, True)
    assert ds.X.n_nib_features == sum(1 for b in nb if 3 <= b <= 16)
    # the packed matrix unpacks to the input
    assert np.array_equal(ds.X.blocked_to_rowmajor().cpu().numpy(), bins)
    p = oracle.make_params(**pk)
    ref = oracle.train(bins, nb, label, p, T, keep_pred_per_tree=True, dump_tree=0)
    bst.train(1)
    TB = ds.ft.total_bins
    tree0 = bst.host_trees()[0]
    for v in orc_has_hist(tree0, p.max_depth, min_split_count(p)):
        cnt, gq = hist_from_device(bst.hist_g, bst.hist_cnt, v, TB)
        assert np.array_equal(cnt, ref["dump_cnt"][v]), ("count", v)
        assert np.array_equal(gq, ref["dump_gq"][v]), ("G", v)
    bst.train(T - 1)
    trees = bst.host_trees()
    for t in range(T):
        compare_tree(trees[t], ref["nodes"][t][: ref["n_nodes"][t]])
    assert np.array_equal(bst.pred.cpu().numpy(), ref["pred"])
    # the layout without the nibble block gives the same bits
    _, b2 = _train(bins, label, nb, pk, T, False)
    b2.train(T)
    assert b2.ds.X.n_nib_features == 0
    assert b"".join(t.tobytes() for t in b2.host_trees()) == b"".join(t.tobytes() for t in trees)
    assert np.array_equal(b2.pred.cpu().numpy(), bst.pred.cpu().numpy())
    # ensemble prediction of held-out rows through the nibble layout
    hb, _, _ = datagen.make_random(2345, case["n_bins"], case["seed"] + 100)
    hds = g.Dataset(hb, np.zeros(hb.shape[0], dtype=np.float32), nb, DEV)
    got = bst.predict(hds.X).cpu().numpy()
    want = oracle.predict(hb, ref["nodes"], ref["n_nodes"], 0.0, p.learning_rate)
    assert np.array_equal(got, want)


def test_nibble_layout_large_tiles():
    """More than 4M rows in a layout with at most one byte block: the
    partition's 4096-row tiles move the nibble words; logistic objective on
    the same layout (its Hessians ride through the same partition)."""
    n = (1 << 22) + 777
    say("nibbles: %d rows" % n)
    bins, label, nb = datagen.make_random(n, [5, 9, 16, 3, 64, 2, 7], 84, bin_kind=1, label_kind=2)
    for objective in (g.OBJECTIVE_SQUARED_ERROR, g.OBJECTIVE_LOGISTIC):
        y = label if objective == 0 else (label > np.median(label)).astype(np.float32)
        pk = dict(max_depth=5, learning_rate=0.3, objective=objective)
        ds, bst = _train(bins, y, nb, pk, 2, True)
        assert ds.X.n_nib_features == 5 and ds.X.n_blocks == 1
        bst.train(2)
        ref = oracle.train(bins, nb, y, oracle.make_params(**pk), 2)
        trees = bst.host_trees()
        for t in range(2):
            compare_tree(trees[t], ref["nodes"][t][: ref["n_nodes"][t]])
        assert np.array_equal(bst.pred.cpu().numpy(), ref["pred"])
