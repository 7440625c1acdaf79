"""Ensemble prediction (gbdt_predict) against the oracle's forward pass.

"Gradient boosted trees (spec model)", section Forward pass: every row is
routed through each tree (bin <= threshold_bin goes left) and the ensemble
adds learning_rate * leaf value tree by tree to the base score.  The trees
come from the GPU's own training (node for node the oracle's trees, which
other tests check); the rows are held-out rows drawn past the training rows,
and the training rows themselves, whose predictions must equal the
training-time predictions bit for bit.  Layouts with and without the bit
block, several column blocks, trees too large for LDS, no trees, and a
malformed tree are covered.
"""
import numpy as np
import pytest
import torch

import datagen
import histogram_split_finding_amd as g
import oracle
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _gpu_trees_as_oracle(bst):
    """The booster's trees as an oracle node array [T][stride] (the oracle's own
    node layout, filled field by field)."""
    stride = int(bst.sizes.max_nodes)
    T = len(bst.trees)
    arr = np.zeros((T, stride), dtype=oracle.NODE_DTYPE)
    counts = np.zeros(T, dtype=np.int32)
    for t, (nodes, nn) in enumerate(bst.trees):
        k = int(nn.item())
        src = g.nodes_to_host(nodes, k)
        counts[t] = k
        for f in ("feature", "threshold_bin", "left", "right", "leaf_value", "gain", "flags", "depth"):
            arr[t, :k][f] = src[f]
    return arr, counts


def _check(bins_train, label, nb, params, T, heldout, pack_bits=True, base=0.0):
    ds = g.Dataset(bins_train, label, nb, DEV, pack_bits=pack_bits)
    bst = g.Booster(ds, params, base_score=base)
    bst.train(T)
    trees, counts = _gpu_trees_as_oracle(bst)
    # training rows: the training-time predictions, bit for bit
    got = bst.predict(ds.X, base_score=base).cpu().numpy()
    assert np.array_equal(got, bst.pred.cpu().numpy())
    # held-out rows against the oracle's forward pass
    hb = np.ascontiguousarray(heldout)
    hds = g.Dataset(hb, np.zeros(hb.shape[0], dtype=np.float32), nb, DEV, pack_bits=pack_bits)
    got = bst.predict(hds.X, base_score=base).cpu().numpy()
    want = oracle.predict(hb, trees, counts, base, params.learning_rate)
    assert np.array_equal(got, want)
    # every prefix of the ensemble, and no trees at all
    for t in (0, 1, T // 2):
        got = bst.predict(hds.X, base_score=base, trees=bst.trees[:t]).cpu().numpy()
        assert np.array_equal(got, oracle.predict(hb, trees[:t], counts[:t], base, params.learning_rate))
    return bst


@pytest.mark.parametrize("pack_bits", [True, False])
@pytest.mark.parametrize("case", [
    dict(n=3000, n_bins=[7, 2, 33, 2, 256, 5, 2, 64], depth=5, T=4, seed=5),
    dict(n=5003, n_bins=[3] * 40 + [2] * 40, depth=3, T=6, seed=6),       # two blocks + two bit words
    dict(n=2049, n_bins=[256] * 70, depth=4, T=3, seed=7),                  # three column blocks
    dict(n=4000, n_bins=[9, 2, 17], depth=13, T=2, seed=8),                 # trees too large for LDS
])
def test_predict_small(case, pack_bits):
    say("predict: %s pack_bits=%s" % (case, pack_bits))
    bins, label, nb = datagen.make_random(case["n"] + 1777, case["n_bins"], case["seed"], label_kind=2)
    p = g.make_params(case["depth"], learning_rate=0.3, min_samples_leaf=3)
    n = case["n"]
    _check(bins[:n], label[:n], nb, p, case["T"], bins[n:], pack_bits=pack_bits, base=0.125)


@pytest.mark.parametrize("k,T,n_out", [(3, 12, 200_000), (5, 2, 1_000_000)])
def test_predict_workload_shapes(k, T, n_out):
    """Held-out rows of the covtype-shaped depth-10 workload and of the
    50M x 28 depth-12 one, with trees grown on the full training matrix."""
    say("predict: workload %d, %d trees, %d held-out rows" % (k, T, n_out))
    bins, label, nb = datagen.make_workload(k)
    wl = dict(datagen.WORKLOADS[k])
    hb, _, _ = datagen.make_heldout(k, n_out)
    _check(bins, label, nb, g.make_params(**wl), T, hb)


def test_predict_rejects_a_malformed_tree():
    bins, label, nb = datagen.make_random(1000, [8, 8], 9)
    ds = g.Dataset(bins, label, nb, DEV)
    bst = g.Booster(ds, g.make_params(3))
    bst.train(2)
    nodes, nn = bst.trees[1]
    arr = g.nodes_to_host(nodes)
    arr[0]["right"] = arr[0]["left"] + 2  # siblings no longer adjacent
    bad = torch.from_numpy(arr.view(np.uint8).copy()).to(DEV)
    out = torch.full((ds.n_rows,), 7.0, dtype=torch.float64, device=DEV)
    stride = int(bst.sizes.max_nodes)
    trees = torch.cat([bst.trees[0][0], bad])
    counts = torch.cat([bst.trees[0][1], nn])
    ws = g.new_workspace(g.gbdt_predict_workspace_bytes(2, stride))
    g.gbdt_predict(ds.X.matrix(), trees, counts, 2, stride, 0.0, 0.3, out, ws)
    assert g.gbdt_read_error(ws) == -1  # GBDT_E_ARG
    assert bool((out == 7.0).all().item())  # nothing written
