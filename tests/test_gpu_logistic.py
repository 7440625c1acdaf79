"""The logistic objective on the GPU against the oracle.

Sigmoid cross-entropy ("Gradient boosted trees (spec model)",
gbtBinaryCrossentropyGradSpec) with the Hessian s(1 - s): gradients and
Hessians on their own fixed-point grids, Hessian histograms next to the
counts, H in min_child_weight, in H > 0, in the gain and in the leaf weight.
Every tree node by node (structure, fixed-point gradient and Hessian sums,
leaf values and gains bit for bit), the Hessian and gradient histograms of
the first tree's nodes, and every prediction.
"""
import numpy as np
import pytest

import datagen
import histogram_split_finding_amd as g
import oracle
from gpu_util import DEV, compare_tree, hist_from_device, min_split_count, orc_has_hist, say

pytestmark = pytest.mark.gpu


def _run(bins, label, nb, T, pack_bits=True, **kw):
    kw = dict(kw)
    kw["objective"] = g.OBJECTIVE_LOGISTIC
    ds = g.Dataset(bins, label, nb, DEV, pack_bits=pack_bits)
    bst = g.Booster(ds, g.make_params(**kw))
    p = oracle.make_params(**kw)
    ref = oracle.train(bins, nb, label, p, T, keep_pred_per_tree=True, dump_tree=0)
    TB = ds.ft.total_bins
    # first tree: histograms of every node the GPU builds or derives
    bst.train(1)
    tree0 = bst.host_trees()[0]
    ms = 2 * max(int(p.min_samples_leaf), 1)
    for v in orc_has_hist(tree0, p.max_depth, ms):
        cnt, gq = hist_from_device(bst.hist_g, bst.hist_cnt, v, TB)
        hq = bst.hist_h[v * TB:(v + 1) * TB].cpu().numpy()
        assert np.array_equal(cnt, ref["dump_cnt"][v]), ("count", v)
        assert np.array_equal(gq, ref["dump_gq"][v]), ("G", v)
        assert np.array_equal(hq, ref["dump_hq"][v]), ("H", v)
    assert np.array_equal(bst.pred.cpu().numpy(), ref["pred_per_tree"][0])
    for t in range(1, T):
        bst.train(1)
        assert np.array_equal(bst.pred.cpu().numpy(), ref["pred_per_tree"][t]), ("pred", t)
    trees = bst.host_trees()
    for t in range(T):
        want = ref["nodes"][t][: ref["n_nodes"][t]]
        compare_tree(trees[t], want)
        assert np.array_equal(trees[t]["hsum"], want["hsum_q"]), (t, "hsum")
    assert np.array_equal(bst.pred.cpu().numpy(), ref["pred"])
    return bst, ref


@pytest.mark.parametrize("pack_bits", [True, False])
@pytest.mark.parametrize("case", [
    dict(n=5000, n_bins=[9, 2, 33, 2, 256, 5], depth=5, T=3, seed=51, msl=1, mcw=0.0, lam=1.0),
    dict(n=7001, n_bins=[3] * 40 + [2] * 40, depth=4, T=3, seed=52, msl=5, mcw=2.0, lam=0.5),
    dict(n=4100, n_bins=[256] * 70, depth=3, T=2, seed=53, msl=1, mcw=0.5, lam=0.0),
])
def test_logistic_small(case, pack_bits):
    say("logistic: %s pack_bits=%s" % (case, pack_bits))
    bins, _, nb = datagen.make_random(case["n"], case["n_bins"], case["seed"])
    rng = np.random.default_rng(case["seed"])
    score = bins[:, 0].astype(np.float64) / nb[0] + bins[:, 2].astype(np.float64) / nb[2] + \
        rng.normal(0.0, 0.3, case["n"])
    label = (score > 1.0).astype(np.float32)
    _run(bins, label, nb, case["T"], pack_bits=pack_bits, max_depth=case["depth"],
         min_samples_leaf=case["msl"], min_child_weight=case["mcw"], reg_lambda=case["lam"],
         learning_rate=0.5, gamma=0.01)


@pytest.mark.parametrize("k,T,cut", [(3, 3, 5.0), (2, 2, 0.0)])
def test_logistic_workload_shapes(k, T, cut):
    """The covtype-shaped depth-10 workload (label >= 5 as the positive class)
    and the 1M x 32 depth-6 one (label > 0), full size."""
    say("logistic: workload %d, %d trees" % (k, T))
    bins, label, nb = datagen.make_workload(k)
    wl = dict(datagen.WORKLOADS[k])
    y = (label >= cut).astype(np.float32) if k == 3 else (label > cut).astype(np.float32)
    _run(bins, y, nb, T, max_depth=wl["max_depth"], min_samples_leaf=wl["min_samples_leaf"],
         reg_lambda=wl["reg_lambda"], learning_rate=wl["learning_rate"])


def test_logistic_over_2_pow_21_rows():
    """More than 2^21 rows: the grids' 30-bit cap no longer binds (52 - e -
    ceil(log2 n) is smaller), the same int32 fixed-point values, larger
    partition tiles."""
    n = (1 << 22) + 12345
    say("logistic: %d rows" % n)
    bins, _, nb = datagen.make_random(n, [64, 64, 2, 16, 256], 61)
    label = ((bins[:, 0].astype(np.int32) + bins[:, 3] * 4) > 80).astype(np.float32)
    _run(bins, label, nb, 2, max_depth=5, learning_rate=0.3)
