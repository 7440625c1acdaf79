"""Index mode of the tree driver: for rows of two or more byte blocks the
partition moves row ids and q only ("Module Design: Training Core", section
6, step 5: a stable partition of row indices) and the histogram reads each
node's rows of the original matrix through the ids.

Trees (node by node), the histograms of every node the first tree builds or
derives, and the predictions must equal the oracle's bit for bit, for two to
eight blocks, skewed and uniform bins, ragged row counts, small nodes, and
more than 4M rows (the 8192-row partition tiles and int32 q) -- gathering
from the block-major matrix itself and from its row-interleaved and
column-major copies (gbdt_interleave_rows, gbdt_column_major), which their
own test checks byte by byte.
"""
import numpy as np
import pytest

import datagen
import histogram_split_finding_amd as g
import oracle
from gpu_util import DEV, compare_tree, hist_from_device, min_split_count, orc_has_hist, say

pytestmark = pytest.mark.gpu

CASES = [
    # two blocks of 17 and 16 columns, ragged n, depth 6
    dict(n=7777, n_bins=[256] * 33, depth=6, T=3, seed=91, bin_kind=0, msl=1),
    # two blocks of 32 columns, Zipf-skewed bins, min_samples_leaf
    dict(n=30011, n_bins=[256] * 64, depth=7, T=2, seed=92, bin_kind=1, msl=25),
    # eight blocks of 32 columns of mixed widths, deep and narrow nodes
    dict(n=5003, n_bins=[256, 3, 17, 64] * 64, depth=9, T=2, seed=93, bin_kind=0, msl=1),
    # three blocks, one row per leaf possible
    dict(n=900, n_bins=[5] * 70, depth=10, T=2, seed=94, bin_kind=0, msl=1),
]


@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_index_mode_trees_match_oracle(case, interleave):
    say("index mode: %s interleave %s" % (case, interleave))
    bins, label, nb = datagen.make_random(case["n"], case["n_bins"], case["seed"], bin_kind=case["bin_kind"])
    pk = dict(max_depth=case["depth"], min_samples_leaf=case["msl"], learning_rate=0.4)
    ds = g.Dataset(bins, label, nb, DEV, pack_bits=False, pack_nibbles=False)
    assert ds.X.n_blocks >= 2
    bst = g.Booster(ds, g.make_params(**pk), interleave=interleave)
    assert bst.moves_ids and bst.pp[0].bins is None
    assert (bst.rows_ix is not None) == interleave and (bst.cols is not None) == interleave
    p = oracle.make_params(**pk)
    ref = oracle.train(bins, nb, label, p, case["T"], keep_pred_per_tree=True, dump_tree=0)
    bst.train(1)
    TB = ds.ft.total_bins
    tree0 = bst.host_trees()[0]
    for v in orc_has_hist(tree0, p.max_depth, min_split_count(p)):
        cnt, gq = hist_from_device(bst.hist_g, bst.hist_cnt, v, TB)
        assert np.array_equal(cnt, ref["dump_cnt"][v]), ("count", v)
        assert np.array_equal(gq, ref["dump_gq"][v]), ("G", v)
    assert np.array_equal(bst.pred.cpu().numpy(), ref["pred_per_tree"][0])
    bst.train(case["T"] - 1)
    trees = bst.host_trees()
    for t in range(case["T"]):
        compare_tree(trees[t], ref["nodes"][t][: ref["n_nodes"][t]])
    assert np.array_equal(bst.pred.cpu().numpy(), ref["pred"])


def test_copy_layouts():
    """gbdt_interleave_rows: row r's block b lands at r P + b block_stride,
    the bytes after a row's blocks zero, with P the row's bytes rounded up to
    a power of two up to 128 and to a multiple of 128 beyond;
    gbdt_column_major: column c's byte of row r at c row_capacity + r -- for
    a ragged row count and three blocks (P 128 and 64) and eight (P 256)."""
    import torch
    n = 3001
    for F, want_P in ((70, 128), (40, 64), (250, 256)):
        bins, label, nb = datagen.make_random(n, [256] * F, 96)
        ds = g.Dataset(bins, label, nb, DEV, pack_bits=False, pack_nibbles=False)
        X = ds.X.matrix()
        nbk, bs, cap = int(X.n_blocks), int(X.block_stride), int(X.row_capacity)
        P = g.gbdt_interleave_pitch(X)
        say("copy layout: F %d blocks %d stride %d pitch %d" % (F, nbk, bs, P))
        assert P == want_P and P >= nbk * bs
        out = torch.full((cap * P + 64,), 0xA5, dtype=torch.uint8, device=DEV)
        g.gbdt_interleave_rows(X, out)
        got = out.cpu().numpy()
        assert (got[cap * P:] == 0xA5).all()  # nothing past the copy is written
        rows = got[: cap * P].reshape(cap, P)
        blocked = ds.X.bins.cpu().numpy()[: nbk * cap * bs].reshape(nbk, cap, bs)
        assert np.array_equal(rows[:, : nbk * bs].reshape(cap, nbk, bs), blocked.transpose(1, 0, 2))
        assert (rows[:, nbk * bs:] == 0).all()
        # the copy's block b, column j of row r is the matrix's bin of that
        # column (no packing: matrix column c is feature c)
        assert not ds.ft.mapped
        bf = int(X.block_features)
        r = np.arange(n)
        for c in sorted({0, 5, bf, min(2 * bf + 1, F - 1), F - 1}):
            b, j = divmod(c, bf)
            assert np.array_equal(rows[r, b * bs + j], bins[r, c])
        cols = torch.full((cap * F + 64,), 0x5A, dtype=torch.uint8, device=DEV)
        g.gbdt_column_major(X, cols)
        got = cols.cpu().numpy()
        assert np.array_equal(got[: cap * F].reshape(F, cap)[:, :n], bins.T)
        assert (got[cap * F:] == 0x5A).all()


@pytest.mark.parametrize("interleave", [False, True])
def test_index_mode_over_4m_rows(interleave):
    """More than 4M rows of two blocks: int32 q and the 8192-row tiles of the
    id-only partition."""
    n = (1 << 22) + 4321
    say("index mode: %d rows interleave %s" % (n, interleave))
    bins, label, nb = datagen.make_random(n, [64] * 40, 95)
    pk = dict(max_depth=5, learning_rate=0.3)
    ds = g.Dataset(bins, label, nb, DEV)
    bst = g.Booster(ds, g.make_params(**pk), interleave=interleave)
    assert bst.moves_ids
    bst.train(2)
    ref = oracle.train(bins, nb, label, oracle.make_params(**pk), 2)
    trees = bst.host_trees()
    for t in range(2):
        compare_tree(trees[t], ref["nodes"][t][: ref["n_nodes"][t]])
    assert np.array_equal(bst.pred.cpu().numpy(), ref["pred"])
