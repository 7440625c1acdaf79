"""gbdt_predict_noalloc (no workspace, the library's per-GPU scratch) against
gbdt_predict (caller's workspace) through the C ABI: two calls in a row, the
second with fewer rows and fewer trees, bit for bit; a size beyond the
scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

import datagen
import histogram_split_finding_amd as g
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _run_both(bst, X, trees, base):
    stride = int(bst.sizes.max_nodes)
    T = len(trees)
    nodes = torch.cat([t[0] for t in trees])
    counts = torch.cat([t[1] for t in trees])
    want = torch.empty(X.n_rows, dtype=torch.float64, device=DEV)
    ws = g.new_workspace(g.gbdt_predict_workspace_bytes(T, stride))
    g.gbdt_predict(X.matrix(), nodes, counts, T, stride, base, bst.params.learning_rate, want, ws)
    assert g.gbdt_read_error(ws) == 0
    got = torch.full((X.n_rows,), -1.0, dtype=torch.float64, device=DEV)
    status = torch.full((1,), 12345, dtype=torch.int32, device=DEV)
    g.gbdt_predict_noalloc(X.matrix(), nodes, counts, T, stride, base, bst.params.learning_rate, got, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(got, want)
    return got


def test_predict_noalloc_matches_predict():
    say("no-alloc predict: two calls against gbdt_predict")
    nb = [9, 2, 33, 2, 256, 5, 2, 64, 17, 3]
    bins, label, nb = datagen.make_random(30000, nb, 41, label_kind=2)
    ds = g.Dataset(bins[:20000], label[:20000], nb, DEV)
    bst = g.Booster(ds, g.make_params(6, learning_rate=0.3))
    bst.train(5)
    big = g.Dataset(bins[20000:], label[20000:], nb, DEV)
    small = g.Dataset(bins[20000:21234], label[20000:21234], nb, DEV)
    a = _run_both(bst, big.X, bst.trees, 0.5)
    b = _run_both(bst, small.X, bst.trees[:3], -0.25)
    assert not torch.equal(a[:1234], b)  # the second call is a different computation
    # a tree set beyond the scratch is refused on the host
    stride = int(bst.sizes.max_nodes)
    too_many = (16 << 20) // (16 * stride) + 1
    out = torch.zeros(small.n_rows, dtype=torch.float64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    nodes = torch.zeros(too_many * stride * 64, dtype=torch.uint8, device=DEV)
    counts = torch.ones(too_many, dtype=torch.int32, device=DEV)
    with pytest.raises(g.GbdtError):
        g.gbdt_predict_noalloc(small.X.matrix(), nodes, counts, too_many, stride, 0.0, 0.3, out, status)
