"""Bin bounds on the GPU (gbdt_feature_bounds) against the oracle, bit for bit.

Equal width over each feature's finite range and quantiles of a row sample
(the readings of the "Quantized" state, Training Core section 5), with the
non-increasing bounds raised to the next FP32 value; then binning with the
derived bounds.  Shapes: ragged row counts, one row, no rows, more rows than
the quantile sample, NaN / +-inf / ties / constant features, 2 to 256 bins.
"""
import numpy as np
import pytest
import torch

import histogram_split_finding_amd as g
import oracle
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _matrix(n, F, seed):
    rng = np.random.default_rng(seed)
    raw = rng.normal(0.0, 1.0, (n, F)).astype(np.float32)
    if F > 1:
        raw[:, 1] = np.round(raw[:, 1] * 3)          # heavy ties
    if F > 2:
        raw[:, 2] = np.float32(7.5)                  # constant
    if F > 3:
        raw[:, 3] = rng.exponential(1e6, n).astype(np.float32) - np.float32(1e6)
    if n > 0 and F > 4:
        raw[rng.integers(0, n, max(1, n // 50)), 4] = np.nan
        raw[0, 4] = np.inf
        raw[n - 1, 4] = -np.inf
    if F > 5:
        raw[:, 5] = np.nan                           # no finite value
    return raw


def _gpu_bounds(raw, nb, method):
    ft = g.FeatureTable(nb, DEV, pack_bits=False)
    n = raw.shape[0]
    t = torch.from_numpy(raw).to(DEV) if n > 0 else torch.zeros((0, raw.shape[1]), dtype=torch.float32, device=DEV)
    up = torch.full((ft.total_bins,), -1.0, dtype=torch.float32, device=DEV)
    ws = g.new_workspace(g.gbdt_workspace_bytes(max(n, 1), 1, ft.total_bins))
    g.gbdt_feature_bounds(t, ft, method, up, ws)
    assert g.gbdt_read_error(ws) == 0
    return up.cpu().numpy(), ft, t


@pytest.mark.parametrize("method", [g.BOUNDS_EQUAL_WIDTH, g.BOUNDS_QUANTILE])
@pytest.mark.parametrize("n,nb,seed", [
    (1000, [4, 8, 2, 64, 256, 3, 255], 1),
    (33, [16] * 9, 2),
    (1, [5, 5, 5, 5, 5, 5], 3),
    (0, [7, 2, 9, 3, 4, 6], 4),
    (32768, [256] * 6, 5),
    (70001, [64, 3, 17, 256, 2, 128, 9, 33], 6),
])
def test_bounds_match_oracle(method, n, nb, seed):
    say("bounds: method %d, n %d, %d features" % (method, n, len(nb)))
    raw = _matrix(n, len(nb), seed)
    got, ft, t = _gpu_bounds(raw, nb, method)
    want = oracle.feature_bounds(raw, nb, method)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    if n > 0:
        # binning with the derived bounds
        out = torch.zeros((n, len(nb)), dtype=torch.uint8, device=DEV)
        ws = g.new_workspace(g.gbdt_workspace_bytes(n, 1, ft.total_bins))
        g.gbdt_bin_features(t, ft, torch.from_numpy(got).to(DEV), out, ws)
        code = g.gbdt_read_error(ws)
        wb, nan = oracle.bin_features(raw, nb, want)
        assert code == (-3 if nan else 0)
        assert np.array_equal(out.cpu().numpy(), wb)


def test_bounds_full_size():
    """The 50M x 28 x 64-bin binning shape: both methods on the GPU against the
    oracle, then binned, sampled rows checked against the oracle."""
    n, F, B = 50_000_000, 28, 64
    say("bounds: full size %d x %d, %d bins" % (n, F, B))
    gen = torch.Generator(device=DEV)
    gen.manual_seed(71)
    raw = torch.randn((n, F), generator=gen, dtype=torch.float32, device=DEV)
    raw[:, 7].mul_(1e3).add_(5.0)
    ft = g.FeatureTable([B] * F, DEV, pack_bits=False)
    host = raw.cpu().numpy()
    ws = g.new_workspace(g.gbdt_workspace_bytes(n, 1, ft.total_bins))
    for method in (g.BOUNDS_EQUAL_WIDTH, g.BOUNDS_QUANTILE):
        up = torch.zeros(ft.total_bins, dtype=torch.float32, device=DEV)
        g.gbdt_feature_bounds(raw, ft, method, up, ws)
        assert g.gbdt_read_error(ws) == 0
        want = oracle.feature_bounds(host, [B] * F, method)
        assert np.array_equal(up.cpu().numpy().view(np.uint32), want.view(np.uint32)), method
        out = torch.empty((n, F), dtype=torch.uint8, device=DEV)
        g.gbdt_bin_features(raw, ft, up, out, ws)
        assert g.gbdt_read_error(ws) == 0
        rows = np.unique(np.random.default_rng(72).integers(0, n, 4096))
        wb, _ = oracle.bin_features(host[rows], [B] * F, want)
        assert np.array_equal(out[torch.from_numpy(rows).to(DEV)].cpu().numpy(), wb)
        if method == g.BOUNDS_QUANTILE:
            # the bins hold about 1/64 of the rows each
            counts = torch.bincount(out[:, 0].to(torch.int64), minlength=B).cpu().numpy()
            assert counts.min() > 0.8 * n / B and counts.max() < 1.2 * n / B
