#!/usr/bin/env python3
"""Writes the oracle's expected outputs for the first trees of the two large
workloads (10,000,000 x 100 Zipf-skewed bins, depth 8; 50,000,000 x 28
uniform 64-bin, depth 12) to tests/golden/fullsize_w<k>.json.gz.

Only the seeded generator (datagen) and the CPU oracle (oracle) are called:
for each tree the oracle grows it from the predictions left by the previous
one (Training Core, section 6, steps 1-7) and dumps every node's histogram.
The file keeps
  - the input fingerprints (FNV-1a-64 of the bin and label bytes), so a test
    can tell that the generator reproduced the same inputs;
  - per tree: the grid exponent S, every node of the breadth-first array
    (feature, threshold bin, children, flags, depth, row count, fixed-point
    gradient sum, and the FP64 leaf value and gain as their IEEE bit
    patterns), the first 64 bits of a SHA-256 of each depth < max_depth node's histogram (uint32
    counts then int64 fixed-point sums, little-endian, in global bin order),
    a SHA-256 of the fixed-point gradients and of the predictions after the
    tree (float64, little-endian, row order), and the predictions of a few
    sampled rows.

Run from the repository root:  python tests/golden/make_fullsize_golden.py [k ...]
Takes a few minutes per tree (single-threaded oracle).
"""
from __future__ import annotations

import gzip
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402
import oracle  # noqa: E402

N_TREES = 2
SAMPLE_ROWS = 64


def sha(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def sample_rows(n: int):
    rng = np.random.default_rng(20261202)
    return sorted(set([0, n - 1] + rng.integers(0, n, size=SAMPLE_ROWS - 2).tolist()))


def make(k: int) -> dict:
    wl = dict(datagen.WORKLOADS[k])
    t0 = time.time()
    bins, label, nb = datagen.make_workload(k)
    n, F = bins.shape
    p = oracle.make_params(**wl)
    out = {
        "source": "written by tests/golden/make_fullsize_golden.py from datagen and the CPU oracle "
                  "(oracle/oracle.c: Training Core, sections 2, 3, 6 and 7)",
        "workload": wl["name"], "k": k, "rows": n, "features": F,
        "bins_fnv1a64": datagen.fingerprint(bins), "label_fnv1a64": datagen.fingerprint(label),
        "max_depth": int(p.max_depth), "sample_rows": sample_rows(n), "trees": [],
    }
    print("workload %d: %d x %d generated in %.1f s" % (k, n, F, time.time() - t0), flush=True)
    pred = np.zeros(n, dtype=np.float64)
    for t in range(N_TREES):
        t1 = time.time()
        r = oracle.train(bins, nb, label, p, 1, pred0=pred, dump_tree=0)
        nn = int(r["n_nodes"][0])
        tree = r["nodes"][0][:nn]
        pred = r["pred"]
        hist = {}
        for v in range(nn):
            if int(tree[v]["depth"]) < p.max_depth:
                hist[str(v)] = sha(r["dump_cnt"][v], r["dump_gq"][v])[:16]
        out["trees"].append({
            "scale": int(r["scale"][0]),
            "n_nodes": nn,
            "feature": tree["feature"].tolist(),
            "threshold_bin": tree["threshold_bin"].tolist(),
            "left": tree["left"].tolist(),
            "right": tree["right"].tolist(),
            "flags": tree["flags"].tolist(),
            "depth": tree["depth"].tolist(),
            "count": tree["count"].tolist(),
            "gsum_q": tree["gsum_q"].tolist(),
            "leaf_value_bits": tree["leaf_value"].view(np.uint64).tolist(),
            "gain_bits": tree["gain"].view(np.uint64).tolist(),
            "hist_sha256": hist,
            "q_sha256": sha(r["dump_k"]),
            "pred_sha256": sha(pred),
            "pred_sample_bits": pred[out["sample_rows"]].view(np.uint64).tolist(),
        })
        print("  tree %d: %d nodes, oracle %.1f s" % (t, nn, time.time() - t1), flush=True)
        del r
    return out


def main():
    ks = [int(a) for a in sys.argv[1:]] or [4, 5]
    for k in ks:
        g = make(k)
        path = os.path.join(HERE, "fullsize_w%d.json.gz" % k)
        with gzip.open(path, "wt", compresslevel=9) as fh:
            json.dump(g, fh, separators=(",", ":"))
        print("wrote %s (%d bytes)" % (path, os.path.getsize(path)), flush=True)


if __name__ == "__main__":
    main()
