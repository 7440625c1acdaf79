#!/usr/bin/env python3
"""Benchmark of the level-wise histogram GBDT hot path on one MI355X.

A step is one boosting iteration: gradients and the fixed-point grid, the
tree grown level by level (histograms of the smaller children, sibling
subtraction, split search, stable partition) and the prediction update,
over the full synthetic workload resident in HBM.

Default workload: 581,012 rows x 54 features (10 Gaussian features in 256
equal-width bins, 44 binary features with ~5% ones; integer label 1..7),
depth 10, 100 trees, lambda 1 -- the covtype-shaped depth-10 configuration.

Output: one JSON line on stdout (progress goes to stderr).
  value      histogram rows*features per second: rows*features the
             histogram build visits -- every directly built node's rows (root
             and smaller children; at a filtered level, gbdt_grow_filtered_levels,
             the parent's rows, which its tiles read and test) -- divided by
             the summed device time of the histogram build (k_hist and the
             reduction of multi-tile partials, k_hist_reduce) over the timed
             trees; value_built_rows_only credits the built nodes' own rows
             only
  roofline   the histogram build against the 8 TB/s HBM peak, algorithmic
             bytes n_v*(F + 4 + 8) + total_bins*12 per built node, n_v the
             rows visited as above; k_hist alone is reported beside it
  rooflines  the partition and the prediction update on the same trees
  trees_per_s / ms_per_step  whole boosting steps, host wall clock
  cpu_baseline  the CPU oracle (single thread) on a bounded sample of trees
  also       the same figures (value, rooflines, trees_per_s, per-kernel
             device time) for further workloads, each timed over its tree
             count after at least W trees and half a second of warm-up: by
             default the 10,000,000 x 100 (Zipf-skewed 256 bins, depth 8,
             20 trees) and the 50,000,000 x 28 (64 uniform bins, depth 12,
             10 trees) ones, whose histogram builds are bound by HBM rather
             than by latency
  binning    raw FP32 values to uint8 bins (the step before the path) at the
             50M x 28 x 64-bin shape: values/s, its HBM roofline and the
             oracle on a 200K-row sample
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DIAG_HIST = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def built_work(trees, n_features, total_bins, max_depth, min_split, filtered=0):
    """(built rows, built nodes) summed over trees: root plus the smaller child
    of every split pair whose larger child can still split.  A node of a
    filtered level (bit d of gbdt_grow_filtered_levels) is built from its
    parent's unmoved rows, so its rows are the parent's."""
    rows = 0
    nodes = 0
    for tr in trees:
        if max_depth >= 1 and int(tr[0]["count"]) >= min_split:
            rows += int(tr[0]["count"])
            nodes += 1
        for nd in tr:
            if nd["flags"] & 1:
                continue
            L, R = tr[int(nd["left"])], tr[int(nd["right"])]
            if int(L["depth"]) >= max_depth:
                continue
            nl, nr = int(L["count"]), int(R["count"])
            if max(nl, nr) >= min_split:
                rows += nl + nr if (filtered >> int(L["depth"])) & 1 else min(nl, nr)
                nodes += 1
    return rows, nodes


DIAG_HIST_REDUCE = 5
DIAG_FIND = 7
DIAG_PARTITION = 10
DIAG_UPDATE = 11


def other_rooflines(trees, kt, n, max_depth, workload_name, filtered=0):
    """HBM rooflines of the partition, the prediction update and the split
    search over the same timed trees, with the algorithmic bytes of each step
    (per row of a splitting node: 4 B row index read + 1 B bin + 4 B index
    written + 16 B of q moved; per row of the update: 4 B index + 16 B pred
    read and written).  Without filtered levels the partition runs after
    levels 0 .. max_depth - 2 over the splitting nodes' rows; with them
    (gbdt_grow_filtered_levels: the odd levels) one two-level partition
    follows each odd level d < max_depth - 1 and moves the rows of every
    level-(d - 1) node that split into a child that splits, counted here as
    one pass (25 B per row), although it advances the rows two levels.  The
    update is two launches per tree (the tree compaction, then the row
    walk), counted as one unit."""
    part_rows = 0
    for tr in trees:
        for nd in tr:
            if nd["flags"] & 1:
                continue
            dep = int(nd["depth"])
            if not filtered:
                if dep <= max_depth - 2:
                    part_rows += int(nd["count"])
            elif dep % 2 == 0 and dep + 2 < max_depth:
                kids = (tr[int(nd["left"])], tr[int(nd["right"])])
                if any(not (k["flags"] & 1) for k in kids):
                    part_rows += int(nd["count"])
    out = {}
    K = len(trees)

    def entry(kind, name, alg, units=None):
        t, launches = kt.get(kind, (0.0, 0))
        if launches == 0 or t <= 0.0:
            return None
        launches = units if units is not None else launches
        a = alg / (t * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBS, "traffic": None, "kernel": name, "launches": launches,
                "avg_launch_us": 1000.0 * t / launches, "alg_bytes_per_launch": alg / launches,
                "ms_per_tree": t / K}

    out["partition"] = entry(DIAG_PARTITION, "k_partition", part_rows * 25)
    if out["partition"] is not None:
        out["partition"]["traffic"] = profiled_traffic(workload_name, "k_partition")
    # two launches per update (the tree compaction, then the row walk)
    out["update"] = entry(DIAG_UPDATE, "k_compact_tree + k_update", K * n * 20, units=K)
    return out


def profiled_traffic(workload_name, kernel="k_hist"):
    """HBM bytes per launch of `kernel` (k_hist: with its reduction) from the
    committed rocprofv3 counter summary of this workload, if it was taken on
    the current kernel source; else None."""
    import hashlib
    if workload_name.startswith("binning"):
        path = os.path.join(ROOT, "profiles", "%s_%s_counters.txt" % (kernel, workload_name))
    else:
        path = os.path.join(ROOT, "profiles", "gbdt_tree_%s_counters.txt" % workload_name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    csrc = os.path.join(ROOT, "histogram_split_finding_amd", "csrc")
    h = hashlib.sha256()
    for name in ("gbdt_kernels.hip", "gbdt_driver.hip", "gbdt_internal.h", "gbdt_device.h"):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256") != h.hexdigest()[:16]:
        return None
    try:
        if workload_name.startswith("binning"):
            return float(fields["traffic_bytes_per_launch"])
        return float(fields["traffic_%s" % kernel])
    except (KeyError, ValueError):
        return None


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and the CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"model": model, "cpus_available": avail, "threads_used": 1}


def cpu_baseline(k, seconds_budget):
    """The oracle as it stands, single-threaded, on the first trees of the same workload."""
    import datagen
    import oracle
    bins, label, nb = datagen.make_workload(k)
    wl = dict(datagen.WORKLOADS[k])
    p = oracle.make_params(**wl)
    # one tree to size the sample
    r = oracle.train(bins, nb, label, p, 1)
    per_tree = max(r["seconds"], 1e-3)
    n_trees = int(max(1, min(wl["n_trees"], seconds_budget // per_tree)))
    r = oracle.train(bins, nb, label, p, n_trees)
    F = bins.shape[1]
    cells = 0
    for t in range(n_trees):
        tr = r["nodes"][t][: r["n_nodes"][t]]
        cells += int(sum(int(nd["count"]) for nd in tr if int(nd["depth"]) < p.max_depth)) * F
    return dict(value=cells / r["hist_seconds"], unit="rows*features/s", cores=1, kind="oracle",
                trees_per_s=n_trees / r["seconds"], host=host_cpu(),
                sample="first %d of %d trees of the workload, every node's histogram built directly "
                       "(no subtraction), single thread" % (n_trees, wl["n_trees"]))


def measure(g, datagen, torch, k, K, W, diag, warm_s=0.0):
    """Grows W untimed trees (more, until warm_s seconds have passed), then K
    timed trees of workload k on the GPU; with diag, K more trees with
    per-kernel events for the histogram roofline."""
    wl = dict(datagen.WORKLOADS[k])
    log("generating workload %d (%s)" % (k, wl["name"]))
    bins, label, nb = datagen.make_workload(k)
    n, F = bins.shape
    fp_bins, fp_label = datagen.fingerprint(bins), datagen.fingerprint(label)
    ds = g.Dataset(bins, label, nb, "cuda")
    del bins
    params = g.make_params(**wl)
    bst = g.Booster(ds, params)
    torch.cuda.synchronize()
    log("dataset on device: %d x %d, %d bins, blocks %d x %d" % (n, F, ds.ft.total_bins,
                                                                 ds.X.n_blocks, ds.X.block_stride))
    t_warm = time.perf_counter()
    for _ in range(W):
        bst.grow_tree()
    torch.cuda.synchronize()
    while time.perf_counter() - t_warm < warm_s:
        bst.grow_tree()
        torch.cuda.synchronize()
        W += 1
    bst.check()
    # back to the starting predictions, so the timed trees are the workload's
    # boosting rounds 1 .. K (the warm-up only settles clocks and caches)
    bst.pred.fill_(0.0)
    torch.cuda.synchronize()
    log("warmup done (%d trees; predictions reset)" % W)

    nodes_bufs = [torch.zeros(bst.sizes.max_nodes * g.NODE_DTYPE.itemsize, dtype=torch.uint8,
                              device="cuda") for _ in range(K)]
    nn_bufs = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        bst.grow_tree(nodes_bufs[i], nn_bufs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    bst.check()
    log("timed %d trees in %.3f s (%.2f trees/s)" % (K, wall, K / wall))

    min_split = 2 * max(int(params.min_samples_leaf), int(np.ceil(params.min_child_weight)), 1)
    TB = ds.ft.total_bins
    out = {
        "metric": "histogram rows*features/sec (HBM % of peak) + trees/sec at depth-10",
        "value": None,
        "unit": "rows*features/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": 1000.0 * wall / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64",
        "data": "synthetic",
        "config": {"workload": wl["name"], "rows": n, "features": F, "total_bins": TB,
                   "max_depth": params.max_depth, "trees": wl["n_trees"],
                   "learning_rate": params.learning_rate, "reg_lambda": params.reg_lambda,
                   "gamma": params.gamma, "min_samples_leaf": params.min_samples_leaf,
                   "min_child_weight": params.min_child_weight,
                   "bins_fnv1a64": fp_bins, "label_fnv1a64": fp_label,
                   "layout": {"byte_blocks": int(ds.X.n_blocks), "block_stride": int(ds.X.block_stride),
                              "bit_features": int(ds.X.n_bit_features),
                              "nibble_features": int(ds.X.n_nib_features),
                              "partition_moves": "row ids" if bst.moves_ids else "rows",
                              "filtered_levels": [d for d in range(params.max_depth)
                                                  if (bst.filtered_levels >> d) & 1],
                              "gather_copies": (["rows interleaved", "column-major"]
                                                if bst.rows_ix is not None else [])}},
        "trees_per_s": K / wall,
    }

    if diag:
        # second pass over the same rounds 1 .. K (predictions reset again):
        # per-kernel device time with events on the library's stream
        bst.pred.fill_(0.0)
        torch.cuda.synchronize()
        lib = g.load()
        cap = 64 * (params.max_depth + 4) * K + 64
        assert lib.gbdt_diag_enable(cap) == 0
        for i in range(K):
            bst.grow_tree(nodes_bufs[i], nn_bufs[i])
        import ctypes
        kinds = np.zeros(cap, dtype=np.int32)
        ms = np.zeros(cap, dtype=np.float32)
        cnt = ctypes.c_int32()
        rc = lib.gbdt_diag_read(cap, kinds.ctypes.data_as(ctypes.c_void_p),
                                ms.ctypes.data_as(ctypes.c_void_p), ctypes.byref(cnt))
        lib.gbdt_diag_disable()
        assert rc == 0
        bst.check()
        kinds, ms = kinds[: cnt.value], ms[: cnt.value]
        trees = [g.nodes_to_host(nodes_bufs[i], int(nn_bufs[i].item())) for i in range(K)]
        rows, nbuilt = built_work(trees, F, TB, params.max_depth, min_split, bst.filtered_levels)
        rows_built_only, _ = built_work(trees, F, TB, params.max_depth, min_split)
        kt = {kk: (float(ms[kinds == kk].sum()), int((kinds == kk).sum())) for kk in set(kinds.tolist())}
        hist_ms, launches = kt.get(DIAG_HIST, (0.0, 0))
        red_ms, red_launches = kt.get(DIAG_HIST_REDUCE, (0.0, 0))
        build_ms = hist_ms + red_ms
        cells = rows * F
        alg_bytes = rows * (F + 4 + 8) + nbuilt * TB * 12
        achieved = alg_bytes / (build_ms * 1e-3) / 1e9
        # the histogram build: k_hist plus the reduction of the partials of
        # nodes covered by several tiles (part of every such node's histogram)
        out["value"] = cells / (build_ms * 1e-3)
        # the same time, crediting only the rows of the nodes built (the
        # filtered levels' smaller children, not the parents' rows their tiles read)
        out["value_built_rows_only"] = rows_built_only * F / (build_ms * 1e-3)
        out["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(wl["name"]),
                           "kernel": "k_hist + k_hist_reduce", "launches": launches,
                           "avg_launch_us": 1000.0 * build_ms / max(launches, 1),
                           "alg_bytes_per_launch": alg_bytes / max(launches, 1),
                           "k_hist_avg_us": 1000.0 * hist_ms / max(launches, 1),
                           "k_hist_reduce_avg_us": 1000.0 * red_ms / max(red_launches, 1),
                           "k_hist_reduce_launches": red_launches,
                           "k_hist_only_frac": alg_bytes / (hist_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           # the same time over the built nodes' own rows only (a filtered
                           # level's smaller children, not the parents' rows its tiles read)
                           "frac_built_rows_only": (rows_built_only * (F + 4 + 8) + nbuilt * TB * 12)
                                                   / (build_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        out["rooflines"] = other_rooflines(trees, kt, n, params.max_depth, wl["name"], bst.filtered_levels)
        names = {1: "grad_max", 2: "grad_q", 3: "plan", 4: "hist", 5: "hist_reduce", 6: "subtract",
                 7: "find", 8: "tree_init", 9: "level", 10: "partition", 11: "update", 12: "pack"}
        out["device_ms_per_tree"] = {names.get(int(kk), str(kk)): kt[kk][0] / K for kk in sorted(kt)}
        out["built_rows_per_tree"] = rows / K
        out["built_rows_only_per_tree"] = rows_built_only / K
        log("histogram build: %d launches, %.3f ms total (k_hist %.3f + reduce %.3f), %.1f GB/s "
            "algorithmic (%.1f%% of 8 TB/s)" % (launches, build_ms, hist_ms, red_ms, achieved,
                                                100 * achieved / HBM_PEAK_GBS))
    del bst, ds
    torch.cuda.empty_cache()
    return out


DIAG_BIN = 13


def measure_binning(g, torch, R, with_cpu):
    """Raw FP32 -> uint8 binning (gbdt_bin_features) at the 50M x 28 x 64-bin
    shape: standard normal values, 63 equal-width bounds per feature over
    [-3, 3].  R timed launches after 3 warm-ups; the kernel's time comes from
    the library's events around each launch on its stream.  Algorithmic bytes:
    4 read + 1 written per value."""
    import ctypes
    n, F, B = 50_000_000, 28, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(61)
    raw = torch.randn((n, F), generator=gen, dtype=torch.float32, device="cuda")
    kk = np.arange(1, B, dtype=np.float64)
    one = np.concatenate([(-3.0 + 6.0 * kk / B).astype(np.float32), np.zeros(1, dtype=np.float32)])
    upper_host = np.tile(one, F)
    upper = torch.from_numpy(upper_host).cuda()
    ft = g.FeatureTable([B] * F, "cuda", pack_bits=False)
    out = torch.empty((n, F), dtype=torch.uint8, device="cuda")
    ws = g.new_workspace(g.gbdt_workspace_bytes(n, 1, 1))
    for _ in range(3):
        g.gbdt_bin_features(raw, ft, upper, out, ws)
    torch.cuda.synchronize()
    lib = g.load()
    assert lib.gbdt_diag_enable(R) == 0
    t0 = time.perf_counter()
    for _ in range(R):
        g.gbdt_bin_features(raw, ft, upper, out, ws)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / R
    kinds = np.zeros(R, dtype=np.int32)
    ms = np.zeros(R, dtype=np.float32)
    cnt = ctypes.c_int32()
    assert lib.gbdt_diag_read(R, kinds.ctypes.data_as(ctypes.c_void_p), ms.ctypes.data_as(ctypes.c_void_p),
                              ctypes.byref(cnt)) == 0
    lib.gbdt_diag_disable()
    if g.gbdt_read_error(ws) != 0:
        raise RuntimeError("binning: device-side error")
    t = float(ms[: cnt.value][kinds[: cnt.value] == DIAG_BIN].mean()) * 1e-3
    alg = 5 * n * F
    res = {"config": {"workload": "binning_50Mx28_b64_equal_width", "rows": n, "features": F, "bins": B},
           "value": n * F / t, "unit": "values/s", "launches": R, "ms_per_launch_wall": wall * 1e3,
           "roofline": {"bound": "hbm", "achieved": alg / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": alg / t / 1e9 / HBM_PEAK_GBS,
                        "traffic": profiled_traffic("binning_50Mx28_b64_equal_width", "k_bin"), "kernel": "k_bin",
                        "avg_launch_us": t * 1e6, "alg_bytes_per_launch": alg}}
    if with_cpu:
        import oracle
        m = 200_000
        sample = raw[:m].cpu().numpy()
        t0 = time.perf_counter()
        oracle.bin_features(sample, [B] * F, upper_host)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": m * F / dt, "unit": "values/s", "cores": 1, "kind": "oracle",
                               "sample": "first %d rows, single thread" % m, "host": host_cpu()}
    del raw, out
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed trees (default: the workload's tree count)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed trees before the timed ones (default: at least 2 trees and "
                         "half a second, so the GPU's clocks have settled; the JSON reports the count)")
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--also", type=int, nargs="*", default=[4, 5],
                    help="further workloads reported under 'also' (default: the 10M x 100 and "
                         "50M x 28 ones, whose histograms are bound by HBM; each its tree count)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-diag", action="store_true", help="skip the per-kernel timing pass")
    ap.add_argument("--no-binning", action="store_true", help="skip the binning measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import datagen
    import histogram_split_finding_amd as g

    if args.calibrate_copy:
        nbytes = 1 << 30
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 3
        print(json.dumps({"calibration": "plain device copy", "bytes_read": nbytes, "bytes_written": nbytes,
                          "copies": 3, "GBps_read_plus_write": 2 * nbytes / dt / 1e9}), flush=True)
        return

    out = None
    secondary = []
    for idx, k in enumerate([args.workload] + [w for w in args.also if w != args.workload]):
        wl = dict(datagen.WORKLOADS[k])
        # the further workloads time their whole tree count after a warm-up
        # of at least half a second (the first trees run at lower clocks), and
        # so does the primary one unless --warmup fixes its count
        K = (args.steps if args.steps is not None else wl["n_trees"]) if idx == 0 else wl["n_trees"]
        W = args.warmup if args.warmup is not None else 2
        warm_s = 0.0 if (idx == 0 and args.warmup is not None) else 0.5
        res = measure(g, datagen, torch, k, K, W, not args.no_diag, warm_s)
        if idx == 0:
            out = res
        else:
            secondary.append({key: res[key] for key in ("config", "value", "value_built_rows_only", "unit",
                                                        "steps", "warmup",
                                                        "ms_per_step",
                                                        "trees_per_s", "roofline", "rooflines",
                                                        "device_ms_per_tree")
                              if key in res})
    if secondary:
        out["also"] = secondary
    if not args.no_binning:
        log("binning 50M x 28 (raw FP32 -> 64 bins)")
        out["binning"] = measure_binning(g, torch, 20, not args.no_cpu_baseline)

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle), ~%.0f s" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
