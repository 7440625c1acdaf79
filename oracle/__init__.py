"""CPU oracle (ctypes wrapper around oracle.c).

TEST INFRASTRUCTURE: only tests/, the smoke check and the bench's CPU-baseline
leg may import this package.  The GPU library and its Python binding never
import, call or link it.

Everything the oracle computes is documented in oracle.c with the passage of
the pages it follows ("Module Design: Training Core", sections 2, 3, 6, 7).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "_liboracle.so")
_lib = None

LEAF = 1

NODE_DTYPE = np.dtype([
    ("feature", "<i4"), ("threshold_bin", "<i4"), ("left", "<i4"), ("right", "<i4"),
    ("leaf_value", "<f8"), ("gain", "<f8"), ("flags", "<u4"), ("depth", "<i4"),
    ("count", "<i8"), ("gsum_q", "<i8"), ("hsum_q", "<i8"),
])
assert NODE_DTYPE.itemsize == 64

SPLIT_DTYPE = np.dtype([
    ("gain", "<f8"), ("feature", "<i4"), ("threshold_bin", "<i4"), ("n_left", "<i8"),
    ("gq_left", "<i8"), ("valid", "<i4"), ("pad", "<i4"), ("h_left", "<f8"),
])
assert SPLIT_DTYPE.itemsize == 48

SQUARED_ERROR = 0
LOGISTIC = 1


class OrcParams(ctypes.Structure):
    _fields_ = [("reg_lambda", ctypes.c_double), ("gamma", ctypes.c_double),
                ("min_child_weight", ctypes.c_double), ("learning_rate", ctypes.c_double),
                ("min_samples_leaf", ctypes.c_int32), ("max_depth", ctypes.c_int32),
                ("objective", ctypes.c_int32), ("pad", ctypes.c_int32)]


def build(force: bool = True) -> str:
    """Compile oracle.c (gcc, -O2, no contraction, no fast-math)."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-mno-fma", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    lib.orc_validate_params.restype = ctypes.c_int
    lib.orc_validate_params.argtypes = [ctypes.POINTER(OrcParams)]
    lib.orc_ceil_log2.restype = ctypes.c_int32
    lib.orc_ceil_log2.argtypes = [ctypes.c_int64]
    lib.orc_gradient_grid.restype = ctypes.c_int
    lib.orc_gradient_grid.argtypes = [ctypes.c_int64, vp, vp, vp, vp, vp]
    lib.orc_node_histogram.restype = ctypes.c_int
    lib.orc_node_histogram.argtypes = [vp, ctypes.c_int32, vp, ctypes.c_int32, vp, ctypes.c_int64,
                                       vp, ctypes.c_int32, vp, vp, vp, vp, vp, ctypes.c_int32, vp]
    lib.orc_exp_neg.restype = ctypes.c_double
    lib.orc_exp_neg.argtypes = [ctypes.c_double]
    lib.orc_logistic_gh.restype = None
    lib.orc_logistic_gh.argtypes = [ctypes.c_double, ctypes.c_double, vp, vp]
    lib.orc_logistic_grid.restype = ctypes.c_int
    lib.orc_logistic_grid.argtypes = [ctypes.c_int64, vp, vp, vp, vp, vp, vp]
    lib.orc_best_split.restype = ctypes.c_int
    lib.orc_best_split.argtypes = [ctypes.c_int32, vp, vp, vp, vp, vp, vp, ctypes.c_double,
                                   ctypes.c_double, ctypes.c_int64, ctypes.POINTER(OrcParams), vp]
    lib.orc_leaf_weight.restype = ctypes.c_double
    lib.orc_leaf_weight.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
    lib.orc_partition.restype = ctypes.c_int64
    lib.orc_partition.argtypes = [vp, ctypes.c_int32, vp, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_int32, vp, vp]
    lib.orc_train.restype = ctypes.c_int
    lib.orc_train.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, vp, vp, ctypes.POINTER(OrcParams),
                              ctypes.c_int32, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp,
                              vp, vp, vp]
    lib.orc_predict.restype = ctypes.c_int
    lib.orc_predict.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, ctypes.c_int32, vp, ctypes.c_int32,
                                vp, ctypes.c_double, ctypes.c_double, vp]
    lib.orc_feature_bounds.restype = ctypes.c_int
    lib.orc_feature_bounds.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, vp, ctypes.c_int32, vp]
    lib.orc_bin_features.restype = ctypes.c_int64
    lib.orc_bin_features.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, vp, vp, vp, vp]
    _lib = lib
    return lib


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.c_void_p)


def make_params(max_depth, reg_lambda=1.0, gamma=0.0, min_child_weight=0.0, learning_rate=0.3,
                min_samples_leaf=1, objective=SQUARED_ERROR, **_ignored) -> OrcParams:
    return OrcParams(float(reg_lambda), float(gamma), float(min_child_weight), float(learning_rate),
                     int(min_samples_leaf), int(max_depth), int(objective), 0)


def validate_params(**kw) -> int:
    p = make_params(**kw)
    return int(_load().orc_validate_params(ctypes.byref(p)))


def ceil_log2(n: int) -> int:
    return int(_load().orc_ceil_log2(n))


def bin_offsets(n_bins) -> np.ndarray:
    nb = np.asarray(n_bins, dtype=np.int64)
    off = np.zeros(nb.shape[0] + 1, dtype=np.int32)
    off[1:] = np.cumsum(nb)
    return off


def gradient_grid(pred, label):
    """(k int64[n], S, g float64[n]) for g = pred - label on the per-tree grid."""
    pred = np.ascontiguousarray(pred, dtype=np.float64)
    label = np.ascontiguousarray(label, dtype=np.float32)
    n = pred.shape[0]
    k = np.empty(n, dtype=np.int64)
    g = np.empty(n, dtype=np.float64)
    S = ctypes.c_int32()
    rc = _load().orc_gradient_grid(n, _p(pred), _p(label), _p(k), ctypes.addressof(S), _p(g))
    if rc:
        raise ValueError("orc_gradient_grid failed (%d)" % rc)
    return k, int(S.value), g


def exp_neg(x: float) -> float:
    """orc_exp_neg: e^x for x <= 0 (Cody-Waite reduction, degree-13 Taylor series)."""
    return float(_load().orc_exp_neg(float(x)))


def logistic_gh(p: float, y: float):
    """(g, h) of the sigmoid cross-entropy at raw score p and label y."""
    g = ctypes.c_double()
    h = ctypes.c_double()
    _load().orc_logistic_gh(float(p), float(y), ctypes.addressof(g), ctypes.addressof(h))
    return g.value, h.value


def logistic_grid(pred, label):
    """(kg int64[n], kh int64[n], Sg, Sh) of the logistic objective."""
    pred = np.ascontiguousarray(pred, dtype=np.float64)
    label = np.ascontiguousarray(label, dtype=np.float32)
    n = pred.shape[0]
    kg = np.empty(n, dtype=np.int64)
    kh = np.empty(n, dtype=np.int64)
    sg = ctypes.c_int32()
    sh = ctypes.c_int32()
    rc = _load().orc_logistic_grid(n, _p(pred), _p(label), _p(kg), _p(kh), ctypes.addressof(sg),
                                   ctypes.addressof(sh))
    if rc:
        raise ValueError("orc_logistic_grid failed (%d)" % rc)
    return kg, kh, int(sg.value), int(sh.value)


def node_histogram(bins, n_bins, rows, k, S, kh=None, Sh=0):
    """Histogram of the rows (in the given order): (cnt uint32[TB], gq int64[TB]),
    plus hq int64[TB] when the logistic Hessians kh are given."""
    bins = np.ascontiguousarray(bins, dtype=np.uint8)
    n_bins = np.ascontiguousarray(n_bins, dtype=np.int32)
    off = bin_offsets(n_bins)
    TB = int(off[-1])
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    k = np.ascontiguousarray(k, dtype=np.int64)
    cnt = np.empty(TB, dtype=np.uint32)
    gq = np.empty(TB, dtype=np.int64)
    g = np.empty(TB, dtype=np.float64)
    h = np.empty(TB, dtype=np.float64)
    hq = np.empty(TB, dtype=np.int64) if kh is not None else None
    khc = np.ascontiguousarray(kh, dtype=np.int64) if kh is not None else None
    rc = _load().orc_node_histogram(_p(bins), bins.shape[1], _p(off), TB, _p(rows), rows.shape[0],
                                    _p(k), S, _p(cnt), _p(gq), _p(g), _p(h), _p(khc), int(Sh), _p(hq))
    if rc:
        raise RuntimeError("orc_node_histogram: FP64 sum differs from its int64 shadow")
    return (cnt, gq) if kh is None else (cnt, gq, hq)


def best_split(cnt, gq, n_bins, node_gq: int, node_n: int, S: int, params: OrcParams, hq=None,
               node_hq: int = 0, Sh: int = 0):
    """Best split of one node from its histogram; returns a SPLIT_DTYPE record.
    With hq (logistic), H comes from the fixed-point Hessian sums on grid Sh."""
    n_bins = np.ascontiguousarray(n_bins, dtype=np.int32)
    off = bin_offsets(n_bins)
    cnt = np.ascontiguousarray(cnt, dtype=np.uint32)
    gq = np.ascontiguousarray(gq, dtype=np.int64)
    g = np.ldexp(gq.astype(np.float64), -S)
    if hq is None:
        h = cnt.astype(np.float64)
        H_v = float(node_n)
    else:
        h = np.ascontiguousarray(np.ldexp(np.asarray(hq, dtype=np.int64).astype(np.float64), -Sh))
        H_v = float(np.ldexp(np.float64(node_hq), -Sh))
    G_v = float(np.ldexp(np.float64(node_gq), -S))
    out = np.zeros(1, dtype=SPLIT_DTYPE)
    _load().orc_best_split(n_bins.shape[0], _p(n_bins), _p(off), _p(cnt), _p(gq), _p(g), _p(h),
                           G_v, H_v, node_n, ctypes.byref(params), _p(out))
    return out[0]


def leaf_weight(G: float, H: float, reg_lambda: float) -> float:
    return float(_load().orc_leaf_weight(G, H, reg_lambda))


def partition(bins, rows, feature: int, threshold_bin: int):
    bins = np.ascontiguousarray(bins, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    left = np.empty(rows.shape[0], dtype=np.int32)
    right = np.empty(rows.shape[0], dtype=np.int32)
    nl = _load().orc_partition(_p(bins), bins.shape[1], _p(rows), rows.shape[0], feature,
                               threshold_bin, _p(left), _p(right))
    return left[:nl].copy(), right[:rows.shape[0] - nl].copy()


def bin_features(raw, n_bins, upper):
    """Bins of a float32 [n][F] matrix: per value, the number of its feature's
    upper bounds strictly below it (bounds of feature f at bin_offset[f] + k,
    k < n_bins[f] - 1).  Returns (uint8 [n][F], NaN count), or (None, -1) when
    the bounds are NaN or not strictly increasing."""
    raw = np.ascontiguousarray(raw, dtype=np.float32)
    nb = np.ascontiguousarray(n_bins, dtype=np.int32)
    off = bin_offsets(nb)
    upper = np.ascontiguousarray(upper, dtype=np.float32)
    if upper.shape[0] < int(off[-1]):
        raise ValueError("upper must hold total_bins entries")
    out = np.zeros(raw.shape, dtype=np.uint8)
    rc = int(_load().orc_bin_features(raw.shape[0], raw.shape[1], _p(raw), _p(nb), _p(off), _p(upper),
                                      _p(out)))
    if rc < 0:
        return None, rc
    return out, rc


def predict(bins, trees, n_nodes, base_score=0.0, learning_rate=0.3):
    """Ensemble forward pass (orc_predict): base + eta*w_1 + eta*w_2 + ... added
    tree by tree.  trees: [T][stride] NODE_DTYPE (oracle node arrays, e.g.
    train()["nodes"]); n_nodes: [T]."""
    bins = np.ascontiguousarray(bins, dtype=np.uint8)
    n, F = bins.shape
    trees = np.ascontiguousarray(trees, dtype=NODE_DTYPE)
    if trees.ndim == 1:
        trees = trees[None, :]
    n_nodes = np.ascontiguousarray(n_nodes, dtype=np.int32)
    out = np.empty(n, dtype=np.float64)
    rc = _load().orc_predict(n, F, _p(bins), trees.shape[0], _p(trees), trees.shape[1], _p(n_nodes),
                             float(base_score), float(learning_rate), _p(out))
    if rc:
        raise ValueError("orc_predict failed (%d)" % rc)
    return out


QUANTILE_SAMPLE = 32768
BOUNDS_EQUAL_WIDTH = 0
BOUNDS_QUANTILE = 1


def feature_bounds(raw, n_bins, method):
    """orc_feature_bounds: float32 [total_bins] bounds (feature f's at
    bin_offset[f] + k) for a float32 [n][F] matrix; method 0 equal width,
    1 quantile of the row sample."""
    raw = np.ascontiguousarray(raw, dtype=np.float32)
    nb = np.ascontiguousarray(n_bins, dtype=np.int32)
    n, F = raw.shape
    out = np.zeros(int(nb.sum()), dtype=np.float32)
    rc = _load().orc_feature_bounds(n, F, _p(raw), _p(nb), int(method), _p(out))
    if rc:
        raise ValueError("orc_feature_bounds failed (%d)" % rc)
    return out


def max_nodes(max_depth: int) -> int:
    return (1 << (max_depth + 1)) - 1


def train(bins, n_bins, label, params: OrcParams, n_trees: int, pred0=None, base_score=0.0,
          dump_tree: int = -1, keep_pred_per_tree: bool = False, dump_hist: bool = True):
    """Boost n_trees trees; returns a dict with nodes, n_nodes, scale, pred and dumps."""
    bins = np.ascontiguousarray(bins, dtype=np.uint8)
    n, F = bins.shape
    n_bins = np.ascontiguousarray(n_bins, dtype=np.int32)
    label = np.ascontiguousarray(label, dtype=np.float32)
    TB = int(np.sum(n_bins, dtype=np.int64))
    mn = max_nodes(params.max_depth)
    pred = (np.full(n, base_score, dtype=np.float64) if pred0 is None
            else np.array(pred0, dtype=np.float64, copy=True))
    nodes = np.zeros((max(n_trees, 1), mn), dtype=NODE_DTYPE)
    n_nodes = np.zeros(max(n_trees, 1), dtype=np.int32)
    scale = np.zeros(max(n_trees, 1), dtype=np.int32)
    ppt = np.zeros((n_trees, n), dtype=np.float64) if keep_pred_per_tree else None
    logistic = int(params.objective) == LOGISTIC
    scale_h = np.zeros(max(n_trees, 1), dtype=np.int32)
    dcnt = dgq = dleaf = dk = dhq = dkh = None
    if dump_tree >= 0:
        if dump_hist:
            dcnt = np.zeros((mn, TB), dtype=np.uint32)
            dgq = np.zeros((mn, TB), dtype=np.int64)
            if logistic:
                dhq = np.zeros((mn, TB), dtype=np.int64)
        dleaf = np.full(n, -1, dtype=np.int32)
        dk = np.zeros(n, dtype=np.int64)
        if logistic:
            dkh = np.zeros(n, dtype=np.int64)
    timing = np.zeros(2, dtype=np.float64)
    rc = _load().orc_train(n, F, _p(bins), _p(n_bins), _p(label), ctypes.byref(params), n_trees,
                           _p(pred), _p(nodes), _p(n_nodes), _p(scale), _p(ppt), dump_tree,
                           _p(dcnt), _p(dgq), _p(dleaf), _p(dk), _p(timing), _p(scale_h), _p(dhq),
                           _p(dkh))
    if rc:
        raise ValueError("orc_train failed (%d)" % rc)
    return dict(nodes=nodes[:n_trees], n_nodes=n_nodes[:n_trees], scale=scale[:n_trees], pred=pred,
                pred_per_tree=ppt, dump_cnt=dcnt, dump_gq=dgq, dump_leaf_of_row=dleaf, dump_k=dk,
                scale_h=scale_h[:n_trees], dump_hq=dhq, dump_kh=dkh,
                seconds=float(timing[0]), hist_seconds=float(timing[1]))
