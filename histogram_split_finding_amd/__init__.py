"""Python binding of libgbdt_hip.so (the C ABI in include/gbdt.h).

Argument marshalling only: torch tensors own the device memory, the current
HIP stream is passed through, and every step of the hot path runs in the
library's HIP kernels.  There is no CPU fallback: if the library is not built
or no GPU is present, the calls raise.

Names mirror the C entry points (gbdt_compute_gradients, gbdt_build_histograms,
gbdt_subtract_histograms, gbdt_find_best_splits, gbdt_partition_rows,
gbdt_update_predictions, gbdt_grow_tree, ...).  `Dataset` and `Booster` hold
the buffers of a training run and call gbdt_grow_tree once per tree.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgbdt_hip.so")

GBDT_OK = 0
GBDT_NODE_LEAF = 1
OBJECTIVE_SQUARED_ERROR = 0
OBJECTIVE_LOGISTIC = 1
GBDT_MAX_DEPTH = 16
STATUS_NAMES = {0: "OK", -1: "ARG", -2: "SHAPE", -3: "RANGE", -4: "OVERFLOW", -5: "DEVICE",
                -6: "UNSUPPORTED", -7: "INTERNAL"}

NODE_DTYPE = np.dtype([
    ("feature", "<i4"), ("threshold_bin", "<i4"), ("left", "<i4"), ("right", "<i4"),
    ("leaf_value", "<f8"), ("gain", "<f8"), ("flags", "<u4"), ("depth", "<i4"),
    ("begin", "<i4"), ("count", "<i4"), ("gsum", "<i8"), ("hsum", "<i8"),
])
assert NODE_DTYPE.itemsize == 64
SPLIT_DTYPE = np.dtype([
    ("gain", "<f8"), ("feature", "<i4"), ("threshold_bin", "<i4"), ("g_left", "<i8"),
    ("n_left", "<i4"), ("valid", "<i4"),
])
assert SPLIT_DTYPE.itemsize == 32
PAIR_DTYPE = np.dtype([("parent", "<i4"), ("smaller", "<i4"), ("larger", "<i4"), ("pad", "<i4")])


class GbdtError(RuntimeError):
    def __init__(self, code, what):
        super().__init__("%s failed: %s (%s)" % (what, STATUS_NAMES.get(code, code), last_error()))
        self.code = code


vp = ctypes.c_void_p
i32 = ctypes.c_int32
i64 = ctypes.c_int64


class Matrix(ctypes.Structure):
    _fields_ = [("bins", vp), ("n_rows", i64), ("row_capacity", i64), ("n_features", i32),
                ("n_blocks", i32), ("block_features", i32), ("block_stride", i32),
                ("n_bit_features", i32), ("bit_stride", i32), ("col_feature", vp),
                ("feature_col", vp), ("n_nib_features", i32), ("nib_stride", i32)]


class Features(ctypes.Structure):
    _fields_ = [("n_features", i32), ("total_bins", i32), ("max_block_bins", i32), ("pad", i32),
                ("n_bins", vp), ("bin_offset", vp), ("bin_feature", vp), ("skip_bin", vp)]


class Rows(ctypes.Structure):
    _fields_ = [("X", Matrix), ("q", vp), ("rid", vp)]


class Params(ctypes.Structure):
    _fields_ = [("reg_lambda", ctypes.c_double), ("gamma", ctypes.c_double),
                ("min_child_weight", ctypes.c_double), ("learning_rate", ctypes.c_double),
                ("min_samples_leaf", i32), ("max_depth", i32), ("objective", i32), ("pad", i32)]


class GrowBuffers(ctypes.Structure):
    _fields_ = [("pp", Rows * 2), ("q", vp), ("hist_g", vp), ("hist_cnt", vp), ("splits", vp),
                ("lists", vp), ("ctrl", vp), ("ws", vp), ("ws_bytes", ctypes.c_size_t),
                ("qh", vp), ("hist_h", vp), ("split_h", vp), ("rows_ix", vp), ("cols", vp)]


class GrowSizes(ctypes.Structure):
    _fields_ = [("max_nodes", i64), ("hist_slots", i64), ("list_words", i64),
                ("ctrl_bytes", i64), ("ws_bytes", i64)]


_lib = None


def load():
    """Loads the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libgbdt_hip.so is not built (run __graft_entry__.build() or "
                          "python histogram_split_finding_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sigs = {
        "gbdt_abi_version": (ctypes.c_int, []),
        "gbdt_last_error": (ctypes.c_char_p, []),
        "gbdt_validate_params": (ctypes.c_int, [P(Params)]),
        "gbdt_workspace_bytes": (ctypes.c_size_t, [i64, i32, i32]),
        "gbdt_choose_blocking": (ctypes.c_int, [i32, vp, P(Matrix), P(i32)]),
        "gbdt_choose_layout": (ctypes.c_int, [i32, vp, i32, P(Matrix), P(i32), vp, vp]),
        "gbdt_pack_matrix": (ctypes.c_int, [vp, P(Matrix), P(Features), vp, ctypes.c_size_t, vp]),
        "gbdt_bin_features": (ctypes.c_int, [vp, i64, P(Features), vp, vp, vp, ctypes.c_size_t, vp]),
        "gbdt_feature_bounds": (ctypes.c_int, [vp, i64, P(Features), i32, vp, vp, ctypes.c_size_t, vp]),
        "gbdt_read_error": (ctypes.c_int, [vp, vp]),
        "gbdt_compute_gradients": (ctypes.c_int, [vp, vp, i64, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "gbdt_build_histograms": (ctypes.c_int, [P(Rows), P(Features), vp, vp, vp, i32, i64, vp, vp,
                                                 vp, ctypes.c_size_t, vp]),
        "gbdt_subtract_histograms": (ctypes.c_int, [vp, vp, i32, vp, vp, i32, vp, ctypes.c_size_t,
                                                    vp]),
        "gbdt_find_best_splits": (ctypes.c_int, [vp, vp, P(Features), vp, vp, vp, i32, P(Params), vp,
                                                 vp, vp, ctypes.c_size_t, vp]),
        "gbdt_partition_rows": (ctypes.c_int, [P(Rows), P(Rows), vp, vp, vp, vp, i32, i64, vp,
                                               ctypes.c_size_t, vp]),
        "gbdt_update_predictions": (ctypes.c_int, [vp, P(Matrix), vp, vp, i32, ctypes.c_double, vp,
                                                   ctypes.c_size_t, vp]),
        "gbdt_diag_enable": (ctypes.c_int, [i32]),
        "gbdt_diag_disable": (ctypes.c_int, []),
        "gbdt_diag_read": (ctypes.c_int, [i32, vp, vp, vp]),
        "gbdt_predict_workspace_bytes": (ctypes.c_size_t, [i32, i32]),
        "gbdt_predict": (ctypes.c_int, [P(Matrix), vp, vp, i32, i32, ctypes.c_double, ctypes.c_double,
                                        vp, vp, ctypes.c_size_t, vp]),
        "gbdt_predict_noalloc": (ctypes.c_int, [P(Matrix), vp, vp, i32, i32, ctypes.c_double,
                                                ctypes.c_double, vp, vp, vp]),
        "gbdt_grow_sizes": (ctypes.c_int, [i64, i32, i32, P(GrowSizes)]),
        "gbdt_grow_moves_ids": (ctypes.c_int, [P(Matrix), i32]),
        "gbdt_grow_filtered_levels": (i64, [P(Matrix), P(Params)]),
        "gbdt_interleave_rows": (ctypes.c_int, [P(Matrix), vp, vp]),
        "gbdt_interleave_pitch": (i32, [P(Matrix)]),
        "gbdt_column_major": (ctypes.c_int, [P(Matrix), vp, vp]),
        "gbdt_grow_tree": (ctypes.c_int, [P(Matrix), P(Features), vp, vp, P(Params), vp, vp,
                                          P(GrowBuffers), vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error() -> str:
    if _lib is None:
        return ""
    s = _lib.gbdt_last_error()
    return s.decode() if s else ""


def _check(rc, what):
    if rc != GBDT_OK:
        raise GbdtError(rc, what)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_params(max_depth, reg_lambda=1.0, gamma=0.0, min_child_weight=0.0, learning_rate=0.3,
                min_samples_leaf=1, objective=OBJECTIVE_SQUARED_ERROR, **_ignored) -> Params:
    return Params(float(reg_lambda), float(gamma), float(min_child_weight), float(learning_rate),
                  int(min_samples_leaf), int(max_depth), int(objective), 0)


# ----------------------------------------------------------- host-only calls --

def gbdt_abi_version() -> int:
    return int(load().gbdt_abi_version())


def gbdt_validate_params(p: Params) -> int:
    return int(load().gbdt_validate_params(ctypes.byref(p)))


def gbdt_workspace_bytes(n_rows: int, max_list: int, total_bins: int) -> int:
    return int(load().gbdt_workspace_bytes(n_rows, max_list, total_bins))


def gbdt_choose_blocking(n_bins):
    nb = np.ascontiguousarray(np.asarray(n_bins, dtype=np.int32))
    X = Matrix()
    mbb = i32()
    rc = load().gbdt_choose_blocking(nb.shape[0], nb.ctypes.data_as(vp), ctypes.byref(X),
                                     ctypes.byref(mbb))
    _check(rc, "gbdt_choose_blocking")
    return X, int(mbb.value)


PACK_BITS = 1
PACK_NIBBLES = 2


def gbdt_choose_layout(n_bins, pack_bits=True, pack_nibbles=False):
    """(Matrix layout fields, max_block_bins, col_feature, feature_col) for the
    features' bin counts; with pack_bits, features of at most 2 bins are bits;
    with pack_nibbles, features of 3 to 16 bins are 4-bit cells."""
    nb = np.ascontiguousarray(np.asarray(n_bins, dtype=np.int32))
    X = Matrix()
    mbb = i32()
    cf = np.zeros(nb.shape[0], dtype=np.int32)
    fc = np.zeros(nb.shape[0], dtype=np.int32)
    flags = (PACK_BITS if pack_bits else 0) | (PACK_NIBBLES if pack_nibbles else 0)
    rc = load().gbdt_choose_layout(nb.shape[0], nb.ctypes.data_as(vp), flags,
                                   ctypes.byref(X), ctypes.byref(mbb), cf.ctypes.data_as(vp),
                                   fc.ctypes.data_as(vp))
    _check(rc, "gbdt_choose_layout")
    return X, int(mbb.value), cf, fc


def gbdt_grow_sizes(n_rows: int, total_bins: int, max_depth: int) -> GrowSizes:
    out = GrowSizes()
    _check(load().gbdt_grow_sizes(n_rows, total_bins, max_depth, ctypes.byref(out)), "gbdt_grow_sizes")
    return out


# ----------------------------------------------------------- device helpers --

def new_workspace(nbytes: int, device="cuda"):
    """Zero-filled workspace tensor (256-byte aligned by the caching allocator)."""
    import torch
    ws = torch.zeros(int(nbytes), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws


class FeatureTable:
    """Device feature table (n_bins, bin_offset, bin_feature, skip_bin) and the
    matrix layout chosen for it (with pack_bits, features of at most 2 bins
    are stored as bits; with pack_nibbles, features of 3 to 16 bins as 4-bit
    cells; the column maps live on the device)."""

    def __init__(self, n_bins, device="cuda", pack_bits=True, pack_nibbles=True):
        import torch
        nb = np.ascontiguousarray(np.asarray(n_bins, dtype=np.int32))
        self.n_bins_host = nb
        self.n_features = int(nb.shape[0])
        off = np.zeros(self.n_features + 1, dtype=np.int32)
        off[1:] = np.cumsum(nb)
        self.bin_offset_host = off
        self.total_bins = int(off[-1])
        bf = np.repeat(np.arange(self.n_features, dtype=np.int32), nb)
        self.layout, self.max_block_bins, cf, fc = gbdt_choose_layout(nb, pack_bits, pack_nibbles)
        self.col_feature_host, self.feature_col_host = cf, fc
        self.mapped = bool(pack_bits or pack_nibbles)
        self.col_feature = torch.from_numpy(cf).to(device) if self.mapped else None
        self.feature_col = torch.from_numpy(fc).to(device) if self.mapped else None
        self.n_bins = torch.from_numpy(nb).to(device)
        self.bin_offset = torch.from_numpy(off).to(device)
        self.bin_feature = torch.from_numpy(bf).to(device)
        self.skip_bin = torch.full((self.n_features,), -1, dtype=torch.int32, device=device)

    def struct(self, use_skip=True) -> Features:
        return Features(self.n_features, self.total_bins, self.max_block_bins, 0,
                        _ptr(self.n_bins), _ptr(self.bin_offset), _ptr(self.bin_feature),
                        _ptr(self.skip_bin) if use_skip else None)


class RowBuffer:
    """A row order: column-blocked bins, q and row ids on the device."""

    def __init__(self, ft: FeatureTable, n_rows: int, device="cuda", with_rid=True, with_bins=True):
        import torch
        L = ft.layout
        self.ft = ft
        self.n_rows = int(n_rows)
        self.row_capacity = max(self.n_rows, 1)
        self.n_blocks, self.block_features, self.block_stride = L.n_blocks, L.block_features, L.block_stride
        self.n_bit_features, self.bit_stride = L.n_bit_features, L.bit_stride
        self.n_nib_features, self.nib_stride = L.n_nib_features, L.nib_stride
        self.n_features = ft.n_features
        self.byte_bytes = self.n_blocks * self.row_capacity * self.block_stride
        # (a row order of row ids only, in the tree driver's index mode, has no bins)
        self.bins = torch.zeros(self.byte_bytes + self.row_capacity * (self.bit_stride + self.nib_stride),
                                dtype=torch.uint8, device=device) if with_bins else None
        self.q = torch.zeros(self.row_capacity, dtype=torch.int64, device=device)
        self.rid = torch.zeros(self.row_capacity, dtype=torch.int32, device=device) if with_rid else None

    def matrix(self) -> Matrix:
        return Matrix(_ptr(self.bins), self.n_rows, self.row_capacity, self.n_features,
                      self.n_blocks, self.block_features, self.block_stride, self.n_bit_features,
                      self.bit_stride, _ptr(self.ft.col_feature), _ptr(self.ft.feature_col),
                      self.n_nib_features, self.nib_stride)

    def rows(self, identity_rid=False) -> Rows:
        return Rows(self.matrix(), _ptr(self.q), None if (identity_rid or self.rid is None) else _ptr(self.rid))

    def blocked_to_rowmajor(self):
        """Bins back in row-major [n, F] order (for tests)."""
        import torch
        n, F = self.n_rows, self.n_features
        out = torch.zeros((n, F), dtype=torch.uint8, device=self.bins.device)
        nbc = F - self.n_bit_features - self.n_nib_features
        cf = torch.from_numpy(self.ft.col_feature_host).long().to(self.bins.device)
        if self.n_blocks > 0:
            b = self.bins[: self.byte_bytes].view(self.n_blocks, self.row_capacity, self.block_stride)[:, :n]
            cols = [b[k, :, : min(self.block_features, nbc - k * self.block_features)]
                    for k in range(self.n_blocks)]
            out[:, cf[:nbc]] = torch.cat(cols, dim=1)
        if self.n_bit_features > 0:
            nw = self.bit_stride // 4
            w = self.bins[self.byte_bytes: self.byte_bytes + self.row_capacity * self.bit_stride].view(
                torch.int32).view(self.row_capacity, nw)[:n]
            k = torch.arange(self.n_bit_features, device=self.bins.device)
            bitv = (w[:, k // 32] >> (k % 32)) & 1
            out[:, cf[F - self.n_bit_features:]] = bitv.to(torch.uint8)
        if self.n_nib_features > 0:
            nw = self.nib_stride // 4
            base = self.byte_bytes + self.row_capacity * self.bit_stride
            w = self.bins[base: base + self.row_capacity * self.nib_stride].view(torch.int32).view(
                self.row_capacity, nw)[:n]
            k = torch.arange(self.n_nib_features, device=self.bins.device)
            nib = (w[:, k // 8] >> (4 * (k % 8))) & 15
            out[:, cf[nbc: nbc + self.n_nib_features]] = nib.to(torch.uint8)
        return out


# -------------------------------------------------------- hot-path wrappers --

def gbdt_pack_matrix(rowmajor, rb: RowBuffer, ft: FeatureTable, ws, stream=None):
    m = rb.matrix()
    f = ft.struct()
    rc = load().gbdt_pack_matrix(_ptr(rowmajor), ctypes.byref(m), ctypes.byref(f), _ptr(ws),
                                 ws.numel(), _stream(stream))
    _check(rc, "gbdt_pack_matrix")


def gbdt_bin_features(raw, ft: FeatureTable, upper, bins_out, ws, stream=None):
    """raw: float32 [n][F] device tensor; upper: float32 [total_bins] (feature f's
    bounds at bin_offset[f] + k); bins_out: uint8 [n][F]."""
    f = ft.struct()
    rc = load().gbdt_bin_features(_ptr(raw), int(raw.shape[0]) if raw.dim() > 0 else 0,
                                  ctypes.byref(f), _ptr(upper), _ptr(bins_out), _ptr(ws), ws.numel(),
                                  _stream(stream))
    _check(rc, "gbdt_bin_features")


BOUNDS_EQUAL_WIDTH = 0
BOUNDS_QUANTILE = 1


def gbdt_feature_bounds(raw, ft: FeatureTable, method, upper, ws, stream=None):
    """raw: float32 [n][F] device tensor; upper: float32 [total_bins] (written)."""
    f = ft.struct()
    rc = load().gbdt_feature_bounds(_ptr(raw), int(raw.shape[0]), ctypes.byref(f), int(method), _ptr(upper),
                                    _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "gbdt_feature_bounds")


def gbdt_read_error(ws, stream=None) -> int:
    return int(load().gbdt_read_error(_ptr(ws), _stream(stream)))


def gbdt_compute_gradients(pred, label, q, scale, gsum, ws, stream=None):
    rc = load().gbdt_compute_gradients(_ptr(pred), _ptr(label), pred.numel(), _ptr(q), _ptr(scale),
                                       _ptr(gsum), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "gbdt_compute_gradients")


def gbdt_build_histograms(src: Rows, ft: Features, nodes, lst, list_len, list_cap, rows_bound,
                          hist_g, hist_cnt, ws, stream=None):
    rc = load().gbdt_build_histograms(ctypes.byref(src), ctypes.byref(ft), _ptr(nodes), _ptr(lst),
                                      _ptr(list_len), int(list_cap), int(rows_bound), _ptr(hist_g),
                                      _ptr(hist_cnt), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "gbdt_build_histograms")


def gbdt_subtract_histograms(hist_g, hist_cnt, total_bins, pairs, n_pairs, pair_cap, ws, stream=None):
    rc = load().gbdt_subtract_histograms(_ptr(hist_g), _ptr(hist_cnt), int(total_bins), _ptr(pairs),
                                         _ptr(n_pairs), int(pair_cap), _ptr(ws), ws.numel(),
                                         _stream(stream))
    _check(rc, "gbdt_subtract_histograms")


def gbdt_find_best_splits(hist_g, hist_cnt, ft: Features, nodes, lst, list_len, list_cap, p: Params,
                          scale, splits, ws, stream=None):
    rc = load().gbdt_find_best_splits(_ptr(hist_g), _ptr(hist_cnt), ctypes.byref(ft), _ptr(nodes),
                                      _ptr(lst), _ptr(list_len), int(list_cap), ctypes.byref(p),
                                      _ptr(scale), _ptr(splits), _ptr(ws), ws.numel(),
                                      _stream(stream))
    _check(rc, "gbdt_find_best_splits")


def gbdt_partition_rows(src: Rows, dst: Rows, nodes, splits, lst, list_len, list_cap, rows_bound, ws,
                        stream=None):
    rc = load().gbdt_partition_rows(ctypes.byref(src), ctypes.byref(dst), _ptr(nodes), _ptr(splits),
                                    _ptr(lst), _ptr(list_len), int(list_cap), int(rows_bound),
                                    _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "gbdt_partition_rows")


def gbdt_update_predictions(pred, X: Matrix, nodes, n_nodes, max_nodes, learning_rate, ws, stream=None):
    rc = load().gbdt_update_predictions(_ptr(pred), ctypes.byref(X), _ptr(nodes), _ptr(n_nodes),
                                        int(max_nodes), float(learning_rate), _ptr(ws), ws.numel(),
                                        _stream(stream))
    _check(rc, "gbdt_update_predictions")


def gbdt_predict_workspace_bytes(n_trees: int, tree_stride: int) -> int:
    return int(load().gbdt_predict_workspace_bytes(n_trees, tree_stride))


def gbdt_predict(X: Matrix, trees, n_nodes, n_trees, tree_stride, base_score, learning_rate, out, ws,
                 stream=None):
    """trees: device bytes of n_trees * tree_stride nodes; n_nodes: int32 [n_trees];
    out: float64 [n_rows]."""
    rc = load().gbdt_predict(ctypes.byref(X), _ptr(trees), _ptr(n_nodes), int(n_trees), int(tree_stride),
                             float(base_score), float(learning_rate), _ptr(out), _ptr(ws), ws.numel(),
                             _stream(stream))
    _check(rc, "gbdt_predict")


def gbdt_interleave_pitch(X: Matrix) -> int:
    """Row pitch in bytes of gbdt_interleave_rows' copy."""
    return int(load().gbdt_interleave_pitch(ctypes.byref(X)))


def gbdt_interleave_rows(X: Matrix, out, stream=None):
    """X's byte blocks interleaved row by row into out (a uint8 device tensor
    of at least row_capacity * gbdt_interleave_pitch(X) bytes)."""
    need = int(X.row_capacity) * gbdt_interleave_pitch(X)
    if out.numel() * out.element_size() < need:
        raise ValueError("out holds fewer than %d bytes" % need)
    _check(load().gbdt_interleave_rows(ctypes.byref(X), _ptr(out), _stream(stream)),
           "gbdt_interleave_rows")


def gbdt_column_major(X: Matrix, out, stream=None):
    """X's byte columns one after another into out (a uint8 device tensor of
    at least row_capacity bytes per byte column)."""
    n_cols = int(X.n_features) - int(X.n_bit_features) - int(X.n_nib_features)
    need = int(X.row_capacity) * n_cols if int(X.n_blocks) > 0 else 0
    if out.numel() * out.element_size() < need:
        raise ValueError("out holds fewer than %d bytes" % need)
    _check(load().gbdt_column_major(ctypes.byref(X), _ptr(out), _stream(stream)), "gbdt_column_major")


def gbdt_predict_noalloc(X: Matrix, trees, n_nodes, n_trees, tree_stride, base_score, learning_rate,
                         out, status, stream=None):
    """gbdt_predict without a workspace (the library's per-GPU scratch);
    status: int32 [1] device tensor, receives the device-side error code."""
    rc = load().gbdt_predict_noalloc(ctypes.byref(X), _ptr(trees), _ptr(n_nodes), int(n_trees),
                                     int(tree_stride), float(base_score), float(learning_rate),
                                     _ptr(out), _ptr(status), _stream(stream))
    _check(rc, "gbdt_predict_noalloc")


# ------------------------------------------------------------ training run --

class Dataset:
    """Bins packed on the device in the column-blocked layout, plus labels."""

    def __init__(self, bins_rowmajor, label, n_bins, device="cuda", use_skip_bins=True, pack_bits=True,
                 pack_nibbles=True):
        import torch
        bins_rowmajor = np.ascontiguousarray(bins_rowmajor, dtype=np.uint8)
        self.n_rows, self.n_features = bins_rowmajor.shape
        self.ft = FeatureTable(n_bins, device, pack_bits=pack_bits, pack_nibbles=pack_nibbles)
        self.use_skip_bins = use_skip_bins
        self.X = RowBuffer(self.ft, self.n_rows, device, with_rid=False)
        self.label = torch.from_numpy(np.ascontiguousarray(label, dtype=np.float32)).to(device)
        ws = new_workspace(gbdt_workspace_bytes(self.n_rows, 1, self.ft.total_bins), device)
        src = torch.from_numpy(bins_rowmajor).to(device)
        gbdt_pack_matrix(src, self.X, self.ft, ws)
        _check(gbdt_read_error(ws), "gbdt_pack_matrix (device check)")
        if not use_skip_bins:
            self.ft.skip_bin.fill_(-1)
        del src, ws


class Booster:
    """Buffers of one training run; grow_tree() runs one boosting step."""

    def __init__(self, ds: Dataset, params: Params, base_score=0.0, device="cuda", interleave=True):
        """interleave: in index mode, also keep a row-interleaved copy of the
        byte blocks (gbdt_interleave_rows) for the histogram's gathers and a
        column-major copy (gbdt_column_major) for the partition's."""
        import torch
        _check(gbdt_validate_params(params), "gbdt_validate_params")
        self.ds = ds
        self.params = params
        n, D, TB = ds.n_rows, params.max_depth, ds.ft.total_bins
        sz = gbdt_grow_sizes(n, TB, D)
        self.sizes = sz
        self.pred = torch.full((n,), float(base_score), dtype=torch.float64, device=device)
        logistic = int(params.objective) == OBJECTIVE_LOGISTIC
        # index mode: the row buffers carry row ids and q only; otherwise bins
        # and q (and, for the logistic objective, its Hessians in the rid arrays)
        X0 = ds.X.matrix()
        self.moves_ids = bool(load().gbdt_grow_moves_ids(ctypes.byref(X0), int(params.objective)))
        # the levels whose histograms are built from the parents' unmoved rows (bit d: level d)
        self.filtered_levels = int(load().gbdt_grow_filtered_levels(ctypes.byref(X0), ctypes.byref(params)))
        self.pp = [RowBuffer(ds.ft, n, device, with_rid=logistic or self.moves_ids,
                             with_bins=not self.moves_ids) for _ in range(2)]
        self.rows_ix = self.cols = None
        if self.moves_ids and interleave:
            cap = int(X0.row_capacity)
            self.rows_ix = torch.empty(cap * gbdt_interleave_pitch(X0), dtype=torch.uint8, device=device)
            gbdt_interleave_rows(X0, self.rows_ix)
            n_cols = int(X0.n_features) - int(X0.n_bit_features) - int(X0.n_nib_features)
            self.cols = torch.empty(cap * n_cols, dtype=torch.uint8, device=device)
            gbdt_column_major(X0, self.cols)
        self.q = torch.zeros(n, dtype=torch.int64, device=device)
        self.qh = torch.zeros(n, dtype=torch.int32, device=device) if logistic else None
        self.hist_h = torch.zeros(sz.hist_slots * TB, dtype=torch.int64, device=device) if logistic else None
        self.split_h = torch.zeros(sz.max_nodes, dtype=torch.int64, device=device) if logistic else None
        self.hist_g = torch.zeros(sz.hist_slots * TB, dtype=torch.int64, device=device)
        self.hist_cnt = torch.zeros(sz.hist_slots * TB, dtype=torch.int32, device=device)
        self.splits = torch.zeros(sz.max_nodes * SPLIT_DTYPE.itemsize, dtype=torch.uint8, device=device)
        self.lists = torch.zeros(sz.list_words, dtype=torch.int32, device=device)
        self.ctrl = torch.zeros(sz.ctrl_bytes, dtype=torch.uint8, device=device)
        self.ws = new_workspace(sz.ws_bytes, device)
        self.n_nodes_dev = torch.zeros(1, dtype=torch.int32, device=device)
        self.trees = []  # (nodes tensor [max_nodes*64 bytes], n_nodes tensor)
        self._buf = GrowBuffers(
            (Rows * 2)(self.pp[0].rows(), self.pp[1].rows()), _ptr(self.q), _ptr(self.hist_g),
            _ptr(self.hist_cnt), _ptr(self.splits), _ptr(self.lists), _ptr(self.ctrl), _ptr(self.ws),
            self.ws.numel(), _ptr(self.qh), _ptr(self.hist_h), _ptr(self.split_h), _ptr(self.rows_ix),
            _ptr(self.cols))
        self._X = ds.X.matrix()
        self._ft = ds.ft.struct(ds.use_skip_bins)

    def grow_tree(self, nodes_out=None, n_nodes_out=None, stream=None):
        """Enqueues one tree (no host synchronisation); returns the device node buffer."""
        import torch
        if nodes_out is None:
            nodes_out = torch.zeros(self.sizes.max_nodes * NODE_DTYPE.itemsize, dtype=torch.uint8,
                                    device=self.pred.device)
        if n_nodes_out is None:
            n_nodes_out = torch.zeros(1, dtype=torch.int32, device=self.pred.device)
        rc = load().gbdt_grow_tree(ctypes.byref(self._X), ctypes.byref(self._ft), _ptr(self.ds.label),
                                   _ptr(self.pred), ctypes.byref(self.params), _ptr(nodes_out),
                                   _ptr(n_nodes_out), ctypes.byref(self._buf), _stream(stream))
        _check(rc, "gbdt_grow_tree")
        return nodes_out, n_nodes_out

    def train(self, n_trees: int, keep_trees=True):
        """Grows n_trees trees (enqueued without host synchronisation), then
        reads the workspace error word once.  After a device-side failure the
        library has left the failed tree and every later one with 0 nodes and
        changed no prediction; those trees are dropped and GbdtError is raised,
        so the booster keeps exactly the trees that completed and pred is the
        prediction after the last of them."""
        new = [self.grow_tree() for _ in range(n_trees)]
        code = gbdt_read_error(self.ws)
        if code != GBDT_OK:
            done = 0
            while done < len(new) and int(new[done][1].item()) > 0:
                done += 1
            if keep_trees:
                self.trees.extend(new[:done])
            raise GbdtError(code, "gbdt_grow_tree (device-side check, tree %d of this call)" % done)
        if keep_trees:
            self.trees.extend(new)
        return self

    def check(self):
        _check(gbdt_read_error(self.ws), "device-side check")

    def predict(self, X: "RowBuffer", base_score=0.0, trees=None):
        """Ensemble prediction (gbdt_predict) of the rows of X -- a RowBuffer in
        the layout of this booster's dataset, e.g. Dataset(...).X of held-out
        rows -- over the kept trees (or `trees`, a list of (nodes, n_nodes)
        pairs as grow_tree returns them).  Returns a float64 device tensor."""
        import torch
        trees = self.trees if trees is None else trees
        dev = self.pred.device
        stride = int(self.sizes.max_nodes)
        if trees:
            nodes = torch.cat([t[0] for t in trees])
            counts = torch.cat([t[1] for t in trees])
        else:
            nodes = torch.zeros(NODE_DTYPE.itemsize, dtype=torch.uint8, device=dev)
            counts = torch.zeros(1, dtype=torch.int32, device=dev)
        out = torch.empty(X.n_rows, dtype=torch.float64, device=dev)
        ws = new_workspace(max(gbdt_predict_workspace_bytes(len(trees), stride), 256), dev)
        gbdt_predict(X.matrix(), nodes, counts, len(trees), stride, base_score,
                     self.params.learning_rate, out, ws)
        _check(gbdt_read_error(ws), "gbdt_predict (device-side check)")
        return out

    def host_trees(self):
        """Node arrays of the kept trees as numpy structured arrays (synchronises)."""
        out = []
        for nodes, nn in self.trees:
            k = int(nn.item())
            arr = np.frombuffer(nodes.cpu().numpy().tobytes(), dtype=NODE_DTYPE)[:k].copy()
            out.append(arr)
        return out


def nodes_to_host(nodes_tensor, n_nodes=None):
    arr = np.frombuffer(nodes_tensor.cpu().numpy().tobytes(), dtype=NODE_DTYPE)
    return arr[:n_nodes].copy() if n_nodes is not None else arr.copy()


def splits_to_host(splits_tensor):
    return np.frombuffer(splits_tensor.cpu().numpy().tobytes(), dtype=SPLIT_DTYPE).copy()
