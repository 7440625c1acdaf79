"""Seeded synthetic workloads for level-wise histogram GBDT training.

Input generation only: the row-major uint8 bin matrix, the float32 labels and
the per-feature bin counts, plus each workload's training parameters.  No
boosting arithmetic lives here, so the oracle and the GPU path can both take
their inputs from this module without sharing any of the method's code.

The C source (``gen.c``) documents the counter-based SplitMix64 recipe.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "_libdatagen.so")
_lib = None

# Training parameters of the five workloads.  Where a workload leaves a value
# open, the plain choice is taken: learning rate 0.3, lambda 1, gamma 0,
# min_samples_leaf 1, min_child_weight 0, base score 0.
WORKLOADS = {
    1: dict(name="w1_4096x8_b32_d3", max_depth=3, n_trees=5, learning_rate=0.3, reg_lambda=1.0,
            gamma=0.0, min_samples_leaf=1, min_child_weight=0.0, base_score=0.0),
    2: dict(name="w2_1Mx32_b256_d6", max_depth=6, n_trees=50, learning_rate=0.3, reg_lambda=1.0,
            gamma=0.0, min_samples_leaf=20, min_child_weight=0.0, base_score=0.0),
    3: dict(name="w3_581012x54_covtype_shape_d10", max_depth=10, n_trees=100, learning_rate=0.3,
            reg_lambda=1.0, gamma=0.0, min_samples_leaf=1, min_child_weight=0.0, base_score=0.0),
    4: dict(name="w4_10Mx100_zipf256_d8", max_depth=8, n_trees=20, learning_rate=0.3, reg_lambda=1.0,
            gamma=0.0, min_samples_leaf=1, min_child_weight=1.0, base_score=0.0),
    5: dict(name="w5_50Mx28_b64_d12", max_depth=12, n_trees=10, learning_rate=0.3, reg_lambda=1.0,
            gamma=0.1, min_samples_leaf=1, min_child_weight=0.0, base_score=0.0),
}


def build(force: bool = True) -> str:
    """Compile gen.c into _libdatagen.so (gcc, OpenMP)."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
           _SRC, "-o", tmp, "-lm"]
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
    lib.dg_u64.restype = ctypes.c_uint64
    lib.dg_u64.argtypes = [ctypes.c_uint64] * 3
    lib.dg_uniform.restype = ctypes.c_double
    lib.dg_uniform.argtypes = [ctypes.c_uint64] * 3
    lib.dg_normal.restype = ctypes.c_double
    lib.dg_normal.argtypes = [ctypes.c_uint64] * 3
    lib.dg_fnv1a64.restype = ctypes.c_uint64
    lib.dg_fnv1a64.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.dg_config_shape.restype = ctypes.c_int
    lib.dg_config_shape.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int32)]
    lib.dg_config_nbins.restype = ctypes.c_int
    lib.dg_config_nbins.argtypes = [ctypes.c_int, ctypes.c_void_p]
    lib.dg_config_rows.restype = ctypes.c_int
    lib.dg_config_rows.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.dg_random.restype = ctypes.c_int
    lib.dg_random.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint64,
                              ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def workload_shape(k: int):
    lib = _load()
    n = ctypes.c_int64()
    f = ctypes.c_int32()
    if lib.dg_config_shape(k, ctypes.byref(n), ctypes.byref(f)):
        raise ValueError("unknown workload %r" % (k,))
    return int(n.value), int(f.value)


def workload_nbins(k: int) -> np.ndarray:
    _, F = workload_shape(k)
    nb = np.zeros(F, dtype=np.int32)
    if _load().dg_config_nbins(k, _ptr(nb)):
        raise ValueError("unknown workload %r" % (k,))
    return nb


def make_workload(k: int, n_rows: int | None = None, row_start: int = 0):
    """Rows [row_start, row_start + n_rows) of workload k.

    Returns (bins uint8 [n, F] row-major, label float32 [n], n_bins int32 [F]).
    """
    n_full, F = workload_shape(k)
    if n_rows is None:
        n_rows = n_full - row_start
    r1 = row_start + n_rows
    bins = np.empty((n_rows, F), dtype=np.uint8)
    label = np.empty(n_rows, dtype=np.float32)
    rc = _load().dg_config_rows(k, row_start, r1, _ptr(bins), _ptr(label))
    if rc:
        raise ValueError("dg_config_rows failed (%d)" % rc)
    return bins, label, workload_nbins(k)


def make_heldout(k: int, n_rows: int):
    """n_rows held-out rows of workload k: rows n .. n + n_rows - 1 of the same
    recipe, past the training rows (bins, label, n_bins)."""
    n_full, _ = workload_shape(k)
    return make_workload(k, n_rows, row_start=n_full)


def make_random(n: int, n_bins, seed: int, bin_kind: int = 0, label_kind: int = 0):
    """Generic test workload: uniform (or skewed) bins, N(0,1) / dyadic / additive labels."""
    nb = np.ascontiguousarray(np.asarray(n_bins, dtype=np.int32))
    F = int(nb.shape[0])
    bins = np.empty((n, F), dtype=np.uint8)
    label = np.empty(n, dtype=np.float32)
    rc = _load().dg_random(n, F, _ptr(nb), seed, bin_kind, label_kind, _ptr(bins), _ptr(label))
    if rc:
        raise ValueError("dg_random failed (%d)" % rc)
    return bins, label, nb


def fingerprint(a: np.ndarray) -> str:
    a = np.ascontiguousarray(a)
    return "%016x" % _load().dg_fnv1a64(_ptr(a), a.nbytes)


def uniform(seed: int, stream: int, c: int) -> float:
    return float(_load().dg_uniform(seed, stream, c))


def u64(seed: int, stream: int, c: int) -> int:
    return int(_load().dg_u64(seed, stream, c))
