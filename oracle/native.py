"""ctypes binding of the threaded C++ oracle (oracle/oracle.cpp -> liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  The library is
plain C++17 (no HIP) and computes what oracle/ref.py computes, bit for bit
(the tests hold the two equal), at the benchmark workloads' full sizes.

build() compiles it with g++; lib() loads it, building it first when no
library is on disk.  The functions take and return NumPy arrays; they
only marshal pointers and sizes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add; no -ffast-math: IEEE semantics,
# subnormals kept, no reassociation.
FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-pthread", "-Wall"]

SUM, MIN, MAX, AVG = 0, 1, 2, 3
F32, BF16, I32 = 0, 1, 2
ORD_RING, ORD_RD, ORD_HD, ORD_TREE, ORD_DBT = 0, 1, 2, 3, 4
NP = {F32: np.float32, BF16: np.uint16, I32: np.int32}

_lib = None


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["g++", *FLAGS, "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_allreduce.argtypes = [vp, vp, i32, i64, i32, i32, i32, vp, i32]
        L.oracle_reduce_scatter.argtypes = [vp, vp, i32, i64, i32, i32, vp, i32]
        L.oracle_allgather.argtypes = [vp, vp, i32, i64, i32, i32]
        L.oracle_alltoallv.argtypes = [vp, vp, i32, vp, i32, i32]
        L.oracle_allreduce_batch.argtypes = [i32, i32, vp, vp, vp, vp, vp, i32]
        L.oracle_fp8_row_bytes.argtypes = [i64, i64]
        L.oracle_fp8_row_bytes.restype = i64
        L.oracle_fp8_encode_rows.argtypes = [vp, i64, i64, i64, vp, i32]
        L.oracle_fp8_dequant_rows.argtypes = [vp, i64, i64, i64, vp, i32]
        L.oracle_moe_combine.argtypes = [vp, vp, vp, vp, vp, i64, i32, i64, i32, i32]
        L.oracle_hardware_threads.argtypes = []
        _lib = L
    return _lib


def hardware_threads() -> int:
    return int(lib().oracle_hardware_threads())


def _threads(nthreads):
    return hardware_threads() if nthreads is None else int(nthreads)


def _ptrs(arrays):
    return (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def _contig(arrays, dtype=None):
    out = []
    for a in arrays:
        a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
        out.append(a)
    return out


def allreduce(xs, op: int, dtype: int, order: int = ORD_RING, scales=None, nthreads=None) -> np.ndarray:
    """The reduced vector every rank receives (oracle_allreduce)."""
    xs = _contig(xs, NP[dtype])
    n = len(xs[0])
    out = np.empty(n, dtype=NP[dtype])
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)
    rc = lib().oracle_allreduce(_ptrs(xs), out.ctypes.data, len(xs), n, dtype, op, order,
                                None if sc is None else sc.ctypes.data, _threads(nthreads))
    _check(rc, "allreduce")
    return out


def reduce_scatter(xs, op: int, dtype: int, scales=None, nthreads=None) -> list[np.ndarray]:
    """Block r of the reduction for every rank r (each x holds p * n)."""
    xs = _contig(xs, NP[dtype])
    p = len(xs)
    n = len(xs[0]) // p
    outs = [np.empty(n, dtype=NP[dtype]) for _ in range(p)]
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)
    rc = lib().oracle_reduce_scatter(_ptrs(xs), _ptrs(outs), p, n, dtype, op,
                                     None if sc is None else sc.ctypes.data, _threads(nthreads))
    _check(rc, "reduce_scatter")
    return outs


def allgather(xs, nthreads=None) -> list[np.ndarray]:
    xs = _contig(xs)
    p, n = len(xs), len(xs[0])
    outs = [np.empty(p * n, dtype=xs[0].dtype) for _ in range(p)]
    rc = lib().oracle_allgather(_ptrs(xs), _ptrs(outs), p, n, xs[0].itemsize, _threads(nthreads))
    _check(rc, "allgather")
    return outs


def alltoallv(xs, counts, nthreads=None) -> list[np.ndarray]:
    """counts[i][j] elements from rank i to rank j; receive buffers packed
    in source order (their lengths are the column sums)."""
    xs = _contig(xs)
    p = len(xs)
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.int64).reshape(p, p))
    outs = [np.empty(int(s), dtype=xs[0].dtype) for s in c.sum(axis=0)]
    rc = lib().oracle_alltoallv(_ptrs(xs), _ptrs(outs), p, c.ctypes.data, xs[0].itemsize, _threads(nthreads))
    _check(rc, "alltoallv")
    return outs


def alltoall(xs, nthreads=None) -> list[np.ndarray]:
    p = len(xs)
    m = len(xs[0]) // p
    return alltoallv(xs, np.full((p, p), m, dtype=np.int64), nthreads)


def allreduce_batch(calls, outs, nthreads=None) -> None:
    """calls: (per-rank inputs, op, dtype) each; outs: one preallocated
    output array per call, written in place."""
    p = len(calls[0][0])
    srcs = []
    for xs, op, dt in calls:
        srcs.extend(_contig(xs, NP[dt]))
    for o, (_, _, dt) in zip(outs, calls):
        assert o.dtype == NP[dt] and o.flags.c_contiguous
    n = np.array([len(c[0][0]) for c in calls], dtype=np.int64)
    dts = np.array([c[2] for c in calls], dtype=np.int32)
    ops = np.array([c[1] for c in calls], dtype=np.int32)
    rc = lib().oracle_allreduce_batch(len(calls), p, n.ctypes.data, dts.ctypes.data, ops.ctypes.data, _ptrs(srcs),
                                      _ptrs(outs), _threads(nthreads))
    _check(rc, "allreduce_batch")


def fp8_row_bytes(hidden: int, group: int) -> int:
    return int(lib().oracle_fp8_row_bytes(hidden, group))


def fp8_encode_rows(tokens_bf16, hidden: int, group: int, nthreads=None) -> np.ndarray:
    """Packed FP8 rows (uint8 [rows * row_bytes]) of bf16 token rows."""
    t = np.ascontiguousarray(tokens_bf16, dtype=np.uint16)
    rows = len(t) // hidden
    out = np.empty(rows * fp8_row_bytes(hidden, group), dtype=np.uint8)
    _check(lib().oracle_fp8_encode_rows(t.ctypes.data, rows, hidden, group, out.ctypes.data, _threads(nthreads)),
           "fp8_encode_rows")
    return out


def fp8_dequant_rows(packed, hidden: int, group: int, nthreads=None) -> np.ndarray:
    """bf16 bits [rows * hidden] of packed FP8 rows."""
    b = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = len(b) // fp8_row_bytes(hidden, group)
    out = np.empty(rows * hidden, dtype=np.uint16)
    _check(lib().oracle_fp8_dequant_rows(b.ctypes.data, rows, hidden, group, out.ctypes.data, _threads(nthreads)),
           "fp8_dequant_rows")
    return out


def moe_combine(rows, slot, weights, k: int, hidden: int, dtype: int, residual=None, nthreads=None) -> np.ndarray:
    """One rank's combine: token t sums w[t*k+s] * rows[slot[t*k+s]] onto the
    residual (fp32, slot order, every product and sum rounded)."""
    r = np.ascontiguousarray(rows, dtype=NP[dtype])
    sl = np.ascontiguousarray(slot, dtype=np.int64)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    T = len(sl) // k
    res = None if residual is None else np.ascontiguousarray(residual, dtype=NP[dtype])
    out = np.empty(T * hidden, dtype=NP[dtype])
    _check(lib().oracle_moe_combine(r.ctypes.data, sl.ctypes.data, w.ctypes.data,
                                    None if res is None else res.ctypes.data, out.ctypes.data, T, k, hidden, dtype,
                                    _threads(nthreads)), "moe_combine")
    return out
