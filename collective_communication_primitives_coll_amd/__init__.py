"""Collective communication primitives over p logical ranks in one MI355X.

Thin ctypes binding of ``libcoll.so`` (C ABI in ``include/coll.h``).  The
functions carry the C names and only marshal arguments: buffers may be
torch tensors (their ``data_ptr()`` is passed) or raw device addresses
(ints).  Every byte of the collective is moved by the library's HIP
kernels; there is no CPU or torch fallback, and a missing library raises.

Calls are asynchronous on ``stream`` (default: torch's current stream on
the current device); synchronise before reading results.
"""
from __future__ import annotations

import ctypes
import os
from typing import Any, Sequence

# Enum values of coll.h
COLL_F32, COLL_BF16, COLL_I32 = 0, 1, 2
COLL_SUM, COLL_MIN, COLL_MAX, COLL_AVG = 0, 1, 2, 3
COLL_OK, COLL_ERR_INVALID_ARG, COLL_ERR_UNSUPPORTED, COLL_ERR_ALIAS, COLL_ERR_HIP = 0, 1, 2, 3, 4
COLL_ALGO_RING, COLL_ALGO_ONEPASS, COLL_ALGO_RING_LITERAL, COLL_ALGO_HALVING_DOUBLING = 0, 1, 2, 3
COLL_ALGO_RECURSIVE_DOUBLING = COLL_ALGO_ONEPASS
COLL_ALGO_TREE, COLL_ALGO_DOUBLE_BINARY_TREE = 4, 5
COLL_MAX_RANKS = 64
COLL_BATCH_CHECK_ALIAS = 1
COLL_BATCH_NOALLOC_MAX_BYTES = 4 << 20

COLL_U8 = 3
COLL_A2A_DIRECT, COLL_A2A_LDS_STAGED = 0, 1
COLL_PROBE_NT_LOADS, COLL_PROBE_NT_STORES, COLL_PROBE_CLAIM, COLL_PROBE_DEVICE_STORES = 1, 2, 4, 8
ELEM_BYTES = {COLL_F32: 4, COLL_BF16: 2, COLL_I32: 4, COLL_U8: 1}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcoll.so")

_lib = None


class CollError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class coll_call_t(ctypes.Structure):
    _fields_ = [
        ("send", ctypes.POINTER(ctypes.c_void_p)),
        ("recv", ctypes.POINTER(ctypes.c_void_p)),
        ("n", ctypes.c_size_t),
        ("dtype", ctypes.c_int),
        ("op", ctypes.c_int),
    ]


def lib() -> ctypes.CDLL:
    """Load libcoll.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with __graft_entry__.build(). "
                           "There is no fallback path.")
    # torch ships its own HIP runtime.  Loaded first, it also serves this
    # library; loaded after it, it would be a second runtime in the process,
    # in which torch's device pointers and streams mean nothing (every call
    # then fails with hipErrorNoDevice).
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, pp, sz, i32 = ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_int
    i64p = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "coll_allreduce": [pp, pp, i32, sz, i32, i32, vp],
        "coll_allreduce_algo": [pp, pp, i32, sz, i32, i32, i32, vp],
        "coll_reduce": [pp, vp, i32, sz, i32, i32, i32, vp],
        "coll_broadcast": [vp, pp, i32, sz, i32, i32, vp],
        "coll_reduce_scatter": [pp, pp, i32, sz, i32, i32, vp],
        "coll_allgather": [pp, pp, i32, sz, i32, vp],
        "coll_alltoall": [pp, pp, i32, sz, i32, vp],
        "coll_alltoall_algo": [pp, pp, i32, sz, i32, i32, vp],
        "coll_alltoallv": [pp, pp, i32, vp, i64p, i64p, vp, i32, vp],
        "coll_gather": [pp, vp, i32, sz, i32, i32, vp],
        "coll_allreduce_premul": [pp, pp, i32, sz, i32, ctypes.POINTER(ctypes.c_float), i32, vp],
        "coll_reduce_scatter_premul": [pp, pp, i32, sz, i32, ctypes.POINTER(ctypes.c_float), vp],
        "coll_alltoallv_transposed": [pp, pp, i32, vp, i64p, i64p, vp, i32, vp],
        "coll_moe_pack": [pp, pp, pp, pp, vp, vp, i32, sz, i32, sz, i32, vp],
        "coll_moe_combine": [pp, pp, pp, pp, pp, i32, sz, i32, sz, i32, vp],
        "coll_scatter": [vp, pp, i32, sz, i32, i32, vp],
        "coll_allreduce_batch": [ctypes.POINTER(coll_call_t), i32, i32, ctypes.c_uint, vp],
        "coll_allreduce_batch_noalloc": [ctypes.POINTER(coll_call_t), i32, i32, ctypes.c_uint, vp],
        "coll_moe_pack_fp8": [pp, pp, pp, pp, vp, vp, vp, i32, sz, i32, sz, sz, vp],
        "coll_moe_dequant_fp8": [pp, pp, i32, vp, i64p, vp, sz, sz, vp],
        "coll_moe_dispatch": [pp, pp, pp, pp, vp, vp, i32, sz, i32, sz, i64p, i32, vp],
        "coll_moe_dispatch_fp8": [pp, pp, pp, pp, vp, vp, vp, i32, sz, i32, sz, sz, i64p, vp],
        "coll_moe_combine_direct": [pp, pp, pp, pp, pp, i32, sz, i32, sz, i64p, i32, vp],
        "coll_stream_probe": [pp, i32, pp, i32, sz, i32, ctypes.c_uint, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.coll_status_string.argtypes = [ctypes.c_int]
    L.coll_status_string.restype = ctypes.c_char_p
    L.coll_last_hip_error.argtypes = []
    L.coll_last_hip_error.restype = ctypes.c_int
    L.coll_version.argtypes = []
    L.coll_version.restype = ctypes.c_int
    L.coll_moe_fp8_row_bytes.argtypes = [sz, sz]
    L.coll_moe_fp8_row_bytes.restype = sz
    L.coll_finalize.argtypes = []
    L.coll_finalize.restype = None
    L.coll_set_grid_limit.argtypes = [ctypes.c_int]
    L.coll_set_grid_limit.restype = None
    _lib = L
    return L


# ----------------------------------------------------------------------------
# Marshalling helpers
# ----------------------------------------------------------------------------

def _addr(x: Any) -> int:
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("buffers must be device tensors")
        if not x.is_contiguous():
            raise ValueError("buffers must be contiguous")
        return x.data_ptr()
    raise TypeError(f"expected a tensor or a device address, got {type(x)}")


def _ptr_array(xs: Sequence[Any]):
    arr = (ctypes.c_void_p * len(xs))(*[_addr(x) for x in xs])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), arr


def _dtype_of(x: Any, dtype: int | None) -> int:
    if dtype is not None:
        return int(dtype)
    import torch
    m = {torch.float32: COLL_F32, torch.bfloat16: COLL_BF16, torch.int32: COLL_I32, torch.uint8: COLL_U8}
    if not hasattr(x, "dtype") or x.dtype not in m:
        raise ValueError("dtype must be given for raw addresses, or tensors must be "
                         "float32/bfloat16/int32/uint8")
    return m[x.dtype]


def _numel(x: Any, n: int | None) -> int:
    if n is not None:
        return int(n)
    if hasattr(x, "numel"):
        return int(x.numel())
    raise ValueError("n must be given for raw addresses")


def _stream(stream: Any) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(status: int, what: str) -> None:
    if status != COLL_OK:
        L = lib()
        msg = L.coll_status_string(status).decode()
        if status == COLL_ERR_HIP:
            msg += f" (hipError {L.coll_last_hip_error()})"
        raise CollError(status, f"{what}: {msg}")


class Prepared:
    """A C-ABI call whose arguments were marshalled once.

    Calling it launches the same collective again on the same buffers and
    stream; it raises CollError on a non-OK status like the direct call.
    """

    def __init__(self, fname: str, args: tuple, what: str, keep: tuple):
        self._f = getattr(lib(), fname)
        self._args = args
        self._what = what
        self._keep = keep   # ctypes arrays the argument pointers refer to

    def __call__(self) -> None:
        _check(self._f(*self._args), self._what)


def _run(fname: str, args: tuple, what: str, defer: bool, keep: tuple = ()):
    """Call fname(*args) now, or with defer=True return it as a Prepared call."""
    if defer:
        return Prepared(fname, args, what, keep)
    _check(getattr(lib(), fname)(*args), what)
    return None


def _check_sizes(xs: Sequence[Any], need: int, what: str) -> None:
    for x in xs:
        if hasattr(x, "numel") and x.numel() < need:
            raise ValueError(f"{what}: buffer of {x.numel()} elements, {need} needed")


def _same_dtype(xs: Sequence[Any], dt: int) -> None:
    for x in xs:
        if hasattr(x, "dtype") and _dtype_of(x, None) != dt:
            raise ValueError("all buffers must share one dtype")


# ----------------------------------------------------------------------------
# The entry points (names and argument order of coll.h; n and dtype are
# taken from the tensors when not given)
# ----------------------------------------------------------------------------

def coll_allreduce(send, recv, op: int = COLL_SUM, n: int | None = None, dtype: int | None = None,
                   stream=None, defer: bool = False):
    return coll_allreduce_algo(send, recv, COLL_ALGO_RING, op, n, dtype, stream, defer)


def coll_allreduce_algo(send, recv, algo: int, op: int = COLL_SUM, n: int | None = None,
                        dtype: int | None = None, stream=None, defer: bool = False):
    p = len(send)
    if len(recv) != p:
        raise ValueError("send and recv must list the same ranks")
    dt = _dtype_of(send[0], dtype)
    n = _numel(send[0], n)
    _same_dtype([*send, *recv], dt)
    _check_sizes([*send, *recv], n, "allreduce")
    s, k1 = _ptr_array(send)
    r, k2 = _ptr_array(recv)
    return _run("coll_allreduce_algo", (s, r, p, n, dt, int(op), int(algo), _stream(stream)),
                "coll_allreduce", defer, (k1, k2))


def coll_allreduce_premul(send, recv, scale: Sequence[float], algo: int = COLL_ALGO_RING, n: int | None = None,
                          dtype: int | None = None, stream=None, defer: bool = False):
    """recv[r] = sum_k scale[k] * send[k] (fp32 products rounded on their own)."""
    p = len(send)
    if len(recv) != p or len(scale) != p:
        raise ValueError("send, recv and scale must list the same ranks")
    dt = _dtype_of(send[0], dtype)
    n = _numel(send[0], n)
    _same_dtype([*send, *recv], dt)
    _check_sizes([*send, *recv], n, "allreduce_premul")
    s, k1 = _ptr_array(send)
    r, k2 = _ptr_array(recv)
    sc = (ctypes.c_float * p)(*[float(v) for v in scale])
    return _run("coll_allreduce_premul", (s, r, p, n, dt, sc, int(algo), _stream(stream)),
                "coll_allreduce_premul", defer, (k1, k2, sc))


def coll_reduce_scatter_premul(send, recv, scale: Sequence[float], n: int | None = None, dtype: int | None = None,
                               stream=None, defer: bool = False):
    """ReduceScatter of sum_k scale[k] * send[k]; n = elements each rank receives."""
    p = len(send)
    if len(scale) != p:
        raise ValueError("one scale per rank")
    dt = _dtype_of(send[0], dtype)
    n = _numel(recv[0], n)
    _same_dtype([*send, *recv], dt)
    _check_sizes(send, p * n, "reduce_scatter_premul send")
    _check_sizes(recv, n, "reduce_scatter_premul recv")
    s, k1 = _ptr_array(send)
    r, k2 = _ptr_array(recv)
    sc = (ctypes.c_float * p)(*[float(v) for v in scale])
    return _run("coll_reduce_scatter_premul", (s, r, p, n, dt, sc, _stream(stream)),
                "coll_reduce_scatter_premul", defer, (k1, k2, sc))


def coll_reduce(send, recv_root, root: int, op: int = COLL_SUM, n: int | None = None,
                dtype: int | None = None, stream=None, defer: bool = False):
    p = len(send)
    dt = _dtype_of(send[0], dtype)
    n = _numel(send[0], n)
    _same_dtype([*send, recv_root], dt)
    _check_sizes([*send, recv_root], n, "reduce")
    s, k = _ptr_array(send)
    return _run("coll_reduce", (s, _addr(recv_root), p, n, dt, int(op), int(root), _stream(stream)),
                "coll_reduce", defer, (k,))


def coll_broadcast(send_root, recv, root: int, n: int | None = None, dtype: int | None = None,
                   stream=None, defer: bool = False):
    p = len(recv)
    dt = _dtype_of(send_root, dtype)
    n = _numel(send_root, n)
    _same_dtype([send_root, *recv], dt)
    _check_sizes([send_root, *recv], n, "broadcast")
    r, k = _ptr_array(recv)
    return _run("coll_broadcast", (_addr(send_root), r, p, n, dt, int(root), _stream(stream)),
                "coll_broadcast", defer, (k,))


def coll_reduce_scatter(send, recv, op: int = COLL_SUM, n: int | None = None, dtype: int | None = None,
                        stream=None, defer: bool = False):
    """n = elements each rank receives; send[r] holds p*n."""
    p = len(send)
    dt = _dtype_of(send[0], dtype)
    n = _numel(recv[0], n)
    _same_dtype([*send, *recv], dt)
    _check_sizes(send, p * n, "reduce_scatter send")
    _check_sizes(recv, n, "reduce_scatter recv")
    s, k1 = _ptr_array(send)
    r, k2 = _ptr_array(recv)
    return _run("coll_reduce_scatter", (s, r, p, n, dt, int(op), _stream(stream)),
                "coll_reduce_scatter", defer, (k1, k2))


def coll_allgather(send, recv, n: int | None = None, dtype: int | None = None, stream=None,
                   defer: bool = False):
    """n = elements each rank sends; recv[r] holds p*n."""
    p = len(send)
    dt = _dtype_of(send[0], dtype)
    n = _numel(send[0], n)
    _same_dtype([*send, *recv], dt)
    _check_sizes(send, n, "allgather send")
    _check_sizes(recv, p * n, "allgather recv")
    s, k1 = _ptr_array(send)
    r, k2 = _ptr_array(recv)
    return _run("coll_allgather", (s, r, p, n, dt, _stream(stream)), "coll_allgather", defer, (k1, k2))


def coll_alltoall(send, recv, n_block: int | None = None, dtype: int | None = None, stream=None,
                  defer: bool = False):
    """send[i] and recv[j] hold p blocks of n_block elements."""
    p = len(send)
    dt = _dtype_of(send[0], dtype)
    if n_block is None:
        n_block = _numel(send[0], None) // p
    _same_dtype([*send, *recv], dt)
    _check_sizes([*send, *recv], p * n_block, "alltoall")
    s, k1 = _ptr_array(send)
    r, k2 = _ptr_array(recv)
    return _run("coll_alltoall", (s, r, p, int(n_block), dt, _stream(stream)), "coll_alltoall", defer,
                (k1, k2))


def coll_alltoall_algo(send, recv, algo: int, n_block: int | None = None, dtype: int | None = None, stream=None,
                       defer: bool = False):
    """coll_alltoall with an explicit data path (COLL_A2A_DIRECT or
    COLL_A2A_LDS_STAGED)."""
    p = len(send)
    dt = _dtype_of(send[0], dtype)
    if n_block is None:
        n_block = _numel(send[0], None) // p
    _same_dtype([*send, *recv], dt)
    _check_sizes([*send, *recv], p * n_block, "alltoall")
    s, k1 = _ptr_array(send)
    r, k2 = _ptr_array(recv)
    return _run("coll_alltoall_algo", (s, r, p, int(n_block), dt, int(algo), _stream(stream)),
                "coll_alltoall_algo", defer, (k1, k2))


def coll_gather(send, recv_root, root: int, n: int | None = None, dtype: int | None = None, stream=None,
                defer: bool = False):
    """n = elements each rank sends; recv_root holds p*n."""
    p = len(send)
    dt = _dtype_of(send[0], dtype)
    n = _numel(send[0], n)
    _same_dtype([*send, recv_root], dt)
    _check_sizes(send, n, "gather send")
    _check_sizes([recv_root], p * n, "gather recv")
    s, k = _ptr_array(send)
    return _run("coll_gather", (s, _addr(recv_root), p, n, dt, int(root), _stream(stream)),
                "coll_gather", defer, (k,))


def coll_scatter(send_root, recv, root: int, n: int | None = None, dtype: int | None = None, stream=None,
                 defer: bool = False):
    """n = elements each rank receives; send_root holds p*n."""
    p = len(recv)
    dt = _dtype_of(send_root, dtype)
    n = _numel(recv[0], n)
    _same_dtype([send_root, *recv], dt)
    _check_sizes([send_root], p * n, "scatter send")
    _check_sizes(recv, n, "scatter recv")
    r, k = _ptr_array(recv)
    return _run("coll_scatter", (_addr(send_root), r, p, n, dt, int(root), _stream(stream)),
                "coll_scatter", defer, (k,))


def coll_alltoallv(send, recv, counts_dev, send_cap: Sequence[int] | None = None,
                   recv_cap: Sequence[int] | None = None, status_dev=None, dtype: int | None = None,
                   stream=None, defer: bool = False):
    """counts_dev: device int64 [p, p] (row = source).  Capacities default to
    the tensors' sizes."""
    p = len(send)
    dt = _dtype_of(send[0], dtype)
    if send_cap is None:
        send_cap = [_numel(x, None) for x in send]
    if recv_cap is None:
        recv_cap = [_numel(x, None) for x in recv]
    if hasattr(counts_dev, "dtype"):
        import torch
        if counts_dev.dtype != torch.int64 or counts_dev.numel() < p * p:
            raise ValueError("counts must be a device int64 tensor with p*p entries")
    _same_dtype([*send, *recv], dt)
    s, k1 = _ptr_array(send)
    r, k2 = _ptr_array(recv)
    sc = (ctypes.c_int64 * p)(*[int(v) for v in send_cap])
    rc = (ctypes.c_int64 * p)(*[int(v) for v in recv_cap])
    st = _addr(status_dev) if status_dev is not None else None
    return _run("coll_alltoallv", (s, r, p, _addr(counts_dev), sc, rc, st, dt, _stream(stream)),
                "coll_alltoallv", defer, (k1, k2, sc, rc))


def coll_alltoallv_transposed(send, recv, counts_dev, send_cap: Sequence[int] | None = None,
                              recv_cap: Sequence[int] | None = None, status_dev=None, dtype: int | None = None,
                              stream=None, defer: bool = False):
    """The reverse exchange of coll_alltoallv: counts_dev is the forward
    [p, p] matrix; rank i sends counts[j][i] elements to rank j."""
    p = len(send)
    dt = _dtype_of(send[0], dtype)
    if send_cap is None:
        send_cap = [_numel(x, None) for x in send]
    if recv_cap is None:
        recv_cap = [_numel(x, None) for x in recv]
    if hasattr(counts_dev, "dtype"):
        import torch
        if counts_dev.dtype != torch.int64 or counts_dev.numel() < p * p:
            raise ValueError("counts must be a device int64 tensor with p*p entries")
    _same_dtype([*send, *recv], dt)
    s, k1 = _ptr_array(send)
    r, k2 = _ptr_array(recv)
    sc = (ctypes.c_int64 * p)(*[int(v) for v in send_cap])
    rc = (ctypes.c_int64 * p)(*[int(v) for v in recv_cap])
    st = _addr(status_dev) if status_dev is not None else None
    return _run("coll_alltoallv_transposed", (s, r, p, _addr(counts_dev), sc, rc, st, dt, _stream(stream)),
                "coll_alltoallv_transposed", defer, (k1, k2, sc, rc))


def coll_moe_pack(tokens, dest, packed, pos, counts_dev, k: int, hidden: int, status_dev=None,
                  tokens_per_rank: int | None = None, dtype: int | None = None, stream=None,
                  defer: bool = False):
    """Dispatch pack: per rank, tokens [T*hidden], dest int32 [T*k] ->
    packed [T*k*hidden], pos int32 [T*k]; counts_dev int64 [p, p] (elements)."""
    p = len(tokens)
    dt = _dtype_of(tokens[0], dtype)
    T = tokens_per_rank if tokens_per_rank is not None else _numel(tokens[0], None) // int(hidden)
    _same_dtype([*tokens, *packed], dt)
    _check_sizes(tokens, T * hidden, "moe_pack tokens")
    _check_sizes(packed, T * k * hidden, "moe_pack packed")
    _check_sizes([*dest, *pos], T * k, "moe_pack dest/pos")
    a1, k1 = _ptr_array(tokens)
    a2, k2 = _ptr_array(dest)
    a3, k3 = _ptr_array(packed)
    a4, k4 = _ptr_array(pos)
    st = _addr(status_dev) if status_dev is not None else None
    return _run("coll_moe_pack", (a1, a2, a3, a4, _addr(counts_dev), st, p, int(T), int(k), int(hidden), dt,
                                  _stream(stream)), "coll_moe_pack", defer, (k1, k2, k3, k4))


def coll_moe_fp8_row_bytes(hidden: int, group: int) -> int:
    """Bytes of one packed FP8 row (codes, scales, padding); 0 if the shape
    is not accepted."""
    return int(lib().coll_moe_fp8_row_bytes(int(hidden), int(group)))


def coll_moe_pack_fp8(tokens, dest, packed, pos, counts_dev, k: int, hidden: int, group: int,
                      counts_hidden_dev=None, status_dev=None, tokens_per_rank: int | None = None,
                      stream=None, defer: bool = False):
    """Quantizing dispatch pack: per rank, bf16 tokens [T*hidden], dest int32
    [T*k] -> packed uint8 [T*k*row_bytes], pos int32 [T*k]; counts_dev int64
    [p, p] in bytes; counts_hidden_dev (optional) int64 [p, p] in rows*hidden."""
    p = len(tokens)
    T = tokens_per_rank if tokens_per_rank is not None else _numel(tokens[0], None) // int(hidden)
    R = coll_moe_fp8_row_bytes(hidden, group)
    if R:
        _check_sizes(packed, T * k * R, "moe_pack_fp8 packed")
    _check_sizes(tokens, T * hidden, "moe_pack_fp8 tokens")
    _check_sizes([*dest, *pos], T * k, "moe_pack_fp8 dest/pos")
    a1, k1 = _ptr_array(tokens)
    a2, k2 = _ptr_array(dest)
    a3, k3 = _ptr_array(packed)
    a4, k4 = _ptr_array(pos)
    st = _addr(status_dev) if status_dev is not None else None
    ch = _addr(counts_hidden_dev) if counts_hidden_dev is not None else None
    return _run("coll_moe_pack_fp8", (a1, a2, a3, a4, _addr(counts_dev), ch, st, p, int(T), int(k), int(hidden),
                                      int(group), _stream(stream)), "coll_moe_pack_fp8", defer, (k1, k2, k3, k4))


def coll_moe_dequant_fp8(recv, out, counts_dev, rows_cap: Sequence[int], hidden: int, group: int,
                         status_dev=None, stream=None, defer: bool = False):
    """bf16 rows of the FP8 rows each rank received (byte counts [p, p] on
    the device, as written by coll_moe_pack_fp8)."""
    p = len(recv)
    R = coll_moe_fp8_row_bytes(hidden, group)
    for r in range(p):
        if R:
            _check_sizes([recv[r]], int(rows_cap[r]) * R, "moe_dequant_fp8 recv")
        _check_sizes([out[r]], int(rows_cap[r]) * hidden, "moe_dequant_fp8 out")
    a1, k1 = _ptr_array(recv)
    a2, k2 = _ptr_array(out)
    cap = (ctypes.c_int64 * p)(*[int(c) for c in rows_cap])
    st = _addr(status_dev) if status_dev is not None else None
    return _run("coll_moe_dequant_fp8", (a1, a2, p, _addr(counts_dev), cap, st, int(hidden), int(group),
                                         _stream(stream)), "coll_moe_dequant_fp8", defer, (k1, k2, cap))


def coll_moe_dispatch(tokens, dest, recv, loc, counts_dev, k: int, hidden: int, recv_cap: Sequence[int] | None = None,
                      status_dev=None, tokens_per_rank: int | None = None, dtype: int | None = None, stream=None,
                      defer: bool = False):
    """Direct dispatch: per rank, tokens [T*hidden], dest int32 [T*k] ->
    recv[j] (rows received by rank j, capacity recv_cap[j] rows, default the
    tensor's size), loc int64 [T*k] ((dest << 32) | row, or -1); counts_dev
    int64 [p, p] in elements; status_dev optional int32 [p + 1]."""
    p = len(tokens)
    dt = _dtype_of(tokens[0], dtype)
    T = tokens_per_rank if tokens_per_rank is not None else _numel(tokens[0], None) // int(hidden)
    _same_dtype([*tokens, *recv], dt)
    if recv_cap is None:
        recv_cap = [_numel(x, None) // int(hidden) for x in recv]
    for r in range(p):
        _check_sizes([recv[r]], int(recv_cap[r]) * hidden, "moe_dispatch recv")
    _check_sizes(tokens, T * hidden, "moe_dispatch tokens")
    _check_sizes([*dest, *loc], T * k, "moe_dispatch dest/loc")
    a1, k1 = _ptr_array(tokens)
    a2, k2 = _ptr_array(dest)
    a3, k3 = _ptr_array(recv)
    a4, k4 = _ptr_array(loc)
    cap = (ctypes.c_int64 * p)(*[int(c) for c in recv_cap])
    st = _addr(status_dev) if status_dev is not None else None
    return _run("coll_moe_dispatch", (a1, a2, a3, a4, _addr(counts_dev), st, p, int(T), int(k), int(hidden), cap, dt,
                                      _stream(stream)), "coll_moe_dispatch", defer, (k1, k2, k3, k4, cap))


def coll_moe_dispatch_fp8(tokens, dest, recv, loc, counts_dev, k: int, hidden: int, group: int,
                          recv_cap: Sequence[int] | None = None, counts_hidden_dev=None, status_dev=None,
                          tokens_per_rank: int | None = None, stream=None, defer: bool = False):
    """Direct FP8 dispatch: bf16 tokens -> encoded rows written straight into
    recv[j] (uint8, capacity recv_cap[j] rows of row_bytes); counts in bytes."""
    p = len(tokens)
    T = tokens_per_rank if tokens_per_rank is not None else _numel(tokens[0], None) // int(hidden)
    R = coll_moe_fp8_row_bytes(hidden, group)
    if recv_cap is None:
        recv_cap = [(_numel(x, None) // R) if R else 0 for x in recv]
    for r in range(p):
        if R:
            _check_sizes([recv[r]], int(recv_cap[r]) * R, "moe_dispatch_fp8 recv")
    _check_sizes(tokens, T * hidden, "moe_dispatch_fp8 tokens")
    _check_sizes([*dest, *loc], T * k, "moe_dispatch_fp8 dest/loc")
    a1, k1 = _ptr_array(tokens)
    a2, k2 = _ptr_array(dest)
    a3, k3 = _ptr_array(recv)
    a4, k4 = _ptr_array(loc)
    cap = (ctypes.c_int64 * p)(*[int(c) for c in recv_cap])
    ch = _addr(counts_hidden_dev) if counts_hidden_dev is not None else None
    st = _addr(status_dev) if status_dev is not None else None
    return _run("coll_moe_dispatch_fp8", (a1, a2, a3, a4, _addr(counts_dev), ch, st, p, int(T), int(k), int(hidden),
                                          int(group), cap, _stream(stream)), "coll_moe_dispatch_fp8", defer,
                (k1, k2, k3, k4, cap))


def coll_moe_combine_direct(y, loc, weights, out, k: int, hidden: int, y_rows: Sequence[int] | None = None,
                            residual=None, tokens_per_rank: int | None = None, dtype: int | None = None,
                            stream=None, defer: bool = False):
    """Combine reading expert outputs in place: y[j] rows (y_rows[j], default
    the tensor's size) addressed by loc from coll_moe_dispatch(_fp8)."""
    p = len(out)
    dt = _dtype_of(out[0], dtype)
    T = tokens_per_rank if tokens_per_rank is not None else _numel(out[0], None) // int(hidden)
    _same_dtype([*y, *out, *(residual or [])], dt)
    if y_rows is None:
        y_rows = [_numel(x, None) // int(hidden) for x in y]
    for j in range(len(y)):
        _check_sizes([y[j]], int(y_rows[j]) * hidden, "moe_combine_direct y")
    _check_sizes(out, T * hidden, "moe_combine_direct out")
    _check_sizes([*loc, *weights], T * k, "moe_combine_direct loc/weights")
    a1, k1 = _ptr_array(y)
    a2, k2 = _ptr_array(loc)
    a3, k3 = _ptr_array(weights)
    a5, k5 = _ptr_array(out)
    if residual is not None:
        a4, k4 = _ptr_array(residual)
    else:
        a4, k4 = None, None
    rows = (ctypes.c_int64 * p)(*[int(c) for c in y_rows])
    return _run("coll_moe_combine_direct", (a1, a2, a3, a4, a5, p, int(T), int(k), int(hidden), rows, dt,
                                            _stream(stream)), "coll_moe_combine_direct", defer,
                (k1, k2, k3, k4, k5, rows))


def coll_moe_combine(back, pos, weights, out, k: int, hidden: int, residual=None,
                     tokens_per_rank: int | None = None, dtype: int | None = None, stream=None,
                     defer: bool = False):
    """Weighted combine: per rank out[t] = residual[t] + sum_s w[t*k+s] * back[pos[t*k+s]]."""
    p = len(back)
    dt = _dtype_of(back[0], dtype)
    T = tokens_per_rank if tokens_per_rank is not None else _numel(out[0], None) // int(hidden)
    _same_dtype([*back, *out, *(residual or [])], dt)
    _check_sizes(back, T * k * hidden, "moe_combine back")
    _check_sizes(out, T * hidden, "moe_combine out")
    _check_sizes([*pos, *weights], T * k, "moe_combine pos/weights")
    a1, k1 = _ptr_array(back)
    a2, k2 = _ptr_array(pos)
    a3, k3 = _ptr_array(weights)
    a5, k5 = _ptr_array(out)
    if residual is not None:
        a4, k4 = _ptr_array(residual)
    else:
        a4, k4 = None, None
    return _run("coll_moe_combine", (a1, a2, a3, a4, a5, p, int(T), int(k), int(hidden), dt, _stream(stream)),
                "coll_moe_combine", defer, (k1, k2, k3, k4, k5))


def coll_allreduce_batch(calls: Sequence[tuple], p: int, flags: int = 0, stream=None,
                         defer: bool = False, noalloc: bool = False):
    """calls: (send list, recv list, n, dtype, op) per AllReduce.  noalloc:
    use coll_allreduce_batch_noalloc (descriptor table in the library's
    static device array; nothing allocated)."""
    keep = []
    arr = (coll_call_t * len(calls))()
    for k, (send, recv, n, dtype, op) in enumerate(calls):
        if len(send) != p or len(recv) != p:
            raise ValueError("every call must list p ranks")
        s, ks = _ptr_array(send)
        r, kr = _ptr_array(recv)
        keep.append((ks, kr))
        arr[k].send, arr[k].recv = s, r
        arr[k].n, arr[k].dtype, arr[k].op = int(n), int(dtype), int(op)
    fname = "coll_allreduce_batch_noalloc" if noalloc else "coll_allreduce_batch"
    return _run(fname, (arr, len(calls), int(p), int(flags), _stream(stream)), fname, defer, (arr, keep))


def coll_status_string(status: int) -> str:
    return lib().coll_status_string(int(status)).decode()


def coll_last_hip_error() -> int:
    return lib().coll_last_hip_error()


def coll_version() -> int:
    return lib().coll_version()


def coll_stream_probe(src, dst, nbytes: int, unroll: int = 4, flags: int = 0, sink=None, stream=None,
                      defer: bool = False):
    """Direction-mix bandwidth probe: len(src) read and len(dst) write
    streams of nbytes each, `unroll` vectors per lane per tile (a
    measurement helper, not a collective)."""
    s, ks = _ptr_array(src) if len(src) else (None, None)
    d, kd = _ptr_array(dst) if len(dst) else (None, None)
    return _run("coll_stream_probe", (s, len(src), d, len(dst), int(nbytes), int(unroll), int(flags),
                                      _addr(sink) if sink is not None else None, _stream(stream)),
                "coll_stream_probe", defer, (ks, kd, src, dst, sink))


def coll_set_grid_limit(workgroups_per_cu: int) -> None:
    lib().coll_set_grid_limit(int(workgroups_per_cu))


def coll_finalize() -> None:
    lib().coll_finalize()
