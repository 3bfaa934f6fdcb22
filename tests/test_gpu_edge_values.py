"""Reductions on the numeric edge cases, through the C ABI, against the
C++ oracle.

"Collective Communication：AllReduce、AllGather、ReduceScatter 与 All-to-All"
(charlestar.github.io) makes the reduction numerics part of correctness.
The operands here (drawn by inputs.edge_buffers) make int32 sums wrap,
fp32 and bf16 sums run through subnormals, overflow to infinities and land
on bf16 rounding ties, and min/max meet signed zeros, NaN and infinities.

Expected values: the oracle in the schedule's order for floating-point
sums; the ring order for min, max and every int32 operation, which the
library folds in ring order under every schedule (integer sums give the
same bits in any order; min and max do not once NaN or signed zeros meet,
so the schedule argument does not reorder them).  Bit-exact, except that a
NaN produced by an addition only has to be a NaN (IEEE 754 leaves its sign
and payload open).
"""
import numpy as np
import pytest

from gpu_util import BF16, F32, I32, assert_bits_equal, assert_bits_equal_nan, empty, to_dev, to_host
from oracle import native
from collective_communication_primitives_coll_amd import inputs

pytestmark = pytest.mark.gpu

CASES = [("int_wrap", I32), ("subnormal", F32), ("subnormal", BF16), ("overflow", F32), ("overflow", BF16),
         ("ties", BF16), ("zero_nan_inf", F32), ("zero_nan_inf", BF16)]
P_N = [(2, 4099), (3, 7001), (4, 3 * 4096 + 5), (6, 5003), (8, 8 * 1024 + 17), (16, 16 * 1024 + 3)]
OPS = (native.SUM, native.AVG, native.MIN, native.MAX)


@pytest.fixture(scope="module")
def coll():
    import torch
    import collective_communication_primitives_coll_amd as c
    torch.cuda.set_device(0)
    c.lib()
    return c


def sync():
    import torch
    torch.cuda.synchronize()


def _check(got, expect, op, what):
    if op in (native.SUM, native.AVG):
        assert_bits_equal_nan(got, expect, what)
    else:
        assert_bits_equal(got, expect, what)


def _algos(coll, p, dtype):
    out = [(coll.COLL_ALGO_RING, native.ORD_RING)]
    if dtype != BF16:
        out.append((coll.COLL_ALGO_RING_LITERAL, native.ORD_RING))
    if p in (2, 4, 8, 16):
        out += [(coll.COLL_ALGO_RECURSIVE_DOUBLING, native.ORD_RD), (coll.COLL_ALGO_HALVING_DOUBLING, native.ORD_HD),
                (coll.COLL_ALGO_TREE, native.ORD_TREE), (coll.COLL_ALGO_DOUBLE_BINARY_TREE, native.ORD_DBT)]
    return out


@pytest.mark.parametrize("kind,dtype", CASES)
@pytest.mark.parametrize("p,n", P_N)
def test_allreduce_edge_values_every_schedule(coll, kind, dtype, p, n):
    hx = inputs.edge_buffers(p, n, dtype, kind, seed=p)
    send = [to_dev(x, dtype) for x in hx]
    recv = [empty(n, dtype) for _ in range(p)]
    for op in OPS:
        ring = native.allreduce(hx, op, dtype, native.ORD_RING)
        for algo, order in _algos(coll, p, dtype):
            fp_sum = dtype != I32 and op in (native.SUM, native.AVG)
            expect = native.allreduce(hx, op, dtype, order) if fp_sum and order != native.ORD_RING else ring
            coll.coll_allreduce_algo(send, recv, algo, op)
            sync()
            for r in range(p):
                _check(to_host(recv[r], dtype), expect, op, f"{kind} p={p} op={op} algo={algo} rank {r}")


@pytest.mark.parametrize("kind,dtype", CASES)
@pytest.mark.parametrize("p,n", [(2, 2049), (3, 1001), (8, 8192 + 3), (16, 2050), (5, 4099)])
def test_reduce_scatter_and_reduce_edge_values(coll, kind, dtype, p, n):
    hx = inputs.edge_buffers(p, p * n, dtype, kind, seed=10 + p)
    send = [to_dev(x, dtype) for x in hx]
    shard = [empty(n, dtype) for _ in range(p)]
    root_out = empty(p * n, dtype)
    for op in OPS:
        expect = native.reduce_scatter(hx, op, dtype)
        coll.coll_reduce_scatter(send, shard, op)
        sync()
        for r in range(p):
            _check(to_host(shard[r], dtype), expect[r], op, f"RS {kind} p={p} op={op} block {r}")
        coll.coll_reduce(send, root_out, p - 1, op)
        sync()
        _check(to_host(root_out, dtype), native.allreduce(hx, op, dtype), op, f"Reduce {kind} p={p} op={op}")


@pytest.mark.parametrize("p", [3, 8, 16])
def test_batch_edge_values(coll, p):
    rng = np.random.default_rng(p)
    calls, host = [], []
    for k in range(48):
        kind, dtype = CASES[k % len(CASES)]
        n = int(rng.choice([1, p + 1, 777, 4097, 20011]))
        op = OPS[(k // len(CASES)) % len(OPS)]
        hx = inputs.edge_buffers(p, n, dtype, kind, seed=1000 + k)
        calls.append(([to_dev(x, dtype) for x in hx], [empty(n, dtype) for _ in range(p)], n, dtype, op))
        host.append((hx, op, dtype))
    coll.coll_allreduce_batch(calls, p)
    sync()
    for k, ((_, recv, n, dtype, op), (hx, _, _)) in enumerate(zip(calls, host)):
        expect = native.allreduce(hx, op, dtype)
        for r in (0, p - 1):
            _check(to_host(recv[r], dtype), expect, op, f"batch call {k} op {op} rank {r}")


# Sizes past the one-tile-per-workgroup bound with enough tiles per
# workgroup that the walking kernel claims part of them (pooled counters
# for AllReduce at p = 8), so the edge semantics are checked there too.
# Claims start at 8 tiles per workgroup: 2048 tiles for one workgroup per
# CU on 256 CUs.  At p = 8 an AllReduce tile holds 2 vectors per lane of
# 256 lanes and a ReduceScatter tile 4; a vector holds 8 bf16 or 4 others.
def _vec_elems(dtype):
    return 8 if dtype == BF16 else 4


BIG_CASES = [("int_wrap", I32), ("subnormal", F32), ("overflow", BF16), ("zero_nan_inf", F32),
             ("zero_nan_inf", BF16)]


@pytest.mark.parametrize("kind,dtype", BIG_CASES)
def test_allreduce_edge_values_claimed_tiles(coll, kind, dtype):
    te = 2 * 256 * _vec_elems(dtype)
    p, n = 8, 2048 * te + 3 * te // 2 + 37
    hx = inputs.edge_buffers(p, n, dtype, kind, seed=21)
    send = [to_dev(x, dtype) for x in hx]
    recv = [empty(n, dtype) for _ in range(p)]
    for op in OPS:
        for algo, order in ((coll.COLL_ALGO_RING, native.ORD_RING), (coll.COLL_ALGO_RECURSIVE_DOUBLING, native.ORD_RD)):
            fp_sum = dtype != I32 and op in (native.SUM, native.AVG)
            expect = native.allreduce(hx, op, dtype, order if fp_sum else native.ORD_RING)
            coll.coll_allreduce_algo(send, recv, algo, op)
            sync()
            for r in range(p):
                _check(to_host(recv[r], dtype), expect, op, f"{kind} p={p} n={n} op={op} algo={algo} rank {r}")


@pytest.mark.parametrize("kind,dtype", BIG_CASES)
def test_reduce_scatter_and_reduce_edge_values_claimed_tiles(coll, kind, dtype):
    te = 4 * 256 * _vec_elems(dtype)
    p, n = 8, 256 * te + 3 * te // 2 + 37  # 8 chunks of n elements
    hx = inputs.edge_buffers(p, p * n, dtype, kind, seed=22)
    send = [to_dev(x, dtype) for x in hx]
    shard = [empty(n, dtype) for _ in range(p)]
    root_out = empty(p * n, dtype)
    for op in OPS:
        expect = native.reduce_scatter(hx, op, dtype)
        coll.coll_reduce_scatter(send, shard, op)
        sync()
        for r in range(p):
            _check(to_host(shard[r], dtype), expect[r], op, f"RS {kind} p={p} n={n} op={op} block {r}")
        coll.coll_reduce(send, root_out, 3, op)
        sync()
        _check(to_host(root_out, dtype), native.allreduce(hx, op, dtype), op, f"Reduce {kind} p={p} n={n} op={op}")
