"""Bandwidth accounting for the collectives.

Two views of one run:

* algbw / busbw, the conventions of "集合通信：原语、算法、NCCL 实现与拓扑映射"
  (llm-infra-atlas, hpc/04), section 2.5 table of correction factors:
  AllReduce 2(p-1)/p; ReduceScatter, AllGather and AllToAll (p-1)/p;
  Broadcast and Reduce 1.  The payload B follows the B convention of
  "Collective Communication：AllReduce、AllGather、ReduceScatter 与 All-to-All"
  (charlestar.github.io, notation section): B is the full logical tensor
  (AllReduce in and out B; AllGather in B/p, out B; ReduceScatter in B,
  out B/p); All-to-All uses each rank's send buffer B_local.
* HBM bytes: with all p ranks in one device memory, the minimum traffic of
  an out-of-place call is every input element read once and every output
  element written once, self-copies included (the pages' wire volume
  leaves self-copies out; in one HBM they are real traffic).
"""
from __future__ import annotations

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak


def busbw_factor(coll: str, p: int) -> float:
    if coll == "allreduce":
        return 2.0 * (p - 1) / p
    if coll in ("reduce_scatter", "allgather", "alltoall", "alltoallv"):
        return (p - 1) / p
    if coll in ("broadcast", "reduce"):
        return 1.0
    if coll in ("gather", "scatter"):
        # not in the section 2.5 table: of the root's p*n elements, the
        # root's own block never crosses a link, so (p-1)/p of B moves
        return (p - 1) / p
    raise ValueError(coll)


def payload_bytes(coll: str, p: int, n: int, d: int) -> int:
    """B in bytes.  n is the per-rank count of the C ABI:
    allreduce/reduce/broadcast: n per rank (B = n*d);
    reduce_scatter: recv n per rank (B = p*n*d, the full tensor);
    allgather: send n per rank (B = p*n*d);
    alltoall: n = block elements (B_local = p*n*d);
    gather/scatter: n = elements per rank (B = p*n*d, the root's buffer);
    alltoallv: n = elements each rank sends on average (B_local = n*d).
    """
    if coll in ("allreduce", "reduce", "broadcast", "alltoallv"):
        return n * d
    if coll in ("reduce_scatter", "allgather", "alltoall", "gather", "scatter"):
        return p * n * d
    raise ValueError(coll)


def hbm_bytes(coll: str, p: int, n: int, d: int, algo: str = "ring") -> int:
    """Algorithmic HBM bytes (reads + writes) of one out-of-place call."""
    if coll == "allreduce":
        if algo == "ring_literal":
            # 2(p-1) steps over chunks of n/p: each reduce-scatter step reads
            # two chunks and writes one per rank, each all-gather step reads
            # and writes one chunk per rank.
            return 5 * (p - 1) * n * d
        return 2 * p * n * d
    if coll == "reduce":
        return (p + 1) * n * d
    if coll == "broadcast":
        return (p + 1) * n * d
    if coll == "reduce_scatter":
        return (p * p + p) * n * d
    if coll == "allgather":
        return (p + p * p) * n * d
    if coll == "alltoall":
        return 2 * p * p * n * d
    if coll == "alltoallv":
        return 2 * p * n * d
    if coll in ("gather", "scatter"):
        return 2 * p * n * d
    raise ValueError(coll)


def algbw_gbps(coll: str, p: int, n: int, d: int, seconds: float) -> float:
    return payload_bytes(coll, p, n, d) / seconds / 1e9


def busbw_gbps(coll: str, p: int, n: int, d: int, seconds: float) -> float:
    return algbw_gbps(coll, p, n, d, seconds) * busbw_factor(coll, p)


def hbm_gbps(coll: str, p: int, n: int, d: int, seconds: float, algo: str = "ring") -> float:
    return hbm_bytes(coll, p, n, d, algo) / seconds / 1e9
