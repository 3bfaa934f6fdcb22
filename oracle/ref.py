"""CPU oracle for the collective primitives.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this file:
only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP path; the two meet only at the seeded input
generators, which hold none of the arithmetic below.

Everything here is plain NumPy, written to be checked by eye against the
definitions on the pages it follows:

* "集合通信：原语、算法、NCCL 实现与拓扑映射" (llm-infra-atlas, hpc/04):
  notation p, [n], elementwise + in {sum, min, max} (chapter preamble);
  primitive table (section 0); Broadcast 1.1, AllGather 1.2, Reduce 1.3
  with its worked example, AllReduce 1.4, ReduceScatter 1.5, AllToAll 1.6,
  the forward/backward duality table 1.7 and the Gather/Scatter note
  after 1.6; ring all-reduce 2.2;
  recursive doubling and halving-doubling 2.3.
* "Collective Communication：AllReduce、AllGather、ReduceScatter 与 All-to-All"
  (charlestar.github.io): ragged All-to-All (counts c_ij, prefix-sum
  offsets), B convention for volumes, numerics of reduction order.
* "详解分布式训练8大集合通信原语：从Send/Recv到All2All" (bjdmk.com.cn):
  Scatter (section 3.3) and Gather (section 4.3).

Readings taken where the pages are silent or inconsistent:

1. Ring order.  The p=4 ring trace in section 2.2 of the hpc/04 page
   contradicts itself about which chunk a rank sends first.  The reading
   used: chunk c starts at rank c+1 and its partial travels c+1, c+2, ...,
   ending on rank c, so that ReduceScatter's block c ends on rank c as
   section 1.5 requires.  Element i of chunk c is therefore reduced in the
   order x_{c+1}, x_{c+2}, ..., x_{c+p-1}, x_c (indices mod p), left fold.
2. Chunking when p does not divide n: q = ceil(n/p), chunk(i) = i // q;
   trailing chunks may be short or empty.
3. bf16: widen exactly to fp32, fold in fp32 (IEEE add, round to nearest
   even), narrow once with round-to-nearest-even.
4. min/max: compare-select, acc = v if v < acc (min) / v > acc (max), in
   fp32 for bf16.  int32 sum wraps modulo 2^32.  AVG: the schedule's sum,
   then one IEEE fp32 division by p (int32: C division, truncating toward
   zero).  PreMulSum: each operand times its rank's fp32 scale, every
   product rounded on its own, then the sum.
5. Reduce uses the AllReduce chunking, so Reduce then Broadcast equals
   AllReduce bit for bit.
6. Alltoallv: recv counts are the columns of the send-count matrix; the
   receive buffer of rank j holds the blocks from sources 0..p-1 in source
   order, packed.
7. Halving-doubling: the page gives message sizes per step, not partner
   distances; the reduce-scatter phase pairs ranks at distance p/2, then
   p/4, ..., 1 (see halving_doubling_simulated).
8. MoE pack/combine: the page lists the steps, not the formats.  Packing
   orders assignments by destination rank, stable in assignment index;
   the combine accumulates in fp32 in slot order with products and sums
   rounded separately (see moe_pack, moe_combine).  The direct dispatch
   and combine (moe_dispatch_direct, moe_combine_direct) give the same
   receive layout and outputs without the staging copies.
"""
from __future__ import annotations

import numpy as np

SUM, MIN, MAX, AVG = 0, 1, 2, 3
F32, BF16, I32 = 0, 1, 2


# ----------------------------------------------------------------------------
# bf16 <-> fp32 (IEEE-754 binary16-brain: sign, 8-bit exponent, 7-bit fraction)
# ----------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening: the bf16 pattern is the upper half of the fp32 pattern."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Narrow fp32 to bf16 with round-to-nearest, ties-to-even.

    The kept part is the upper 16 bits of the fp32 pattern; the dropped
    part is the lower 16 bits.  Round up when the dropped part exceeds half
    an ulp (0x8000), or equals it and the kept part is odd.  Carry out of
    the fraction moves into the exponent, which gives the right result up
    to and including overflow to infinity.  NaN maps to a quiet NaN with
    the same sign.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    kept = u >> np.uint32(16)
    dropped = u & np.uint32(0xFFFF)
    up = (dropped > 0x8000) | ((dropped == 0x8000) & ((kept & np.uint32(1)) == 1))
    out = (kept + up.astype(np.uint32)).astype(np.uint32)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    out = np.where(nan, (kept & np.uint32(0x8000)) | np.uint32(0x7FC0), out)
    return out.astype(np.uint16)


# ----------------------------------------------------------------------------
# The reduction: a left fold in a given rank order
# ----------------------------------------------------------------------------

def ring_order(c: int, p: int) -> list[int]:
    """Ranks visited by chunk c's partial: c+1, c+2, ..., c (mod p)."""
    return [(c + k) % p for k in range(1, p + 1)]


def _widen(v: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == BF16:
        return bf16_to_f32(v)
    if dtype == F32:
        return np.asarray(v, dtype=np.float32)
    if dtype == I32:
        return np.asarray(v, dtype=np.int32)
    raise ValueError(dtype)


def _combine(acc: np.ndarray, v: np.ndarray, op: int) -> np.ndarray:
    if op in (SUM, AVG):
        with np.errstate(over="ignore", invalid="ignore"):
            return acc + v          # fp32 IEEE add (RNE) / int32 add mod 2^32
    if op == MIN:
        return np.where(v < acc, v, acc)
    if op == MAX:
        return np.where(v > acc, v, acc)
    raise ValueError(op)


def _finish(acc: np.ndarray, op: int, dtype: int, p: int) -> np.ndarray:
    """After the fold: AVG divides the sum by p (one IEEE fp32 division;
    int32: C division of the wrapped sum, truncating toward zero), then
    bf16 is narrowed once."""
    if op == AVG:
        if dtype == I32:
            a = np.asarray(acc).astype(np.int64)
            acc = (np.sign(a) * (np.abs(a) // p)).astype(np.int32)
        else:
            acc = (np.asarray(acc, dtype=np.float32) / np.float32(p)).astype(np.float32)
    if dtype == BF16:
        return f32_to_bf16_rne(acc)
    return acc


def fold(vals_in_order: list[np.ndarray], op: int, dtype: int, scales=None) -> np.ndarray:
    """acc = v0; acc = acc (+) v1; ...; then _finish.

    With scales (PreMulSum, sum only) operand k is first multiplied by
    scales[k] in fp32, each product rounded on its own."""
    def operand(k):
        w = _widen(vals_in_order[k], dtype)
        if scales is not None:
            w = (np.float32(scales[k]) * w.astype(np.float32)).astype(np.float32)
        return w
    acc = operand(0).copy()
    for k in range(1, len(vals_in_order)):
        acc = _combine(acc, operand(k), op)
    return _finish(acc, op, dtype, len(vals_in_order))


def reduce_elements(cols: np.ndarray, chunk: np.ndarray, op: int, dtype: int, scales=None) -> np.ndarray:
    """Reduce selected elements.

    cols[r, e] is rank r's value of element e; chunk[e] is the chunk that
    element belongs to.  Element e is folded in ring_order(chunk[e], p).
    scales[r] (PreMulSum) multiplies rank r's operand.  Used both for whole
    buffers and for sampled elements of large ones.
    """
    cols = np.asarray(cols)
    p, m = cols.shape
    chunk = np.asarray(chunk, dtype=np.int64)
    e = np.arange(m)
    ranks = [(chunk + k) % p for k in range(1, p + 1)]
    ordered = [cols[r, e] for r in ranks]
    if scales is None:
        return fold(ordered, op, dtype)
    sc = np.asarray(scales, dtype=np.float32)
    return fold(ordered, op, dtype, scales=[sc[r] for r in ranks])


def chunk_len(n: int, p: int) -> int:
    """q = ceil(n / p) elements per chunk."""
    return -(-n // p) if n > 0 else 0


def chunk_of(idx: np.ndarray, n: int, p: int) -> np.ndarray:
    q = chunk_len(n, p)
    return np.asarray(idx, dtype=np.int64) // max(q, 1)


# ----------------------------------------------------------------------------
# The primitives (section 0 primitive table of the hpc/04 page)
# ----------------------------------------------------------------------------

def allreduce(xs: list[np.ndarray], op: int, dtype: int, scales=None) -> list[np.ndarray]:
    """out_r[i] = (+)_{r'} x_{r'}[i] on every rank r (section 1.4).

    op AVG: the sum divided by p, the average that the page notes older
    NCCL lacked (section 1.4, sum then divide by the world size).
    scales: PreMulSum, out = sum_r scales[r] * x_r ("Collective
    Communication" page: NCCL's constrained custom reduction)."""
    p = len(xs)
    n = len(xs[0])
    if n == 0:
        return [xs[0][:0].copy() for _ in range(p)]
    res = reduce_elements(np.stack(xs), chunk_of(np.arange(n), n, p), op, dtype, scales)
    return [res.copy() for _ in range(p)]


def reduce(xs: list[np.ndarray], op: int, dtype: int, root: int) -> np.ndarray:
    """Only the root receives (+)_r x_r (section 1.3).  Same order as allreduce."""
    assert 0 <= root < len(xs)
    return allreduce(xs, op, dtype)[root]


def broadcast(x_root: np.ndarray, p: int) -> list[np.ndarray]:
    """Every rank receives the root's [n] (section 1.1)."""
    return [np.array(x_root, copy=True) for _ in range(p)]


def reduce_scatter(xs: list[np.ndarray], op: int, dtype: int, scales=None) -> list[np.ndarray]:
    """Each rank holds [p*n]; rank r keeps block r of the reduction (section 1.5).

    Block r is reduced in ring_order(r, p); scales as in allreduce.
    """
    p = len(xs)
    total = len(xs[0])
    assert total % p == 0
    n = total // p
    out = []
    for r in range(p):
        order = ring_order(r, p)
        blk = [xs[k][r * n:(r + 1) * n] for k in order]
        sc = None if scales is None else [scales[k] for k in order]
        out.append(fold(blk, op, dtype, sc) if n > 0 else xs[0][:0].copy())
    return out


def allgather(xs: list[np.ndarray]) -> list[np.ndarray]:
    """Every rank receives [x_0 | x_1 | ... | x_{p-1}] in rank order (section 1.2)."""
    cat = np.concatenate(xs)
    return [cat.copy() for _ in xs]


def gather(xs: list[np.ndarray], root: int) -> np.ndarray:
    """Only the root receives [x_0 | x_1 | ... | x_{p-1}] in rank order:
    AllGather with a single receiver ("详解分布式训练8大集合通信原语" page,
    section 4.3; the hpc/04 page's note after section 1.6)."""
    assert 0 <= root < len(xs)
    return np.concatenate(xs)


def scatter(x_root: np.ndarray, p: int, root: int) -> list[np.ndarray]:
    """The root's [p*n] is cut into p blocks of n; rank r receives block r
    (the same page, section 3.3: every rank gets one slice of the whole)."""
    assert 0 <= root < p
    total = len(x_root)
    assert total % p == 0
    n = total // p
    return [np.array(x_root[r * n:(r + 1) * n], copy=True) for r in range(p)]


def alltoall(xs: list[np.ndarray]) -> list[np.ndarray]:
    """recv[j] block i = send[i] block j: a transpose of the block matrix (section 1.6)."""
    p = len(xs)
    m = len(xs[0]) // p
    return [np.concatenate([xs[i][j * m:(j + 1) * m] for i in range(p)]) for j in range(p)]


def alltoallv(xs: list[np.ndarray], counts: np.ndarray) -> list[np.ndarray]:
    """Variable-split All-to-All.

    counts[i][j] elements go from source i to destination j.  Send offsets
    are the exclusive prefix sums along each row; destination j packs the
    blocks from sources 0..p-1 in source order.
    """
    counts = np.asarray(counts, dtype=np.int64)
    p = len(xs)
    send_off = np.zeros((p, p), dtype=np.int64)
    for i in range(p):
        for j in range(1, p):
            send_off[i, j] = send_off[i, j - 1] + counts[i, j - 1]
    out = []
    for j in range(p):
        parts = [xs[i][send_off[i, j]:send_off[i, j] + counts[i, j]] for i in range(p)]
        out.append(np.concatenate(parts) if parts else xs[0][:0].copy())
    return out


def alltoallv_recv_counts(counts: np.ndarray) -> np.ndarray:
    """Elements each destination receives: the column sums of the count matrix."""
    return np.asarray(counts, dtype=np.int64).sum(axis=0)


# ----------------------------------------------------------------------------
# MoE dispatch and combine around the ragged exchange ("Collective
# Communication" page: Ragged All-to-All flow; Expert Parallel section)
# ----------------------------------------------------------------------------

def moe_pack(tokens: np.ndarray, dest: np.ndarray, k: int, hidden: int, p: int):
    """One rank's dispatch pack.

    tokens: [T*hidden] (row t = token t); dest[a] = destination rank of
    assignment a = t*k + s (token t, slot s).  Assignments are ordered by
    destination rank, stable in a (the page's "count assignments per
    destination -> prefix-sum offsets -> pack/permute payload").

    Returns (counts, pos, packed): counts[j] = hidden * (assignments to j),
    in elements as the ragged exchange takes them; pos[a] = packed row of
    assignment a; packed row pos[a] = token a // k.
    """
    dest = np.asarray(dest, dtype=np.int64)
    A = len(dest)
    assert np.all((dest >= 0) & (dest < p))
    rows = np.zeros(p, dtype=np.int64)
    for a in range(A):
        rows[dest[a]] += 1
    offset = np.zeros(p, dtype=np.int64)
    for j in range(1, p):
        offset[j] = offset[j - 1] + rows[j - 1]
    cursor = offset.copy()
    pos = np.zeros(A, dtype=np.int64)
    for a in range(A):
        pos[a] = cursor[dest[a]]
        cursor[dest[a]] += 1
    packed = np.zeros(A * hidden, dtype=np.asarray(tokens).dtype)
    for a in range(A):
        t = a // k
        packed[pos[a] * hidden:(pos[a] + 1) * hidden] = tokens[t * hidden:(t + 1) * hidden]
    return rows * hidden, pos, packed


def moe_combine(back: np.ndarray, pos: np.ndarray, weights: np.ndarray, k: int, hidden: int, dtype: int,
                residual: np.ndarray | None = None) -> np.ndarray:
    """One rank's weighted combine after the reverse exchange.

    back holds the rows returned in packed order; for token t,
    out[t] = r[t] + w[t*k] * y_0 + w[t*k+1] * y_1 + ... with y_s = row
    pos[t*k + s] of back and r the residual (or +0 without one): the page's
    "weighted combine + residual".  Reading: fp32 accumulation in slot
    order, each product and each sum rounded to fp32 separately (no fused
    multiply-add), bf16 narrowed once at the end.
    """
    A = len(pos)
    T = A // k
    w = np.asarray(weights, dtype=np.float32)
    rows = _widen(back, dtype).reshape(A, hidden)
    if residual is not None:
        acc = _widen(residual, dtype).reshape(T, hidden).copy()
    else:
        acc = np.zeros((T, hidden), dtype=np.float32)
    for s in range(k):
        a = np.arange(T) * k + s
        prod = (w[a][:, None] * rows[pos[a]]).astype(np.float32)
        acc = (acc + prod).astype(np.float32)
    acc = acc.reshape(-1)
    return f32_to_bf16_rne(acc) if dtype == BF16 else acc


def moe_dispatch_direct(tokens: list[np.ndarray], dests: list[np.ndarray], k: int, hidden: int):
    """Dispatch without a staging copy: every assignment's token row lands
    directly in its destination's receive buffer.

    recv[j] holds, for source ranks i = 0, 1, ..., p-1 in turn, the rows of
    rank i's assignments to j in assignment order: the same receive layout
    as pack followed by the ragged exchange (the "Collective Communication"
    page's flow, with the pack and the exchange writing one buffer; the
    load/store peer access of the hpc/04 page, section 3.9).  slot[i][a] is
    the row of assignment a inside recv[dest[i][a]].  counts[i][j] =
    hidden * (assignments of rank i to rank j), as moe_pack."""
    p = len(tokens)
    recv_rows = [[] for _ in range(p)]
    slots = []
    counts = np.zeros((p, p), dtype=np.int64)
    for i in range(p):
        d = np.asarray(dests[i], dtype=np.int64)
        slot = np.zeros(len(d), dtype=np.int64)
        for j in range(p):
            for a in range(len(d)):
                if d[a] == j:
                    slot[a] = len(recv_rows[j])
                    t = a // k
                    recv_rows[j].append(np.asarray(tokens[i])[t * hidden:(t + 1) * hidden])
                    counts[i, j] += hidden
        slots.append(slot)
    dt = np.asarray(tokens[0]).dtype
    recv = [np.concatenate(r) if r else np.zeros(0, dtype=dt) for r in recv_rows]
    return counts, slots, recv


def moe_combine_direct(ys: list[np.ndarray], dest: np.ndarray, slot: np.ndarray, weights: np.ndarray, k: int,
                       hidden: int, dtype: int, residual: np.ndarray | None = None) -> np.ndarray:
    """One rank's weighted combine reading every expert output where it
    lies: y_s = row slot[t*k+s] of ys[dest[t*k+s]].  Same arithmetic as
    moe_combine (fp32, slot order, products and sums rounded separately)."""
    A = len(dest)
    rows = [np.asarray(ys[int(dest[a])])[int(slot[a]) * hidden:(int(slot[a]) + 1) * hidden] for a in range(A)]
    back = np.concatenate(rows) if rows else np.zeros(0, dtype=np.asarray(ys[0]).dtype)
    return moe_combine(back, np.arange(A), weights, k, hidden, dtype, residual)


# ----------------------------------------------------------------------------
# The ring all-reduce of section 2.2, simulated step by step
# ----------------------------------------------------------------------------

def ring_allreduce_simulated(xs: list[np.ndarray], op: int, dtype: int,
                             return_after_rs: bool = False):
    """2(p-1) neighbour steps over per-rank buffers.

    Each rank's buffer is cut into p chunks of q = ceil(n/p) elements.
    Reduce-scatter phase, step s = 1..p-1: every rank X sends its current
    copy of chunk (X - s) mod p to rank X+1, which combines it with its own
    copy (received partial on the left).  All-gather phase, step t =
    1..p-1: every rank X sends chunk (X + 1 - t) mod p, which it holds in
    final form, to rank X+1, which stores it.  Sends of a step read the
    buffers as they were before that step.

    Partials stay in fp32 for bf16 and are narrowed once at the end.
    With return_after_rs the per-rank buffers after the first phase are
    returned (widened), so tests can check where each reduced chunk lands.
    """
    p = len(xs)
    n = len(xs[0])
    q = chunk_len(n, p)
    buf = [_widen(x, dtype).copy() for x in xs]

    def sl(c):
        return slice(min(c * q, n), min((c + 1) * q, n))

    for s in range(1, p):
        snap = [b.copy() for b in buf]
        for x in range(p):
            c = (x - s) % p
            dst = (x + 1) % p
            buf[dst][sl(c)] = _combine(snap[x][sl(c)], buf[dst][sl(c)], op)
    if return_after_rs:
        return buf
    for t in range(1, p):
        snap = [b.copy() for b in buf]
        for x in range(p):
            c = (x + 1 - t) % p
            dst = (x + 1) % p
            buf[dst][sl(c)] = snap[x][sl(c)]
    return [_finish(b, op, dtype, p) for b in buf]


# ----------------------------------------------------------------------------
# Recursive doubling and halving-doubling (section 2.3 of the hpc/04 page)
# ----------------------------------------------------------------------------

def _is_pow2(p: int) -> bool:
    return p >= 1 and (p & (p - 1)) == 0


def recursive_doubling_simulated(xs: list[np.ndarray], op: int, dtype: int) -> list[np.ndarray]:
    """log2(p) steps; at step k every rank exchanges its whole vector with
    the peer at distance 2^k (rank XOR 2^k) and both keep the combination.

    The lower rank's partial is the left operand.  Partials stay in fp32 for
    bf16 and are narrowed once at the end.  p must be a power of two.
    """
    p = len(xs)
    assert _is_pow2(p)
    buf = [_widen(x, dtype).copy() for x in xs]
    d = 1
    while d < p:
        snap = [b.copy() for b in buf]
        for r in range(p):
            lo, hi = min(r, r ^ d), max(r, r ^ d)
            buf[r] = _combine(snap[lo], snap[hi], op)
        d *= 2
    return [_finish(b, op, dtype, p) for b in buf]


def halving_doubling_simulated(xs: list[np.ndarray], op: int, dtype: int) -> list[np.ndarray]:
    """Reduce-scatter by recursive halving, then all-gather by recursive
    doubling.

    Reading of the page (it gives the message sizes, not the partner
    distances): the halving phase pairs ranks at distance p/2, p/4, ..., 1
    (Rabenseifner's order).  At each step a rank splits the range it holds
    in two, keeps the lower half if its distance bit is 0 and the upper
    half otherwise, and combines its partial of the kept half with the
    peer's partial of the same half (lower rank's partial on the left).
    After log2(p) steps rank r holds block r of the result; the doubling
    phase copies the blocks back to every rank (distances 1, 2, ..., p/2).
    Blocks are q = ceil(n/p) elements; p must be a power of two.
    """
    p = len(xs)
    assert _is_pow2(p)
    n = len(xs[0])
    q = chunk_len(n, p)
    buf = [_widen(x, dtype).copy() for x in xs]
    blk = [(0, p) for _ in range(p)]          # block range [b0, b1) each rank holds
    d = p // 2
    while d >= 1:
        snap = [b.copy() for b in buf]
        new_blk = []
        for r in range(p):
            b0, b1 = blk[r]
            mid = (b0 + b1) // 2
            keep = (b0, mid) if (r & d) == 0 else (mid, b1)
            sl = slice(min(keep[0] * q, n), min(keep[1] * q, n))
            lo, hi = min(r, r ^ d), max(r, r ^ d)
            buf[r][sl] = _combine(snap[lo][sl], snap[hi][sl], op)
            new_blk.append(keep)
        blk = new_blk
        d //= 2
    assert all(blk[r] == (r, r + 1) for r in range(p))
    d = 1
    while d < p:
        snap = [b.copy() for b in buf]
        new_blk = []
        for r in range(p):
            (a0, a1), (c0, c1) = blk[r], blk[r ^ d]
            sl = slice(min(c0 * q, n), min(c1 * q, n))
            buf[r][sl] = snap[r ^ d][sl]
            new_blk.append((min(a0, c0), max(a1, c1)))
        blk = new_blk
        d *= 2
    return [_finish(b, op, dtype, p) for b in buf]


# ----------------------------------------------------------------------------
# Tree AllReduce and the double binary tree (hpc/04 page, sections 2.3 and
# 2.4; the "Collective Communication" page's Tree AllReduce: reduce up the
# tree to the root, then broadcast down)
# ----------------------------------------------------------------------------

def tree_reduce_to_root(vals: list[np.ndarray], ranks: list[int], op: int, dtype: int):
    """Binary tree in heap order over the listed ranks: node v (rank
    ranks[v]) has children 2v+1 and 2v+2.  Each node waits for its
    children's partials and sends partial(v) = (x_v (+) partial(2v+1))
    (+) partial(2v+2) to its parent (reading: own value first, then the
    left subtree, then the right).  Returns the root's partial, widened."""
    p = len(ranks)
    partial = [None] * p
    for v in range(p - 1, -1, -1):          # leaves first: every child is done before its parent
        acc = _widen(vals[ranks[v]], dtype).copy()
        for c in (2 * v + 1, 2 * v + 2):
            if c < p:
                acc = _combine(acc, partial[c], op)
        partial[v] = acc
    return partial[0]


def tree_allreduce_simulated(xs: list[np.ndarray], op: int, dtype: int) -> list[np.ndarray]:
    """Tree AllReduce: reduce up the heap-ordered binary tree rooted at rank
    0, then broadcast the root's result down the same tree."""
    p = len(xs)
    root = _finish(tree_reduce_to_root(xs, list(range(p)), op, dtype), op, dtype, p)
    return [root.copy() for _ in range(p)]


def double_binary_tree_simulated(xs: list[np.ndarray], op: int, dtype: int) -> list[np.ndarray]:
    """Double binary tree (section 2.4): two complementary trees, tree A the
    heap order over ranks 0, 1, ..., p-1 and tree B its mirror (node v on
    rank p-1-v), so every rank is inner in one tree and a leaf in the
    other.  Reading of how the data is split between them: the AllReduce
    chunks c < p/2 (chunk c = elements [c*q, (c+1)*q), q = ceil(n/p)) go
    through tree A, the others through tree B; each tree reduces its chunks
    to its root and broadcasts them back."""
    p = len(xs)
    n = len(xs[0])
    if n == 0:
        return [xs[0][:0].copy() for _ in range(p)]
    q = chunk_len(n, p)
    out_parts = []
    for c in range(p):
        lo, hi = min(n, c * q), min(n, (c + 1) * q)
        if lo == hi:
            continue
        ranks = list(range(p)) if c < p // 2 else list(range(p - 1, -1, -1))
        part = tree_reduce_to_root([x[lo:hi] for x in xs], ranks, op, dtype)
        out_parts.append(_finish(part, op, dtype, p))
    res = np.concatenate(out_parts)
    return [res.copy() for _ in range(p)]


def fold_tree(vals: list[np.ndarray], op: int, dtype: int, first_stride: str) -> np.ndarray:
    """Balanced pairwise tree over ranks 0..p-1 (p a power of two).

    first_stride "low": pairs (0,1), (2,3), ... first, then pairs of pairs
    (the recursive-doubling order); "high": pairs (k, k + p/2) first, then
    (k, k + p/4), ... (the halving-doubling order).  Operands are the
    values of ranks in rank order (not rotated); narrowed once for bf16.
    """
    p = len(vals)
    assert _is_pow2(p)
    a = [_widen(v, dtype).copy() for v in vals]
    if first_stride == "low":
        s = 1
        while s < p:
            for k in range(0, p, 2 * s):
                a[k] = _combine(a[k], a[k + s], op)
            s *= 2
    else:
        s = p // 2
        while s >= 1:
            for k in range(s):
                a[k] = _combine(a[k], a[k + s], op)
            s //= 2
    return _finish(a[0], op, dtype, p)


# ----------------------------------------------------------------------------
# Batched small AllReduce: each call independently
# ----------------------------------------------------------------------------

def allreduce_batch(calls: list[tuple[list[np.ndarray], int, int]]) -> list[np.ndarray]:
    """calls: (per-rank inputs, op, dtype).  Returns the reduced vector per call."""
    return [allreduce(xs, op, dt)[0] for xs, op, dt in calls]
