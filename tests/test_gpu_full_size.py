"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (same entry points, default grids, same seeded inputs).

The oracle cannot reduce gigabytes in seconds, so reductions are checked on
sampled elements it computes one by one (random positions plus every tile
and chunk boundary nearby), and copies are checked whole against the
oracle's definitions.  Properties that hold at any size (every rank of an
AllReduce holds the same bits; AllGather is the rank-order concatenation of
what ReduceScatter produced) are checked on the device over every element.
"""
import numpy as np
import pytest

from gpu_util import BF16, F32, I32, assert_bf16_within_ulp, assert_bits_equal, assert_fp32_close, to_host
from oracle import ref
from collective_communication_primitives_coll_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import collective_communication_primitives_coll_amd as c
    torch.cuda.set_device(0)
    c.lib()
    return torch, c


def dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def sample_positions(n, seed, tile, extra=()):
    """Random positions plus the neighbourhood of every tile boundary among
    the first and last few tiles, and of the given extra boundaries."""
    rng = np.random.default_rng(seed)
    pos = set(rng.integers(0, n, 20000).tolist())
    for b in list(range(0, min(n, 4 * tile) + 1, tile)) + list(range(max(0, n - 3 * tile), n + 1, tile)) + list(extra):
        for d in (-2, -1, 0, 1, 2):
            if 0 <= b + d < n:
                pos.add(b + d)
    pos.update({0, n - 1})
    return np.array(sorted(pos), dtype=np.int64)


def gather_host(torch, t, idx, dtype):
    """t[idx] copied to the host (bit patterns for bf16)."""
    sel = t[torch.from_numpy(idx).cuda()]
    return to_host(sel, dtype)


def test_zero_rs_ag_full_size(env):
    """ReduceScatter (sum) then AllGather, p=8, 2^26 bf16 per rank ~ N(0, 1e-3)."""
    torch, coll = env
    p, total = 8, 1 << 26
    n = total // p
    hx = inputs.rank_buffers(inputs.WL_ZERO_RS_AG, p, total, inputs.BF16, dist="normal", sigma=1e-3)
    send = [dev(torch, x) for x in hx]
    shard = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    full = [torch.empty(total, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    coll.coll_reduce_scatter(send, shard, coll.COLL_SUM)
    coll.coll_allgather(shard, full)
    torch.cuda.synchronize()
    stacked = np.stack(hx)
    tile = 4 * 256 * 8   # ReduceScatter tile of bf16 at p=8: 4 vectors per lane
    for r in range(p):
        j = sample_positions(n, 1000 + r, tile)
        cols = stacked[:, r * n + j]
        expect = ref.reduce_elements(cols, np.full(len(j), r), ref.SUM, ref.BF16)
        got = gather_host(torch, shard[r], j, BF16)
        assert_bits_equal(got, expect, f"RS full size, block {r}")
    # AllGather: every rank holds the rank-order concatenation of the shards
    for r in range(p):
        for s in range(p):
            assert torch.equal(full[r][s * n:(s + 1) * n].view(torch.int16), shard[s].view(torch.int16)), \
                f"AG full size rank {r} block {s}"


def test_dp_allreduce_full_size(env):
    """AllReduce sum, p=8, 2^26 fp32 per rank ~ N(0,1): fused ring, recursive
    doubling, halving-doubling, the tree, the double binary tree and the
    literal 14-step ring, each bit-exact
    against the oracle's order for that schedule; the recursive-doubling
    result is also held to 1e-5 * sum|x| of the ring order."""
    torch, coll = env
    p, n = 8, 1 << 26
    hx = inputs.rank_buffers(inputs.WL_DP_RING_AR, p, n, inputs.F32, dist="normal")
    send = [dev(torch, x) for x in hx]
    recv = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(p)]
    stacked = np.stack(hx)
    q = -(-n // p)
    j = sample_positions(n, 7, 2 * 256 * 4, extra=[c * q for c in range(p)])
    cols = stacked[:, j]
    expect = ref.reduce_elements(cols, ref.chunk_of(j, n, p), ref.SUM, ref.F32)
    abs_sum = np.sum(np.abs(cols.astype(np.float64)), axis=0)
    per_rank = [cols[r] for r in range(p)]
    tree_a = ref.tree_reduce_to_root(per_rank, list(range(p)), ref.SUM, ref.F32)
    tree_b = ref.tree_reduce_to_root(per_rank, list(range(p - 1, -1, -1)), ref.SUM, ref.F32)
    trees = {coll.COLL_ALGO_RECURSIVE_DOUBLING: ref.fold_tree(per_rank, ref.SUM, ref.F32, "low"),
             coll.COLL_ALGO_HALVING_DOUBLING: ref.fold_tree(per_rank, ref.SUM, ref.F32, "high"),
             coll.COLL_ALGO_TREE: tree_a,
             coll.COLL_ALGO_DOUBLE_BINARY_TREE: np.where(ref.chunk_of(j, n, p) < p // 2, tree_a, tree_b)}
    for algo in (coll.COLL_ALGO_RING, coll.COLL_ALGO_RECURSIVE_DOUBLING, coll.COLL_ALGO_HALVING_DOUBLING,
                 coll.COLL_ALGO_TREE, coll.COLL_ALGO_DOUBLE_BINARY_TREE, coll.COLL_ALGO_RING_LITERAL):
        for t in recv:
            t.fill_(float("nan"))
        coll.coll_allreduce_algo(send, recv, algo, coll.COLL_SUM)
        torch.cuda.synchronize()
        for r in range(1, p):
            assert torch.equal(recv[r].view(torch.int32), recv[0].view(torch.int32)), f"algo {algo}: rank {r} differs"
        got = gather_host(torch, recv[0], j, F32)
        assert_bits_equal(got, trees.get(algo, expect), f"algo {algo} full size")
        if algo == coll.COLL_ALGO_RECURSIVE_DOUBLING:
            assert_fp32_close(got, expect, abs_sum, 1e-5, "recursive doubling vs ring order")


def test_small_allreduce_full_size(env):
    """AllReduce p=4, 2^20 per rank: fp32 sum, int32 min and max; whole arrays."""
    torch, coll = env
    p, n = 4, 1 << 20
    for dt, op in ((inputs.F32, ref.SUM), (inputs.I32, ref.MIN), (inputs.I32, ref.MAX)):
        hx = inputs.rank_buffers(inputs.WL_AR_SMALL, p, n, dt)
        send = [dev(torch, x) for x in hx]
        recv = [torch.empty_like(s) for s in send]
        coll.coll_allreduce(send, recv, op)
        torch.cuda.synchronize()
        expect = ref.allreduce(hx, op, dt)
        for r in range(p):
            assert_bits_equal(to_host(recv[r], dt), expect[r], f"AR p=4 dt={dt} op={op} rank {r}")


def test_moe_alltoall_full_size(env):
    """All-to-All and Alltoallv, p=8, 4096 x 7168 bf16 per rank; whole arrays."""
    torch, coll = env
    p, tokens, hidden = 8, 4096, 7168
    per = tokens * hidden
    hx = inputs.rank_buffers(inputs.WL_MOE_A2A, p, per, inputs.BF16, dist="normal")
    send = [dev(torch, x) for x in hx]
    recv = [torch.empty(per, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    coll.coll_alltoall(send, recv, per // p)
    torch.cuda.synchronize()
    expect = ref.alltoall(hx)
    for jr in range(p):
        assert_bits_equal(to_host(recv[jr], BF16), expect[jr], f"A2A full size dest {jr}")
    for r in recv:
        r.zero_()
    coll.coll_alltoall_algo(send, recv, coll.COLL_A2A_LDS_STAGED, per // p)
    torch.cuda.synchronize()
    for jr in range(p):
        assert_bits_equal(to_host(recv[jr], BF16), expect[jr], f"A2A LDS-staged full size dest {jr}")
    del recv, expect
    counts = inputs.moe_token_counts(p, tokens) * hidden
    cols = counts.sum(axis=0)
    recv = [torch.empty(int(c), dtype=torch.bfloat16, device="cuda") for c in cols]
    cdev = torch.from_numpy(counts.reshape(-1).copy()).cuda()
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    coll.coll_alltoallv(send, recv, cdev, status_dev=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    expect = ref.alltoallv(hx, counts)
    for jr in range(p):
        assert_bits_equal(to_host(recv[jr], BF16), expect[jr], f"A2Av full size dest {jr}")


def test_small_batch_full_plan(env):
    """The 10,000-call batched AllReduce plan at p=16 in one launch; a seeded
    sample of calls (plus the first and last) checked whole."""
    torch, coll = env
    p = 16
    plan, out_elems = inputs.small_batch_plan(10000)
    pf, pi = inputs.small_batch_pools(p)
    dpf = [dev(torch, x) for x in pf]
    dpi = [dev(torch, x) for x in pi]
    outs = [torch.empty(out_elems, dtype=torch.int32, device="cuda") for _ in range(p)]
    bf = [t.data_ptr() for t in dpf]
    bi = [t.data_ptr() for t in dpi]
    bo = [t.data_ptr() for t in outs]
    calls = []
    for c in plan:
        src = bf if c.dtype == inputs.F32 else bi
        calls.append(([b + 4 * c.src_off for b in src], [b + 4 * c.dst_off for b in bo], c.n, c.dtype, c.op))
    coll.coll_allreduce_batch(calls, p)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    pick = sorted(set(rng.choice(len(plan), 150, replace=False).tolist()) | {0, len(plan) - 1})
    for k in pick:
        c = plan[k]
        pool = pf if c.dtype == inputs.F32 else pi
        xs = [pool[r][c.src_off:c.src_off + c.n] for r in range(p)]
        expect = ref.allreduce(xs, c.op, c.dtype)
        for r in (0, 7, 15):
            got = outs[r][c.dst_off:c.dst_off + c.n].cpu().numpy()
            if c.dtype == inputs.F32:
                got = got.view(np.float32)
            assert_bits_equal(got, expect[r], f"batch call {k} rank {r}")


def test_moe_round_trip_full_size(env):
    """MoE dispatch and combine at p=8, 4096 tokens x 7168 bf16 per rank,
    top-2 routing uniform over ranks: pack, dispatch exchange, reverse
    exchange and weighted combine with residual, whole arrays against the
    oracle at every stage."""
    torch, coll = env
    p, T, H, k = 8, 4096, 7168, 2
    toks = inputs.rank_buffers(inputs.WL_MOE_A2A, p, T * H, inputs.BF16, dist="normal")
    routes = inputs.moe_routes(p, T, k)
    weights = inputs.moe_weights(p, T, k)
    dtok = [dev(torch, x) for x in toks]
    packed = [torch.empty(T * k * H, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    pos = [torch.empty(T * k, dtype=torch.int32, device="cuda") for _ in range(p)]
    counts = torch.empty(p * p, dtype=torch.int64, device="cuda")
    coll.coll_moe_pack(dtok, [dev(torch, r) for r in routes], packed, pos, counts, k, H)
    torch.cuda.synchronize()
    C = counts.cpu().numpy().reshape(p, p)
    packs = [ref.moe_pack(toks[i], routes[i], k, H, p) for i in range(p)]
    assert np.array_equal(C, np.stack([pk[0] for pk in packs]))
    for i in range(p):
        assert pos[i].cpu().numpy().tolist() == packs[i][1].tolist()
        assert_bits_equal(to_host(packed[i], BF16), packs[i][2], f"packed rank {i}")
    cols = C.sum(axis=0)
    recv = [torch.empty(int(c), dtype=torch.bfloat16, device="cuda") for c in cols]
    coll.coll_alltoallv(packed, recv, counts)
    back = [torch.empty(T * k * H, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    coll.coll_alltoallv_transposed(recv, back, counts)
    torch.cuda.synchronize()
    for i in range(p):
        assert torch.equal(back[i].view(torch.int16), packed[i].view(torch.int16)), f"round trip rank {i}"
    residual = inputs.rank_buffers(inputs.WL_MOE_A2A, p, T * H, inputs.BF16, dist="normal", extra=(5,))
    out = [dev(torch, r) for r in residual]
    coll.coll_moe_combine(back, pos, [dev(torch, w) for w in weights], out, k, H, residual=out)
    torch.cuda.synchronize()
    for i in range(p):
        expect = ref.moe_combine(packs[i][2], packs[i][1], weights[i], k, H, BF16, residual[i])
        assert_bits_equal(to_host(out[i], BF16), expect, f"combine rank {i}")


def test_moe_fp8_round_trip_full_size(env):
    """The FP8 dispatch at p=8, 4096 tokens x 7168 bf16 per rank, top-2,
    one scale per 128 elements: routing, counts and pos whole; packed rows,
    dequantized rows, returned rows and combined tokens on a seeded sample
    of assignments (the oracle encodes row by row)."""
    from oracle import fp8
    torch, coll = env
    p, T, H, k, G = 8, 4096, 7168, 2, 128
    A = T * k
    R = fp8.row_bytes(H, G)
    toks = inputs.rank_buffers(inputs.WL_MOE_A2A, p, T * H, inputs.BF16, dist="normal")
    routes = inputs.moe_routes(p, T, k)
    weights = inputs.moe_weights(p, T, k)
    packed = [torch.empty(A * R, dtype=torch.uint8, device="cuda") for _ in range(p)]
    pos = [torch.empty(A, dtype=torch.int32, device="cuda") for _ in range(p)]
    counts = torch.empty(p * p, dtype=torch.int64, device="cuda")
    counts_h = torch.empty(p * p, dtype=torch.int64, device="cuda")
    coll.coll_moe_pack_fp8([dev(torch, x) for x in toks], [dev(torch, r) for r in routes], packed, pos, counts,
                           k, H, G, counts_hidden_dev=counts_h)
    torch.cuda.synchronize()
    C = counts.cpu().numpy().reshape(p, p)
    rng = np.random.default_rng(17)
    poss = []
    for i in range(p):
        rows_per_dest, epos, _ = ref.moe_pack(np.arange(T), routes[i], k, 1, p)
        assert list(C[i]) == list(rows_per_dest * R), f"byte counts rank {i}"
        got_pos = pos[i].cpu().numpy()
        assert np.array_equal(got_pos, epos), f"pos rank {i}"
        poss.append(got_pos)
        for a in rng.choice(A, 48, replace=False).tolist() + [0, A - 1]:
            row = packed[i][int(got_pos[a]) * R:(int(got_pos[a]) + 1) * R].cpu().numpy()
            x = ref.bf16_to_f32(toks[i][(a // k) * H:(a // k + 1) * H])
            assert_bits_equal(row, fp8.encode_row(x, G), f"fp8 row rank {i} assignment {a}")
    assert np.array_equal(counts_h.cpu().numpy().reshape(p, p), C // R * H)
    rows = C.sum(axis=0) // R
    recv = [torch.empty(int(r) * R, dtype=torch.uint8, device="cuda") for r in rows]
    ex_in = [torch.empty(int(r) * H, dtype=torch.bfloat16, device="cuda") for r in rows]
    back = [torch.empty(A * H, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    coll.coll_alltoallv(packed, recv, counts)
    coll.coll_moe_dequant_fp8(recv, ex_in, counts, [int(r) for r in rows], H, G, status_dev=status)
    coll.coll_alltoallv_transposed(ex_in, back, counts_h)
    residual = inputs.rank_buffers(inputs.WL_MOE_A2A, p, T * H, inputs.BF16, dist="normal", extra=(9,))
    out = [dev(torch, r) for r in residual]
    coll.coll_moe_combine(back, pos, [dev(torch, w) for w in weights], out, k, H, residual=out)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in range(p):
        bk = to_host(back[i], BF16).reshape(A, H)
        ot = to_host(out[i], BF16).reshape(T, H)
        for t in rng.choice(T, 24, replace=False).tolist() + [0, T - 1]:
            x = ref.bf16_to_f32(toks[i][t * H:(t + 1) * H])
            deq = fp8.dequantize_rows(fp8.encode_row(x, G), H, G)
            for s in range(k):
                assert_bits_equal(bk[poss[i][t * k + s]], deq, f"returned row rank {i} token {t} slot {s}")
            back_t = np.concatenate([deq] * k)
            expect = ref.moe_combine(back_t, np.arange(k), weights[i][t * k:(t + 1) * k], k, H, BF16,
                                     residual[i][t * H:(t + 1) * H])
            assert_bits_equal(ot[t], expect, f"combined token rank {i} token {t}")


def test_moe_direct_full_size(env):
    """Direct dispatch and in-place combine at p=8, 4096 tokens x 7168 bf16
    per rank, top-2: counts and every location whole; received rows,
    combined tokens on a seeded sample (expert = identity, so the combine
    reads the received rows)."""
    torch, coll = env
    p, T, H, k = 8, 4096, 7168, 2
    A = T * k
    toks = inputs.rank_buffers(inputs.WL_MOE_A2A, p, T * H, inputs.BF16, dist="normal")
    routes = inputs.moe_routes(p, T, k)
    weights = inputs.moe_weights(p, T, k)
    rows = np.zeros(p, dtype=np.int64)
    for r in routes:
        rows += np.bincount(r, minlength=p)
    recv = [torch.empty(int(r) * H, dtype=torch.bfloat16, device="cuda") for r in rows]
    loc = [torch.empty(A, dtype=torch.int64, device="cuda") for _ in range(p)]
    counts = torch.empty(p * p, dtype=torch.int64, device="cuda")
    status = torch.full((p + 1,), -1, dtype=torch.int32, device="cuda")
    coll.coll_moe_dispatch([dev(torch, x) for x in toks], [dev(torch, r) for r in routes], recv, loc, counts, k, H,
                           status_dev=status)
    residual = inputs.rank_buffers(inputs.WL_MOE_A2A, p, T * H, inputs.BF16, dist="normal", extra=(11,))
    out = [dev(torch, r) for r in residual]
    coll.coll_moe_combine_direct(recv, loc, [dev(torch, w) for w in weights], out, k, H, residual=out)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0] * (p + 1)
    C = counts.cpu().numpy().reshape(p, p)
    exp_rows = np.stack([np.bincount(r, minlength=p) for r in routes])
    assert np.array_equal(C, exp_rows * H)
    roff = np.concatenate([np.zeros((1, p), np.int64), np.cumsum(exp_rows, axis=0)[:-1]])
    rng = np.random.default_rng(23)
    for i in range(p):
        got = loc[i].cpu().numpy()
        d = routes[i].astype(np.int64)
        # row of assignment a in recv[d]: sources before i, then i's earlier assignments to d
        nth = np.zeros(A, dtype=np.int64)
        seen = np.zeros(p, dtype=np.int64)
        for a in range(A):
            nth[a] = seen[d[a]]
            seen[d[a]] += 1
        assert np.array_equal(got, (d << 32) | (roff[i, d] + nth)), f"locations rank {i}"
        ot = to_host(out[i], BF16).reshape(T, H)
        for t in rng.choice(T, 24, replace=False).tolist() + [0, T - 1]:
            for s in range(k):
                a = t * k + s
                row = recv[d[a]][int(got[a] & 0xffffffff) * H:(int(got[a] & 0xffffffff) + 1) * H]
                assert_bits_equal(to_host(row, BF16), toks[i][(a // k) * H:(a // k + 1) * H], f"row rank {i} a {a}")
            expect = ref.moe_combine(np.concatenate([toks[i][t * H:(t + 1) * H]] * k), np.arange(k),
                                     weights[i][t * k:(t + 1) * k], k, H, BF16, residual[i][t * H:(t + 1) * H])
            assert_bits_equal(ot[t], expect, f"combined token rank {i} token {t}")
