"""Calls past 2^31 elements per buffer (4 GiB and more per rank of bf16),
where any 32-bit element or byte offset would wrap.

At p = 2 the ring order folds each element as one fp32 sum of the two
operands, rounded once to bf16, which is exactly torch's bf16 addition
(fp32 arithmetic, round to nearest even): every output element is checked
against that on the device, and sampled elements, including those either
side of 2^31, against the oracle.
"""
import numpy as np
import pytest

from gpu_util import BF16, assert_bits_equal
from oracle import native

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def coll():
    import torch
    import collective_communication_primitives_coll_amd as c
    torch.cuda.set_device(0)
    c.lib()
    return c


def _bits(t):
    import torch
    return t.view(torch.int16)


def _sample_check(send, got, n, what):
    """got at sampled positions against the oracle's p = 2 fold of the
    same positions of the inputs."""
    import torch
    rng = np.random.default_rng(2031)
    j = np.unique(np.concatenate([rng.integers(0, n, 100000),
                                  np.array([0, 1, (1 << 31) - 1, 1 << 31, (1 << 31) + 1, n - 2, n - 1])]))
    idx = torch.from_numpy(j).cuda()
    ops = [_bits(s[idx]).cpu().numpy().view(np.uint16) for s in send]
    expect = native.allreduce(ops, native.SUM, native.BF16)
    assert_bits_equal(_bits(got[idx]).cpu().numpy().view(np.uint16), expect, what)


def test_allreduce_and_reduce_scatter_past_2_31_elements(coll):
    import torch
    p, n = 2, (1 << 31) + 4099
    g = torch.Generator(device="cuda").manual_seed(31)
    send = [torch.randn(n, generator=g, device="cuda").to(torch.bfloat16) for _ in range(p)]
    expect = (send[0].float() + send[1].float()).to(torch.bfloat16)
    recv = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    for t in recv:
        t.fill_(float("nan"))
    coll.coll_allreduce(send, recv, coll.COLL_SUM)
    torch.cuda.synchronize()
    for r in range(p):
        assert torch.equal(_bits(recv[r]), _bits(expect)), f"AllReduce n={n} rank {r}"
    _sample_check(send, recv[1], n, f"AllReduce n={n} sampled")

    blk = (1 << 30) + 2049          # send buffers of 2 * blk > 2^31 elements
    shard = [t[:blk] for t in recv]
    for t in shard:
        t.fill_(float("nan"))
    coll.coll_reduce_scatter([s[:p * blk] for s in send], shard, coll.COLL_SUM)
    torch.cuda.synchronize()
    for r in range(p):
        assert torch.equal(_bits(shard[r]), _bits(expect[r * blk:(r + 1) * blk])), f"ReduceScatter block {r}"


def test_allgather_and_alltoall_past_2_31_elements(coll):
    """AllGather of 2^30 + 2049-element bf16 shards and All-to-All of blocks
    of that size, p = 2: each receive (and All-to-All send) buffer holds
    more than 2^31 elements; every element checked against slices of the
    inputs."""
    import torch
    p, blk = 2, (1 << 30) + 2049
    g = torch.Generator(device="cuda").manual_seed(32)
    send = [torch.randn(p * blk, generator=g, device="cuda").to(torch.bfloat16) for _ in range(p)]
    recv = [torch.empty(p * blk, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    shards = [s[:blk] for s in send]
    for t in recv:
        t.fill_(float("nan"))
    coll.coll_allgather(shards, recv)
    torch.cuda.synchronize()
    for r in range(p):
        for s in range(p):
            assert torch.equal(_bits(recv[r][s * blk:(s + 1) * blk]), _bits(shards[s])), f"AllGather rank {r} block {s}"
    for t in recv:
        t.fill_(float("nan"))
    coll.coll_alltoall(send, recv, blk)
    torch.cuda.synchronize()
    for j in range(p):
        for i in range(p):
            assert torch.equal(_bits(recv[j][i * blk:(i + 1) * blk]), _bits(send[i][j * blk:(j + 1) * blk])), \
                f"All-to-All dest {j} block {i}"


def test_reduce_and_broadcast_past_2_31_elements(coll):
    """Reduce to root 1 and Broadcast from root 0, p = 2, 2^31 + 4099 bf16
    elements: the root's sum against torch's bf16 addition (the p = 2 fold)
    and every receiver against the root's buffer, whole."""
    import torch
    p, n = 2, (1 << 31) + 4099
    g = torch.Generator(device="cuda").manual_seed(33)
    send = [torch.randn(n, generator=g, device="cuda").to(torch.bfloat16) for _ in range(p)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(float("nan"))
    coll.coll_reduce(send, out, 1, coll.COLL_SUM)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits((send[0].float() + send[1].float()).to(torch.bfloat16))), "Reduce"
    recv = [out, torch.empty(n, dtype=torch.bfloat16, device="cuda")]
    for t in recv:
        t.fill_(float("nan"))
    coll.coll_broadcast(send[0], recv, 0)
    torch.cuda.synchronize()
    for r in range(p):
        assert torch.equal(_bits(recv[r]), _bits(send[0])), f"Broadcast rank {r}"


def test_alltoallv_past_2_31_elements(coll):
    """Alltoallv, p = 2, 2^31 + 4099 bf16 elements per send buffer, with
    counts that leave the blocks at differing 16-byte offsets (so both the
    aligned and the byte-shifted copy paths run) and receive buffers of more
    than 2^31 elements: every block checked whole against its source."""
    import torch
    p, n = 2, (1 << 31) + 4099
    counts = np.array([[(1 << 30) + 5, (1 << 30) + 4094], [(1 << 30) + 4000, (1 << 30) + 99]], dtype=np.int64)
    assert (counts.sum(axis=1) == n).all()
    g = torch.Generator(device="cuda").manual_seed(34)
    send = [torch.randn(n, generator=g, device="cuda").to(torch.bfloat16) for _ in range(p)]
    cols = counts.sum(axis=0)
    recv = [torch.empty(int(c), dtype=torch.bfloat16, device="cuda").fill_(float("nan")) for c in cols]
    cdev = torch.from_numpy(counts.reshape(-1).copy()).cuda()
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    coll.coll_alltoallv(send, recv, cdev, status_dev=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for j in range(p):
        ro = 0
        for i in range(p):
            so = int(counts[i, :j].sum())
            c = int(counts[i, j])
            assert torch.equal(_bits(recv[j][ro:ro + c]), _bits(send[i][so:so + c])), f"Alltoallv {i} -> {j}"
            ro += c


def test_gather_and_scatter_past_2_31_elements(coll):
    """Gather to root 1 and Scatter from root 0, p = 2, blocks of 2^30 + 2049
    bf16 elements: the root buffer holds more than 2^31 elements; every
    block checked whole."""
    import torch
    p, blk = 2, (1 << 30) + 2049
    g = torch.Generator(device="cuda").manual_seed(35)
    ranks = [torch.randn(blk, generator=g, device="cuda").to(torch.bfloat16) for _ in range(p)]
    root_buf = torch.empty(p * blk, dtype=torch.bfloat16, device="cuda").fill_(float("nan"))
    coll.coll_gather(ranks, root_buf, 1)
    torch.cuda.synchronize()
    for r in range(p):
        assert torch.equal(_bits(root_buf[r * blk:(r + 1) * blk]), _bits(ranks[r])), f"Gather block {r}"
    out = [torch.empty(blk, dtype=torch.bfloat16, device="cuda").fill_(float("nan")) for _ in range(p)]
    coll.coll_scatter(root_buf, out, 0)
    torch.cuda.synchronize()
    for r in range(p):
        assert torch.equal(_bits(out[r]), _bits(ranks[r])), f"Scatter rank {r}"
