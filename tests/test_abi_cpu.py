"""Host-side checks of the C ABI that need no GPU: the library loads,
exports every function coll.h declares, and rejects invalid calls before
touching the device."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

import collective_communication_primitives_coll_amd as coll


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Calls below pass made-up device addresses.  They are all invalid and must
# be rejected on the host; on a machine with a GPU they are not run at all,
# so a regression that accepted one could never launch a kernel on them.
host_only = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: host-only machine")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "coll.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coll_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = coll.lib()
    names = declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(L, name), f"{name} declared in coll.h but not exported"


def test_status_strings_and_version():
    assert coll.coll_status_string(coll.COLL_OK) == "COLL_OK"
    for s in range(1, 5):
        assert coll.coll_status_string(s).startswith("COLL_ERR_")
    assert "unknown" in coll.coll_status_string(99)
    assert coll.coll_version() >= 100
    assert coll.coll_last_hip_error() == 0


def _arr(vals):
    a = (ctypes.c_void_p * len(vals))(*vals)
    return ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)), a


def test_zero_elements_is_ok_without_pointers():
    L = coll.lib()
    assert L.coll_allreduce(None, None, 4, 0, 0, 0, None) == coll.COLL_OK
    assert L.coll_reduce_scatter(None, None, 4, 0, 0, 0, None) == coll.COLL_OK
    assert L.coll_allgather(None, None, 4, 0, 1, None) == coll.COLL_OK
    assert L.coll_alltoall(None, None, 4, 0, 1, None) == coll.COLL_OK
    assert L.coll_broadcast(None, None, 4, 0, 2, 0, None) == coll.COLL_OK
    assert L.coll_reduce(None, None, 4, 0, 2, 1, 3, None) == coll.COLL_OK
    assert L.coll_allreduce_batch(None, 0, 4, 0, None) == coll.COLL_OK
    assert L.coll_gather(None, None, 4, 0, 0, 1, None) == coll.COLL_OK
    assert L.coll_scatter(None, None, 4, 0, 0, 1, None) == coll.COLL_OK
    assert L.coll_allreduce_premul(None, None, 4, 0, 0, None, 0, None) == coll.COLL_OK
    assert L.coll_reduce_scatter_premul(None, None, 4, 0, 1, None, None) == coll.COLL_OK
    assert L.coll_alltoall(None, None, 4, 0, 3, None) == coll.COLL_OK       # bytes


@host_only
def test_invalid_arguments_rejected():
    L = coll.lib()
    INV = coll.COLL_ERR_INVALID_ARG
    base = 0x7F0000000000
    s, _ks = _arr([base + 0x100000 * r for r in range(4)])
    r, _kr = _arr([base + 0x10000000 + 0x100000 * i for i in range(4)])
    n = 1000
    assert L.coll_allreduce(s, r, 0, n, 0, 0, None) == INV            # p = 0
    assert L.coll_allreduce(s, r, 65, n, 0, 0, None) == INV           # p > 64
    assert L.coll_allreduce(s, r, 4, n, 3, 0, None) == INV            # bytes: no arithmetic
    assert L.coll_allreduce(s, r, 4, n, 4, 0, None) == INV            # bad dtype
    assert L.coll_reduce_scatter(s, r, 4, n, 3, 0, None) == INV
    assert L.coll_reduce(s, base + 0x20000000, 4, n, 3, 0, 0, None) == INV
    assert L.coll_allreduce(s, r, 4, n, 0, 4, None) == INV            # bad op (4 is internal)
    assert L.coll_allreduce(s, r, 4, n, 0, -1, None) == INV           # bad op
    assert L.coll_allreduce_premul(s, r, 4, n, 0, None, 0, None) == INV   # no scales
    assert L.coll_reduce_scatter_premul(s, r, 4, n, 0, None, None) == INV
    one = (ctypes.c_float * 4)(1, 1, 1, 1)
    assert L.coll_allreduce_premul(s, r, 4, n, 2, one, 0, None) == coll.COLL_ERR_UNSUPPORTED  # int32
    assert L.coll_allreduce_premul(s, r, 4, n, 0, one, 2, None) == coll.COLL_ERR_UNSUPPORTED  # literal ring
    assert L.coll_reduce_scatter_premul(s, r, 4, n, 2, one, None) == coll.COLL_ERR_UNSUPPORTED
    assert L.coll_allreduce_algo(s, r, 4, n, 0, 0, 7, None) == INV    # bad algo
    assert L.coll_allreduce_algo(s, r, 4, n, 0, 0, 6, None) == INV
    # schedules outside their rank counts (pointer lists of 32 ranks)
    s32, _ks32 = _arr([base + 0x100000 * i for i in range(32)])
    r32, _kr32 = _arr([base + 0x10000000 + 0x100000 * i for i in range(32)])
    one32 = (ctypes.c_float * 32)(*([1.0] * 32))
    assert L.coll_allreduce_algo(s32, r32, 3, n, 0, 0, 1, None) == coll.COLL_ERR_UNSUPPORTED   # recursive doubling, p = 3
    assert L.coll_allreduce_algo(s32, r32, 6, n, 0, 0, 3, None) == coll.COLL_ERR_UNSUPPORTED   # halving-doubling, p = 6
    assert L.coll_allreduce_algo(s32, r32, 17, n, 0, 0, 4, None) == coll.COLL_ERR_UNSUPPORTED  # tree, p = 17
    assert L.coll_allreduce_algo(s32, r32, 32, n, 0, 0, 5, None) == coll.COLL_ERR_UNSUPPORTED  # double tree, p = 32
    assert L.coll_allreduce_premul(s32, r32, 5, n, 0, one32, 1, None) == coll.COLL_ERR_UNSUPPORTED  # RD, p = 5
    assert L.coll_alltoall_algo(s, r, 4, n, 1, 2, None) == INV       # bad All-to-All data path
    assert L.coll_alltoall_algo(s, r, 4, n, 1, -1, None) == INV
    assert L.coll_alltoall_algo(s, r, 4, n, 4, 1, None) == INV       # bad dtype
    assert L.coll_alltoall_algo(s, r, 0, n, 1, 1, None) == INV       # p = 0
    assert L.coll_alltoall_algo(s, r, 4, 0, 1, 7, None) == INV       # algo checked before the n = 0 no-op
    assert L.coll_allreduce(None, r, 4, n, 0, 0, None) == INV         # null array
    assert L.coll_allreduce(s, r, 4, 1 << 61, 0, 0, None) == INV      # size overflow
    z, _kz = _arr([base, 0, base + 0x200000, base + 0x300000])
    assert L.coll_allreduce(z, r, 4, n, 0, 0, None) == INV            # null entry
    m, _km = _arr([base + 2, base + 0x100000, base + 0x200000, base + 0x300000])
    assert L.coll_allreduce(m, r, 4, n, 0, 0, None) == INV            # fp32 pointer not 4-byte aligned
    assert L.coll_reduce(s, base + 0x20000000, 4, n, 0, 0, 4, None) == INV   # root out of range
    assert L.coll_reduce(s, base + 0x20000000, 4, n, 0, 0, -1, None) == INV
    assert L.coll_broadcast(base, r, 4, n, 0, 9, None) == INV
    assert L.coll_broadcast(None, r, 4, n, 0, 0, None) == INV
    caps = (ctypes.c_int64 * 4)(10, 10, 10, 10)
    neg = (ctypes.c_int64 * 4)(10, -1, 10, 10)
    huge = (ctypes.c_int64 * 4)(1 << 60, 10, 10, 10)
    assert L.coll_alltoallv(s, r, 4, None, caps, caps, None, 0, None) == INV         # no counts
    assert L.coll_alltoallv(s, r, 4, base + 0x40000000, neg, caps, None, 0, None) == INV
    assert L.coll_alltoallv(s, r, 4, base + 0x40000000, huge, caps, None, 0, None) == INV
    assert L.coll_alltoallv(s, r, 4, base + 0x40000004, caps, caps, None, 0, None) == INV  # counts misaligned
    assert L.coll_allreduce_batch(None, 3, 4, 0, None) == INV
    assert L.coll_allreduce_batch(None, 0, 4, 8, None) == INV        # unknown flag
    assert L.coll_gather(s, base + 0x20000000, 4, n, 0, 4, None) == INV     # root out of range
    assert L.coll_gather(s, None, 4, n, 0, 0, None) == INV                  # null root buffer
    assert L.coll_gather(s, base + 0x20000002, 4, n, 0, 0, None) == INV     # misaligned root buffer
    assert L.coll_scatter(base, r, 4, n, 0, -1, None) == INV
    assert L.coll_scatter(None, r, 4, n, 0, 0, None) == INV
    assert L.coll_scatter(base, r, 4, n, 5, 0, None) == INV                 # bad dtype
    cnt = base + 0x50000000
    assert L.coll_moe_pack(s, s, r, r, cnt, None, 4, 10, 0, 16, 1, None) == INV   # k = 0
    assert L.coll_moe_pack(s, s, r, r, cnt, None, 4, 10, 9, 16, 1, None) == INV   # k > 8
    assert L.coll_moe_pack(s, s, r, r, cnt, None, 4, 10, 2, 0, 1, None) == INV    # hidden = 0
    assert L.coll_moe_pack(s, s, r, r, None, None, 4, 10, 2, 16, 1, None) == INV  # no counts
    assert L.coll_moe_pack(s, s, r, r, cnt + 4, None, 4, 10, 2, 16, 1, None) == INV  # counts misaligned
    assert L.coll_moe_combine(s, s, s, None, r, 4, 10, 2, 16, 2, None) == coll.COLL_ERR_UNSUPPORTED  # int32
    assert L.coll_moe_combine(s, s, s, None, None, 4, 10, 2, 16, 0, None) == INV  # no outputs
    assert L.coll_alltoallv_transposed(s, r, 4, None, caps, caps, None, 0, None) == INV
    assert L.coll_moe_combine(s, s, s, None, r, 4, 10, 2, 16, 3, None) == INV    # bytes: no arithmetic


def test_fp8_row_bytes():
    rb = coll.coll_moe_fp8_row_bytes
    assert rb(7168, 128) == 7168 + 56 * 4
    assert rb(7168, 7168) == 7168 + 16          # one scale, padded to 16 bytes
    assert rb(16384, 16384) == 16384 + 16
    assert rb(96, 16) == 96 + 32
    assert rb(2048, 2048) == 2048 + 16 and rb(6144, 3072) == 6144 + 16
    assert rb(32768, 1024) == 32768 + 128       # column-local groups: any hidden size
    for hidden, group in [(100, 16), (7168, 48), (7168, 0), (0, 16), (32768, 2048), (96, 8), (3072, 1536),
                          (1 << 31, 1024)]:
        assert rb(hidden, group) == 0, (hidden, group)


@host_only
def test_fp8_invalid_arguments_rejected():
    L = coll.lib()
    INV, UNS = coll.COLL_ERR_INVALID_ARG, coll.COLL_ERR_UNSUPPORTED
    base = 0x7F0000000000
    tok, _k1 = _arr([base + 0x1000000 * r for r in range(4)])
    dst, _k2 = _arr([base + 0x10000000 + 0x1000000 * r for r in range(4)])
    pk, _k3 = _arr([base + 0x20000000 + 0x1000000 * r for r in range(4)])
    ps, _k4 = _arr([base + 0x30000000 + 0x1000000 * r for r in range(4)])
    cnt = base + 0x40000000
    T, k, H = 10, 2, 256
    assert L.coll_moe_pack_fp8(tok, dst, pk, ps, cnt, None, None, 4, T, k, 192, 48, None) == UNS  # group shape
    assert L.coll_moe_pack_fp8(tok, dst, pk, ps, cnt, None, None, 4, T, k, 100, 16, None) == INV  # group does not divide
    assert L.coll_moe_pack_fp8(tok, dst, pk, ps, cnt, None, None, 4, T, k, 32768, 2048, None) == UNS  # row too wide
    assert L.coll_moe_pack_fp8(tok, dst, pk, ps, cnt, None, None, 4, T, 0, H, 128, None) == INV   # k = 0
    assert L.coll_moe_pack_fp8(tok, dst, pk, ps, None, None, None, 4, T, k, H, 128, None) == INV  # no counts
    bad, _k5 = _arr([base + 8, base + 0x1000000, base + 0x2000000, base + 0x3000000])
    assert L.coll_moe_pack_fp8(bad, dst, pk, ps, cnt, None, None, 4, T, k, H, 128, None) == INV  # tokens not 16-aligned
    assert L.coll_moe_pack_fp8(tok, dst, bad, ps, cnt, None, None, 4, T, k, H, 128, None) == INV  # packed not 16-aligned
    assert L.coll_moe_pack_fp8(tok, dst, tok, ps, cnt, None, None, 4, T, k, H, 128, None) == coll.COLL_ERR_ALIAS
    caps = (ctypes.c_int64 * 4)(10, 10, 10, 10)
    neg = (ctypes.c_int64 * 4)(10, -1, 10, 10)
    assert L.coll_moe_dequant_fp8(pk, tok, 4, cnt, None, None, H, 128, None) == INV        # no capacities
    assert L.coll_moe_dequant_fp8(pk, tok, 4, cnt, neg, None, H, 128, None) == INV
    assert L.coll_moe_dequant_fp8(pk, tok, 4, None, caps, None, H, 128, None) == INV       # no counts
    assert L.coll_moe_dequant_fp8(bad, tok, 4, cnt, caps, None, H, 128, None) == INV       # recv not 16-aligned
    assert L.coll_moe_dequant_fp8(pk, tok, 4, cnt, caps, None, 192, 48, None) == UNS
    assert L.coll_moe_dequant_fp8(pk, pk, 4, cnt, caps, None, H, 128, None) == coll.COLL_ERR_ALIAS


@host_only
def test_illegal_aliasing_rejected():
    L = coll.lib()
    AL = coll.COLL_ERR_ALIAS
    base = 0x7F0000000000
    n, p, d = 256, 4, 4
    nb = n * d
    send = [base + 0x100000 * i for i in range(p)]
    recv = [base + 0x10000000 + 0x100000 * i for i in range(p)]
    s, _k1 = _arr(send)
    # AllReduce: recv[0] overlaps send[1]
    r, _k2 = _arr([send[1] + 4] + recv[1:])
    assert L.coll_allreduce(s, r, p, n, 0, 0, None) == AL
    # AllReduce: two outputs overlap
    r, _k3 = _arr([recv[0], recv[0] + 8, recv[2], recv[3]])
    assert L.coll_allreduce(s, r, p, n, 0, 0, None) == AL
    # AllReduce: recv[1] == send[0] (in place only with its own rank)
    r, _k4 = _arr([recv[0], send[0], recv[2], recv[3]])
    assert L.coll_allreduce(s, r, p, n, 0, 0, None) == AL
    # ReduceScatter: recv[2] inside send[2] but at block 0 instead of block 2
    big = [base + 0x1000000 * i for i in range(p)]
    sb, _k5 = _arr(big)
    r, _k6 = _arr([recv[0], recv[1], big[2], recv[3]])
    assert L.coll_reduce_scatter(sb, r, p, n, 0, 0, None) == AL
    # AllGather: send[1] inside recv[1] at the wrong block
    rg = [base + 0x1000000 * i for i in range(p)]
    r, _k7 = _arr(rg)
    sg, _k8 = _arr([send[0], rg[1], send[2], send[3]])
    assert L.coll_allgather(sg, r, p, n, 0, None) == AL
    # AllToAll: any overlap of recv with send
    r, _k9 = _arr([send[0]] + recv[1:])
    assert L.coll_alltoall(s, r, p, n // p, 0, None) == AL
    # Broadcast: recv[1] == send_root while root is 0
    r, _k10 = _arr([recv[0], send[0], recv[2], recv[3]])
    assert L.coll_broadcast(send[0], r, p, n, 0, 0, None) == AL
    # Reduce: root buffer overlaps a non-root input
    assert L.coll_reduce(s, send[2], p, n, 0, 0, 1, None) == AL
    # Alltoallv: counts array inside a receive buffer
    caps = (ctypes.c_int64 * 4)(n, n, n, n)
    r, _k11 = _arr(recv)
    assert L.coll_alltoallv(s, r, p, recv[1] + 64, caps, caps, None, 0, None) == AL
    # Gather: send[1] inside the root buffer, but the root is 2
    root_buf = base + 0x30000000
    sg2, _k12 = _arr([send[0], root_buf + 1 * nb, send[2], send[3]])
    assert L.coll_gather(sg2, root_buf, p, n, 0, 2, None) == AL
    # Gather: the root's own block in place is accepted
    sg3, _k13 = _arr([send[0], send[1], root_buf + 2 * nb, send[3]])
    assert L.coll_gather(sg3, root_buf, p, n, 0, 2, None) != AL
    # Scatter: two outputs overlap
    r, _k14 = _arr([recv[0], recv[0] + 4, recv[2], recv[3]])
    assert L.coll_scatter(root_buf, r, p, n, 0, 0, None) == AL
    # Scatter: recv[0] inside the root buffer while the root is 1
    r, _k15 = _arr([root_buf, recv[1], recv[2], recv[3]])
    assert L.coll_scatter(root_buf, r, p, n, 0, 1, None) == AL
    # MoE combine: an output overlapping a returned-rows buffer is rejected
    T, k, H = 8, 2, 16
    back = [base + 0x60000000 + 0x100000 * i for i in range(p)]
    outs = [base + 0x70000000 + 0x100000 * i for i in range(p)]
    posb = [base + 0x78000000 + 0x100000 * i for i in range(p)]
    wb = [base + 0x7c000000 + 0x100000 * i for i in range(p)]
    b_, _k16 = _arr(back)
    pz, _k17 = _arr(posb)
    wz, _k18 = _arr(wb)
    o_, _k19 = _arr([back[0]] + outs[1:])
    assert L.coll_moe_combine(b_, pz, wz, None, o_, p, T, k, H, 0, None) == AL
    # ... and out == residual (in place) is accepted by the alias check
    o_, _k20 = _arr(outs)
    assert L.coll_moe_combine(b_, pz, wz, o_, o_, p, T, k, H, 0, None) != AL
    # MoE pack: pos overlapping packed is rejected
    pk = [base + 0x40000000 + 0x1000000 * i for i in range(p)]
    pk_, _k21 = _arr(pk)
    ps_, _k22 = _arr([pk[0]] + [base + 0x48000000 + 0x10000 * i for i in range(1, p)])
    assert L.coll_moe_pack(s, s, pk_, ps_, base + 0x4f000000, None, p, T, k, H, 0, None) == AL
    assert nb > 0


@host_only
def test_direct_moe_invalid_arguments_rejected():
    L = coll.lib()
    INV, UNS, AL = coll.COLL_ERR_INVALID_ARG, coll.COLL_ERR_UNSUPPORTED, coll.COLL_ERR_ALIAS
    base = 0x7F0000000000
    tok, _k1 = _arr([base + 0x1000000 * r for r in range(4)])
    dst, _k2 = _arr([base + 0x10000000 + 0x1000000 * r for r in range(4)])
    rcv, _k3 = _arr([base + 0x20000000 + 0x1000000 * r for r in range(4)])
    loc, _k4 = _arr([base + 0x30000000 + 0x1000000 * r for r in range(4)])
    cnt = base + 0x40000000
    T, k, H = 10, 2, 256
    caps = (ctypes.c_int64 * 4)(20, 20, 20, 20)
    neg = (ctypes.c_int64 * 4)(20, -1, 20, 20)
    big = (ctypes.c_int64 * 4)(20, 1 << 31, 20, 20)
    assert L.coll_moe_dispatch(tok, dst, rcv, loc, cnt, None, 4, T, 0, H, caps, 1, None) == INV     # k = 0
    assert L.coll_moe_dispatch(tok, dst, rcv, loc, cnt, None, 4, T, k, 0, caps, 1, None) == INV     # hidden 0
    assert L.coll_moe_dispatch(tok, dst, rcv, loc, cnt, None, 4, T, k, H, None, 1, None) == INV     # no caps
    assert L.coll_moe_dispatch(tok, dst, rcv, loc, cnt, None, 4, T, k, H, neg, 1, None) == INV
    assert L.coll_moe_dispatch(tok, dst, rcv, loc, cnt, None, 4, T, k, H, big, 1, None) == INV     # > 2^31 - 1 rows
    assert L.coll_moe_dispatch(tok, dst, rcv, loc, None, None, 4, T, k, H, caps, 1, None) == INV    # no counts
    assert L.coll_moe_dispatch(tok, dst, rcv, loc, cnt, None, 4, T, k, H, caps, 9, None) == INV     # bad dtype
    odd, _k5 = _arr([base + 0x30000004, base + 0x31000000, base + 0x32000000, base + 0x33000000])
    assert L.coll_moe_dispatch(tok, dst, rcv, odd, cnt, None, 4, T, k, H, caps, 1, None) == INV     # loc not 8-aligned
    assert L.coll_moe_dispatch(tok, dst, tok, loc, cnt, None, 4, T, k, H, caps, 1, None) == AL      # recv = tokens
    assert L.coll_moe_dispatch(tok, dst, rcv, loc, cnt, loc[0], 4, T, k, H, caps, 1, None) == AL    # status in loc
    assert L.coll_moe_dispatch_fp8(tok, dst, rcv, loc, cnt, None, None, 4, T, k, 192, 48, caps, None) == UNS
    assert L.coll_moe_dispatch_fp8(tok, dst, rcv, loc, cnt, None, None, 4, T, k, 100, 16, caps, None) == INV
    mis, _k6 = _arr([base + 0x20000008, base + 0x21000000, base + 0x22000000, base + 0x23000000])
    assert L.coll_moe_dispatch_fp8(tok, dst, mis, loc, cnt, None, None, 4, T, k, H, 128, caps, None) == INV
    assert L.coll_moe_dispatch_fp8(tok, dst, rcv, loc, cnt, cnt, None, 4, T, k, H, 128, caps, None) == AL
    w, _k7 = _arr([base + 0x50000000 + 0x1000000 * r for r in range(4)])
    out, _k8 = _arr([base + 0x60000000 + 0x1000000 * r for r in range(4)])
    assert L.coll_moe_combine_direct(rcv, loc, w, None, out, 4, T, k, H, None, 1, None) == INV     # no y_rows
    assert L.coll_moe_combine_direct(rcv, loc, w, None, out, 4, T, k, H, neg, 1, None) == INV
    assert L.coll_moe_combine_direct(rcv, loc, w, None, out, 4, T, k, H, caps, 2, None) == UNS     # int32
    assert L.coll_moe_combine_direct(rcv, loc, w, None, out, 4, T, k, H, caps, 3, None) == INV     # bytes
    assert L.coll_moe_combine_direct(rcv, odd, w, None, out, 4, T, k, H, caps, 1, None) == INV
    assert L.coll_moe_combine_direct(rcv, loc, w, None, rcv, 4, T, k, H, caps, 1, None) == AL      # out = y
    assert L.coll_moe_combine_direct(rcv, loc, w, None, out, 4, 0, k, H, caps, 1, None) == coll.COLL_OK  # T = 0


@host_only
def test_stream_probe_rejects_invalid_calls():
    L = coll.lib()
    a, ka = _arr([0x10000, 0x20000])
    b, kb = _arr([0x40000])
    sink = 0x80000
    # no stream at all, bytes not a multiple of 16, unknown flag
    assert L.coll_stream_probe(None, 0, None, 0, 64, 4, 0, sink, None) == coll.COLL_ERR_INVALID_ARG
    assert L.coll_stream_probe(a, 1, b, 1, 40, 4, 0, None, None) == coll.COLL_ERR_INVALID_ARG
    assert L.coll_stream_probe(a, 1, b, 1, 64, 4, 16, None, None) == coll.COLL_ERR_INVALID_ARG
    assert L.coll_stream_probe(a, 1, b, 1, 64, 0, 0, None, None) == coll.COLL_ERR_INVALID_ARG
    # a mix or a tile size the probe does not build
    assert L.coll_stream_probe(a, 2, None, 0, 64, 4, 0, sink, None) == coll.COLL_ERR_UNSUPPORTED
    assert L.coll_stream_probe(a, 1, b, 1, 64, 3, 0, None, None) == coll.COLL_ERR_UNSUPPORTED
    big, kbig = _arr([0x100000 * (i + 1) for i in range(16)])
    assert L.coll_stream_probe(big, 16, b, 1, 64, 4, 0, None, None) == coll.COLL_ERR_UNSUPPORTED  # 64 loads
    # read-only mixes need an aligned sink; pointers must be 16-byte aligned
    assert L.coll_stream_probe(a, 1, None, 0, 64, 4, 0, None, None) == coll.COLL_ERR_INVALID_ARG
    assert L.coll_stream_probe(a, 1, None, 0, 64, 4, 0, sink + 4, None) == coll.COLL_ERR_INVALID_ARG
    c, kc = _arr([0x10004])
    assert L.coll_stream_probe(c, 1, b, 1, 64, 4, 0, None, None) == coll.COLL_ERR_INVALID_ARG
    # a destination overlapping a source
    d, kd = _arr([0x10010])
    assert L.coll_stream_probe(a, 1, d, 1, 64, 4, 0, None, None) == coll.COLL_ERR_ALIAS
    # zero bytes is a no-op
    assert L.coll_stream_probe(a, 1, b, 1, 0, 4, 0, None, None) == coll.COLL_OK


def test_noalloc_batch_rejects_invalid_calls_on_the_host():
    L = coll.lib()
    assert L.coll_allreduce_batch_noalloc(None, 0, 4, 0, None) == coll.COLL_OK        # nothing to do
    assert L.coll_allreduce_batch_noalloc(None, 1, 4, 0, None) == coll.COLL_ERR_INVALID_ARG
    assert L.coll_allreduce_batch_noalloc(None, -1, 4, 0, None) == coll.COLL_ERR_INVALID_ARG
    assert L.coll_allreduce_batch_noalloc(None, 0, 0, 0, None) == coll.COLL_ERR_INVALID_ARG
    assert L.coll_allreduce_batch_noalloc(None, 0, 4, 8, None) == coll.COLL_ERR_INVALID_ARG
    # calls of n == 0 are valid and launch nothing
    calls = (coll.coll_call_t * 3)()
    for c in calls:
        c.n, c.dtype, c.op = 0, coll.COLL_F32, coll.COLL_SUM
    assert L.coll_allreduce_batch_noalloc(calls, 3, 4, 0, None) == coll.COLL_OK
    calls[1].op = 9
    assert L.coll_allreduce_batch_noalloc(calls, 3, 4, 0, None) == coll.COLL_ERR_INVALID_ARG


def test_binding_shares_torchs_hip_runtime():
    """Loading the library before torch is imported still leaves one HIP
    runtime in the process (torch's), so torch's device pointers and streams
    are valid in the library's calls."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import collective_communication_primitives_coll_amd as c\n"
            "c.lib()\n"
            "import torch\n"
            "m = sorted(set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l))\n"
            "print(len(m), m)\n"
            "assert len(m) == 1, m\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
