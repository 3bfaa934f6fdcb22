"""Pins for the CPU oracle: values the pages print, closed forms, invariants
and brute force on tiny inputs.  Each test is chosen so that a plausible
mistake in the oracle (a dropped rank, a wrong rotation, a transposed
block, a bad rounding rule) fails it.  No value here comes from the GPU.
"""
import itertools
import math
import struct

import numpy as np
import pytest

from conftest import read_golden
from oracle import ref
from collective_communication_primitives_coll_amd import inputs, metrics

OPS = (ref.SUM, ref.MIN, ref.MAX)
DTYPES = (ref.F32, ref.BF16, ref.I32)


def _as_dtype(int_vals, dtype):
    a = np.asarray(int_vals, dtype=np.int64)
    if dtype == ref.I32:
        return a.astype(np.int32)
    if dtype == ref.F32:
        return a.astype(np.float32)
    # small integers are exact in bf16: take the upper half of the fp32 bits
    return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _to_float(vals, dtype):
    if dtype == ref.BF16:
        return ref.bf16_to_f32(vals).astype(np.float64)
    return np.asarray(vals).astype(np.float64)


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


# ----------------------------------------------------------------------------
# The pages' worked example (hpc/04 sections 1.3 and 1.4)
# ----------------------------------------------------------------------------

def _worked_example():
    rows = read_golden("reduce_worked_example.txt")
    xs = [[int(v) for v in r[2:]] for r in rows if r[0] == "in"]
    out = [int(v) for r in rows if r[0] == "out" for v in r[2:]]
    return xs, out


@pytest.mark.parametrize("dtype", DTYPES)
def test_worked_example_sum(dtype):
    xs, expect = _worked_example()
    arrs = [_as_dtype(x, dtype) for x in xs]
    for r_out in ref.allreduce(arrs, ref.SUM, dtype):
        assert list(_to_float(r_out, dtype)) == expect
    for root in range(len(xs)):
        assert list(_to_float(ref.reduce(arrs, ref.SUM, dtype, root), dtype)) == expect


@pytest.mark.parametrize("dtype", DTYPES)
def test_worked_example_min_max(dtype):
    # Derived from the same inputs with the definition of min / max.
    xs, _ = _worked_example()
    arrs = [_as_dtype(x, dtype) for x in xs]
    assert list(_to_float(ref.allreduce(arrs, ref.MIN, dtype)[0], dtype)) == [0, 1]
    assert list(_to_float(ref.allreduce(arrs, ref.MAX, dtype)[0], dtype)) == [6, 7]


# ----------------------------------------------------------------------------
# Brute force over every small integer input (order-independent ops)
# ----------------------------------------------------------------------------

def _py_reduce(vals, op):
    return {ref.SUM: sum, ref.MIN: min, ref.MAX: max}[op](vals)


@pytest.mark.parametrize("p,n", [(1, 1), (1, 2), (2, 1), (2, 2), (3, 1), (3, 2), (4, 1), (4, 2)])
@pytest.mark.parametrize("dtype", DTYPES)
def test_bruteforce_all_small_inputs(p, n, dtype):
    """Every input in {-2..2}^(p*n): reduce_elements against Python's
    sum/min/max, plus allreduce() on a sample of the cases."""
    vals = np.array(list(itertools.product(range(-2, 3), repeat=p * n)), dtype=np.int64)  # cases x (p*n)
    cases = vals.shape[0]
    per_rank = vals.reshape(cases, p, n)                       # case, rank, elem
    cols = per_rank.transpose(1, 0, 2).reshape(p, cases * n)   # rank, (case, elem)
    chunk = ref.chunk_of(np.tile(np.arange(n), cases), n, p)
    for op in OPS:
        got = _to_float(ref.reduce_elements(_as_dtype(cols, dtype), chunk, op, dtype), dtype)
        expect = [_py_reduce(list(cols[:, e]), op) for e in range(cols.shape[1])]
        assert got.tolist() == expect
    rng = np.random.default_rng(p * 10 + n)
    for case in rng.choice(cases, size=min(cases, 300), replace=False):
        xs = [_as_dtype(per_rank[case, r], dtype) for r in range(p)]
        for op in OPS:
            expect = [_py_reduce(list(per_rank[case, :, e]), op) for e in range(n)]
            for out in ref.allreduce(xs, op, dtype):
                assert _to_float(out, dtype).tolist() == expect


# ----------------------------------------------------------------------------
# Order-dependent fp32 / bf16 sums: pure-Python fold with exact rounding
# ----------------------------------------------------------------------------

def _f32(x: float) -> float:
    """Round a Python float (binary64) to binary32, nearest-even."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _py_add_f32(a: float, b: float) -> float:
    # a + b is exact or correctly rounded in binary64; rounding that to
    # binary32 equals one correct rounding of the exact sum because 53 >=
    # 2*24 + 2 (double rounding is innocuous for +).
    return _f32(a + b)


def _py_bf16_rne(x: float) -> float:
    """Nearest bf16 to the binary32 value x, ties to the even pattern,
    found by comparing distances to the two bf16 neighbours."""
    if x == 0.0 or math.isinf(x):
        return x
    bits = struct.unpack("<I", struct.pack("<f", x))[0]
    lo_bits = bits & 0xFFFF0000
    hi_bits = lo_bits + 0x10000
    lo = struct.unpack("<f", struct.pack("<I", lo_bits))[0]
    # the next bf16 away from zero; past the largest finite value it is inf
    hi = struct.unpack("<f", struct.pack("<I", hi_bits & 0xFFFFFFFF))[0]
    dlo, dhi = abs(x - lo), abs(hi - x)
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if ((lo_bits >> 16) & 1) == 0 else hi


def _py_ring_fold(vals_by_rank, c, dtype):
    p = len(vals_by_rank)
    order = [(c + k) % p for k in range(1, p + 1)]
    acc = vals_by_rank[order[0]]
    for r in order[1:]:
        acc = _py_add_f32(acc, vals_by_rank[r])
    return _py_bf16_rne(acc) if dtype == ref.BF16 else acc


@pytest.mark.parametrize("dtype", [ref.F32, ref.BF16])
def test_fp_sum_order_against_pure_python(dtype):
    rng = np.random.default_rng(1234)
    for trial in range(60):
        p = int(rng.integers(1, 7))
        n = int(rng.integers(1, 12))
        scale = float(10.0 ** rng.integers(-3, 4))
        xs = [(rng.standard_normal(n) * scale).astype(np.float32) for _ in range(p)]
        if dtype == ref.BF16:
            xs = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in xs]
        got = _to_float(ref.allreduce(xs, ref.SUM, dtype)[0], dtype)
        q = -(-n // p)
        widened = [_to_float(x, dtype) for x in xs]
        for i in range(n):
            expect = _py_ring_fold([float(w[i]) for w in widened], i // q, dtype)
            assert got[i] == expect, (trial, p, n, i)


def test_fp_sum_order_matters_here():
    """Guard for the previous test: the chosen data does distinguish orders."""
    rng = np.random.default_rng(5)
    xs = [rng.standard_normal(4096).astype(np.float32) for _ in range(8)]
    ring = ref.allreduce(xs, ref.SUM, ref.F32)[0]
    natural = xs[0].copy()
    for x in xs[1:]:
        natural = natural + x
    assert not np.array_equal(ring.view(np.uint32), natural.view(np.uint32))


def test_bf16_rne_pins():
    one = 1.0
    cases = [  # (fp32 value, bf16 pattern); a list because 0.0 == -0.0 as dict keys
        (one, 0x3F80),
        (one + 2.0 ** -8, 0x3F80),                # exact tie, even kept part
        (one + 3 * 2.0 ** -8, 0x3F82),            # exact tie, odd kept part rounds up
        (one + 2.0 ** -8 + 2.0 ** -20, 0x3F81),   # just above the tie
        (one + 2.0 ** -9, 0x3F80),                # below the tie
        (-(one + 3 * 2.0 ** -8), 0xBF82),
        (float.fromhex("0x1.fffffep127"), 0x7F80),  # largest fp32 rounds to +inf
        (float.fromhex("0x1.fefffep127"), 0x7F7F),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (float("inf"), 0x7F80),
        (2.0 ** -133, 0x0001),                    # smallest bf16 subnormal, exact
        (2.0 ** -134, 0x0000),                    # half of it: tie, even kept part (zero)
        (2.0 ** -134 + 2.0 ** -149, 0x0001),      # just above that tie
        (2.0 ** -126, 0x0080),
    ]
    xs = np.array([c[0] for c in cases], dtype=np.float32)
    got = ref.f32_to_bf16_rne(xs)
    assert [int(g) for g in got] == [c[1] for c in cases]
    nan = ref.f32_to_bf16_rne(np.array([np.nan, -np.nan], dtype=np.float32))
    assert all((int(v) & 0x7F80) == 0x7F80 and (int(v) & 0x7F) != 0 for v in nan)


def test_bf16_rne_against_pure_python_and_torch():
    rng = np.random.default_rng(9)
    base = rng.standard_normal(20000).astype(np.float32) * np.float32(1e3)
    # add exact ties and near-ties
    u = base.view(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    near = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)).view(np.float32)
    xs = np.concatenate([base, ties, near])
    got = ref.f32_to_bf16_rne(xs)
    py = np.array([_py_bf16_rne(float(v)) for v in xs[:3000]])
    assert np.array_equal(ref.bf16_to_f32(got[:3000]).astype(np.float64), py)
    torch = pytest.importorskip("torch")
    tb = torch.from_numpy(xs.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, tb)


# ----------------------------------------------------------------------------
# The ring of section 2.2 simulated step by step == the closed-form order
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_ring_simulator_equals_closed_form(dtype, op):
    rng = np.random.default_rng(100 + dtype * 3 + op)
    for p in range(1, 10):
        for n in (1, p - 1 if p > 1 else 1, p, 2 * p + 1, 37, 64):
            xs = inputs.rank_buffers(inputs.WL_TEST, p, n, dtype, dist="normal", extra=(p, n))
            sim = ref.ring_allreduce_simulated(xs, op, dtype)
            closed = ref.allreduce(xs, op, dtype)
            for r in range(p):
                assert np.array_equal(_bits(sim[r]), _bits(closed[r])), (p, n, r)


def test_ring_reduce_scatter_phase_lands_chunk_c_on_rank_c():
    """After the p-1 reduce-scatter steps, rank c holds chunk c fully
    reduced (section 1.5 placement), checked with exact integer data."""
    for p in (2, 3, 4, 5, 8):
        n = 4 * p + (p // 2)
        xs = inputs.rank_buffers(inputs.WL_TEST, p, n, ref.I32, extra=(7, p))
        bufs = ref.ring_allreduce_simulated(xs, ref.SUM, ref.I32, return_after_rs=True)
        total = np.sum(np.stack(xs).astype(np.int64), axis=0)
        q = -(-n // p)
        for c in range(p):
            sl = slice(min(c * q, n), min((c + 1) * q, n))
            assert np.array_equal(bufs[c][sl].astype(np.int64), total[sl])
            # and no other rank holds it complete (p > 1 and values non-trivial)
            if p > 2:
                other = (c + 1) % p
                assert not np.array_equal(bufs[other][sl].astype(np.int64), total[sl]) or sl.start == sl.stop


def test_ring_message_count_and_volume():
    """Section 2.2: 2(p-1) messages, 2n(p-1)/p bytes per rank (n bytes per rank)."""
    for p in (2, 4, 8, 16):
        n_bytes = 1024 * p
        sends_per_rank = 2 * (p - 1)            # one chunk per step, 2(p-1) steps
        assert sends_per_rank * (n_bytes // p) == 2 * n_bytes * (p - 1) // p


# ----------------------------------------------------------------------------
# Identities (section 0: AllReduce == Reduce then Broadcast ==
# ReduceScatter then AllGather) and duality (section 1.7)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_identity_allreduce_is_rs_then_ag(dtype, op):
    for p in (1, 2, 3, 4, 8):
        nb = 5
        xs = inputs.rank_buffers(inputs.WL_TEST, p, p * nb, dtype, dist="normal", extra=(11, p))
        ar = ref.allreduce(xs, op, dtype)
        ag = ref.allgather(ref.reduce_scatter(xs, op, dtype))
        for r in range(p):
            assert np.array_equal(_bits(ar[r]), _bits(ag[r]))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_identity_allreduce_is_reduce_then_broadcast(dtype, op):
    for p in (1, 2, 3, 5, 8):
        n = 3 * p + 2
        xs = inputs.rank_buffers(inputs.WL_TEST, p, n, dtype, dist="normal", extra=(12, p))
        ar = ref.allreduce(xs, op, dtype)
        for root in range(p):
            bc = ref.broadcast(ref.reduce(xs, op, dtype, root), p)
            for r in range(p):
                assert np.array_equal(_bits(ar[r]), _bits(bc[r]))


def test_duality_allgather_reduce_scatter_adjoint():
    rng = np.random.default_rng(3)
    for p in (1, 2, 3, 4, 8):
        n = 6
        x = [rng.integers(-50, 50, n).astype(np.int32) for _ in range(p)]
        y = [rng.integers(-50, 50, p * n).astype(np.int32) for _ in range(p)]
        lhs = sum(int(np.dot(a.astype(np.int64), b.astype(np.int64))) for a, b in zip(ref.allgather(x), y))
        rs = ref.reduce_scatter(y, ref.SUM, ref.I32)
        rhs = sum(int(np.dot(a.astype(np.int64), b.astype(np.int64))) for a, b in zip(x, rs))
        assert lhs == rhs


def test_duality_broadcast_reduce_adjoint():
    rng = np.random.default_rng(4)
    for p in (1, 2, 5, 8):
        n = 7
        x = rng.integers(-50, 50, n).astype(np.int32)
        y = [rng.integers(-50, 50, n).astype(np.int32) for _ in range(p)]
        lhs = sum(int(np.dot(a.astype(np.int64), b.astype(np.int64))) for a, b in zip(ref.broadcast(x, p), y))
        for root in range(p):
            red = ref.reduce(y, ref.SUM, ref.I32, root)
            assert lhs == int(np.dot(x.astype(np.int64), red.astype(np.int64)))


# ----------------------------------------------------------------------------
# Symbolic layouts printed on the pages
# ----------------------------------------------------------------------------

def _symbol_codes(rows):
    syms = sorted({s for r in rows if r[0] == "in" for s in r[2:]})
    return {s: 1 << i for i, s in enumerate(syms)}


def test_allgather_symbolic():
    rows = read_golden("allgather_symbolic.txt")
    code = _symbol_codes(rows)
    xs = [np.array([code[s] for s in r[2:]], dtype=np.int32) for r in rows if r[0] == "in"]
    expect = [code[s] for r in rows if r[0] == "out" for s in r[2:]]
    for out in ref.allgather(xs):
        assert out.tolist() == expect


def test_reduce_scatter_symbolic():
    rows = read_golden("reduce_scatter_symbolic.txt")
    code = _symbol_codes(rows)
    xs = [np.array([code[s] for s in r[2:]], dtype=np.int32) for r in rows if r[0] == "in"]
    got = ref.reduce_scatter(xs, ref.SUM, ref.I32)
    for r in rows:
        if r[0] == "out":
            expect = sum(code[s] for s in r[2].split("+"))
            assert got[int(r[1])].tolist() == [expect]


@pytest.mark.parametrize("name", ["alltoall_symbolic.txt", "alltoall_three_rank.txt"])
def test_alltoall_symbolic(name):
    rows = read_golden(name)
    code = _symbol_codes(rows)
    xs = [np.array([code[s] for s in r[2:]], dtype=np.int32) for r in rows if r[0] == "in"]
    got = ref.alltoall(xs)
    for r in rows:
        if r[0] == "out":
            assert got[int(r[1])].tolist() == [code[s] for s in r[2:]]


def test_broadcast_symbolic():
    rows = read_golden("broadcast_symbolic.txt")
    code = _symbol_codes(rows)
    root = int([r for r in rows if r[0] == "root"][0][1])
    x = np.array([code[s] for r in rows if r[0] == "in" for s in r[2:]], dtype=np.int32)
    expect = [code[s] for r in rows if r[0] == "out" for s in r[2:]]
    for out in ref.broadcast(x, 4):
        assert out.tolist() == expect
    assert root == 0


def test_alltoall_twice_is_identity():
    for p in (1, 2, 3, 8):
        for m in (0, 1, 5):
            xs = inputs.rank_buffers(inputs.WL_TEST, p, p * m, ref.I32, extra=(21, p, m))
            back = ref.alltoall(ref.alltoall(xs))
            assert all(np.array_equal(a, b) for a, b in zip(xs, back))


def test_alltoallv_then_transposed_counts_is_identity():
    rng = np.random.default_rng(8)
    for p in (1, 2, 3, 5, 8):
        for _ in range(5):
            counts = rng.integers(0, 6, size=(p, p))
            counts[rng.random((p, p)) < 0.2] = 0
            xs = [rng.integers(-100, 100, int(counts[i].sum())).astype(np.int32) for i in range(p)]
            mid = ref.alltoallv(xs, counts)
            assert [len(m) for m in mid] == ref.alltoallv_recv_counts(counts).tolist()
            back = ref.alltoallv(mid, counts.T)
            assert all(np.array_equal(a, b) for a, b in zip(xs, back))


def test_alltoallv_small_explicit():
    # p = 2: source 0 sends 1 element to 0 and 2 to 1; source 1 sends 3 to 0 and 0 to 1.
    xs = [np.array([10, 11, 12], dtype=np.int32), np.array([20, 21, 22], dtype=np.int32)]
    counts = np.array([[1, 2], [3, 0]])
    out = ref.alltoallv(xs, counts)
    assert out[0].tolist() == [10, 20, 21, 22]
    assert out[1].tolist() == [11, 12]


def test_alltoallv_equal_counts_match_alltoall():
    for p in (2, 4, 8):
        m = 3
        xs = inputs.rank_buffers(inputs.WL_TEST, p, p * m, ref.I32, extra=(31, p))
        a = ref.alltoall(xs)
        b = ref.alltoallv(xs, np.full((p, p), m))
        assert all(np.array_equal(u, v) for u, v in zip(a, b))


# ----------------------------------------------------------------------------
# Error bound of the fp32 fold against the exact sum
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("p", [2, 8, 16])
def test_fp32_sum_within_recursive_summation_bound(p):
    n = 2048
    xs = inputs.rank_buffers(inputs.WL_TEST, p, n, ref.F32, dist="normal", extra=(41, p))
    got = ref.allreduce(xs, ref.SUM, ref.F32)[0].astype(np.float64)
    u = 2.0 ** -24
    gamma = (p - 1) * u / (1 - (p - 1) * u)
    for i in range(0, n, 7):
        vals = [float(x[i]) for x in xs]
        exact = math.fsum(vals)
        bound = gamma * sum(abs(v) for v in vals)
        assert abs(got[i] - exact) <= bound + 1e-45


# ----------------------------------------------------------------------------
# Bandwidth conventions (section 2.5 table)
# ----------------------------------------------------------------------------

def test_busbw_factors_match_table():
    for name, a, b, den in read_golden("busbw_factors.txt"):
        for p in (2, 4, 8, 16):
            expect = int(a) * (p + int(b)) / p if den == "p" else float(a)
            assert metrics.busbw_factor(name, p) == pytest.approx(expect, rel=0, abs=1e-15)


def test_hbm_to_busbw_ratio():
    # Out-of-place AllReduce: HBM bytes / busbw bytes = p^2/(p-1).
    for p in (4, 8, 16):
        n, d = 1 << 20, 4
        hbm = metrics.hbm_bytes("allreduce", p, n, d)
        bus = metrics.payload_bytes("allreduce", p, n, d) * metrics.busbw_factor("allreduce", p)
        assert hbm / bus == pytest.approx(p * p / (p - 1))
    # ReduceScatter / AllGather: p(p+1)/(p-1)
    for coll in ("reduce_scatter", "allgather"):
        p = 8
        hbm = metrics.hbm_bytes(coll, p, 1000, 2)
        bus = metrics.payload_bytes(coll, p, 1000, 2) * metrics.busbw_factor(coll, p)
        assert hbm / bus == pytest.approx(p * (p + 1) / (p - 1))


# ----------------------------------------------------------------------------
# Input recipes
# ----------------------------------------------------------------------------

def test_input_recipes():
    g = inputs.rng_for(inputs.WL_TEST, 0)
    u = inputs.uniform_f32(g, 100000)
    assert u.dtype == np.float32 and u.min() >= -1.0 and u.max() < 1.0
    assert not np.any((u == 0) & np.signbit(u))
    assert np.all(np.mod(u.astype(np.float64) * 2 ** 23, 1.0) == 0)
    i = inputs.uniform_i32(g, 100000)
    assert i.min() >= -1000 and i.max() <= 1000
    nb = inputs.normal_bf16_bits(inputs.rng_for(2, 0), 200000, 1e-3)
    vals = ref.bf16_to_f32(nb)
    assert abs(float(np.std(vals)) - 1e-3) < 2e-5
    # determinism
    a = inputs.rank_buffers(inputs.WL_TEST, 3, 10, inputs.F32)
    b = inputs.rank_buffers(inputs.WL_TEST, 3, 10, inputs.F32)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    c = inputs.moe_token_counts()
    assert c.shape == (8, 8) and np.all(c.sum(axis=1) == 4096)
    calls, pool = inputs.small_batch_plan(2000)
    sizes = np.array([c.n * 4 for c in calls])
    assert sizes.min() >= 4096 - 3 and sizes.max() < 1 << 20
    assert all(c.src_off % 64 == 0 and c.dst_off % 64 == 0 for c in calls)
    assert [c.op for c in calls[:6]] == [0, 1, 2, 0, 1, 2]
    assert [c.dtype for c in calls[:6]] == [0, 0, 0, 2, 2, 2]


# ----------------------------------------------------------------------------
# Recursive doubling and halving-doubling (hpc/04 section 2.3)
# ----------------------------------------------------------------------------

def _py_tree(vals, first_stride, dtype):
    """Pure-Python pairwise tree with struct-rounded fp32 adds."""
    a = list(vals)
    p = len(a)
    if first_stride == "low":
        s = 1
        while s < p:
            for k in range(0, p, 2 * s):
                a[k] = _py_add_f32(a[k], a[k + s])
            s *= 2
    else:
        s = p // 2
        while s >= 1:
            for k in range(s):
                a[k] = _py_add_f32(a[k], a[k + s])
            s //= 2
    return _py_bf16_rne(a[0]) if dtype == ref.BF16 else a[0]


@pytest.mark.parametrize("dtype", [ref.F32, ref.BF16])
@pytest.mark.parametrize("p", [1, 2, 4, 8, 16])
def test_doubling_schedules_simulated_equal_their_trees(dtype, p):
    """The step-by-step simulations give, on every rank, the balanced tree of
    their pairing order, checked element by element against a pure-Python
    tree with struct-rounded fp32 additions."""
    rng = np.random.default_rng(77 + p)
    for n in (1, p - 1 if p > 1 else 1, 3 * p + 1, 37):
        xs = [(rng.standard_normal(n) * 10.0 ** rng.integers(-2, 3)).astype(np.float32) for _ in range(p)]
        if dtype == ref.BF16:
            xs = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in xs]
        widened = [_to_float(x, dtype) for x in xs]
        for sim, stride in ((ref.recursive_doubling_simulated, "low"), (ref.halving_doubling_simulated, "high")):
            outs = sim(xs, ref.SUM, dtype)
            tree = ref.fold_tree(xs, ref.SUM, dtype, stride)
            for r in range(p):
                assert np.array_equal(_bits(outs[r]), _bits(tree)), (sim.__name__, p, n, r)
            got = _to_float(tree, dtype)
            for i in range(n):
                assert got[i] == _py_tree([float(w[i]) for w in widened], stride, dtype), (stride, p, n, i)


@pytest.mark.parametrize("p", [2, 4, 8])
def test_doubling_schedules_exact_on_integers(p):
    """Brute-force style: integer data (exact in every order) gives the plain
    sum, min and max on every rank, for int32 and for small fp32 integers."""
    rng = np.random.default_rng(p)
    for n in (1, 5, 2 * p + 3):
        ints = [rng.integers(-50, 51, n) for _ in range(p)]
        for dtype in (ref.I32, ref.F32):
            xs = [_as_dtype(v, dtype) for v in ints]
            for op, fn in ((ref.SUM, np.sum), (ref.MIN, np.min), (ref.MAX, np.max)):
                expect = fn(np.stack(ints), axis=0)
                for sim in (ref.recursive_doubling_simulated, ref.halving_doubling_simulated):
                    for out in sim(xs, op, dtype):
                        assert list(_to_float(out, dtype)) == list(expect.astype(np.float64))


def test_halving_doubling_leaves_block_r_on_rank_r():
    """After the halving phase rank r owns block r (the reduce-scatter
    placement of section 1.5); the simulator asserts it internally, and the
    all-gather phase then gives every rank the full vector."""
    p, n = 8, 8 * 5
    xs = [np.full(n, float(r + 1), dtype=np.float32) for r in range(p)]
    outs = ref.halving_doubling_simulated(xs, ref.SUM, ref.F32)
    for o in outs:
        assert np.all(o == sum(range(1, p + 1)))


def test_doubling_orders_differ_from_ring_and_each_other():
    """Guard: at p = 8 the three orders give different bits on this data,
    so a kernel using the wrong one fails its parity test."""
    rng = np.random.default_rng(9)
    xs = [rng.standard_normal(4096).astype(np.float32) for _ in range(8)]
    ring = ref.allreduce(xs, ref.SUM, ref.F32)[0]
    rd = ref.fold_tree(xs, ref.SUM, ref.F32, "low")
    hd = ref.fold_tree(xs, ref.SUM, ref.F32, "high")
    assert not np.array_equal(_bits(ring), _bits(rd))
    assert not np.array_equal(_bits(ring), _bits(hd))
    assert not np.array_equal(_bits(rd), _bits(hd))


@pytest.mark.parametrize("stride", ["low", "high"])
def test_tree_orders_within_summation_bound(stride):
    """A balanced tree over p = 16 values has depth 4: |tree - fsum| <= gamma_4 sum|x|."""
    p, n = 16, 1024
    xs = inputs.rank_buffers(inputs.WL_TEST, p, n, ref.F32, dist="normal", extra=(43, p))
    got = ref.fold_tree(xs, ref.SUM, ref.F32, stride).astype(np.float64)
    u = 2.0 ** -24
    gamma = 4 * u / (1 - 4 * u)
    for i in range(0, n, 5):
        vals = [float(x[i]) for x in xs]
        assert abs(got[i] - math.fsum(vals)) <= gamma * sum(abs(v) for v in vals) + 1e-45


# ----------------------------------------------------------------------------
# Gather and Scatter (single-root forms of AllGather and Broadcast)
# ----------------------------------------------------------------------------

def test_gather_scatter_symbolic():
    rows = read_golden("gather_scatter_symbolic.txt")
    gin = {int(r[1]): r[2:] for r in rows if r[0] == "gather_in"}
    gout = [r for r in rows if r[0] == "gather_out"][0]
    p = len(gin)
    root = int(gout[1])
    # symbols -> integer codes so the oracle runs on arrays
    sym = sorted({v for vs in gin.values() for v in vs})
    code = {v: i for i, v in enumerate(sym)}
    xs = [np.array([code[v] for v in gin[r]], dtype=np.int32) for r in range(p)]
    got = ref.gather(xs, root)
    assert [sym[i] for i in got] == gout[2:]
    sin = [r for r in rows if r[0] == "scatter_in"][0]
    sroot, svals = int(sin[1]), sin[2:]
    scode = {v: i for i, v in enumerate(svals)}
    outs = ref.scatter(np.array([scode[v] for v in svals], dtype=np.int32), p, sroot)
    for r in rows:
        if r[0] == "scatter_out":
            assert [svals[i] for i in outs[int(r[1])]] == r[2:]


def test_gather_is_allgather_at_root_and_scatter_inverts_it():
    rng = np.random.default_rng(31)
    for p in (1, 2, 5, 8):
        n = int(rng.integers(1, 9))
        xs = [rng.integers(-100, 100, n).astype(np.int32) for _ in range(p)]
        for root in range(p):
            g = ref.gather(xs, root)
            assert np.array_equal(g, ref.allgather(xs)[root])
            back = ref.scatter(g, p, root)
            assert all(np.array_equal(a, b) for a, b in zip(back, xs))
            whole = rng.integers(-100, 100, p * n).astype(np.int32)
            assert np.array_equal(ref.gather(ref.scatter(whole, p, root), root), whole)


def test_gather_scatter_adjoint():
    """<Gather(x), y> = <x, Scatter(y)>: one copy map is the other's transpose
    (the duality of the hpc/04 page's section 1.7 applied to the single-root
    pair), exact in int64."""
    rng = np.random.default_rng(32)
    for p in (2, 3, 8):
        n = 5
        xs = [rng.integers(-1000, 1000, n).astype(np.int64) for _ in range(p)]
        y = rng.integers(-1000, 1000, p * n).astype(np.int64)
        lhs = int(np.dot(ref.gather(xs, 0), y))
        rhs = sum(int(np.dot(x, s)) for x, s in zip(xs, ref.scatter(y, p, 0)))
        assert lhs == rhs


# ----------------------------------------------------------------------------
# MoE dispatch pack and combine ("Collective Communication" page, Ragged
# All-to-All flow and Expert Parallel section)
# ----------------------------------------------------------------------------

def _route(rng, p, T, k):
    return rng.integers(0, p, T * k).astype(np.int32)


@pytest.mark.parametrize("p,T,k", [(1, 3, 1), (2, 5, 2), (3, 7, 1), (4, 9, 3), (8, 16, 2)])
def test_moe_pack_order_and_counts(p, T, k):
    """The packed order is Python's sorted() by (destination, assignment);
    counts are the destination histogram times the row length."""
    rng = np.random.default_rng(p * 100 + T)
    H = 3
    tokens = rng.integers(-9, 10, T * H).astype(np.int32)
    dest = _route(rng, p, T, k)
    counts, pos, packed = ref.moe_pack(tokens, dest, k, H, p)
    order = sorted(range(T * k), key=lambda a: (int(dest[a]), a))
    assert [int(pos[a]) for a in order] == list(range(T * k))
    assert list(counts) == [H * int((dest == j).sum()) for j in range(p)]
    for row, a in enumerate(order):
        t = a // k
        assert list(packed[row * H:(row + 1) * H]) == list(tokens[t * H:(t + 1) * H])


@pytest.mark.parametrize("dtype", [ref.F32, ref.BF16])
def test_moe_round_trip_is_identity(dtype):
    """pack -> ragged exchange -> reverse exchange (transposed counts) ->
    combine with one slot of weight 1 returns every rank's tokens exactly;
    two slots of weight 1/2 do too (halving and the sum are exact)."""
    rng = np.random.default_rng(4)
    p, T, H = 4, 11, 5
    toks = [(rng.standard_normal(T * H)).astype(np.float32) for _ in range(p)]
    if dtype == ref.BF16:
        toks = [(t.view(np.uint32) >> 16).astype(np.uint16) for t in toks]
    for k, w in ((1, [1.0]), (2, [0.5, 0.5])):
        routes = [_route(rng, p, T, k) for _ in range(p)]
        packs = [ref.moe_pack(toks[i], routes[i], k, H, p) for i in range(p)]
        C = np.stack([pk[0] for pk in packs])
        recv = ref.alltoallv([pk[2] for pk in packs], C)
        back = ref.alltoallv(recv, C.T)
        for i in range(p):
            assert np.array_equal(back[i], packs[i][2])
            weights = np.tile(np.array(w, dtype=np.float32), T)
            out = ref.moe_combine(back[i], packs[i][1], weights, k, H, dtype)
            assert np.array_equal(_bits(out), _bits(toks[i])), (k, i)


def test_moe_combine_against_pure_python():
    rng = np.random.default_rng(8)
    T, k, H = 6, 3, 4
    A = T * k
    back = rng.standard_normal(A * H).astype(np.float32)
    pos = rng.permutation(A)
    w = rng.random(A).astype(np.float32)
    res = rng.standard_normal(T * H).astype(np.float32)
    for residual in (None, res):
        got = ref.moe_combine(back, pos, w, k, H, ref.F32, residual)
        for t in range(T):
            for h in range(H):
                acc = 0.0 if residual is None else float(residual[t * H + h])
                for s_ in range(k):
                    a = t * k + s_
                    prod = struct.unpack("f", struct.pack("f", float(w[a]) * float(back[pos[a] * H + h])))[0]
                    acc = _py_add_f32(acc, prod)
                assert got[t * H + h] == np.float32(acc)


# ----------------------------------------------------------------------------
# AVG and PreMulSum (hpc/04 section 1.4 note; "Collective Communication"
# numerics section on NCCL's constrained custom reduction)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_avg_on_worked_example(dtype):
    """The worked example's sum [10 14] over p = 4 ranks: the average is
    [2.5 3.5]; int32 truncates toward zero to [2 3]; bf16 holds 2.5 and 3.5
    exactly."""
    xs, _ = _worked_example()
    arrs = [_as_dtype(x, dtype) for x in xs]
    expect = [2, 3] if dtype == ref.I32 else [2.5, 3.5]
    for out in ref.allreduce(arrs, ref.AVG, dtype):
        assert list(_to_float(out, dtype)) == expect


@pytest.mark.parametrize("p", [1, 2, 3, 4])
def test_avg_int32_bruteforce_truncates(p):
    """Every int32 input in {-3..3}^p: AVG is the sum divided by p,
    truncated toward zero (C division), for one element."""
    for vals in itertools.product(range(-3, 4), repeat=p):
        xs = [np.array([v], dtype=np.int32) for v in vals]
        got = int(ref.allreduce(xs, ref.AVG, ref.I32)[0][0])
        s_ = sum(vals)
        assert got == int(s_ / p) == (abs(s_) // p) * (1 if s_ >= 0 else -1)


@pytest.mark.parametrize("dtype", [ref.F32, ref.BF16])
def test_avg_is_rounded_sum_over_p(dtype):
    """fp32 AVG = fl(fl_sum / p) with one IEEE division; checked against
    Python's float division of the pure-Python ring-order sum, including a
    p that is not a power of two."""
    rng = np.random.default_rng(21)
    for p in (3, 5, 8):
        xs = [rng.standard_normal(64).astype(np.float32) for _ in range(p)]
        if dtype == ref.BF16:
            xs = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in xs]
        n = 64
        q = -(-n // p)
        got = _to_float(ref.allreduce(xs, ref.AVG, dtype)[0], dtype)
        widened = [_to_float(x, dtype) for x in xs]
        for i in range(n):
            ssum = _py_ring_fold([float(w[i]) for w in widened], i // q, ref.F32)
            # the double quotient rounded to fp32; differs from one rounding only
            # if the double lands exactly on an fp32 tie (probability ~2^-28)
            quo = struct.unpack("f", struct.pack("f", ssum / p))[0]
            expect = _py_bf16_rne(quo) if dtype == ref.BF16 else quo
            assert got[i] == expect, (p, i)


@pytest.mark.parametrize("dtype", [ref.F32, ref.BF16])
def test_premulsum_special_cases(dtype):
    """Scales of 1 give the plain sum bit for bit; scales of 1/p with p a
    power of two give AVG bit for bit (scaling by a power of two commutes
    with rounding); integer scales on small integers give the exact sum."""
    rng = np.random.default_rng(22)
    p, n = 8, 300
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(p)]
    if dtype == ref.BF16:
        xs = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in xs]
    ones = np.ones(p, dtype=np.float32)
    assert np.array_equal(_bits(ref.allreduce(xs, ref.SUM, dtype, scales=ones)[0]),
                          _bits(ref.allreduce(xs, ref.SUM, dtype)[0]))
    inv = np.full(p, 1.0 / p, dtype=np.float32)
    assert np.array_equal(_bits(ref.allreduce(xs, ref.SUM, dtype, scales=inv)[0]),
                          _bits(ref.allreduce(xs, ref.AVG, dtype)[0]))
    ints = [rng.integers(-20, 21, n) for _ in range(p)]
    sc = rng.integers(-3, 4, p).astype(np.float32)
    got = _to_float(ref.allreduce([_as_dtype(v, dtype) for v in ints], ref.SUM, dtype, scales=sc)[0], dtype)
    assert list(got) == list(sum(float(sc[r]) * ints[r].astype(np.float64) for r in range(p)))


def test_premulsum_reduce_scatter_matches_allreduce_blocks():
    rng = np.random.default_rng(23)
    p, n = 4, 50
    xs = [rng.standard_normal(p * n).astype(np.float32) for _ in range(p)]
    sc = rng.random(p).astype(np.float32) + 0.5
    rs = ref.reduce_scatter(xs, ref.SUM, ref.F32, scales=sc)
    ar = ref.allreduce(xs, ref.SUM, ref.F32, scales=sc)[0]
    for r in range(p):
        assert np.array_equal(_bits(rs[r]), _bits(ar[r * n:(r + 1) * n]))


@pytest.mark.parametrize("sim", ["recursive_doubling_simulated", "halving_doubling_simulated",
                                 "ring_allreduce_simulated"])
def test_avg_under_every_schedule_is_sum_divided(sim):
    rng = np.random.default_rng(24)
    p, n = 8, 40
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(p)]
    s_ = getattr(ref, sim)(xs, ref.SUM, ref.F32)
    a_ = getattr(ref, sim)(xs, ref.AVG, ref.F32)
    for r in range(p):
        assert np.array_equal(_bits(a_[r]), _bits((s_[r] / np.float32(p)).astype(np.float32)))


# ----------------------------------------------------------------------------
# Direct MoE dispatch and combine: equal to pack -> exchange -> reverse ->
# combine, bit for bit
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("p,T,k,H", [(1, 5, 1, 3), (3, 17, 2, 4), (4, 30, 3, 2), (8, 25, 2, 5)])
def test_direct_dispatch_equals_pack_then_exchange(p, T, k, H):
    rng = np.random.default_rng(60 + p * T)
    toks = [rng.integers(-50, 50, T * H).astype(np.int32) for _ in range(p)]
    dests = [rng.integers(0, p, T * k).astype(np.int64) for _ in range(p)]
    counts, slots, recv = ref.moe_dispatch_direct(toks, dests, k, H)
    packs = [ref.moe_pack(toks[i], dests[i], k, H, p) for i in range(p)]
    C = np.stack([pk[0] for pk in packs])
    assert np.array_equal(counts, C)
    via_exchange = ref.alltoallv([pk[2] for pk in packs], C)
    for j in range(p):
        assert np.array_equal(recv[j], via_exchange[j])
    rows = C // H
    for i in range(p):
        soff = np.concatenate([[0], np.cumsum(rows[i])[:-1]])
        for a in range(T * k):
            j = int(dests[i][a])
            t = a // k
            # the slot's row is the token, and it is where the exchange put the packed row
            assert np.array_equal(recv[j][slots[i][a] * H:(slots[i][a] + 1) * H], toks[i][t * H:(t + 1) * H])
            assert slots[i][a] == rows[:i, j].sum() + (packs[i][1][a] - soff[j])


@pytest.mark.parametrize("with_residual", [False, True])
def test_direct_combine_equals_reverse_then_combine(with_residual):
    p, T, k, H = 4, 23, 2, 6
    rng = np.random.default_rng(71)
    toks = [ref.f32_to_bf16_rne(rng.standard_normal(T * H).astype(np.float32)) for _ in range(p)]
    dests = [rng.integers(0, p, T * k).astype(np.int64) for _ in range(p)]
    w = [rng.random(T * k).astype(np.float32) for _ in range(p)]
    res = [ref.f32_to_bf16_rne(rng.standard_normal(T * H).astype(np.float32)) for _ in range(p)]
    counts, slots, recv = ref.moe_dispatch_direct(toks, dests, k, H)
    # experts: any per-row map; use a row-dependent scaling
    ys = [ref.f32_to_bf16_rne((ref.bf16_to_f32(r).reshape(-1, H) *
                               (1 + np.arange(len(r) // H, dtype=np.float32))[:, None] / 7).reshape(-1))
          for r in recv]
    packs = [ref.moe_pack(toks[i], dests[i], k, H, p) for i in range(p)]
    C = np.stack([pk[0] for pk in packs])
    back = ref.alltoallv(ys, C.T.copy())          # reverse exchange: the transposed matrix
    for i in range(p):
        a = ref.moe_combine_direct(ys, dests[i], slots[i], w[i], k, H, ref.BF16, res[i] if with_residual else None)
        b = ref.moe_combine(back[i], packs[i][1], w[i], k, H, ref.BF16, res[i] if with_residual else None)
        assert np.array_equal(a, b)


def test_direct_fp8_dispatch_equals_pack_then_exchange():
    from oracle import fp8
    p, T, k, H, G = 3, 11, 2, 64, 32
    rng = np.random.default_rng(72)
    toks = [ref.f32_to_bf16_rne(rng.standard_normal(T * H).astype(np.float32)) for _ in range(p)]
    dests = [rng.integers(0, p, T * k).astype(np.int64) for _ in range(p)]
    counts, slots, recv = fp8.moe_dispatch_direct_fp8(toks, dests, k, H, G)
    packs = [fp8.moe_pack_fp8(toks[i], dests[i], k, H, G, p) for i in range(p)]
    C = np.stack([pk[0] for pk in packs])
    assert np.array_equal(counts, C)
    via = ref.alltoallv([pk[2] for pk in packs], C)
    for j in range(p):
        assert np.array_equal(recv[j], via[j])


# ----------------------------------------------------------------------------
# Tree AllReduce and the double binary tree
# ----------------------------------------------------------------------------

def _py_heap_tree(vals_by_rank, ranks, dtype):
    """The heap-ordered tree fold written out with struct-rounded Python
    floats: partial(v) = (x_v + partial(2v+1)) + partial(2v+2)."""
    def part(v):
        acc = vals_by_rank[ranks[v]]
        for c in (2 * v + 1, 2 * v + 2):
            if c < len(ranks):
                acc = _py_add_f32(acc, part(c))
        return acc
    r = part(0)
    return _py_bf16_rne(r) if dtype == ref.BF16 else _f32(r)


@pytest.mark.parametrize("dtype", [ref.F32, ref.BF16])
@pytest.mark.parametrize("p", [2, 3, 4, 7, 8, 16])
def test_tree_allreduce_against_pure_python(dtype, p):
    rng = np.random.default_rng(80 + p)
    n = 2 * p + 3
    xs = [_as_dtype((rng.standard_normal(n) * 1e3).astype(np.float64), dtype) for _ in range(p)]
    got = ref.tree_allreduce_simulated(xs, ref.SUM, dtype)
    dbt = ref.double_binary_tree_simulated(xs, ref.SUM, dtype)
    q = ref.chunk_len(n, p)
    for i in range(n):
        vals = [float(_to_float([x[i]], dtype)[0]) for x in xs]
        a = _py_heap_tree(vals, list(range(p)), dtype)
        b = _py_heap_tree(vals, list(range(p - 1, -1, -1)), dtype) if i // q >= p // 2 else a
        for r in range(p):
            assert float(_to_float([got[r][i]], dtype)[0]) == a
            assert float(_to_float([dbt[r][i]], dtype)[0]) == b


def test_tree_orders_written_out_at_p4():
    """p = 4, heap order: partial(1) = x1 + x3, partial(0) = (x0 + partial(1)) + x2;
    the mirror (tree B) gives (x3 + (x2 + x0)) + x1."""
    big, one = np.float32(2.0 ** 24), np.float32(1.0)
    xs = [np.array([v], dtype=np.float32) for v in (big, one, -big, one)]
    # tree A: x1 + x3 = 2 exactly; big + 2 = big + 2; + (-big) = 2
    assert ref.tree_allreduce_simulated(xs, ref.SUM, ref.F32)[0][0] == np.float32(2.0)
    # a case that separates the two trees:
    zs = [np.array([v], dtype=np.float32) for v in (big, one, one, -big)]
    a = ref.tree_reduce_to_root(zs, [0, 1, 2, 3], ref.SUM, ref.F32)
    b = ref.tree_reduce_to_root(zs, [3, 2, 1, 0], ref.SUM, ref.F32)
    # tree A: x1 + x3 = 1 - big = -(big - 1) exact; x0 + that = 1; + x2 = 2
    assert a[0] == np.float32(2.0)
    # tree B: x2 + x0 = 1 + big -> big (round to even); x3 + big = 0; + x1 = 1
    assert b[0] == np.float32(1.0)


@pytest.mark.parametrize("op", [ref.SUM, ref.MIN, ref.MAX, ref.AVG])
def test_tree_orders_exact_on_integers(op):
    rng = np.random.default_rng(90)
    p, n = 8, 50
    xs = [rng.integers(-100, 100, n).astype(np.int32) for _ in range(p)]
    expect = ref.allreduce(xs, op, ref.I32)
    for sim in (ref.tree_allreduce_simulated, ref.double_binary_tree_simulated):
        got = sim(xs, op, ref.I32)
        for r in range(p):
            assert np.array_equal(got[r], expect[r])


def test_tree_orders_differ_from_the_others_on_floats():
    rng = np.random.default_rng(91)
    p, n = 8, 4096
    xs = [(rng.standard_normal(n) * np.exp(rng.uniform(-8, 8, n))).astype(np.float32) for _ in range(p)]
    results = [ref.allreduce(xs, ref.SUM, ref.F32)[0], ref.recursive_doubling_simulated(xs, ref.SUM, ref.F32)[0],
               ref.halving_doubling_simulated(xs, ref.SUM, ref.F32)[0],
               ref.tree_allreduce_simulated(xs, ref.SUM, ref.F32)[0],
               ref.double_binary_tree_simulated(xs, ref.SUM, ref.F32)[0]]
    for i in range(len(results)):
        for j in range(i + 1, len(results)):
            assert not np.array_equal(results[i], results[j]), (i, j)


def test_tree_shapes_match_the_figure(monkeypatch):
    """The hpc/04 page's double-binary-tree figure (section 2.4): tree A has
    0 -> (1, 2), 1 -> (3, 4), 2 -> (5, 6); tree B has 7 -> (6, 5),
    6 -> (4, 3), 5 -> (2, 1).  Symbolic operands record every combine;
    at p = 8 the heap order adds 3 -> 7 (tree A) and 4 -> 0 (tree B)."""
    monkeypatch.setattr(ref, "_widen", lambda v, dtype: np.asarray(v, dtype=object))
    monkeypatch.setattr(ref, "_combine", lambda a, b, op: np.array([f"({x}+{y})" for x, y in zip(a, b)], dtype=object))
    xs = [np.array([f"x{r}"], dtype=object) for r in range(8)]
    a = ref.tree_reduce_to_root(xs, list(range(8)), ref.SUM, ref.F32)[0]
    b = ref.tree_reduce_to_root(xs, list(range(7, -1, -1)), ref.SUM, ref.F32)[0]
    assert a == "((x0+((x1+(x3+x7))+x4))+((x2+x5)+x6))"
    assert b == "((x7+((x6+(x4+x0))+x3))+((x5+x2)+x1))"
