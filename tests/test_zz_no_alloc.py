"""coll_allreduce_batch_noalloc (descriptor table in the library's static
device array) against coll_allreduce_batch (library-allocated table), bit
for bit, on two batches issued back to back on one stream, the second
smaller; and the size limit, rejected on the host before anything runs."""
import numpy as np
import pytest

from gpu_util import BF16, F32, I32, empty, to_dev, to_host
from collective_communication_primitives_coll_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def coll():
    import torch
    import collective_communication_primitives_coll_amd as c
    torch.cuda.set_device(0)
    c.lib()
    return c


def _batch(p, ncalls, seed, max_n):
    rng = np.random.default_rng(seed)
    host, calls_a, calls_b = [], [], []
    for k in range(ncalls):
        n = int(rng.integers(1, max_n))
        dtype = (F32, I32, BF16)[k % 3]
        op = k % 4 if dtype != BF16 else k % 3
        hx = inputs.rank_buffers(inputs.WL_TEST, p, n, dtype, dist="uniform", extra=(seed, k))
        send = [to_dev(x, dtype) for x in hx]
        calls_a.append((send, [empty(n, dtype, fill=0) for _ in range(p)], n, dtype, op))
        calls_b.append((send, [empty(n, dtype, fill=1) for _ in range(p)], n, dtype, op))
        host.append(dtype)
    return calls_a, calls_b, host


def test_noalloc_batch_matches_allocating_batch_twice(coll):
    import torch
    p = 16
    first = _batch(p, 300, 1, 20000)
    second = _batch(p, 40, 2, 3000)          # smaller: fewer calls, smaller calls
    for calls_a, calls_b, _ in (first, second):
        coll.coll_allreduce_batch(calls_a, p)
    # the two no-alloc batches back to back, no synchronisation in between
    coll.coll_allreduce_batch(first[1], p, noalloc=True)
    coll.coll_allreduce_batch(second[1], p, noalloc=True)
    torch.cuda.synchronize()
    for name, (calls_a, calls_b, dts) in (("first", first), ("second", second)):
        for k, (ca, cb, dt) in enumerate(zip(calls_a, calls_b, dts)):
            for r in range(p):
                a, b = to_host(ca[1][r], dt), to_host(cb[1][r], dt)
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{name} batch call {k} rank {r}"


def test_noalloc_batch_rejects_tables_over_the_limit(coll):
    p = 16
    ncalls = (coll.COLL_BATCH_NOALLOC_MAX_BYTES // (16 * p)) + 10
    t = empty(1, F32)
    calls = [([t] * p, [t] * p, 0, F32, 0)] * (ncalls - 1) + [([t] * p, [empty(1, F32) for _ in range(p)], 1, F32, 0)]
    # every call but the last is empty; only the size of the table is too large
    with pytest.raises(coll.CollError) as e:
        coll.coll_allreduce_batch(calls, p, noalloc=True)
    assert e.value.status == coll.COLL_ERR_INVALID_ARG
