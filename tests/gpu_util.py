"""Host <-> device helpers for the GPU tests (plumbing only)."""
from __future__ import annotations

import numpy as np

F32, BF16, I32 = 0, 1, 2


def torch_dtype(dtype: int):
    import torch
    return {F32: torch.float32, BF16: torch.bfloat16, I32: torch.int32}[dtype]


def to_dev(a: np.ndarray, dtype: int, dev="cuda"):
    import torch
    if dtype == BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dev)


def to_host(t, dtype: int) -> np.ndarray:
    import torch
    t = t.detach()
    if dtype == BF16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty(n: int, dtype: int, dev="cuda", fill=None):
    import torch
    t = torch.empty(n, dtype=torch_dtype(dtype), device=dev)
    if fill is not None:
        if dtype == BF16:
            v = fill & 0xFFFF
            t.view(torch.int16).fill_(v - 0x10000 if v >= 0x8000 else v)
        else:
            v = fill & 0xFFFFFFFF
            t.view(torch.int32).fill_(v - (1 << 32) if v >= 0x80000000 else v)
    return t


def bits(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


def assert_bits_equal(got: np.ndarray, expect: np.ndarray, what: str = "") -> None:
    g, e = bits(got), bits(expect)
    assert g.shape == e.shape, (what, g.shape, e.shape)
    if not np.array_equal(g, e):
        bad = np.nonzero(g != e)[0]
        i = int(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {len(g)} elements differ; first at {i}: "
                             f"got {got[i]!r} expected {expect[i]!r}")


def bf16_ordered(u16: np.ndarray) -> np.ndarray:
    """Map bf16 patterns to integers whose order is the numeric order."""
    v = u16.astype(np.int32)
    return np.where(v & 0x8000, -(v & 0x7FFF), v & 0x7FFF)


def assert_fp32_close(got: np.ndarray, expect: np.ndarray, abs_sum: np.ndarray, rel: float = 1e-5,
                      what: str = "") -> None:
    """|got - expect| <= rel * sum_r |x_r| elementwise."""
    d = np.abs(got.astype(np.float64) - expect.astype(np.float64))
    lim = rel * abs_sum.astype(np.float64)
    if not np.all(d <= lim):
        i = int(np.argmax(d - lim))
        raise AssertionError(f"{what}: element {i} off by {d[i]} > {lim[i]}")


def assert_bf16_within_ulp(got: np.ndarray, expect: np.ndarray, ulps: int = 1, what: str = "") -> None:
    dg, de = bf16_ordered(got), bf16_ordered(expect)
    diff = np.abs(dg - de)
    if not np.all(diff <= ulps):
        i = int(np.argmax(diff))
        raise AssertionError(f"{what}: element {i} differs by {diff[i]} bf16 ulps")


def nan_mask(a: np.ndarray) -> np.ndarray:
    """NaN positions of an fp32 array or of bf16 bit patterns (uint16)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return ((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)
    if a.dtype == np.float32:
        return np.isnan(a)
    return np.zeros(a.shape, dtype=bool)


def assert_bits_equal_nan(got: np.ndarray, expect: np.ndarray, what: str = "") -> None:
    """Bit-exact except where the oracle's result is a NaN made by an
    addition: IEEE 754 leaves the sign and payload of such a NaN open, so
    there the kernel's result only has to be a NaN too."""
    gm, em = nan_mask(got), nan_mask(expect)
    if not np.array_equal(gm, em):
        i = int(np.nonzero(gm != em)[0][0])
        raise AssertionError(f"{what}: NaN positions differ; first at {i}: got {got[i]!r} expected {expect[i]!r}")
    keep = ~em
    assert_bits_equal(np.asarray(got)[keep], np.asarray(expect)[keep], what)
