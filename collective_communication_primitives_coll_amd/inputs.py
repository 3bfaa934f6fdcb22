"""Seeded synthetic inputs for the collective primitives.

This module only draws numbers; it holds none of the reduction or
re-placement arithmetic.  Both the GPU path (tests, bench) and the CPU
oracle consume what it produces, so it is the one piece they share.

Every array is produced on the host with NumPy's PCG64 generator, seeded
by ``[workload_id, rank, *extra]``.  Element types are given as NumPy
dtypes; bf16 data is carried as ``uint16`` bit patterns (NumPy has no
bf16 type).

Recipes (sizes follow the workloads the collectives are measured on):

* uniform fp32 in [-1, 1): ``random(float32) * 2 - 1`` (exact in fp32,
  never -0.0 and never 1.0);
* uniform int32 in [-1000, 1000];
* normal fp32 ``N(0, sigma)`` with sigma the standard deviation;
* normal bf16: the fp32 normal truncated to its upper 16 bits (round
  toward zero).  Truncation keeps this module free of the round-to-nearest
  narrowing that the reductions themselves perform.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Workload identifiers (the first seed word).
WL_AR_SMALL = 1       # AllReduce, p=4, 2^20 elements per rank
WL_ZERO_RS_AG = 2     # ReduceScatter then AllGather, p=8, 2^26 bf16 per rank
WL_DP_RING_AR = 3     # AllReduce, p=8, 256 MiB fp32 per rank
WL_MOE_A2A = 4        # All-to-All(v), p=8, 4096 x 7168 bf16 per rank
WL_SMALL_BATCH = 5    # 10,000 small AllReduce calls, p=16
WL_TEST = 100         # free-form test inputs


def rng_for(workload: int, rank: int, *extra: int) -> np.random.Generator:
    """PCG64 stream for (workload, rank, extra...)."""
    return np.random.default_rng([int(workload), int(rank), *[int(e) for e in extra]])


def uniform_f32(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.random(n, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)


def uniform_i32(rng: np.random.Generator, n: int, lo: int = -1000, hi: int = 1000) -> np.ndarray:
    return rng.integers(lo, hi + 1, n, dtype=np.int32)


def normal_f32(rng: np.random.Generator, n: int, sigma: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def normal_bf16_bits(rng: np.random.Generator, n: int, sigma: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, sigma), truncated from fp32."""
    x = normal_f32(rng, n, sigma)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def uniform_bf16_bits(rng: np.random.Generator, n: int) -> np.ndarray:
    x = uniform_f32(rng, n)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# dtype codes shared with the C ABI enum values (F32=0, BF16=1, I32=2)
F32, BF16, I32 = 0, 1, 2
NP_DTYPE = {F32: np.float32, BF16: np.uint16, I32: np.int32}
ELEM_BYTES = {F32: 4, BF16: 2, I32: 4}


def rank_buffers(workload: int, p: int, n: int, dtype: int, dist: str = "uniform",
                 sigma: float = 1.0, extra: tuple = ()) -> list[np.ndarray]:
    """One array of ``n`` elements per rank, seeded by (workload, rank, *extra)."""
    out = []
    for r in range(p):
        g = rng_for(workload, r, *extra)
        if dtype == F32:
            out.append(uniform_f32(g, n) if dist == "uniform" else normal_f32(g, n, sigma))
        elif dtype == I32:
            out.append(uniform_i32(g, n))
        elif dtype == BF16:
            out.append(uniform_bf16_bits(g, n) if dist == "uniform" else normal_bf16_bits(g, n, sigma))
        else:
            raise ValueError(f"unknown dtype code {dtype}")
    return out


# ----------------------------------------------------------------------------
# Workload 4: MoE dispatch counts
# ----------------------------------------------------------------------------

def moe_token_counts(p: int = 8, tokens: int = 4096, seed_extra: int = 0) -> np.ndarray:
    """Token counts C_tok[src][dst] ~ Multinomial(tokens, 1/p) per source row."""
    rows = []
    for i in range(p):
        g = rng_for(WL_MOE_A2A, i, 1000 + seed_extra)
        rows.append(g.multinomial(tokens, [1.0 / p] * p))
    return np.asarray(rows, dtype=np.int64)


# ----------------------------------------------------------------------------
# Workload 5: small-message AllReduce batch
# ----------------------------------------------------------------------------

@dataclass
class SmallCall:
    n: int            # elements per rank
    dtype: int        # F32 or I32
    op: int           # 0 sum, 1 min, 2 max
    src_off: int      # element offset into the per-rank pool of this dtype
    dst_off: int      # element offset into the per-rank output pool


def small_batch_plan(ncalls: int = 10000, lo_bytes: int = 4096, hi_bytes: int = 1 << 20,
                     pool_bytes: int = 32 << 20) -> tuple[list[SmallCall], int]:
    """Message sizes log-uniform in [lo_bytes, hi_bytes), ops cycling sum/min/max,
    dtypes alternating fp32/int32 every three calls.  Sources are 256-byte
    aligned slices of a per-rank pool; destinations are packed back to back
    (each 256-byte aligned) in a per-rank output pool.

    Returns (calls, output pool size in elements).
    """
    g = rng_for(WL_SMALL_BATCH, 0, 7)
    u = g.random(ncalls)
    sizes = np.floor(np.exp(math.log(lo_bytes) + u * (math.log(hi_bytes) - math.log(lo_bytes))))
    sizes = (sizes.astype(np.int64) // 4) * 4
    pool_elems = pool_bytes // 4
    calls = []
    dst = 0
    for k in range(ncalls):
        n = int(sizes[k] // 4)
        max_off_256 = (pool_bytes - int(sizes[k])) // 256
        off = int(g.integers(0, max_off_256 + 1)) * 64  # 64 elements = 256 B
        assert off + n <= pool_elems
        calls.append(SmallCall(n=n, dtype=(F32, I32)[(k // 3) % 2], op=k % 3,
                               src_off=off, dst_off=dst))
        dst += ((n + 63) // 64) * 64
    return calls, dst


def small_batch_pools(p: int = 16, pool_bytes: int = 32 << 20) -> tuple[list[np.ndarray], list[np.ndarray]]:
    """Per-rank fp32 and int32 source pools for workload 5."""
    ne = pool_bytes // 4
    f = [uniform_f32(rng_for(WL_SMALL_BATCH, r, 1), ne) for r in range(p)]
    i = [uniform_i32(rng_for(WL_SMALL_BATCH, r, 2), ne) for r in range(p)]
    return f, i


# ----------------------------------------------------------------------------
# MoE routing: destination rank per assignment and combine weights
# ----------------------------------------------------------------------------

def moe_routes(p: int, tokens: int, k: int, workload: int = WL_MOE_A2A, extra: int = 0) -> list[np.ndarray]:
    """Per rank, int32 [tokens*k]: destination rank of assignment t*k + s,
    uniform over the p ranks (so per-pair token counts are multinomial)."""
    return [rng_for(workload, r, 2000 + extra, k).integers(0, p, tokens * k).astype(np.int32) for r in range(p)]


def moe_routes_skewed(p: int, tokens: int, k: int, alpha: float, extra: int = 0) -> list[np.ndarray]:
    """Per rank, int32 [tokens*k]: destinations drawn from probabilities that
    are themselves drawn from a symmetric Dirichlet(alpha) per source rank;
    small alpha concentrates most assignments on a few hot destinations."""
    out = []
    for r in range(p):
        g = rng_for(WL_TEST, r, 4000 + extra, k)
        prob = g.dirichlet(np.full(p, alpha))
        out.append(g.choice(p, size=tokens * k, p=prob).astype(np.int32))
    return out


def moe_weights(p: int, tokens: int, k: int, workload: int = WL_MOE_A2A, extra: int = 0) -> list[np.ndarray]:
    """Per rank, fp32 [tokens*k] combine weights uniform in [0, 1)."""
    return [rng_for(workload, r, 3000 + extra, k).random(tokens * k, dtype=np.float32) for r in range(p)]


# ----------------------------------------------------------------------------
# Special values: operands that exercise the numeric edge cases of the
# reductions (wrap-around, subnormals, overflow, rounding ties, signed zeros,
# NaN and infinities).  These only draw bit patterns from fixed pools.
# ----------------------------------------------------------------------------

EDGE_KINDS = ("int_wrap", "subnormal", "overflow", "ties", "zero_nan_inf")

_F32_SPECIAL = np.array([0x00000000, 0x80000000, 0x7FC00000, 0xFFC00000, 0x7F800000, 0xFF800000,
                         0x3F800000, 0xBF800000, 0x40000000, 0xC0000000], dtype=np.uint32)
_BF16_SPECIAL = np.array([0x0000, 0x8000, 0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x3F80, 0xBF80, 0x4000, 0xC000],
                         dtype=np.uint16)
# zero, -zero, quiet NaN (both signs), +-inf, +-1, +-2; weights favour the zeros
_SPECIAL_P = np.array([0.2, 0.2, 0.06, 0.04, 0.05, 0.05, 0.1, 0.1, 0.1, 0.1])
# bf16 values whose fp32 sums often land exactly halfway between two bf16
# neighbours: +-1, +-2^-8, +-2^-7, +-(1 + 2^-7), +-3*2^-9, +-2^-9
_BF16_TIES = np.array([0x3F80, 0xBF80, 0x3B80, 0xBB80, 0x3C00, 0xBC00, 0x3F81, 0xBF81, 0x3BC0, 0xBBC0, 0x3B00,
                       0xBB00], dtype=np.uint16)


def edge_buffers(p: int, n: int, dtype: int, kind: str, seed: int = 0) -> list[np.ndarray]:
    """Per rank, n elements of special operands (bit patterns for bf16):

    int_wrap      int32 within 1000 of INT32_MAX or INT32_MIN (sums wrap);
    subnormal     fp32 / bf16 subnormals of either sign, with some normals
                  of the smallest exponents;
    overflow      fp32 / bf16 values within a few ulps of the largest finite
                  value, either sign (sums overflow);
    ties          bf16 values whose fp32 sums often fall halfway between two
                  bf16 neighbours;
    zero_nan_inf  fp32 / bf16 +-0, quiet NaN, +-inf, +-1, +-2.
    """
    out = []
    for r in range(p):
        g = rng_for(WL_TEST, r, 7000 + EDGE_KINDS.index(kind), seed)
        if kind == "int_wrap":
            if dtype != I32:
                raise ValueError("int_wrap is int32")
            hi = g.integers(2**31 - 1000, 2**31, n, dtype=np.int64)
            lo = g.integers(-2**31, -2**31 + 1000, n, dtype=np.int64)
            out.append(np.where(g.random(n) < 0.5, hi, lo).astype(np.int32))
            continue
        if dtype == I32:
            raise ValueError(f"{kind} is a floating-point kind")
        if kind == "subnormal":
            if dtype == F32:
                mant = g.integers(1, 1 << 23, n, dtype=np.uint32)
                normal = g.integers(0x00800000, 0x00A00000, n, dtype=np.uint32)  # exponent field 1
                bits = np.where(g.random(n) < 0.8, mant, normal)
                out.append((bits | (g.integers(0, 2, n, dtype=np.uint32) << np.uint32(31))).view(np.float32))
            else:
                mant = g.integers(1, 0x80, n, dtype=np.uint16)
                normal = g.integers(0x0080, 0x00A0, n, dtype=np.uint16)
                bits = np.where(g.random(n) < 0.8, mant, normal).astype(np.uint16)
                out.append(bits | (g.integers(0, 2, n, dtype=np.uint16) << np.uint16(15)))
        elif kind == "overflow":
            sign = g.integers(0, 2, n)
            if dtype == F32:
                bits = g.integers(0x7F7FFFF0, 0x7F800000, n, dtype=np.uint32)
                bits = np.where(g.random(n) < 0.7, bits, g.integers(0x7F000000, 0x7F7FFFFF, n, dtype=np.uint32))
                out.append((bits.astype(np.uint32) | (sign.astype(np.uint32) << np.uint32(31))).view(np.float32))
            else:
                bits = g.integers(0x7F70, 0x7F80, n, dtype=np.uint16)
                bits = np.where(g.random(n) < 0.7, bits, g.integers(0x7E00, 0x7F70, n, dtype=np.uint16))
                out.append((bits.astype(np.uint16) | (sign.astype(np.uint16) << np.uint16(15))).astype(np.uint16))
        elif kind == "ties":
            if dtype != BF16:
                raise ValueError("ties is bf16")
            out.append(g.choice(_BF16_TIES, n))
        elif kind == "zero_nan_inf":
            if dtype == F32:
                out.append(g.choice(_F32_SPECIAL, n, p=_SPECIAL_P).view(np.float32))
            else:
                out.append(g.choice(_BF16_SPECIAL, n, p=_SPECIAL_P))
        else:
            raise ValueError(kind)
    return out
