"""CPU oracle for the quantized MoE dispatch (FP8 e4m3 payload).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this file:
only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP path.

What the pages fix: "集合通信：原语、算法、NCCL 实现与拓扑映射" (hpc/04),
section 4.3 (quantized communication): MoE dispatch sends its payload as
FP8 e4m3 and the combine stays in BF16, halving the All-to-All bytes.
The pages name the format and nothing more.  Readings taken:

F1. e4m3 is the OCP 8-bit floating point format E4M3: sign bit, 4
    exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
    the subnormals m * 2^-9; no infinities; S.1111.111 is NaN; the
    largest finite value is 448 (S.1111.110).
F2. Encoding rounds to nearest, ties to even, and saturates: every
    magnitude at or above 448 encodes as +-448.  NaN encodes as S.1111.111.
F3. Scaling: each token row is cut into groups of G consecutive elements
    (G divides the hidden size).  A group's amax is the largest |x| of its
    bf16 values (exact in fp32), floored at 2^-110 so that all-zero groups
    and tiny values keep finite factors.  In fp32, with each operation
    rounded to nearest even: inv = 448 / amax, scale = amax / 448,
    code = encode(x * inv).  The element that attains amax encodes as
    +-448.
F4. Row format: the G-groups' codes (hidden bytes), then the groups' fp32
    scales, then zero bytes up to a multiple of 16 bytes:
    row_bytes = hidden + 16 * ceil(4 * (hidden / G) / 16).
F5. Dequantization for a consumer that wants bf16: y = bf16_rne(decode(code)
    * scale), the product rounded to fp32 first.
F6. Packing and routing are those of the bf16 dispatch (ref.moe_pack):
    assignments grouped by destination, stable in assignment index; the
    exchange counts are in bytes (rows * row_bytes).
"""
from __future__ import annotations

import numpy as np

from . import ref

E4M3_MAX = 448.0
AMAX_FLOOR = np.float32(2.0 ** -110)
_MIN_NORMAL = 2.0 ** -6
_SUB_QUANTUM = 2.0 ** -9


# ----------------------------------------------------------------------------
# The e4m3 format (reading F1, F2)
# ----------------------------------------------------------------------------

def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of every code, as float32 (exact: every e4m3 value is an fp32)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * _SUB_QUANTUM, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return (sign * mag).astype(np.float32)


def e4m3_encode(values: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code (ties to even mantissa), saturating at +-448."""
    v = np.asarray(values, dtype=np.float32).astype(np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))      # saturation
    # spacing of the e4m3 values around a: 2^(e-3) for a in [2^e, 2^(e+1)),
    # and the subnormal quantum 2^-9 below the smallest normal 2^-6
    _, ex = np.frexp(a)                                   # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    quantum = np.exp2(e - 3.0)
    q = np.rint(a / quantum) * quantum                    # exact in fp64; rint ties to even
    # code of the representable value q
    _, qx = np.frexp(q)
    qe = qx.astype(np.int64) - 1
    normal = q >= _MIN_NORMAL
    qe_n = np.where(normal, qe, 0)
    mant = np.where(normal, (q / np.exp2(qe_n) - 1.0) * 8.0, q / _SUB_QUANTUM)
    field = np.where(normal, qe_n + 7, 0)
    code = (field << 3) | np.rint(mant).astype(np.int64)
    code = np.where(nan, 0x7F, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


# ----------------------------------------------------------------------------
# Group scaling and the row format (readings F3, F4, F5)
# ----------------------------------------------------------------------------

def row_bytes(hidden: int, group: int) -> int:
    ngroups = hidden // group
    return hidden + 16 * ((4 * ngroups + 15) // 16)


def quantize_row(x: np.ndarray, group: int):
    """x: one token row as float32 (widened bf16).  Returns (codes uint8
    [hidden], scales float32 [hidden / group])."""
    x = np.asarray(x, dtype=np.float32)
    g = x.reshape(-1, group)
    amax = np.max(np.abs(g), axis=1).astype(np.float32)
    amax = np.maximum(amax, AMAX_FLOOR)
    inv = (np.float32(E4M3_MAX) / amax).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    y = (g * inv[:, None]).astype(np.float32)
    return e4m3_encode(y).reshape(-1), scale


def encode_row(x: np.ndarray, group: int) -> np.ndarray:
    """One packed row (reading F4) of a float32 token row."""
    codes, scale = quantize_row(x, group)
    out = np.zeros(row_bytes(len(x), group), dtype=np.uint8)
    out[:len(x)] = codes
    out[len(x):len(x) + 4 * len(scale)] = scale.astype("<f4").view(np.uint8)
    return out


def dequantize_rows(rows: np.ndarray, hidden: int, group: int) -> np.ndarray:
    """bf16 bits [N * hidden] of N packed rows (reading F5)."""
    R = row_bytes(hidden, group)
    rows = np.asarray(rows, dtype=np.uint8).reshape(-1, R)
    ng = hidden // group
    codes = rows[:, :hidden]
    scales = np.ascontiguousarray(rows[:, hidden:hidden + 4 * ng]).view("<f4").reshape(-1, ng)
    vals = e4m3_decode(codes).reshape(len(rows), ng, group)
    y = (vals * scales[:, :, None].astype(np.float32)).astype(np.float32)
    return ref.f32_to_bf16_rne(y.reshape(-1))


# ----------------------------------------------------------------------------
# Dispatch pack (reading F6)
# ----------------------------------------------------------------------------

def moe_pack_fp8(tokens_bf16: np.ndarray, dest: np.ndarray, k: int, hidden: int, group: int, p: int):
    """One rank's quantized dispatch pack.

    Returns (counts, pos, packed): counts[j] = bytes sent to rank j;
    pos[a] = packed row of assignment a; packed = rows of row_bytes bytes,
    row pos[a] holding the encoded token a // k."""
    T = len(tokens_bf16) // hidden
    # routing only: a payload of one element per token (its index)
    rows_per_dest, pos, _ = ref.moe_pack(np.arange(T), dest, k, 1, p)
    R = row_bytes(hidden, group)
    x = ref.bf16_to_f32(np.asarray(tokens_bf16, dtype=np.uint16)).reshape(T, hidden)
    enc = [encode_row(x[t], group) for t in range(T)]
    A = len(pos)
    packed = np.zeros(A * R, dtype=np.uint8)
    for a in range(A):
        packed[pos[a] * R:(pos[a] + 1) * R] = enc[a // k]
    return rows_per_dest * R, pos, packed


def moe_dispatch_direct_fp8(tokens_bf16: list[np.ndarray], dests: list[np.ndarray], k: int, hidden: int,
                            group: int):
    """The direct dispatch (ref.moe_dispatch_direct) of encoded rows: recv[j]
    holds row_bytes-byte rows; counts are in bytes."""
    R = row_bytes(hidden, group)
    enc = []
    for tok in tokens_bf16:
        x = ref.bf16_to_f32(np.asarray(tok, dtype=np.uint16)).reshape(-1, hidden)
        enc.append(np.concatenate([encode_row(x[t], group) for t in range(len(x))]) if len(x) else
                   np.zeros(0, dtype=np.uint8))
    counts, slots, recv = ref.moe_dispatch_direct(enc, dests, k, R)
    return counts, slots, recv

