// CPU oracle for the collective primitives, threaded C++17.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path links or loads
// this library: only the tests, the smoke check and the benchmark's
// CPU-baseline leg do.  It includes no HIP header and shares no code with
// the HIP path.  It computes exactly what oracle/ref.py computes (the tests
// hold the two bit-identical), fast enough to check the benchmark
// workloads whole.
//
// Definitions followed (page titles as printed):
//   "集合通信：原语、算法、NCCL 实现与拓扑映射" (llm-infra-atlas, hpc/04):
//     chapter preamble (p ranks, [n] per rank, elementwise sum/min/max);
//     AllGather 1.2, Reduce 1.3, AllReduce 1.4, ReduceScatter 1.5,
//     AllToAll 1.6; the ring all-reduce 2.2 (which fixes the order in
//     which a chunk's partial visits the ranks); recursive doubling and
//     halving-doubling 2.3; the double binary tree 2.4; quantized
//     communication 4.3 (FP8 e4m3 dispatch, bf16 combine).
//   "Collective Communication：AllReduce、AllGather、ReduceScatter 与
//     All-to-All" (charlestar.github.io): ragged All-to-All (per-pair
//     counts, prefix-sum offsets, the MoE pack/combine steps); reduction
//     numerics (the accumulator type and the summation order are part of
//     the result).
//
// Readings (the same as oracle/ref.py's):
//   * Ring order: element i of chunk c (c = i / q, q = ceil(n / p)) is
//     folded left to right over ranks c+1, c+2, ..., c+p (mod p).
//     ReduceScatter's block r is chunk r.
//   * fp32: IEEE binary32 add, round to nearest even, no contraction, no
//     flush of subnormals.  bf16: widened exactly to fp32, folded in fp32,
//     narrowed once with round to nearest even.  int32: add modulo 2^32.
//   * min / max: compare-select, acc = (v < acc) ? v : acc (max: v > acc);
//     ties and NaN operands keep the partial.
//   * AVG: the sum, then one IEEE fp32 division by p (int32: C division,
//     truncating toward zero).  PreMulSum: each operand times its rank's
//     fp32 scale, the product rounded on its own, then the sum.
//   * Tree orders over ranks listed in rank order: recursive doubling pairs
//     neighbours first (distance 1, 2, 4, ...), halving-doubling pairs ranks
//     p/2 apart first; the tree all-reduce folds in heap order (node v:
//     own value, then the subtree at 2v+1, then the subtree at 2v+2); the
//     double binary tree sends chunks c < p/2 through that tree and the
//     others through its mirror (node v on rank p-1-v).
//   * Alltoallv: counts[i][j] elements from rank i to rank j, send offsets
//     the prefix sums along row i, destination j packing sources 0..p-1 in
//     order.
//   * FP8 e4m3 (OCP E4M3): bias 7, subnormals m * 2^-9, no infinities,
//     largest finite 448; round to nearest even, saturating at 448.  A
//     group of G elements: amax = max(max |x|, 2^-110); inv = 448 / amax;
//     scale = amax / 448; code = e4m3(x * inv).  Packed row: the codes, the
//     group scales (fp32, little endian), zero bytes to a multiple of 16.
//     Dequantized value: bf16(decode(code) * scale).
//   * MoE combine: out[t] = residual[t] (or +0) + w_0 * y_0 + w_1 * y_1 ...
//     in fp32, slot order, every product and sum rounded, bf16 narrowed once.
//
// Threads split the element (or row, or call) range into contiguous parts.
// Every element's arithmetic is fixed by the definitions above, so the
// results do not depend on the thread count.
//
// Build: g++ -O2 -std=c++17 -fPIC -shared -ffp-contract=off -pthread
// (no -ffast-math: it would allow reassociation and flush subnormals).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

namespace {

enum { F32 = 0, BF16 = 1, I32 = 2 };
enum { SUM = 0, MIN = 1, MAX = 2, AVG = 3 };
enum { ORD_RING = 0, ORD_RD = 1, ORD_HD = 2, ORD_TREE = 3, ORD_DBT = 4 };
constexpr int kMaxP = 64;

// ---------------------------------------------------------------------------
// Threads over [0, count): part t gets a contiguous range.
// ---------------------------------------------------------------------------
void parallel_for(int64_t count, int nthreads, const std::function<void(int64_t, int64_t)>& body) {
  if (count <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > count) nthreads = (int)count;
  if (nthreads == 1) {
    body(0, count);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(nthreads);
  for (int t = 0; t < nthreads; ++t) {
    const int64_t lo = count * t / nthreads, hi = count * (t + 1) / nthreads;
    th.emplace_back([&body, lo, hi] { body(lo, hi); });
  }
  for (auto& x : th) x.join();
}

// ---------------------------------------------------------------------------
// bf16 (sign, 8 exponent bits, 7 fraction bits: the upper half of binary32)
// ---------------------------------------------------------------------------
float bf16_to_f32(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Round to nearest, ties to even, on the bit pattern: keep the upper 16
// bits, add one when the dropped lower half exceeds 0x8000, or equals it
// and the kept part is odd.  A carry moves into the exponent (up to
// infinity).  NaN becomes the quiet NaN 0x7fc0 with the input's sign.
uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if (std::isnan(f)) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
  const uint32_t kept = u >> 16, dropped = u & 0xffffu;
  const bool up = dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u));
  return (uint16_t)(kept + (up ? 1u : 0u));
}

// ---------------------------------------------------------------------------
// One operand and the elementwise combine.
// ---------------------------------------------------------------------------
// Accumulator: fp32 for fp32 and bf16, int32 for int32.
struct Acc {
  float f;
  int32_t i;
};

Acc load(const void* base, int dtype, int64_t idx) {
  Acc a{0.0f, 0};
  if (dtype == F32) a.f = ((const float*)base)[idx];
  else if (dtype == BF16) a.f = bf16_to_f32(((const uint16_t*)base)[idx]);
  else a.i = ((const int32_t*)base)[idx];
  return a;
}

Acc scaled(Acc a, int dtype, const float* scales, int rank) {
  if (scales && dtype != I32) a.f = scales[rank] * a.f;  // one rounded product
  return a;
}

Acc combine(Acc acc, Acc v, int dtype, int op) {
  if (dtype == I32) {
    if (op == SUM || op == AVG) acc.i = (int32_t)((uint32_t)acc.i + (uint32_t)v.i);  // mod 2^32
    else if (op == MIN) acc.i = (v.i < acc.i) ? v.i : acc.i;
    else acc.i = (v.i > acc.i) ? v.i : acc.i;
  } else {
    if (op == SUM || op == AVG) acc.f = acc.f + v.f;
    else if (op == MIN) acc.f = (v.f < acc.f) ? v.f : acc.f;
    else acc.f = (v.f > acc.f) ? v.f : acc.f;
  }
  return acc;
}

void store(void* base, int dtype, int64_t idx, Acc acc, int op, int p) {
  if (op == AVG) {
    if (dtype == I32) acc.i = acc.i / p;        // C division truncates toward zero
    else acc.f = acc.f / (float)p;              // one IEEE division
  }
  if (dtype == F32) ((float*)base)[idx] = acc.f;
  else if (dtype == BF16) ((uint16_t*)base)[idx] = f32_to_bf16(acc.f);
  else ((int32_t*)base)[idx] = acc.i;
}

// Rank listed k-th in the ring order of chunk c.
int ring_rank(int c, int k, int p) { return (c + 1 + k) % p; }

// The reduction of element `idx` of p operand buffers, in the given order,
// for an element of chunk c.  Returns the accumulator before AVG/narrowing.
Acc reduce_one(const void* const* xs, int p, int64_t idx, int c, int dtype, int op, int order,
               const float* scales) {
  if (order == ORD_RING) {
    Acc acc = scaled(load(xs[ring_rank(c, 0, p)], dtype, idx), dtype, scales, ring_rank(c, 0, p));
    for (int k = 1; k < p; ++k) {
      const int r = ring_rank(c, k, p);
      acc = combine(acc, scaled(load(xs[r], dtype, idx), dtype, scales, r), dtype, op);
    }
    return acc;
  }
  // Tree orders: operand v is listed rank v (the double binary tree's
  // second tree lists the ranks mirrored).
  Acc a[kMaxP];
  const bool mirror = order == ORD_DBT && c >= p / 2;
  for (int v = 0; v < p; ++v) {
    const int r = mirror ? p - 1 - v : v;
    a[v] = scaled(load(xs[r], dtype, idx), dtype, scales, r);
  }
  if (order == ORD_RD) {
    for (int st = 1; st < p; st *= 2)
      for (int k = 0; k + st < p; k += 2 * st) a[k] = combine(a[k], a[k + st], dtype, op);
  } else if (order == ORD_HD) {
    for (int st = p / 2; st >= 1; st /= 2)
      for (int k = 0; k < st; ++k) a[k] = combine(a[k], a[k + st], dtype, op);
  } else {
    // heap order, leaves first: every subtree is complete before its parent
    for (int v = p - 1; v >= 0; --v) {
      if (2 * v + 1 < p) a[v] = combine(a[v], a[2 * v + 1], dtype, op);
      if (2 * v + 2 < p) a[v] = combine(a[v], a[2 * v + 2], dtype, op);
    }
  }
  return a[0];
}

bool is_pow2(int p) { return p >= 1 && (p & (p - 1)) == 0; }

bool args_ok(int p, int dtype, int op, int order) {
  if (p < 1 || p > kMaxP) return false;
  if (dtype < F32 || dtype > I32 || op < SUM || op > AVG) return false;
  if (order < ORD_RING || order > ORD_DBT) return false;
  if ((order == ORD_RD || order == ORD_HD) && !is_pow2(p)) return false;
  return true;
}

// ---------------------------------------------------------------------------
// FP8 e4m3 (OCP E4M3)
// ---------------------------------------------------------------------------
constexpr double kE4m3Max = 448.0;

double e4m3_value(uint8_t code) {
  const int e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? m * std::ldexp(1.0, -9) : (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
  return (code & 0x80) ? -mag : mag;
}

// Nearest code, ties to the even mantissa, saturating at 448.
uint8_t e4m3_encode(float x) {
  const uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  if (std::isnan(x)) return sign | 0x7f;
  double a = std::fabs((double)x);
  if (a > kE4m3Max) a = kE4m3Max;
  // spacing of the representable values around a: 2^(e-3) in [2^e, 2^(e+1))
  // for e >= -6, the subnormal quantum 2^-9 below 2^-6
  int ex = 0;
  std::frexp(a, &ex);                       // a = f * 2^ex, f in [0.5, 1)
  int e = a == 0.0 ? -6 : ex - 1;
  if (e < -6) e = -6;
  const double quantum = std::ldexp(1.0, e - 3);
  const double q = std::nearbyint(a / quantum) * quantum;  // default mode: ties to even
  if (q < std::ldexp(1.0, -6)) return sign | (uint8_t)std::nearbyint(q / std::ldexp(1.0, -9));
  int qx = 0;
  std::frexp(q, &qx);
  const int qe = qx - 1;
  const int mant = (int)std::nearbyint((q / std::ldexp(1.0, qe) - 1.0) * 8.0);
  return sign | (uint8_t)(((qe + 7) << 3) | mant);
}

int64_t fp8_row_bytes(int64_t hidden, int64_t group) {
  const int64_t ng = hidden / group;
  return hidden + 16 * ((4 * ng + 15) / 16);
}

// One packed row of the bf16 token row x.
void fp8_encode_row(const uint16_t* x, int64_t hidden, int64_t group, uint8_t* row) {
  const int64_t ng = hidden / group;
  std::memset(row, 0, (size_t)fp8_row_bytes(hidden, group));
  for (int64_t g = 0; g < ng; ++g) {
    float amax = 0.0f;
    for (int64_t e = 0; e < group; ++e) {
      const float v = std::fabs(bf16_to_f32(x[g * group + e]));
      if (v > amax) amax = v;
    }
    const float floor_ = std::ldexp(1.0f, -110);
    if (amax < floor_) amax = floor_;
    const float inv = (float)kE4m3Max / amax;
    const float scale = amax / (float)kE4m3Max;
    for (int64_t e = 0; e < group; ++e) row[g * group + e] = e4m3_encode(bf16_to_f32(x[g * group + e]) * inv);
    std::memcpy(row + hidden + 4 * g, &scale, 4);
  }
}

}  // namespace

#define ORACLE_EXPORT extern "C" __attribute__((visibility("default")))

// All functions return 0 on success and -1 on an invalid argument.

// AllReduce ([A] 1.4): out[i] = the reduction of x_0[i], ..., x_{p-1}[i]
// in the order `order` (0 ring, 1 recursive doubling, 2 halving-doubling,
// 3 tree, 4 double binary tree) with chunks of q = ceil(n/p).  Every rank
// receives the same vector, so there is one output.  scales (optional, p
// fp32 values): PreMulSum, fp32 and bf16 sums only.
ORACLE_EXPORT int oracle_allreduce(const void* const* xs, void* out, int p, int64_t n, int dtype, int op, int order,
                                   const float* scales, int nthreads) {
  if (!args_ok(p, dtype, op, order) || n < 0) return -1;
  if (scales && (dtype == I32 || op != SUM)) return -1;
  const int64_t q = n > 0 ? (n + p - 1) / p : 1;
  parallel_for(n, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) {
      const int c = (int)(i / q);
      store(out, dtype, i, reduce_one(xs, p, i, c, dtype, op, order, scales), op, p);
    }
  });
  return 0;
}

// ReduceScatter ([A] 1.5): every rank holds [p * n]; rank r receives
// block r of the reduction, folded in the ring order of chunk r.
ORACLE_EXPORT int oracle_reduce_scatter(const void* const* xs, void* const* outs, int p, int64_t n, int dtype,
                                        int op, const float* scales, int nthreads) {
  if (!args_ok(p, dtype, op, ORD_RING) || n < 0) return -1;
  if (scales && (dtype == I32 || op != SUM)) return -1;
  parallel_for((int64_t)p * n, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t g = lo; g < hi; ++g) {
      const int r = (int)(g / n);
      const int64_t j = g - (int64_t)r * n;
      store(outs[r], dtype, j, reduce_one(xs, p, (int64_t)r * n + j, r, dtype, op, ORD_RING, scales), op, p);
    }
  });
  return 0;
}

// AllGather ([A] 1.2): out[r] = x_0 | x_1 | ... | x_{p-1} for every r.
ORACLE_EXPORT int oracle_allgather(const void* const* xs, void* const* outs, int p, int64_t n, int elem_bytes,
                                   int nthreads) {
  if (p < 1 || p > kMaxP || n < 0 || elem_bytes < 1) return -1;
  const int64_t nb = n * elem_bytes;
  parallel_for((int64_t)p * p, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t g = lo; g < hi; ++g) {
      const int r = (int)(g / p), s = (int)(g % p);
      std::memcpy((char*)outs[r] + s * nb, xs[s], (size_t)nb);
    }
  });
  return 0;
}

// Alltoallv ("Collective Communication" page, ragged All-to-All):
// counts[i * p + j] elements of rank i, from offset sum_{k<j} counts[i][k],
// go to rank j at offset sum_{k<i} counts[k][j].  The equal-split
// All-to-All ([A] 1.6) is the case of equal counts.
ORACLE_EXPORT int oracle_alltoallv(const void* const* xs, void* const* outs, int p, const int64_t* counts,
                                   int elem_bytes, int nthreads) {
  if (p < 1 || p > kMaxP || !counts || elem_bytes < 1) return -1;
  for (int64_t k = 0; k < (int64_t)p * p; ++k)
    if (counts[k] < 0) return -1;
  parallel_for((int64_t)p * p, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t g = lo; g < hi; ++g) {
      const int i = (int)(g / p), j = (int)(g % p);
      int64_t soff = 0, roff = 0;
      for (int k = 0; k < j; ++k) soff += counts[i * p + k];
      for (int k = 0; k < i; ++k) roff += counts[k * p + j];
      std::memcpy((char*)outs[j] + roff * elem_bytes, (const char*)xs[i] + soff * elem_bytes,
                  (size_t)(counts[i * p + j] * elem_bytes));
    }
  });
  return 0;
}

// Independent AllReduces in ring order: call k reduces src[k * p + r]
// (rank r's input, n[k] elements of dtype[k]) with op[k] into out[k].
ORACLE_EXPORT int oracle_allreduce_batch(int ncalls, int p, const int64_t* n, const int* dtype, const int* op,
                                         const void* const* src, void* const* out, int nthreads) {
  if (ncalls < 0 || p < 1 || p > kMaxP) return -1;
  for (int k = 0; k < ncalls; ++k)
    if (!args_ok(p, dtype[k], op[k], ORD_RING) || n[k] < 0) return -1;
  parallel_for(ncalls, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t k = lo; k < hi; ++k) oracle_allreduce(src + k * p, out[k], p, n[k], dtype[k], op[k], ORD_RING,
                                                       nullptr, 1);
  });
  return 0;
}

// Bytes of one packed FP8 row.
ORACLE_EXPORT int64_t oracle_fp8_row_bytes(int64_t hidden, int64_t group) {
  if (hidden <= 0 || group <= 0 || hidden % group) return -1;
  return fp8_row_bytes(hidden, group);
}

// Packed FP8 rows ([A] 4.3) of `rows` bf16 token rows of `hidden` elements.
ORACLE_EXPORT int oracle_fp8_encode_rows(const uint16_t* tokens, int64_t rows, int64_t hidden, int64_t group,
                                         uint8_t* out, int nthreads) {
  if (rows < 0 || hidden <= 0 || group <= 0 || hidden % group) return -1;
  const int64_t R = fp8_row_bytes(hidden, group);
  parallel_for(rows, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t) fp8_encode_row(tokens + t * hidden, hidden, group, out + t * R);
  });
  return 0;
}

// bf16 rows of `rows` packed FP8 rows: bf16(decode(code) * scale).
ORACLE_EXPORT int oracle_fp8_dequant_rows(const uint8_t* packed, int64_t rows, int64_t hidden, int64_t group,
                                          uint16_t* out, int nthreads) {
  if (rows < 0 || hidden <= 0 || group <= 0 || hidden % group) return -1;
  const int64_t R = fp8_row_bytes(hidden, group);
  parallel_for(rows, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t) {
      const uint8_t* row = packed + t * R;
      for (int64_t e = 0; e < hidden; ++e) {
        float scale;
        std::memcpy(&scale, row + hidden + 4 * (e / group), 4);
        out[t * hidden + e] = f32_to_bf16((float)e4m3_value(row[e]) * scale);
      }
    }
  });
  return 0;
}

// One rank's MoE weighted combine: for token t,
// out[t] = residual[t] (or +0) + sum_s w[t*k+s] * rows[slot[t*k+s]]
// (fp32, slot order, each product and sum rounded; bf16 narrowed once).
// rows: the returned expert rows ([rows_total x hidden], dtype 0 or 1).
ORACLE_EXPORT int oracle_moe_combine(const void* rows, const int64_t* slot, const float* w, const void* residual,
                                     void* out, int64_t tokens, int k, int64_t hidden, int dtype, int nthreads) {
  if (tokens < 0 || k < 1 || hidden <= 0 || (dtype != F32 && dtype != BF16)) return -1;
  parallel_for(tokens, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t)
      for (int64_t e = 0; e < hidden; ++e) {
        float acc = residual ? load(residual, dtype, t * hidden + e).f : 0.0f;
        for (int s = 0; s < k; ++s) {
          const int64_t a = t * k + s;
          const float prod = w[a] * load(rows, dtype, slot[a] * hidden + e).f;
          acc = acc + prod;
        }
        store(out, dtype, t * hidden + e, Acc{acc, 0}, SUM, 1);
      }
  });
  return 0;
}

// Threads a machine offers (std::thread::hardware_concurrency, at least 1).
ORACLE_EXPORT int oracle_hardware_threads(void) {
  const unsigned h = std::thread::hardware_concurrency();
  return h ? (int)h : 1;
}
