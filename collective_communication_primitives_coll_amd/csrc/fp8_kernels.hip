// Quantized MoE dispatch: FP8 e4m3 payload with one fp32 scale per group.
//
// "集合通信：原语、算法、NCCL 实现与拓扑映射" (hpc/04), section 4.3: the
// dispatch direction of an MoE layer may travel as FP8 e4m3 while the
// combine direction stays bf16, which halves the dispatch bytes.  The
// format is the OCP E4M3 one (bias 7, subnormals m * 2^-9, no infinities,
// S.1111.111 = NaN, largest finite 448).
//
// Pack: one wave per (rank, token).  The token row is loaded once into
// registers (16 elements = two 16-byte vectors per unit, units j =
// u*64 + lane), every group's amax is reduced with lane shuffles (groups
// of up to 1024 elements sit inside one unit column of the wave; larger
// groups span whole unit columns), each element is multiplied by
// 448/amax and encoded, and the codes, scales and padding are written to
// the packed row of every slot (assignment) of the token.
//
// Encoding rescales |y| by a power of two so that its e4m3 neighbours
// become consecutive integers, rounds to even there, and assembles the
// code; one formula serves the normal and the subnormal range.
//
// Dequant: one wave per received row; codes decode exactly to fp32, are
// multiplied by the group scale and narrowed to bf16 (round to nearest
// even).  Rows per rank come from the byte counts on the device.
#include "device_common.h"

namespace coll {

namespace {

constexpr int kLanes = 64;
constexpr int kDeqBatch = 4;  // units per lane loaded together in the dequant

__device__ __forceinline__ uint64_t fp8_wave_id() {
  return (uint64_t)blockIdx.x * (kBlock / kLanes) + (uint64_t)__builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
}
__device__ __forceinline__ uint64_t fp8_wave_count() { return (uint64_t)gridDim.x * (kBlock / kLanes); }

// e4m3 code of an fp32 value: nearest, ties to even, saturating at +-448.
// With E = max(exponent of |y|, -6), the e4m3 neighbours of |y| are the
// multiples of 2^(E-3), so m = rint(|y| * 2^(3-E)) is the rounded
// significand: 8..16 in the normal range (16 carries into the next
// binade) and 0..8 for |y| < 2^-6 (the subnormals, 8 being 2^-6).  Then
// code = ((E + 7) << 3) + m - 8 covers both ranges.  Clamping |y| to 448
// first gives the saturation.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t a = min(u & 0x7fffffffu, 0x43e00000u);  // |y| clamped to 448
  const uint32_t eb = max(a >> 23, 121u);                // biased exponent, at least 127 - 6
  const float m = __builtin_rintf(__builtin_ldexpf(__uint_as_float(a), 130 - (int)eb));
  uint32_t c = ((eb - 120u) << 3) + (uint32_t)m - 8u;
  if ((u & 0x7fffffffu) > 0x7f800000u) c = 0x7fu;        // NaN
  return c | ((u >> 24) & 0x80u);
}

// Exact fp32 value of an e4m3 code.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  if (e == 15u && m == 7u) v = __uint_as_float(0x7fc00000u);
  return (c & 0x80u) ? -v : v;
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Largest |x| of 16 bf16 elements, as a bf16 pattern: for finite values
// the magnitude order is the integer order of the low 15 bits, so the two
// halves of every word are compared with one packed 16-bit max.
__device__ __forceinline__ uint32_t unit_amax_bits(const u32x4& x0, const u32x4& x1) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x0[e] & 0x7fff7fffu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x1[e] & 0x7fff7fffu));
  }
  return m[0] > m[1] ? m[0] : m[1];
}

// Codes of 16 bf16 elements (x0: elements 0..7, x1: 8..15) times inv.
__device__ __forceinline__ u32x4 unit_codes(const u32x4& x0, const u32x4& x1, float inv) {
  u32x4 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4& x = q < 2 ? x0 : x1;
    const uint32_t w0 = x[2 * (q & 1)], w1 = x[2 * (q & 1) + 1];
    out[q] = e4m3_code(bf16_lo(w0) * inv) | (e4m3_code(bf16_hi(w0) * inv) << 8) |
             (e4m3_code(bf16_lo(w1) * inv) << 16) | (e4m3_code(bf16_hi(w1) * inv) << 24);
  }
  return out;
}

}  // namespace

// UMAX: units (16 elements) per lane the row needs, rounded up to a power
// of two; hidden <= 64 * 16 * UMAX.
template <int UMAX>
COLL_STREAM_KERNEL void moe_pack_fp8_kernel(Fp8Args a) {
#pragma clang fp contract(off)
  const int lane = (int)(threadIdx.x % kLanes);
  const uint64_t H = a.hidden, R = a.row_bytes;
  const int k = a.k;
  const uint64_t A = a.tokens * (uint64_t)k;
  const uint32_t nunits = (uint32_t)(H / 16);             // <= 1024
  const uint32_t g16 = (uint32_t)(a.group / 16);          // units per group
  const uint32_t gu = g16 > kLanes ? g16 / kLanes : 1u;   // unit columns per group (large groups)
  const uint32_t ngroups = (uint32_t)(H / a.group);
  const uint32_t npad = (uint32_t)((R - H) / 4) - ngroups;  // zero scale slots
  const uint64_t rows = a.tokens * (uint64_t)a.p;
  for (uint64_t r = fp8_wave_id(); r < rows; r += fp8_wave_count()) {
    const int rank = (int)(r / a.tokens);
    const uint64_t t = r - (uint64_t)rank * a.tokens;
    const int32_t* pp = a.pos[rank] + t * (uint64_t)k;
    bool any = false;
    for (int s = 0; s < k; ++s) {
      const int32_t ps = pp[s];
      any |= ps >= 0 && (uint64_t)ps < A;
    }
    if (!any) continue;
    const u32x4* src = reinterpret_cast<const u32x4*>((const uint16_t*)a.src[rank] + t * H);
    u32x4 x[UMAX][2];
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
      const uint32_t j = (uint32_t)(u * kLanes + lane);
      if (j < nunits) {
        x[u][0] = ld16<true>(src + 2 * j);
        x[u][1] = ld16<true>(src + 2 * j + 1);
      } else {
        x[u][0] = u32x4{0, 0, 0, 0};
        x[u][1] = u32x4{0, 0, 0, 0};
      }
    }
    uint32_t mb[UMAX];  // group amax as a bf16 magnitude pattern
#pragma unroll
    for (int u = 0; u < UMAX; ++u) mb[u] = unit_amax_bits(x[u][0], x[u][1]);
    if (g16 <= (uint32_t)kLanes) {
      // a group is g16 adjacent lanes of one unit column
#pragma unroll
      for (int u = 0; u < UMAX; ++u)
        for (uint32_t off = 1; off < g16; off <<= 1) mb[u] = max(mb[u], (uint32_t)__shfl_xor((int)mb[u], (int)off));
    } else {
      // a group is gu whole unit columns
#pragma unroll
      for (int u = 0; u < UMAX; ++u)
#pragma unroll
        for (int off = 1; off < kLanes; off <<= 1) mb[u] = max(mb[u], (uint32_t)__shfl_xor((int)mb[u], off));
      uint32_t gm[UMAX];
#pragma unroll
      for (int u = 0; u < UMAX; ++u) {
        const uint32_t gi = (uint32_t)u / gu;
        uint32_t m = 0;
#pragma unroll
        for (int v = 0; v < UMAX; ++v)
          if ((uint32_t)v / gu == gi) m = max(m, mb[v]);
        gm[u] = m;
      }
#pragma unroll
      for (int u = 0; u < UMAX; ++u) mb[u] = gm[u];
    }
    // quantize in place: x[u][0] becomes the unit's 16 codes, am[u] its scale
    float am[UMAX];
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
      const float amax = fmaxf(__uint_as_float(mb[u] << 16), 0x1p-110f);
      x[u][0] = unit_codes(x[u][0], x[u][1], 448.0f / amax);
      am[u] = amax / 448.0f;
    }
    for (int s = 0; s < k; ++s) {
      const int32_t ps = pp[s];
      if (ps < 0 || (uint64_t)ps >= A) continue;
      uint8_t* row = (uint8_t*)a.dst[rank] + (uint64_t)ps * R;
      u32x4* vc = reinterpret_cast<u32x4*>(row);
      float* sc = reinterpret_cast<float*>(row + H);
#pragma unroll
      for (int u = 0; u < UMAX; ++u) {
        const uint32_t j = (uint32_t)(u * kLanes + lane);
        if (j < nunits) {
          st16<true>(vc + j, x[u][0]);
          const bool lead = g16 <= (uint32_t)kLanes ? (j % g16) == 0 : (lane == 0 && (uint32_t)u % gu == 0);
          if (lead) sc[j / g16] = am[u];
        }
      }
      if ((uint32_t)lane < npad) sc[ngroups + lane] = 0.0f;
    }
  }
}

// out[rank] rows = dequantized received rows, in the order they arrived.
COLL_STREAM_KERNEL void moe_dequant_fp8_kernel(Fp8Args a) {
#pragma clang fp contract(off)
  __shared__ int64_t start[kMaxRanks + 1];
  __shared__ int bad;
  const int p = a.p;
  const int tid = threadIdx.x;
  const uint64_t H = a.hidden, R = a.row_bytes;
  if (tid == 0) bad = 0;
  __syncthreads();
  if (tid < p) {
    const int64_t cap = a.rows_cap[tid] * (int64_t)R;
    int64_t tot = 0;
    bool ok = true;
    for (int i = 0; i < p; ++i) {
      const int64_t c = a.counts[(int64_t)i * p + tid];
      if (c < 0 || c > cap || c % (int64_t)R) ok = false;
      else tot += c;
    }
    if (tot > cap) ok = false;
    if (!ok) bad = 1;
    start[tid + 1] = tot / (int64_t)R;
  }
  __syncthreads();
  if (tid == 0) {
    start[0] = 0;
    for (int r = 0; r < p; ++r) start[r + 1] += start[r];
  }
  __syncthreads();
  const bool reject = bad != 0;
  if (blockIdx.x == 0 && tid == 0 && a.status) *a.status = reject ? 1 : 0;
  if (reject) return;
  const int lane = tid % kLanes;
  const uint64_t nunits = H / 16;
  const uint64_t g16 = a.group / 16;
  const uint64_t total = (uint64_t)start[p];
  for (uint64_t g = fp8_wave_id(); g < total; g += fp8_wave_count()) {
    int rk = 0;
    while ((uint64_t)start[rk + 1] <= g) ++rk;
    const uint64_t row = g - (uint64_t)start[rk];
    const uint8_t* src = (const uint8_t*)a.src[rk] + row * R;
    const u32x4* vc = reinterpret_cast<const u32x4*>(src);
    const float* sc = reinterpret_cast<const float*>(src + H);
    u32x4* dst = reinterpret_cast<u32x4*>((uint16_t*)a.dst[rk] + row * H);
    for (uint64_t j0 = 0; j0 < nunits; j0 += (uint64_t)kDeqBatch * kLanes) {
      u32x4 c[kDeqBatch];
      float s[kDeqBatch];
#pragma unroll
      for (int b = 0; b < kDeqBatch; ++b) {
        const uint64_t j = j0 + (uint64_t)b * kLanes + lane;
        if (j < nunits) {
          c[b] = ld16<true>(vc + j);
          s[b] = sc[j / g16];
        }
      }
#pragma unroll
      for (int b = 0; b < kDeqBatch; ++b) {
        const uint64_t j = j0 + (uint64_t)b * kLanes + lane;
        if (j >= nunits) continue;
        u32x4 y0, y1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = c[b][q];
          const uint32_t lo = bf16_pack(e4m3_value(w & 0xffu) * s[b], e4m3_value((w >> 8) & 0xffu) * s[b]);
          const uint32_t hi = bf16_pack(e4m3_value((w >> 16) & 0xffu) * s[b], e4m3_value(w >> 24) * s[b]);
          u32x4& y = q < 2 ? y0 : y1;
          y[2 * (q & 1)] = lo;
          y[2 * (q & 1) + 1] = hi;
        }
        st16<true>(dst + 2 * j, y0);
        st16<true>(dst + 2 * j + 1, y1);
      }
    }
  }
}

int launch_moe_pack_fp8(const Fp8Args& a, int max_grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const uint64_t rows = a.tokens * (uint64_t)a.p;
  const uint64_t wg_needed = (rows + (kBlock / kLanes) - 1) / (kBlock / kLanes);
  const int grid = (int)(wg_needed < (uint64_t)max_grid ? wg_needed : (uint64_t)max_grid);
  if (grid == 0) return 0;
  const uint64_t per_lane = (a.hidden / 16 + kLanes - 1) / kLanes;
  if (per_lane <= 1) hipLaunchKernelGGL((moe_pack_fp8_kernel<1>), dim3(grid), dim3(kBlock), 0, s, a);
  else if (per_lane <= 2) hipLaunchKernelGGL((moe_pack_fp8_kernel<2>), dim3(grid), dim3(kBlock), 0, s, a);
  else if (per_lane <= 4) hipLaunchKernelGGL((moe_pack_fp8_kernel<4>), dim3(grid), dim3(kBlock), 0, s, a);
  else if (per_lane <= 8) hipLaunchKernelGGL((moe_pack_fp8_kernel<8>), dim3(grid), dim3(kBlock), 0, s, a);
  else if (per_lane <= 16) hipLaunchKernelGGL((moe_pack_fp8_kernel<16>), dim3(grid), dim3(kBlock), 0, s, a);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_moe_dequant_fp8(const Fp8Args& a, int max_grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(moe_dequant_fp8_kernel, dim3(max_grid), dim3(kBlock), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace coll
