// Device-side building blocks shared by the collective kernels (gfx950).
//
// Data moves in 16-byte vectors (global_load/store_dwordx4) with the
// non-temporal hint: every byte is touched once, so nothing is worth
// keeping in L2 or the Infinity Cache.  Element ranges whose start is not
// 16-byte aligned, or whose source and destination are misaligned
// differently, fall back to element-wide accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_args.h"

namespace coll {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;  // threads per workgroup (4 wave64s)

template <int DT> struct Traits;
template <> struct Traits<kF32> {
  using S = float;     // storage type
  using A = float;     // accumulation type
  static constexpr int V = 4;  // elements per 16-byte vector
  static constexpr int B = 4;  // bytes per element
};
template <> struct Traits<kBF16> {
  using S = uint16_t;
  using A = float;
  static constexpr int V = 8;
  static constexpr int B = 2;
};
template <> struct Traits<kI32> {
  using S = int32_t;
  using A = int32_t;
  static constexpr int V = 4;
  static constexpr int B = 4;
};

// ---------------------------------------------------------------------------
// Loads and stores
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
template <typename S>
__device__ __forceinline__ S ld1(const S* p) {
  return __builtin_nontemporal_load(p);
}
template <typename S>
__device__ __forceinline__ void st1(S* p, S v) {
  __builtin_nontemporal_store(v, p);
}

// ---------------------------------------------------------------------------
// Widening and narrowing.  bf16 widens exactly (the pattern is the upper
// half of the fp32 pattern) and narrows with round-to-nearest-even through
// the gfx950 conversion instruction (v_cvt_pk_bf16_f32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

template <int DT>
__device__ __forceinline__ void widen(u32x4 v, typename Traits<DT>::A (&a)[Traits<DT>::V]) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = __uint_as_float(v[e]);
  } else if constexpr (DT == kI32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = (int32_t)v[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[2 * e] = bf16_lo(v[e]);
      a[2 * e + 1] = bf16_hi(v[e]);
    }
  }
}

template <int DT>
__device__ __forceinline__ u32x4 narrow(const typename Traits<DT>::A (&a)[Traits<DT>::V]) {
  u32x4 v;
  if constexpr (DT == kF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(a[e]);
  } else if constexpr (DT == kI32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (uint32_t)a[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = bf16_pack(a[2 * e], a[2 * e + 1]);
  }
  return v;
}

template <int DT>
__device__ __forceinline__ typename Traits<DT>::A widen1(typename Traits<DT>::S s) {
  if constexpr (DT == kBF16) return __uint_as_float((uint32_t)s << 16);
  else return s;
}
template <int DT>
__device__ __forceinline__ typename Traits<DT>::S narrow1(typename Traits<DT>::A a) {
  if constexpr (DT == kBF16) return (uint16_t)bf16_bits(a);
  else return a;
}

// ---------------------------------------------------------------------------
// The elementwise operation.  acc is the running partial, v the next
// rank's value; min/max keep acc on ties.
// ---------------------------------------------------------------------------
template <int OP, typename A>
__device__ __forceinline__ A combine(A acc, A v) {
  if constexpr (OP == kSum) return acc + v;
  else if constexpr (OP == kMin) return (v < acc) ? v : acc;
  else return (v > acc) ? v : acc;
}

template <int OP, int DT>
__device__ __forceinline__ void combine_vec(typename Traits<DT>::A (&acc)[Traits<DT>::V],
                                            const typename Traits<DT>::A (&v)[Traits<DT>::V]) {
#pragma unroll
  for (int e = 0; e < Traits<DT>::V; ++e) acc[e] = combine<OP>(acc[e], v[e]);
}

// ---------------------------------------------------------------------------
// Tile geometry.  A segment is a run of `len` elements that starts at the
// same element offset in every source (and at one offset in every
// destination).  It is cut into tiles of kTileVec vectors' worth of
// elements; within a tile the 16-byte aligned middle goes through vector
// accesses and the misaligned head and tail element by element.
// ---------------------------------------------------------------------------
struct TileSpan {
  uint64_t begin;  // first element of the tile (segment-relative)
  uint64_t head;   // elements before the first aligned vector
  uint64_t nvec;   // aligned vectors
  uint64_t tail;   // elements after the last vector
  bool vec;        // false: every element goes through the element path
};

// mis: byte misalignment (0..15) of the segment start, common to all
// sources and destinations, or -1 when they differ.
template <int B, int V>
__device__ __forceinline__ TileSpan tile_span(uint64_t len, uint64_t tile_elems, uint64_t t, int mis) {
  TileSpan s;
  s.begin = t * tile_elems;
  uint64_t n = len - s.begin;
  if (n > tile_elems) n = tile_elems;
  if (mis < 0 || mis % B != 0) {
    s.vec = false;
    s.head = n;
    s.nvec = 0;
    s.tail = 0;
    return s;
  }
  s.vec = true;
  // tile_elems * B is a multiple of 16, so every tile of the segment shares
  // the segment's misalignment.
  uint64_t h = (uint64_t)(((16 - mis) & 15) / B);
  if (h > n) h = n;
  s.head = h;
  s.nvec = (n - h) / V;
  s.tail = n - h - s.nvec * V;
  return s;
}

__device__ __forceinline__ uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// First tile index t >= 0 of a segment whose flat index base + t is
// congruent to the workgroup id modulo the grid size.
__device__ __forceinline__ uint64_t first_tile(uint64_t base, uint64_t wg, uint64_t grid) {
  uint64_t r = base % grid;
  return (wg + grid - r) % grid;
}

}  // namespace coll
