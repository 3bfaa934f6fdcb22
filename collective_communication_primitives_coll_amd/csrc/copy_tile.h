// Tiles of a plain copy from one source to one or more destinations.
//
// A lane loads kCopyUnroll 16-byte vectors, then stores each to every
// destination of the segment; the copy is type-blind apart from the
// element width used for misaligned heads and tails.  Stores are
// non-temporal; the caller picks the load policy.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace coll {

template <int B>
struct Word;
template <>
struct Word<1> {
  using T = uint8_t;
};
template <>
struct Word<2> {
  using T = uint16_t;
};
template <>
struct Word<4> {
  using T = uint32_t;
};

constexpr int kCopyU = (int)kCopyUnroll;
constexpr uint64_t kCopyTV = (uint64_t)kCopyU * kBlock;  // vectors per copy tile

// Copy tile: U vectors per lane from src (at the segment's first aligned
// vector) to ND destinations (ND = 0: nd, known only at run time), with
// non-temporal stores, of device scope for the fan-outs (ND != 1).
// j0 = tile * kCopyTV + lane.  hook(tok) runs once the loads have returned,
// before the stores (as in reduce_vec_tile; tok is an opaque zero that
// keeps what the hook reads after the loads).
template <bool NTL, bool FULL, int ND, int CU = kCopyU, typename GD, typename Hook = NoHook>
__device__ __forceinline__ void copy_vec_tile(const u32x4* src, const GD& gdst, int nd, uint64_t j0,
                                              uint64_t nvec, const Hook& hook = Hook{}) {
  constexpr bool kHook = !std::is_same<Hook, NoHook>::value;
  u32x4 r[CU];
#pragma unroll
  for (int u = 0; u < CU; ++u) {
    const uint64_t j = j0 + (uint64_t)u * kBlock;
    if (FULL || j < nvec) r[u] = ld16<NTL>(src + j);
    else if (kHook) r[u] = u32x4{0, 0, 0, 0};  // defined input for the hook's token
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads of the tile before the first store
  if constexpr (kHook) {
    uint32_t tok = 0;
    asm volatile("" : "+v"(tok) : "v"(r[0]), "v"(r[CU - 1]));
    hook(tok);
  }
  const int ndst = ND ? ND : nd;
#pragma unroll
  for (int d = 0; d < ndst; ++d) {
    u32x4* dv = gdst(d);
    if constexpr (ND != 1) {
      // fan-outs: non-temporal stores of device scope
      store_tile<kStNTDevice, CU, kBlock, FULL>(dv, j0, nvec, r);
    } else {
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const uint64_t j = j0 + (uint64_t)u * kBlock;
        if (FULL || j < nvec) st16<true>(dv + j, r[u]);
      }
    }
  }
}

// Bytes [16q + r, 16q + r + 16) of the 32 bytes lo | hi, for a
// wave-uniform shift 16q + r in [1, 16): each output word joins two
// adjacent input words with v_alignbyte.
__device__ __forceinline__ u32x4 shift_bytes(const u32x4& lo, const u32x4& hi, int q, int r) {
  const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  u32x4 o;
  switch (q) {
    case 0:
      o = u32x4{__builtin_amdgcn_alignbyte(w[1], w[0], r), __builtin_amdgcn_alignbyte(w[2], w[1], r),
                __builtin_amdgcn_alignbyte(w[3], w[2], r), __builtin_amdgcn_alignbyte(w[4], w[3], r)};
      break;
    case 1:
      o = u32x4{__builtin_amdgcn_alignbyte(w[2], w[1], r), __builtin_amdgcn_alignbyte(w[3], w[2], r),
                __builtin_amdgcn_alignbyte(w[4], w[3], r), __builtin_amdgcn_alignbyte(w[5], w[4], r)};
      break;
    case 2:
      o = u32x4{__builtin_amdgcn_alignbyte(w[3], w[2], r), __builtin_amdgcn_alignbyte(w[4], w[3], r),
                __builtin_amdgcn_alignbyte(w[5], w[4], r), __builtin_amdgcn_alignbyte(w[6], w[5], r)};
      break;
    default:
      o = u32x4{__builtin_amdgcn_alignbyte(w[4], w[3], r), __builtin_amdgcn_alignbyte(w[5], w[4], r),
                __builtin_amdgcn_alignbyte(w[6], w[5], r), __builtin_amdgcn_alignbyte(w[7], w[6], r)};
      break;
  }
  return o;
}

// Copy tile for a source that is `m` bytes (0 < m < 16) past the 16-byte
// alignment of the destinations: destination vector j (16-byte aligned)
// is bytes [m, m + 16) of the aligned source vectors j and j + 1 (vs is the
// source rounded down to 16 bytes).  Each lane loads both vectors (the
// second is its neighbour's first, served by the vector cache), shifts and
// stores one aligned vector to each of ND destinations (ND = 0: nd, known
// only at run time).  The second load of the last vector reads at most 15
// bytes past the segment, inside the aligned 16-byte block that holds its
// last byte.
template <bool FULL, int ND, int CU = kCopyU, typename GD>
__device__ __forceinline__ void copy_shift_tile(const u32x4* vs, const GD& gdst, int nd, uint64_t j0, uint64_t nvec,
                                                int m) {
  u32x4 a[CU], b[CU];
#pragma unroll
  for (int u = 0; u < CU; ++u) {
    const uint64_t j = j0 + (uint64_t)u * kBlock;
    if (FULL || j < nvec) {
      a[u] = ld16<false>(vs + j);
      b[u] = ld16<false>(vs + j + 1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int q = m >> 2, r = m & 3;
#pragma unroll
  for (int u = 0; u < CU; ++u) a[u] = shift_bytes(a[u], b[u], q, r);
  const int ndst = ND ? ND : nd;
#pragma unroll
  for (int d = 0; d < ndst; ++d) {
    u32x4* dv = gdst(d);
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const uint64_t j = j0 + (uint64_t)u * kBlock;
      if (FULL || j < nvec) st16<true>(dv + j, a[u]);
    }
  }
}

// Geometry of a segment copied from src to dst (element-aligned pointers):
// an element-wise head up to the destination's next kLineAlign boundary,
// nvec aligned destination vectors, an element-wise tail; `m` is the
// source's byte offset past 16-byte alignment after the head (0: plain
// vector tiles, else copy_shift_tile).
struct ShiftSpan {
  uint64_t head, nvec, tail;
  int m;
};
template <int B>
__device__ __forceinline__ ShiftSpan shift_span(const void* src, const void* dst, uint64_t len) {
  constexpr uint64_t V = 16 / B;
  ShiftSpan s;
  uint64_t h = (uint64_t)(((uint64_t)kLineAlign - ((uintptr_t)dst & (kLineAlign - 1))) & (kLineAlign - 1)) / B;
  if (h > len) h = len;
  s.head = h;
  s.nvec = (len - h) / V;
  s.tail = len - h - s.nvec * V;
  s.m = (int)(((uintptr_t)src + h * B) & 15);
  return s;
}

// Copy one segment of len elements: this workgroup's vector tiles and,
// if it owns the segment, the element-wise head and tail.  gdst(d) gives
// destination d's element pointer at the segment start.  Returns the
// segment's tile count.
// A copy segment's geometry follows its destinations: `mis` is their
// common address modulo 16 at the segment start (-1: the segment goes
// element by element), `damis` their common address modulo kLineAlign
// (-1: unknown).  The head runs to the destinations' next kLineAlign
// boundary when damis is known, else to their 16-byte alignment: a wave
// whose stores start off a 128-byte line shares a partly written line
// with each neighbouring wave, and those lines cost far more than their
// bytes.  SHIFT: a source that then sits m bytes past its own
// alignment takes copy_shift_tile, otherwise plain vector tiles; without
// SHIFT (the launcher found every segment's source and destinations
// agreeing modulo 16) only plain vector tiles are compiled, so the common
// aligned loop keeps the code and waits it had without the shift path.
//
// Tiles of a copy segment as copy_segment counts them, and whether this
// workgroup works any of them or the head and tail (see copy_segment);
// lets a workgroup skip a segment's pointer setup.
template <int B, int CU = kCopyU>
__device__ __forceinline__ uint64_t copy_segment_tiles(const SegSpan& sp, uint64_t len) {
  return sp.vec ? ceil_div(sp.nvec, (uint64_t)CU * kBlock) : ceil_div(len, (uint64_t)kBlock * 4);
}

// Whether this workgroup is the one the partial last tile of a vectorized
// segment is dealt to although it lies at or beyond lim (partial tiles
// are never claimed).  Flat indices stay below 2^32.
template <int CU = kCopyU>
__device__ __forceinline__ bool copy_owns_partial(const SegSpan& sp, uint64_t base, uint64_t lim) {
  constexpr uint64_t TV = (uint64_t)CU * kBlock;
  const uint64_t nfull = sp.nvec / TV;
  return sp.vec && nfull * TV < sp.nvec && nfull >= lim &&
         (uint32_t)(base + nfull) % gridDim.x == blockIdx.x;
}

template <int B, int CU = kCopyU>
__device__ __forceinline__ bool copy_segment_owned(uint64_t len, int dmis, int damis, uint64_t base,
                                                   uint64_t* nt_out, uint64_t lim = ~0ull) {
  const SegSpan sp = seg_span_a<B>(len, dmis, damis);
  const uint64_t nt = copy_segment_tiles<B, CU>(sp, len);
  *nt_out = nt;
  const uint64_t ft = first_tile32(base, blockIdx.x, gridDim.x);
  return ft < (nt < lim ? nt : lim) || (ft == 0 && (sp.head || sp.tail)) || copy_owns_partial<CU>(sp, base, lim);
}

// Copy one segment of len elements: this workgroup's share of the first
// lim vector tiles (and of the partial last tile when that lies beyond
// lim) and, if it owns the segment, the element-wise head and tail.
// gdst(d) gives destination d's element pointer at the segment start.
// Returns the segment's tile count.  lim applies to vector tiles without
// SHIFT only (the claimed tails copy no other kind).
template <int B, bool NTL, int ND, bool SHIFT, int CU = kCopyU, typename GD>
__device__ __forceinline__ uint64_t copy_segment(const typename Word<B>::T* src, const GD& gdst, int nd,
                                                 uint64_t len, int dmis, int damis, uint64_t base,
                                                 uint64_t lim = ~0ull) {
  using W = typename Word<B>::T;
  constexpr uint64_t V = 16 / B;
  constexpr uint64_t TVU = (uint64_t)CU * kBlock;  // vectors per tile
  const uint64_t grid = gridDim.x, wg = blockIdx.x;
  const int ndst = ND ? ND : nd;
  auto elem_at = [&](uint64_t e) {
    const W w = ld1<NTL>(src + e);
#pragma unroll
    for (int d = 0; d < ndst; ++d) st1<true>(gdst(d) + e, w);
  };
  auto elems = [&](uint64_t from, uint64_t cnt) {
    for (uint64_t i = threadIdx.x; i < cnt; i += kBlock) elem_at(from + i);
  };
  const SegSpan sp = seg_span_a<B>(len, dmis, damis);
  if (!sp.vec) {
    constexpr uint64_t TE = (uint64_t)kBlock * 4;
    const uint64_t nt = ceil_div(len, TE);
    for (uint64_t t = first_tile(base, wg, grid); t < nt; t += grid) {
      const uint64_t from = t * TE;
      elems(from, (len - from) < TE ? (len - from) : TE);
    }
    return nt;
  }
  const uint64_t nt = ceil_div(sp.nvec, TVU);
  if (sp.nvec) {
    const int m = SHIFT ? (int)(((uintptr_t)src + sp.head * B) & 15) : 0;
    auto vd = [&](int d) -> u32x4* { return reinterpret_cast<u32x4*>(gdst(d) + sp.head); };
    const uint64_t nfull = sp.nvec / TVU;
    if (m == 0) {
      const u32x4* vs = reinterpret_cast<const u32x4*>(src + sp.head);
      const uint64_t nd_t = nt < lim ? nt : lim;
      for (uint64_t t = first_tile(base, wg, grid); t < nd_t; t += grid) {
        const uint64_t j0 = t * TVU + threadIdx.x;
        if (t < nfull) copy_vec_tile<NTL, true, ND, CU>(vs, vd, nd, j0, sp.nvec);
        else copy_vec_tile<NTL, false, ND, CU>(vs, vd, nd, j0, sp.nvec);
      }
      if (copy_owns_partial<CU>(sp, base, nd_t))
        copy_vec_tile<NTL, false, ND, CU>(vs, vd, nd, nfull * TVU + threadIdx.x, sp.nvec);
    } else if constexpr (SHIFT) {
      const u32x4* vs = reinterpret_cast<const u32x4*>((uintptr_t)(src + sp.head) & ~(uintptr_t)15);
      for (uint64_t t = first_tile(base, wg, grid); t < nt; t += grid) {
        const uint64_t j0 = t * TVU + threadIdx.x;
        if (t < nfull) copy_shift_tile<true, ND, CU>(vs, vd, nd, j0, sp.nvec, m);
        else copy_shift_tile<false, ND, CU>(vs, vd, nd, j0, sp.nvec, m);
      }
    }
  }
  if ((sp.head || sp.tail) && first_tile(base, wg, grid) == 0) {
    // head and tail together (below kLineAlign + 16 bytes)
    for (uint64_t i = threadIdx.x; i < sp.head + sp.tail; i += kBlock)
      elem_at(i < sp.head ? i : sp.head + sp.nvec * V + (i - sp.head));
  }
  return nt;
}

}  // namespace coll
