// Tiles of a plain copy from one source to one or more destinations.
//
// A lane loads kCopyUnroll 16-byte vectors, then stores each to every
// destination of the segment; the copy is type-blind apart from the
// element width used for misaligned heads and tails.  Stores are
// non-temporal; the caller picks the load policy.
#pragma once

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
// vector) to ND destinations (ND = 0: nd, known only at run time).
// j0 = tile * kCopyTV + lane.
template <bool NTL, bool FULL, int ND, typename GD>
__device__ __forceinline__ void copy_vec_tile(const u32x4* src, const GD& gdst, int nd, uint64_t j0,
                                              uint64_t nvec) {
  u32x4 r[kCopyU];
#pragma unroll
  for (int u = 0; u < kCopyU; ++u) {
    const uint64_t j = j0 + (uint64_t)u * kBlock;
    if (FULL || j < nvec) r[u] = ld16<NTL>(src + j);
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads of the tile before the first store
  const int ndst = ND ? ND : nd;
#pragma unroll
  for (int d = 0; d < ndst; ++d) {
    u32x4* dv = gdst(d);
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint64_t j = j0 + (uint64_t)u * kBlock;
      if (FULL || j < nvec) st16<true>(dv + j, r[u]);
    }
  }
}

// Copy one segment of len elements: this workgroup's vector tiles and,
// if it owns the segment, the element-wise head and tail.  gdst(d) gives
// destination d's element pointer at the segment start.  Returns the
// segment's tile count.
// Tiles of a copy segment as copy_segment counts them, and whether this
// workgroup works any of them or the head and tail (see copy_segment);
// lets a workgroup skip a segment's pointer setup.
template <int B>
__device__ __forceinline__ bool copy_segment_owned(uint64_t len, int mis, uint64_t base, uint64_t* nt_out) {
  const SegSpan sp = seg_span<B>(len, mis);
  const uint64_t nt = sp.vec ? ceil_div(sp.nvec, kCopyTV) : ceil_div(len, (uint64_t)kBlock * 4);
  *nt_out = nt;
  const uint64_t ft = first_tile32(base, blockIdx.x, gridDim.x);
  return ft < nt || (ft == 0 && (sp.head || sp.tail));
}

template <int B, bool NTL, int ND, typename GD>
__device__ __forceinline__ uint64_t copy_segment(const typename Word<B>::T* src, const GD& gdst, int nd,
                                                 uint64_t len, int mis, uint64_t base) {
  using W = typename Word<B>::T;
  constexpr uint64_t V = 16 / B;
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
  const SegSpan sp = seg_span<B>(len, mis);
  if (!sp.vec) {
    constexpr uint64_t TE = (uint64_t)kBlock * 4;
    const uint64_t nt = ceil_div(len, TE);
    for (uint64_t t = first_tile(base, wg, grid); t < nt; t += grid) {
      const uint64_t from = t * TE;
      elems(from, (len - from) < TE ? (len - from) : TE);
    }
    return nt;
  }
  const uint64_t nt = ceil_div(sp.nvec, kCopyTV);
  if (sp.nvec) {
    const u32x4* vs = reinterpret_cast<const u32x4*>(src + sp.head);
    auto vd = [&](int d) -> u32x4* { return reinterpret_cast<u32x4*>(gdst(d) + sp.head); };
    const uint64_t nfull = sp.nvec / kCopyTV;
    for (uint64_t t = first_tile(base, wg, grid); t < nt; t += grid) {
      const uint64_t j0 = t * kCopyTV + threadIdx.x;
      if (t < nfull) copy_vec_tile<NTL, true, ND>(vs, vd, nd, j0, sp.nvec);
      else copy_vec_tile<NTL, false, ND>(vs, vd, nd, j0, sp.nvec);
    }
  }
  if ((sp.head || sp.tail) && first_tile(base, wg, grid) == 0) {
    // head and tail in one pass (each is shorter than a vector)
    const uint64_t i = threadIdx.x;
    if (i < sp.head + sp.tail) elem_at(i < sp.head ? i : sp.head + sp.nvec * V + (i - sp.head));
  }
  return nt;
}

}  // namespace coll
