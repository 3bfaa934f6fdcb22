// Tiles of a p-way elementwise reduction.
//
// The operands of every element are folded left to right in the order the
// caller lists the sources.  The callers list chunk c's sources as
// x_{c+1}, x_{c+2}, ..., x_c: the ring all-reduce of
// "集合通信：原语、算法、NCCL 实现与拓扑映射" (hpc/04, section 2.2) with the
// partial held in registers across its p-1 combine steps, and for
// AllReduce the p all-gather stores issued from the same registers.
// The tree orders instead sum the operands, listed in rank order, as a
// balanced pairwise tree: kOrdRD pairs neighbours first, as recursive
// doubling does (section 2.3 there: exchange at distance 1, 2, 4, ...);
// kOrdHD pairs ranks p/2 apart first, as the recursive-halving
// reduce-scatter of halving-doubling does.  kOrdTree and kOrdDBT fold the
// listed operands as a binary tree in heap order (the tree all-reduce's
// reduce to the root; section 2.4's double binary tree lists the ranks in
// mirrored order for its second tree): operand v adds its left subtree
// (2v+1) and then its right subtree (2v+2), leaves first.
//
// A lane handles U vectors of a tile.  It issues all P*U loads before the
// first combine, source by source, so it keeps P*U 16-byte requests in
// flight.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace coll {

// Vectors per lane in a reduction tile.  Reductions that store once keep
// 32 loads in flight per lane; AllReduce, which also stores p times,
// keeps 16.
template <int P, bool ALL>
struct ReduceUnroll {
  static constexpr int raw = P == 0 ? 1 : (ALL ? 16 / P : 32 / P);
  static constexpr int value = raw < 1 ? 1 : (raw > 8 ? 8 : raw);
};

// a[k] <- a[(k + s) mod P] for a wave-uniform s in [0, P): one conditional
// rotation per bit of s (by 1, 2, 4, ...), each with indices that are
// compile-time constants, so the array stays in scalar registers and its
// elements can be fetched with constant offsets (wide scalar loads issued
// together).  Rotations compose modulo P, so this holds for any P, not only
// powers of two.  Indexing the source array with a run-time rank instead
// makes the compiler fetch every element with its own dependent scalar load.
template <int P, typename T>
__device__ __forceinline__ void rotate_left(T (&a)[P], int s) {
#pragma unroll
  for (int b = 1; b < P; b <<= 1) {
    const bool on = (s & b) != 0;
    T t[P];
#pragma unroll
    for (int k = 0; k < P; ++k) t[k] = a[(k + b) % P];
#pragma unroll
    for (int k = 0; k < P; ++k) a[k] = on ? t[k] : a[k];
  }
}

// a[k] <- a[P - 1 - k] when `on` (wave-uniform).
template <int P, typename T>
__device__ __forceinline__ void reverse_if(T (&a)[P], bool on) {
  T t[P];
#pragma unroll
  for (int k = 0; k < P; ++k) t[k] = a[P - 1 - k];
#pragma unroll
  for (int k = 0; k < P; ++k) a[k] = on ? t[k] : a[k];
}

// Per-rank values (pointers, scales) a[r], indexed by rank, reordered in
// place into the order in which chunk c lists its operands: the ring
// rotation x_{c+1}, ..., x_c, or rank order for the trees (mirrored for
// the double binary tree's second half of the chunks).
template <int ORD, int P, typename T>
__device__ __forceinline__ void list_for_chunk(T (&a)[P], int c) {
  if constexpr (ORD == kOrdRing) rotate_left<P>(a, (c + 1) % P);
  else if constexpr (ORD == kOrdDBT) reverse_if<P>(a, c >= P / 2);
}

// Per-operand scales of a pre-multiplied sum, in the order the operands
// are listed.
template <int P>
struct Scales {
  float s[P];
};

// Operand k widened (and scaled by its rank's factor for kPreMul, the
// product rounded to fp32 on its own).
template <int DT, int OP, int P>
__device__ __forceinline__ void operand(u32x4 r, const Scales<P>& sc, int k,
                                        typename Traits<DT>::A (&a)[Traits<DT>::V]) {
#pragma clang fp contract(off)
  widen<DT>(r, a);
  if constexpr (OP == kPreMul) {
#pragma unroll
    for (int x = 0; x < Traits<DT>::V; ++x) a[x] = sc.s[k] * a[x];
  }
}

// After the fold: kAvg divides by the rank count p (one IEEE division for
// floats, C division for int32).
template <int OP, typename A>
__device__ __forceinline__ A finish(A acc, int p) {
  if constexpr (OP == kAvg) return acc / (A)p;
  else return acc;
}

// Fold of P operands, in list order or as one of the trees.
template <int DT, int OP, int P, int ORD>
__device__ __forceinline__ u32x4 fold_vectors(const u32x4 (&r)[P], const Scales<P>& sc, int avg_p) {
#pragma clang fp contract(off)
  using A = typename Traits<DT>::A;
  constexpr int V = Traits<DT>::V;
  A acc[V];
  if constexpr (ORD == kOrdRD) {
    A a[P][V];
#pragma unroll
    for (int k = 0; k < P; ++k) operand<DT, OP, P>(r[k], sc, k, a[k]);
#pragma unroll
    for (int st = 1; st < P; st *= 2)
#pragma unroll
      for (int k = 0; k + st < P; k += 2 * st) combine_vec<OP, DT>(a[k], a[k + st]);
#pragma unroll
    for (int x = 0; x < V; ++x) acc[x] = a[0][x];
  } else if constexpr (ORD == kOrdHD) {
    A a[P][V];
#pragma unroll
    for (int k = 0; k < P; ++k) operand<DT, OP, P>(r[k], sc, k, a[k]);
#pragma unroll
    for (int st = P / 2; st >= 1; st /= 2)
#pragma unroll
      for (int k = 0; k < st; ++k) combine_vec<OP, DT>(a[k], a[k + st]);
#pragma unroll
    for (int x = 0; x < V; ++x) acc[x] = a[0][x];
  } else if constexpr (ORD == kOrdTree || ORD == kOrdDBT) {
    A a[P][V];
#pragma unroll
    for (int k = 0; k < P; ++k) operand<DT, OP, P>(r[k], sc, k, a[k]);
#pragma unroll
    for (int v = P - 1; v >= 0; --v) {
      if (2 * v + 1 < P) combine_vec<OP, DT>(a[v], a[2 * v + 1]);
      if (2 * v + 2 < P) combine_vec<OP, DT>(a[v], a[2 * v + 2]);
    }
#pragma unroll
    for (int x = 0; x < V; ++x) acc[x] = a[0][x];
  } else {
    operand<DT, OP, P>(r[0], sc, 0, acc);
#pragma unroll
    for (int k = 1; k < P; ++k) {
      A t[V];
      operand<DT, OP, P>(r[k], sc, k, t);
      combine_vec<OP, DT>(acc, t);
    }
  }
#pragma unroll
  for (int x = 0; x < V; ++x) acc[x] = finish<OP>(acc[x], avg_p);
  return narrow<DT>(acc);
}

// One vector tile worked by LANES lanes (a workgroup or a single wave).
// src[k] and dst[d] point at the segment's first aligned vector;
// j0 = tile * U * LANES + lane is this lane's first vector index.
// FULL: every vector of the tile lies inside the segment (nvec unused).
// NTS: non-temporal stores (AllReduce with workgroup tiles; of device
// scope for wave tiles, i.e. the batch: 11.48 against 11.54 ms for 10,000
// calls at p = 16, while the single AllReduce took 742-756 us against
// 737 us with either device-scope policy at p = 8, 256 MiB fp32 per rank);
// otherwise device-scope stores (ReduceScatter, Reduce; see kStDevice).
// hook(tok) runs after the fold, before the stores: every load of the tile
// has then returned, and with it everything the wave issued before them.
// tok is a zero the compiler cannot see through, produced after the fold:
// adding it to what the hook reads keeps that read after the fold (code
// motion would otherwise hoist it among the loads, where it would wait
// for them).
template <int DT, int OP, int P, int ORD, int ND, bool NTS, int U, bool FULL, int LANES = kBlock,
          typename Hook = NoHook>
__device__ __forceinline__ void reduce_vec_tile(const typename Traits<DT>::S* const (&src)[P],
                                                typename Traits<DT>::S* const (&dst)[ND],
                                                uint64_t j0, uint64_t nvec, const Scales<P>& sc,
                                                int avg_p, const Hook& hook = Hook{}) {
  constexpr int V = Traits<DT>::V;
  u32x4 raw[U][P];
#pragma unroll
  for (int k = 0; k < P; ++k)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t j = j0 + (uint64_t)u * LANES;
      if (FULL || j < nvec) raw[u][k] = ld16<true>(src[k] + j * V);
      else raw[u][k] = u32x4{0, 0, 0, 0};
    }
  u32x4 out[U];
#pragma unroll
  for (int u = 0; u < U; ++u) out[u] = fold_vectors<DT, OP, P, ORD>(raw[u], sc, avg_p);
  if constexpr (!std::is_same<Hook, NoHook>::value) {
    uint32_t tok = 0;
    asm volatile("" : "+v"(tok) : "v"(out[0]), "v"(out[U - 1]));
    hook(tok);
  }
  constexpr int SP = !NTS ? kStDevice : LANES == kBlock ? kStNT : kStNTDevice;
  if constexpr (SP == kStNT) {
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t j = j0 + (uint64_t)u * LANES;
        if (FULL || j < nvec) st16<true>(dst[d] + j * V, out[u]);
      }
  } else {
#pragma unroll
    for (int d = 0; d < ND; ++d)
      store_tile<SP, U, LANES, FULL>(reinterpret_cast<u32x4*>(dst[d]), j0, nvec, out);
  }
}

// One element e of the segment (src/dst at the segment start): the p
// operands in the schedule's order, the result to every destination.
template <int DT, int OP, int P, int ORD, int ND, bool NTS>
__device__ __forceinline__ void reduce_elem_at(const typename Traits<DT>::S* const (&src)[P],
                                               typename Traits<DT>::S* const (&dst)[ND], uint64_t e,
                                               const Scales<P>& sc, int avg_p) {
#pragma clang fp contract(off)
  using A = typename Traits<DT>::A;
  A a[P];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    a[k] = widen1<DT>(ld1<true>(src[k] + e));
    if constexpr (OP == kPreMul) a[k] = sc.s[k] * a[k];
  }
  A acc;
  if constexpr (ORD == kOrdRD) {
#pragma unroll
    for (int st = 1; st < P; st *= 2)
#pragma unroll
      for (int k = 0; k + st < P; k += 2 * st) a[k] = combine<OP>(a[k], a[k + st]);
    acc = a[0];
  } else if constexpr (ORD == kOrdHD) {
#pragma unroll
    for (int st = P / 2; st >= 1; st /= 2)
#pragma unroll
      for (int k = 0; k < st; ++k) a[k] = combine<OP>(a[k], a[k + st]);
    acc = a[0];
  } else if constexpr (ORD == kOrdTree || ORD == kOrdDBT) {
#pragma unroll
    for (int v = P - 1; v >= 0; --v) {
      if (2 * v + 1 < P) a[v] = combine<OP>(a[v], a[2 * v + 1]);
      if (2 * v + 2 < P) a[v] = combine<OP>(a[v], a[2 * v + 2]);
    }
    acc = a[0];
  } else {
    acc = a[0];
#pragma unroll
    for (int k = 1; k < P; ++k) acc = combine<OP>(acc, a[k]);
  }
  const auto out = narrow1<DT>(finish<OP>(acc, avg_p));
#pragma unroll
  for (int d = 0; d < ND; ++d) st1<NTS>(dst[d] + e, out);
}

// Element-wise path: cnt elements from element offset `from` of the
// segment (src/dst at the segment start), one element per lane; `lane`
// of LANES lanes.
template <int DT, int OP, int P, int ORD, int ND, bool NTS, int LANES = kBlock>
__device__ __forceinline__ void reduce_elems(const typename Traits<DT>::S* const (&src)[P],
                                             typename Traits<DT>::S* const (&dst)[ND], uint64_t from,
                                             uint64_t cnt, const Scales<P>& sc, int avg_p, int lane = -1) {
  const uint64_t l0 = lane < 0 ? threadIdx.x : (uint64_t)lane;
  for (uint64_t i = l0; i < cnt; i += LANES)
    reduce_elem_at<DT, OP, P, ORD, ND, NTS>(src, dst, from + i, sc, avg_p);
}

// The element-wise head (elements [0, head)) and tail (tail elements from
// tail_from) of a vectorized segment together: lane i < head takes element
// i, lane head + i element tail_from + i, LANES lanes at a time.  The head
// reaches the next line boundary (below kLineAlign bytes) and the tail is
// shorter than one vector, so a workgroup covers both in one pass and a
// wave in at most three, one memory round trip each.
template <int DT, int OP, int P, int ORD, int ND, bool NTS, int LANES = kBlock>
__device__ __forceinline__ void reduce_edges(const typename Traits<DT>::S* const (&src)[P],
                                             typename Traits<DT>::S* const (&dst)[ND], uint64_t head,
                                             uint64_t tail_from, uint64_t tail, const Scales<P>& sc, int avg_p,
                                             int lane) {
  for (uint64_t i = (uint64_t)lane; i < head + tail; i += LANES)
    reduce_elem_at<DT, OP, P, ORD, ND, NTS>(src, dst, i < head ? i : tail_from + (i - head), sc, avg_p);
}

// Workgroup tiles of a segment (vector tiles of U * kBlock vectors, or
// element tiles of 4 * kBlock elements when the buffers disagree modulo 16).
template <int DT, int P, int ND>
__device__ __forceinline__ uint64_t segment_tiles(const SegSpan& sp, uint64_t len) {
  constexpr int U = ReduceUnroll<P, (ND > 1)>::value;
  constexpr uint64_t TV = (uint64_t)U * kBlock;
  return sp.vec ? ceil_div(sp.nvec, TV) : ceil_div(len, (uint64_t)kBlock * 4);
}

// Whether this workgroup is the one tile nfull of a vectorized segment
// (its last tile, when partial) is dealt to although it lies at or beyond
// lim: partial tiles are never claimed.  Flat indices stay below 2^32.
template <int P, int ND>
__device__ __forceinline__ bool owns_partial(const SegSpan& sp, uint64_t base, uint64_t lim) {
  constexpr uint64_t TV = (uint64_t)ReduceUnroll<P, (ND > 1)>::value * kBlock;
  const uint64_t nfull = sp.nvec / TV;
  return sp.vec && nfull * TV < sp.nvec && nfull >= lim && (uint32_t)(base + nfull) % gridDim.x == blockIdx.x;
}

// Tiles of a segment as reduce_segment counts them, and whether workgroup
// wg (of grid) works any of them, or the head and tail, when the segment's
// flat tile indices start at base and only its first lim tiles (and its
// partial last tile) are dealt out.  Lets a workgroup skip a segment's
// pointer setup when it has nothing to do there (small calls, where the
// setup would dominate).
template <int DT, int P, int ND>
__device__ __forceinline__ bool segment_owned(uint64_t len, int mis, int amis, uint64_t base, uint64_t* nt_out,
                                              uint64_t lim = ~0ull) {
  const SegSpan sp = seg_span_a<Traits<DT>::B>(len, mis, amis);
  const uint64_t nt = segment_tiles<DT, P, ND>(sp, len);
  *nt_out = nt;
  const uint64_t ft = first_tile32(base, blockIdx.x, gridDim.x);
  return ft < (nt < lim ? nt : lim) || (ft == 0 && (sp.head || sp.tail)) || owns_partial<P, ND>(sp, base, lim);
}

// A whole segment as seen by one workgroup: its share of the segment's
// first lim tiles (flat tile indices congruent to the workgroup id modulo
// the grid, counting from `base`), the partial last tile if that is its
// and lies beyond lim, and, for the owning workgroup, the head and tail.
// amis: the sources' address modulo kLineAlign at the segment start, or
// -1.  Returns the segment's tile count (the caller advances base by it).
template <int DT, int OP, int P, int ORD, int ND, bool NTS>
__device__ __forceinline__ uint64_t reduce_segment(const typename Traits<DT>::S* const (&src)[P],
                                                   typename Traits<DT>::S* const (&dst)[ND],
                                                   uint64_t len, int mis, int amis, uint64_t base,
                                                   const Scales<P>& sc, int avg_p, uint64_t lim = ~0ull) {
  using S = typename Traits<DT>::S;
  constexpr int V = Traits<DT>::V;
  constexpr int U = ReduceUnroll<P, (ND > 1)>::value;
  constexpr uint64_t TV = (uint64_t)U * kBlock;
  const uint64_t grid = gridDim.x, wg = blockIdx.x;
  const SegSpan sp = seg_span_a<Traits<DT>::B>(len, mis, amis);
  if (!sp.vec) {
    // element path over tiles of kBlock * 4 elements
    constexpr uint64_t TE = (uint64_t)kBlock * 4;
    const uint64_t nt = ceil_div(len, TE);
    const uint64_t nd = nt < lim ? nt : lim;
    for (uint64_t t = first_tile(base, wg, grid); t < nd; t += grid) {
      const uint64_t from = t * TE;
      const uint64_t cnt = (len - from) < TE ? (len - from) : TE;
      reduce_elems<DT, OP, P, ORD, ND, NTS>(src, dst, from, cnt, sc, avg_p);
    }
    return nt;
  }
  const uint64_t nt = ceil_div(sp.nvec, TV);
  if (sp.nvec) {
    const S* vs[P];
    S* vd[ND];
#pragma unroll
    for (int k = 0; k < P; ++k) vs[k] = src[k] + sp.head;
#pragma unroll
    for (int d = 0; d < ND; ++d) vd[d] = dst[d] + sp.head;
    const uint64_t nfull = sp.nvec / TV;
    const uint64_t nd = nt < lim ? nt : lim;
    for (uint64_t t = first_tile(base, wg, grid); t < nd; t += grid) {
      const uint64_t j0 = t * TV + threadIdx.x;
      if (t < nfull) reduce_vec_tile<DT, OP, P, ORD, ND, NTS, U, true>(vs, vd, j0, sp.nvec, sc, avg_p);
      else reduce_vec_tile<DT, OP, P, ORD, ND, NTS, U, false>(vs, vd, j0, sp.nvec, sc, avg_p);
    }
    if (owns_partial<P, ND>(sp, base, nd))
      reduce_vec_tile<DT, OP, P, ORD, ND, NTS, U, false>(vs, vd, nfull * TV + threadIdx.x, sp.nvec, sc, avg_p);
  }
  if ((sp.head || sp.tail) && first_tile(base, wg, grid) == 0)
    reduce_edges<DT, OP, P, ORD, ND, NTS>(src, dst, sp.head, sp.head + sp.nvec * V, sp.tail, sc, avg_p,
                                          (int)threadIdx.x);
  return nt;
}

}  // namespace coll
