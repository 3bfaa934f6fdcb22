// One tile of a p-way elementwise reduction.
//
// The k-th operand of the fold comes from gsrc(k) and the result goes to
// gdst(0..ndst-1); both return element pointers already offset to the
// segment start.  With the ring order the fold is a left fold in the
// order gsrc(0), gsrc(1), ..., which the callers rotate so that chunk c is
// folded x_{c+1}, x_{c+2}, ..., x_c: the ring all-reduce of
// "集合通信：原语、算法、NCCL 实现与拓扑映射" (hpc/04, section 2.2) with the
// partial kept in registers across its p-1 combine steps and the p
// all-gather stores issued from the same registers.  TREE instead sums
// the operands as a balanced pairwise tree (a one-pass reassociated sum).
//
// All p loads of a lane are issued before the first combine, so a lane
// keeps p (x UNROLL) 16-byte requests in flight.
#pragma once

#include "device_common.h"

namespace coll {

template <int P>
struct ReduceUnroll {
  static constexpr int value = (P == 0 || P >= 8) ? 1 : 8 / P;
};

template <int DT, int OP, int P, bool TREE, bool DSTALL, typename GS, typename GD>
__device__ __forceinline__ void reduce_elems(const GS& gsrc, const GD& gdst, int p, uint64_t from,
                                             uint64_t cnt) {
  using T = Traits<DT>;
  using A = typename T::A;
  const int np = P ? P : p;
  for (uint64_t i = threadIdx.x; i < cnt; i += kBlock) {
    const uint64_t e = from + i;
    A acc;
    if constexpr (TREE) {
      static_assert(P > 0, "tree order needs a compile-time rank count");
      A a[P];
#pragma unroll
      for (int k = 0; k < P; ++k) a[k] = widen1<DT>(ld1(gsrc(k) + e));
#pragma unroll
      for (int s = 1; s < P; s *= 2)
#pragma unroll
        for (int k = 0; k + s < P; k += 2 * s) a[k] = combine<OP>(a[k], a[k + s]);
      acc = a[0];
    } else {
      acc = widen1<DT>(ld1(gsrc(0) + e));
      if constexpr (P > 0) {
#pragma unroll
        for (int k = 1; k < P; ++k) acc = combine<OP>(acc, widen1<DT>(ld1(gsrc(k) + e)));
      } else {
        for (int k = 1; k < np; ++k) acc = combine<OP>(acc, widen1<DT>(ld1(gsrc(k) + e)));
      }
    }
    const auto out = narrow1<DT>(acc);
    if constexpr (DSTALL) {
      if constexpr (P > 0) {
#pragma unroll
        for (int k = 0; k < P; ++k) st1(gdst(k) + e, out);
      } else {
        for (int k = 0; k < np; ++k) st1(gdst(k) + e, out);
      }
    } else {
      st1(gdst(0) + e, out);
    }
  }
}

template <int DT, int OP, int P, bool TREE, bool DSTALL, int U, typename GS, typename GD>
__device__ __forceinline__ void reduce_vectors(const GS& gsrc, const GD& gdst, int p, uint64_t v0,
                                               uint64_t nvec) {
  using T = Traits<DT>;
  using S = typename T::S;
  using A = typename T::A;
  constexpr int V = T::V;
  const uint64_t tid = threadIdx.x;
  if constexpr (P > 0) {
    const S* s[P];
#pragma unroll
    for (int k = 0; k < P; ++k) s[k] = gsrc(k);
    u32x4 raw[U][P];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t vi = (uint64_t)u * kBlock + tid;
      if (vi < nvec) {
        const uint64_t e = v0 + vi * V;
#pragma unroll
        for (int k = 0; k < P; ++k) raw[u][k] = ld16(s[k] + e);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t vi = (uint64_t)u * kBlock + tid;
      if (vi < nvec) {
        const uint64_t e = v0 + vi * V;
        A acc[V];
        if constexpr (TREE) {
          A a[P][V];
#pragma unroll
          for (int k = 0; k < P; ++k) widen<DT>(raw[u][k], a[k]);
#pragma unroll
          for (int st = 1; st < P; st *= 2)
#pragma unroll
            for (int k = 0; k + st < P; k += 2 * st) combine_vec<OP, DT>(a[k], a[k + st]);
#pragma unroll
          for (int x = 0; x < V; ++x) acc[x] = a[0][x];
        } else {
          widen<DT>(raw[u][0], acc);
#pragma unroll
          for (int k = 1; k < P; ++k) {
            A t[V];
            widen<DT>(raw[u][k], t);
            combine_vec<OP, DT>(acc, t);
          }
        }
        const u32x4 out = narrow<DT>(acc);
        if constexpr (DSTALL) {
#pragma unroll
          for (int k = 0; k < P; ++k) st16(gdst(k) + e, out);
        } else {
          st16(gdst(0) + e, out);
        }
      }
    }
  } else {
    // Rank count known only at run time: operands in groups of 8, each
    // group's loads issued before its combines.
    const uint64_t vi = tid;
    if (vi < nvec) {
      const uint64_t e = v0 + vi * V;
      A acc[V];
      widen<DT>(ld16(gsrc(0) + e), acc);
      for (int k0 = 1; k0 < p; k0 += 8) {
        u32x4 r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (k0 + j < p) r[j] = ld16(gsrc(k0 + j) + e);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (k0 + j < p) {
            A t[V];
            widen<DT>(r[j], t);
            combine_vec<OP, DT>(acc, t);
          }
      }
      const u32x4 out = narrow<DT>(acc);
      if constexpr (DSTALL) {
        for (int k = 0; k < p; ++k) st16(gdst(k) + e, out);
      } else {
        st16(gdst(0) + e, out);
      }
    }
  }
}

// Tile elements for a reduction: U vectors per lane, one workgroup.
template <int DT, int P>
constexpr uint64_t reduce_tile_elems() {
  return (uint64_t)ReduceUnroll<P>::value * kBlock * Traits<DT>::V;
}

template <int DT, int OP, int P, bool TREE, bool DSTALL, typename GS, typename GD>
__device__ __forceinline__ void reduce_tile(const GS& gsrc, const GD& gdst, int p, const TileSpan& sp) {
  constexpr int U = (P == 0) ? 1 : ReduceUnroll<P>::value;
  constexpr int V = Traits<DT>::V;
  if (sp.vec) {
    if (sp.nvec) reduce_vectors<DT, OP, P, TREE, DSTALL, U>(gsrc, gdst, p, sp.begin + sp.head, sp.nvec);
    if (sp.head) reduce_elems<DT, OP, P, TREE, DSTALL>(gsrc, gdst, p, sp.begin, sp.head);
    if (sp.tail)
      reduce_elems<DT, OP, P, TREE, DSTALL>(gsrc, gdst, p, sp.begin + sp.head + sp.nvec * V, sp.tail);
  } else {
    reduce_elems<DT, OP, P, TREE, DSTALL>(gsrc, gdst, p, sp.begin, sp.head);
  }
}

}  // namespace coll
