// AllReduce, Reduce and ReduceScatter: one kernel family.
//
// Segment c is chunk c of the operation: for AllReduce and Reduce the
// elements [c*q, (c+1)*q) with q = ceil(n/p); for ReduceScatter block c of
// every rank's [p*n] input.  Every workgroup walks the segments in order
// and takes the tiles whose flat index is congruent to its id modulo the
// grid, so all p segments spread over the whole chip.  The destination
// mode picks where a segment's result goes:
//   all    every rank's buffer at the segment offset (AllReduce: the
//          reduce-scatter result of chunk c and its all-gather to every
//          rank come out of one pass),
//   fixed  the root buffer at the segment offset (Reduce),
//   owner  rank c's buffer from its start (ReduceScatter, block c lands on
//          rank c: "集合通信：原语、算法、NCCL 实现与拓扑映射", section 1.5).
#include "reduce_tile.h"

namespace coll {

template <int DT, int OP, int P, bool TREE, bool DSTALL>
__global__ __launch_bounds__(kBlock) void reduce_kernel(RankPtrs ptrs, ReduceGeom g) {
  using T = Traits<DT>;
  using S = typename T::S;
  constexpr uint64_t TE = reduce_tile_elems<DT, P>();
  const int p = P ? P : g.p;
  const uint64_t grid = gridDim.x;
  const uint64_t wg = blockIdx.x;
  uint64_t base = 0;
  for (int c = 0; c < p; ++c) {
    uint64_t lo = (uint64_t)c * g.stride;
    uint64_t hi = lo + g.stride;
    if (lo > g.total) lo = g.total;
    if (hi > g.total) hi = g.total;
    const uint64_t len = hi - lo;
    if (len == 0) continue;
    const uint64_t ntiles = ceil_div(len, TE);
    const uint64_t dst_off = (g.dst_mode == kDstOwner) ? 0 : lo;
    int mis = -1;
    if (g.src_mis >= 0 && g.dst_mis >= 0) {
      const int sm = (int)((g.src_mis + lo * T::B) & 15);
      const int dm = (int)((g.dst_mis + dst_off * T::B) & 15);
      if (sm == dm) mis = sm;
    }
    S* const dfix = (g.dst_mode == kDstOwner) ? (S*)ptrs.dst[c] : (S*)ptrs.dst[0] + lo;
    auto gsrc = [&](int k) -> const S* {
      const int r = TREE ? k : (c + 1 + k) % p;
      return (const S*)ptrs.src[r] + lo;
    };
    auto gdst = [&](int k) -> S* {
      if constexpr (DSTALL) return (S*)ptrs.dst[k] + lo;
      else return dfix;
    };
    for (uint64_t t = first_tile(base, wg, grid); t < ntiles; t += grid) {
      const TileSpan sp = tile_span<T::B, T::V>(len, TE, t, mis);
      reduce_tile<DT, OP, P, TREE, DSTALL>(gsrc, gdst, p, sp);
    }
    base += ntiles;
  }
}

template <int DT, int OP, int P, bool TREE>
static void launch_p(const RankPtrs& ptrs, const ReduceGeom& g, int grid, hipStream_t s) {
  if (g.dst_mode == kDstAll)
    hipLaunchKernelGGL((reduce_kernel<DT, OP, P, TREE, true>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
  else
    hipLaunchKernelGGL((reduce_kernel<DT, OP, P, TREE, false>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
}

template <int DT, int P>
static uint64_t count_tiles(const ReduceGeom& g) {
  constexpr uint64_t TE = reduce_tile_elems<DT, P>();
  uint64_t total = 0;
  for (int c = 0; c < g.p; ++c) {
    uint64_t lo = (uint64_t)c * g.stride, hi = lo + g.stride;
    if (lo > g.total) lo = g.total;
    if (hi > g.total) hi = g.total;
    total += (hi - lo + TE - 1) / TE;
  }
  return total;
}

static int clamp_grid(uint64_t tiles, int max_grid) {
  if (tiles == 0) return 0;
  return (int)(tiles < (uint64_t)max_grid ? tiles : (uint64_t)max_grid);
}

template <int DT, int OP>
static int launch_dt_op(bool tree, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                        hipStream_t s) {
  int grid = 0;
#define COLL_RING_CASE(PV)                                              \
  case PV:                                                              \
    grid = clamp_grid(count_tiles<DT, PV>(g), max_grid);                \
    if (grid) launch_p<DT, OP, PV, false>(ptrs, g, grid, s);            \
    break;
  if constexpr ((DT == kF32 || DT == kBF16) && OP == kSum) {
    if (tree) {
      switch (g.p) {
#define COLL_TREE_CASE(PV)                                              \
  case PV:                                                              \
    grid = clamp_grid(count_tiles<DT, PV>(g), max_grid);                \
    if (grid) launch_p<DT, OP, PV, true>(ptrs, g, grid, s);             \
    break;
        COLL_TREE_CASE(2)
        COLL_TREE_CASE(4)
        COLL_TREE_CASE(8)
        COLL_TREE_CASE(16)
#undef COLL_TREE_CASE
        default:
          return (int)hipErrorInvalidValue;
      }
      return (int)hipGetLastError();
    }
  }
  switch (g.p) {
    COLL_RING_CASE(2)
    COLL_RING_CASE(4)
    COLL_RING_CASE(8)
    COLL_RING_CASE(16)
    default:
      grid = clamp_grid(count_tiles<DT, 0>(g), max_grid);
      if (grid) launch_p<DT, OP, 0, false>(ptrs, g, grid, s);
      break;
  }
#undef COLL_RING_CASE
  return (int)hipGetLastError();
}

template <int DT>
static int launch_dt(int op, bool tree, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                     hipStream_t s) {
  switch (op) {
    case kSum: return launch_dt_op<DT, kSum>(tree, ptrs, g, max_grid, s);
    case kMin: return launch_dt_op<DT, kMin>(tree, ptrs, g, max_grid, s);
    case kMax: return launch_dt_op<DT, kMax>(tree, ptrs, g, max_grid, s);
  }
  return (int)hipErrorInvalidValue;
}

int launch_reduce(int dtype, int op, int algo_tree, const RankPtrs& ptrs, const ReduceGeom& g,
                  int max_grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const bool tree = algo_tree != 0;
  switch (dtype) {
    case kF32: return launch_dt<kF32>(op, tree, ptrs, g, max_grid, s);
    case kBF16: return launch_dt<kBF16>(op, tree, ptrs, g, max_grid, s);
    case kI32: return launch_dt<kI32>(op, tree, ptrs, g, max_grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
