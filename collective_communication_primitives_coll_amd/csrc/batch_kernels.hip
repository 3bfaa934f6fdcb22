// Batched AllReduce: many independent AllReduces in one launch.
//
// Small collectives are dominated by the fixed per-call cost (the alpha
// term of the alpha-beta model, "集合通信：原语、算法、NCCL 实现与拓扑映射"
// section 2.1); fusing them into one launch pays it once, as bucketing and
// group calls do (sections 4.2 and 3.9 there; "Collective Communication"
// page, group calls).
//
// The host lays out, per call, p chunks of ceil(n/p) elements, each cut
// into tiles_per_chunk tiles, and a prefix of tile counts over the calls.
// Each workgroup takes one contiguous run of the flat tile range, finds
// its first call by binary search and then steps forward through the
// calls, so the descriptor lookups per tile are a single comparison.
// Within a tile the work is exactly the single-call AllReduce's: ring
// order, partial in registers, p stores.
#include "reduce_tile.h"

namespace coll {

template <int DT, int OP, int P>
__device__ __forceinline__ void batch_tile(const BatchCall& bc, const void* const* pt, int p, uint64_t local) {
  using T = Traits<DT>;
  using S = typename T::S;
  constexpr uint64_t TE = (uint64_t)kBlock * T::V;  // one vector per lane
  const uint64_t tpc = bc.tiles_per_chunk;
  const int c = (int)(local / tpc);
  const uint64_t ti = local - (uint64_t)c * tpc;
  const uint64_t q = (bc.n + p - 1) / p;
  uint64_t lo = (uint64_t)c * q, hi = lo + q;
  if (lo > bc.n) lo = bc.n;
  if (hi > bc.n) hi = bc.n;
  const uint64_t len = hi - lo;
  if (ti * TE >= len) return;
  const int mis = bc.mis < 0 ? -1 : (int)((bc.mis + lo * T::B) & 15);
  auto gsrc = [&](int k) -> const S* { return (const S*)pt[(c + 1 + k) % p] + lo; };
  auto gdst = [&](int k) -> S* { return (S*)pt[p + k] + lo; };
  const TileSpan sp = tile_span<T::B, T::V>(len, TE, ti, mis);
  // P > 0 instantiations use UNROLL 1 here: the tile is one vector per lane.
  if (sp.vec) {
    if (sp.nvec) reduce_vectors<DT, OP, P, false, true, 1>(gsrc, gdst, p, sp.begin + sp.head, sp.nvec);
    if (sp.head) reduce_elems<DT, OP, P, false, true>(gsrc, gdst, p, sp.begin, sp.head);
    if (sp.tail)
      reduce_elems<DT, OP, P, false, true>(gsrc, gdst, p, sp.begin + sp.head + sp.nvec * T::V, sp.tail);
  } else {
    reduce_elems<DT, OP, P, false, true>(gsrc, gdst, p, sp.begin, sp.head);
  }
}

template <int P>
__device__ __forceinline__ void batch_dispatch(const BatchCall& bc, const void* const* pt, int p, uint64_t local) {
  switch (bc.dtype * 3 + bc.op) {
    case kF32 * 3 + kSum: batch_tile<kF32, kSum, P>(bc, pt, p, local); break;
    case kF32 * 3 + kMin: batch_tile<kF32, kMin, P>(bc, pt, p, local); break;
    case kF32 * 3 + kMax: batch_tile<kF32, kMax, P>(bc, pt, p, local); break;
    case kBF16 * 3 + kSum: batch_tile<kBF16, kSum, P>(bc, pt, p, local); break;
    case kBF16 * 3 + kMin: batch_tile<kBF16, kMin, P>(bc, pt, p, local); break;
    case kBF16 * 3 + kMax: batch_tile<kBF16, kMax, P>(bc, pt, p, local); break;
    case kI32 * 3 + kSum: batch_tile<kI32, kSum, P>(bc, pt, p, local); break;
    case kI32 * 3 + kMin: batch_tile<kI32, kMin, P>(bc, pt, p, local); break;
    case kI32 * 3 + kMax: batch_tile<kI32, kMax, P>(bc, pt, p, local); break;
    default: break;
  }
}

template <int P>
__global__ __launch_bounds__(kBlock) void batch_kernel(BatchArgs a) {
  const int p = P ? P : a.p;
  const uint64_t total = a.calls[a.ncalls].first_tile;
  const uint64_t grid = gridDim.x;
  const uint64_t per = (total + grid - 1) / grid;
  uint64_t t = (uint64_t)blockIdx.x * per;
  uint64_t end = t + per;
  if (end > total) end = total;
  if (t >= end) return;
  // binary search: last call whose first tile is <= t
  int lo = 0, hi = a.ncalls;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.calls[mid].first_tile <= t) lo = mid;
    else hi = mid;
  }
  int k = lo;
  uint64_t next_first = a.calls[k + 1].first_tile;
  for (; t < end; ++t) {
    while (t >= next_first) {
      ++k;
      next_first = a.calls[k + 1].first_tile;
    }
    const BatchCall bc = a.calls[k];
    batch_dispatch<P>(bc, a.ptrs + (size_t)k * 2 * p, p, t - bc.first_tile);
  }
}

int launch_batch(const BatchArgs& a, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.p == 16)
    hipLaunchKernelGGL((batch_kernel<16>), dim3(grid), dim3(kBlock), 0, s, a);
  else if (a.p == 8)
    hipLaunchKernelGGL((batch_kernel<8>), dim3(grid), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((batch_kernel<0>), dim3(grid), dim3(kBlock), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace coll
