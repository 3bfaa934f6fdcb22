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
// order, partial in registers, p stores; tile 0 of a chunk also does the
// chunk's misaligned head and tail.
#include "reduce_tile.h"

namespace coll {

// Elements of a batch tile: one vector tile of the AllReduce kernel.
template <int DT, int P>
__host__ __device__ constexpr uint64_t batch_tile_elems() {
  return (uint64_t)ReduceUnroll<P, true>::value * kBlock * Traits<DT>::V;
}

template <int DT, int OP, int P>
__device__ __forceinline__ void batch_tile(const BatchCall& bc, const void* const* pt, uint64_t local) {
  using T = Traits<DT>;
  using S = typename T::S;
  constexpr int U = ReduceUnroll<P, true>::value;
  constexpr uint64_t TV = (uint64_t)U * kBlock;
  constexpr int V = T::V;
  const uint64_t tpc = bc.tiles_per_chunk;
  const int c = (int)(local / tpc);
  const uint64_t t = local - (uint64_t)c * tpc;
  const uint64_t q = (bc.n + P - 1) / P;
  uint64_t lo = (uint64_t)c * q, hi = lo + q;
  if (lo > bc.n) lo = bc.n;
  if (hi > bc.n) hi = bc.n;
  const uint64_t len = hi - lo;
  if (len == 0) return;
  const S* src[P];
  S* dst[P];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    src[k] = (const S*)pt[(c + 1 + k) % P] + lo;
    dst[k] = (S*)pt[P + k] + lo;
  }
  const int mis = bc.mis < 0 ? -1 : (int)((bc.mis + lo * T::B) & 15);
  const SegSpan sp = seg_span<T::B>(len, mis);
  if (!sp.vec) {
    const uint64_t from = t * TV * V;
    if (from < len) {
      const uint64_t cnt = (len - from) < TV * V ? (len - from) : TV * V;
      reduce_elems<DT, OP, P, false, P, true>(src, dst, from, cnt);
    }
    return;
  }
  if (t * TV < sp.nvec) {
    const S* vs[P];
    S* vd[P];
#pragma unroll
    for (int k = 0; k < P; ++k) {
      vs[k] = src[k] + sp.head;
      vd[k] = dst[k] + sp.head;
    }
    reduce_vec_tile<DT, OP, P, false, P, true, U, false>(vs, vd, t * TV + threadIdx.x, sp.nvec);
  }
  if (t == 0) {
    if (sp.head) reduce_elems<DT, OP, P, false, P, true>(src, dst, 0, sp.head);
    if (sp.tail) reduce_elems<DT, OP, P, false, P, true>(src, dst, sp.head + sp.nvec * V, sp.tail);
  }
}

// Any rank count: element path with pointers read from the table.
template <int DT, int OP>
__device__ __forceinline__ void batch_tile_any(const BatchCall& bc, const void* const* pt, int p, uint64_t local) {
  using T = Traits<DT>;
  using S = typename T::S;
  using A = typename T::A;
  constexpr uint64_t TE = (uint64_t)kBlock * T::V;
  const uint64_t tpc = bc.tiles_per_chunk;
  const int c = (int)(local / tpc);
  const uint64_t t = local - (uint64_t)c * tpc;
  const uint64_t q = (bc.n + p - 1) / p;
  uint64_t lo = (uint64_t)c * q, hi = lo + q;
  if (lo > bc.n) lo = bc.n;
  if (hi > bc.n) hi = bc.n;
  const uint64_t len = hi - lo;
  for (uint64_t e = t * TE + threadIdx.x; e < len && e < (t + 1) * TE; e += kBlock) {
    A acc = widen1<DT>(ld1<true>((const S*)pt[(c + 1) % p] + lo + e));
    for (int k = 1; k < p; ++k) acc = combine<OP>(acc, widen1<DT>(ld1<true>((const S*)pt[(c + 1 + k) % p] + lo + e)));
    const S out = narrow1<DT>(acc);
    for (int k = 0; k < p; ++k) st1<true>((S*)pt[p + k] + lo + e, out);
  }
}

template <int P>
__device__ __forceinline__ void batch_dispatch(const BatchCall& bc, const void* const* pt, int p, uint64_t local) {
#define COLL_BATCH_CASE(DTV, OPV)                                          \
  case DTV * 3 + OPV:                                                      \
    if constexpr (P > 0) batch_tile<DTV, OPV, P>(bc, pt, local);           \
    else batch_tile_any<DTV, OPV>(bc, pt, p, local);                       \
    break;
  switch (bc.dtype * 3 + bc.op) {
    COLL_BATCH_CASE(kF32, kSum)
    COLL_BATCH_CASE(kF32, kMin)
    COLL_BATCH_CASE(kF32, kMax)
    COLL_BATCH_CASE(kBF16, kSum)
    COLL_BATCH_CASE(kBF16, kMin)
    COLL_BATCH_CASE(kBF16, kMax)
    COLL_BATCH_CASE(kI32, kSum)
    COLL_BATCH_CASE(kI32, kMin)
    COLL_BATCH_CASE(kI32, kMax)
    default: break;
  }
#undef COLL_BATCH_CASE
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

uint64_t batch_tile_elems_host(int dtype, int p) {
  const bool bf = dtype == kBF16;
  switch (p) {
    case 2: return bf ? batch_tile_elems<kBF16, 2>() : batch_tile_elems<kF32, 2>();
    case 4: return bf ? batch_tile_elems<kBF16, 4>() : batch_tile_elems<kF32, 4>();
    case 8: return bf ? batch_tile_elems<kBF16, 8>() : batch_tile_elems<kF32, 8>();
    case 16: return bf ? batch_tile_elems<kBF16, 16>() : batch_tile_elems<kF32, 16>();
    default: return (uint64_t)kBlock * (bf ? 8 : 4);
  }
}

int launch_batch(const BatchArgs& a, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (a.p) {
    case 2: hipLaunchKernelGGL((batch_kernel<2>), dim3(grid), dim3(kBlock), 0, s, a); break;
    case 4: hipLaunchKernelGGL((batch_kernel<4>), dim3(grid), dim3(kBlock), 0, s, a); break;
    case 8: hipLaunchKernelGGL((batch_kernel<8>), dim3(grid), dim3(kBlock), 0, s, a); break;
    case 16: hipLaunchKernelGGL((batch_kernel<16>), dim3(grid), dim3(kBlock), 0, s, a); break;
    default: hipLaunchKernelGGL((batch_kernel<0>), dim3(grid), dim3(kBlock), 0, s, a); break;
  }
  return (int)hipGetLastError();
}

}  // namespace coll
