// The ring all-reduce of "集合通信：原语、算法、NCCL 实现与拓扑映射" (hpc/04,
// section 2.2) executed literally: every neighbour step is one kernel
// launch and every partial goes through HBM.
//
// The receive buffers hold the ring's per-rank working copies.  With
// q = ceil(n/p) elements per chunk:
//   reduce-scatter step s (1..p-1): every rank X sends chunk (X - s) mod p
//     to X+1, which combines it with its own input:
//       recv[X+1][c] = (s == 1 ? send[X][c] : recv[X][c]) (+) send[X+1][c]
//   all-gather step t (1..p-1): every rank X forwards chunk (X + 1 - t) mod p:
//       recv[X+1][c] = recv[X][c]
// Chunk c's partial visits ranks c+1, c+2, ..., c and is finished on rank
// c, so the result equals the fused ring kernel bit for bit.  Sends of one
// step never touch the chunk the sender receives in that step, so the
// ranks of a step run concurrently without races; steps are ordered by the
// stream.  Combining in HBM costs (p-1)*3 + (p-1)*2 chunk passes per rank
// instead of the fused kernel's single read and write.
#include "device_common.h"

namespace coll {

template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void ring_step_kernel(RankPtrs ptrs, RingStepGeom g) {
  using T = Traits<DT>;
  using S = typename T::S;
  using A = typename T::A;
  constexpr int V = T::V;
  constexpr int U = 2;
  constexpr uint64_t TE = (uint64_t)U * kBlock * V;
  const int p = g.p;
  const uint64_t grid = gridDim.x, wg = blockIdx.x;
  const uint64_t tid = threadIdx.x;
  uint64_t base = 0;
  for (int x = 0; x < p; ++x) {
    const int nxt = (x + 1) % p;
    const int c = g.phase == 0 ? ((x - g.step) % p + p) % p : ((x + 1 - g.step) % p + p) % p;
    uint64_t lo = (uint64_t)c * g.q, hi = lo + g.q;
    if (lo > g.n) lo = g.n;
    if (hi > g.n) hi = g.n;
    const uint64_t len = hi - lo;
    if (len == 0) continue;
    const uint64_t ntiles = ceil_div(len, TE);
    const S* a = (g.phase == 0 && g.step == 1) ? (const S*)ptrs.src[x] + lo : (const S*)ptrs.dst[x] + lo;
    const S* b = (const S*)ptrs.src[nxt] + lo;
    S* d = (S*)ptrs.dst[nxt] + lo;
    const int mis = g.mis < 0 ? -1 : (int)((g.mis + lo * T::B) & 15);
    for (uint64_t t = first_tile(base, wg, grid); t < ntiles; t += grid) {
      const TileSpan sp = tile_span<T::B, V>(len, TE, t, mis);
      auto elems = [&](uint64_t from, uint64_t cnt) {
        for (uint64_t i = tid; i < cnt; i += kBlock) {
          const uint64_t e = from + i;
          if (g.phase == 0)
            st1(d + e, narrow1<DT>(combine<OP>(widen1<DT>(ld1(a + e)), widen1<DT>(ld1(b + e)))));
          else
            st1(d + e, ld1(a + e));
        }
      };
      if (!sp.vec) {
        elems(sp.begin, sp.head);
        continue;
      }
      const uint64_t v0 = sp.begin + sp.head;
      u32x4 ra[U], rb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t vi = (uint64_t)u * kBlock + tid;
        if (vi < sp.nvec) {
          ra[u] = ld16(a + v0 + vi * V);
          if (g.phase == 0) rb[u] = ld16(b + v0 + vi * V);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t vi = (uint64_t)u * kBlock + tid;
        if (vi < sp.nvec) {
          if (g.phase == 0) {
            A acc[V], t2[V];
            widen<DT>(ra[u], acc);
            widen<DT>(rb[u], t2);
            combine_vec<OP, DT>(acc, t2);
            st16(d + v0 + vi * V, narrow<DT>(acc));
          } else {
            st16(d + v0 + vi * V, ra[u]);
          }
        }
      }
      if (sp.head) elems(sp.begin, sp.head);
      if (sp.tail) elems(sp.begin + sp.head + sp.nvec * V, sp.tail);
    }
    base += ntiles;
  }
}

template <int DT>
static int launch_dt(int op, const RankPtrs& ptrs, const RingStepGeom& g, int grid, hipStream_t s) {
  switch (op) {
    case kSum:
      hipLaunchKernelGGL((ring_step_kernel<DT, kSum>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
      break;
    case kMin:
      hipLaunchKernelGGL((ring_step_kernel<DT, kMin>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
      break;
    case kMax:
      hipLaunchKernelGGL((ring_step_kernel<DT, kMax>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_ring_step(int dtype, int op, const RankPtrs& ptrs, const RingStepGeom& g, int max_grid,
                     void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const uint64_t te = 2ull * kBlock * (dtype == kBF16 ? 8 : 4);
  uint64_t tiles = (uint64_t)g.p * ((g.q + te - 1) / te);
  if (tiles == 0) return 0;
  const int grid = (int)(tiles < (uint64_t)max_grid ? tiles : (uint64_t)max_grid);
  switch (dtype) {
    case kF32: return launch_dt<kF32>(op, ptrs, g, grid, s);
    case kI32: return launch_dt<kI32>(op, ptrs, g, grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
