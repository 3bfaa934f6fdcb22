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
#include "copy_tile.h"
#include "reduce_tile.h"

namespace coll {

template <int DT, int OP>
COLL_STREAM_KERNEL void ring_step_kernel(RankPtrs ptrs, RingStepGeom g) {
  using T = Traits<DT>;
  using S = typename T::S;
  const int p = g.p;
  uint64_t base = 0;
  for (int x = 0; x < p; ++x) {
    const int nxt = (x + 1) % p;
    const int c = g.phase == 0 ? ((x - g.step) % p + p) % p : ((x + 1 - g.step) % p + p) % p;
    uint64_t lo = (uint64_t)c * g.q, hi = lo + g.q;
    if (lo > g.n) lo = g.n;
    if (hi > g.n) hi = g.n;
    const uint64_t len = hi - lo;
    if (len == 0) continue;
    const int mis = g.mis < 0 ? -1 : (int)((g.mis + lo * T::B) & 15);
    const S* partial = (g.phase == 0 && g.step == 1) ? (const S*)ptrs.src[x] + lo : (const S*)ptrs.dst[x] + lo;
    S* d = (S*)ptrs.dst[nxt] + lo;
    if (g.phase == 0) {
      // received partial on the left, the receiver's own input on the right;
      // an average is a sum until the last step, which divides by p
      const S* src[2] = {partial, (const S*)ptrs.src[nxt] + lo};
      S* dst[1] = {d};
      const Scales<2> sc{};
      if (OP == kAvg && g.step == p - 1)
        base += reduce_segment<DT, kAvg, 2, kOrdRing, 1, false>(src, dst, len, mis, -1, base, sc, p);
      else
        base += reduce_segment<DT, OP == kAvg ? kSum : OP, 2, kOrdRing, 1, false>(src, dst, len, mis, -1, base, sc, p);
    } else {
      using W = typename Word<T::B>::T;
      auto gdst = [&](int) -> W* { return (W*)d; };
      base += copy_segment<T::B, true, 1, false>((const W*)partial, gdst, 1, len, mis, -1, base);
    }
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
    case kAvg:
      hipLaunchKernelGGL((ring_step_kernel<DT, kAvg>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_ring_step(int dtype, int op, const RankPtrs& ptrs, const RingStepGeom& g, int max_grid,
                     void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const uint64_t te = (uint64_t)ReduceUnroll<2, false>::value * kBlock * (dtype == kBF16 ? 8 : 4);
  const uint64_t tiles = (uint64_t)g.p * ((g.q + te - 1) / te + 1);
  if (g.q == 0) return 0;
  const int grid = (int)(tiles < (uint64_t)max_grid ? tiles : (uint64_t)max_grid);
  switch (dtype) {
    case kF32: return launch_dt<kF32>(op, ptrs, g, grid, s);
    case kI32: return launch_dt<kI32>(op, ptrs, g, grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
