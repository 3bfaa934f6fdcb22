// All-to-All through LDS: the p x p block transpose of
// "集合通信：原语、算法、NCCL 实现与拓扑映射" section 1.6 (block j of rank
// i becomes block i of rank j), with every 16-byte vector staged in LDS on
// its way from the source block to the destination block.
//
// gfx950 loads global memory straight into LDS (global_load_lds_dwordx4):
// the loaded bytes occupy no VGPRs, so a wave can keep a deep stage in
// flight.  Each wave is an independent worker with two private stages of
// kA2aLdsU vectors per lane (kA2aLdsU KiB each).  While the vectors of one
// stage are read back from LDS and stored to the destination, the loads of
// the wave's next tile fill the other stage.
//
// The compiler does not order an LDS read after an earlier
// global-to-LDS load of the same bytes, so each wave waits for its
// outstanding vector-memory operations (vmcnt 0) before it reads a stage
// back.  Stages are private to a wave, so no workgroup barrier is needed.
//
// This is the vector path only: every segment (i, j) must share one
// 16-byte misalignment (common source and destination misalignment and a
// block size that is a multiple of 16 bytes).  The host sends other
// layouts to the direct copy kernel.  The misaligned head and tail of each
// segment (shorter than one vector) are copied element by element.
#include "copy_tile.h"

namespace coll {

constexpr int kA2aLdsU = 8;                   // vectors per lane per stage
constexpr int kWavesPerWg = kBlock / 64;      // 4
constexpr uint64_t kA2aLdsTV = (uint64_t)kA2aLdsU * 64;  // vectors per wave tile

// s_waitcnt with vmcnt(0) and the other counters left alone (gfx9
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_sched_barrier(0);
}

// Where a wave tile lives: its source and destination vectors (at the
// segment's first aligned vector) and its first vector index.
struct LdsTile {
  const u32x4* src;
  u32x4* dst;
  uint64_t j0;
  bool full;  // all kA2aLdsTV vectors lie inside the segment
};

template <int B>
COLL_STREAM_KERNEL void alltoall_lds_kernel(RankPtrs ptrs, CopyGeom g, uint64_t head, uint64_t nvec,
                                            uint64_t tail) {
  using W = typename Word<B>::T;
  // [wave][stage][u * 64 + lane]: 4 * 2 * 8 * 64 * 16 B = 64 KiB
  __shared__ u32x4 stage[kWavesPerWg][2][kA2aLdsU * 64];
  const int p = g.p;
  const uint64_t n = g.n;
  const int lane = (int)(threadIdx.x & 63);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The host sends calls with 2^32 or more wave tiles to the direct
  // kernel, so tile indices fit 32 bits (and 32-bit division).
  const uint32_t nw = gridDim.x * (uint32_t)kWavesPerWg;
  const uint32_t wid = blockIdx.x * (uint32_t)kWavesPerWg + (uint32_t)wave;
  const uint32_t tps = (uint32_t)((nvec + kA2aLdsTV - 1) / kA2aLdsTV);  // wave tiles per segment
  const uint32_t total = (uint32_t)p * (uint32_t)p * tps;

  auto locate = [&](uint32_t f) {
    const uint32_t sg = f / tps;
    const uint32_t t = f - sg * tps;
    const uint32_t i = sg / (uint32_t)p, j = sg - i * (uint32_t)p;
    LdsTile x;
    x.src = (const u32x4*)((const W*)ptrs.src[i] + (uint64_t)j * n + head);
    x.dst = (u32x4*)((W*)ptrs.dst[j] + (uint64_t)i * n + head);
    x.j0 = (uint64_t)t * kA2aLdsTV;
    x.full = x.j0 + kA2aLdsTV <= nvec;
    return x;
  };
  // Lanes past the end of a partial tile load the segment's last vector
  // again (in bounds, and never stored), so the loads need no branch.
  auto issue = [&](const LdsTile& x, int st) {
#pragma unroll
    for (int u = 0; u < kA2aLdsU; ++u) {
      uint64_t jv = x.j0 + (uint64_t)u * 64 + lane;
      jv = jv < nvec ? jv : nvec - 1;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(x.src + jv),
                                       (__attribute__((address_space(3))) void*)&stage[wave][st][u * 64],
                                       16, 0, 0);
    }
  };

  if (wid < total) {
    int st = 0;
    LdsTile cur = locate(wid);
    issue(cur, 0);
    for (uint32_t f = wid; f < total; f += nw) {
      wait_vmem_all();  // stage st has landed (and the previous stores are done)
      LdsTile nxt;
      const bool more = f + nw < total;
      if (more) {
        nxt = locate(f + nw);
        issue(nxt, st ^ 1);
      }
      u32x4 r[kA2aLdsU];
#pragma unroll
      for (int u = 0; u < kA2aLdsU; ++u) r[u] = stage[wave][st][u * 64 + lane];
      if (cur.full) {
#pragma unroll
        for (int u = 0; u < kA2aLdsU; ++u) st16<true>(cur.dst + cur.j0 + (uint64_t)u * 64 + lane, r[u]);
      } else {
#pragma unroll
        for (int u = 0; u < kA2aLdsU; ++u) {
          const uint64_t jv = cur.j0 + (uint64_t)u * 64 + lane;
          if (jv < nvec) st16<true>(cur.dst + jv, r[u]);
        }
      }
      if (more) cur = nxt;
      st ^= 1;
    }
  }

  // Heads and tails, one segment per wave.
  if (head || tail) {
    for (uint32_t sg = wid; sg < (uint32_t)p * (uint32_t)p; sg += nw) {
      const uint32_t i = sg / (uint32_t)p, j = sg - i * (uint32_t)p;
      const W* s = (const W*)ptrs.src[i] + (uint64_t)j * n;
      W* d = (W*)ptrs.dst[j] + (uint64_t)i * n;
      const uint64_t e = (uint64_t)lane;
      if (e < head + tail) {
        const uint64_t x = e < head ? e : head + nvec * (16 / B) + (e - head);
        st1<true>(d + x, ld1<true>(s + x));
      }
    }
  }
}

// Host side.  Returns hipErrorInvalidValue when the layout needs the
// direct kernel (the caller checks can_stage_alltoall first).
bool can_stage_alltoall(int elem_bytes, const CopyGeom& g) {
  if (!(g.src_mis >= 0 && g.src_mis == g.dst_mis && g.src_mis % elem_bytes == 0 &&
        (g.n * (uint64_t)elem_bytes) % 16 == 0))
    return false;
  // the kernel counts wave tiles in 32 bits
  const uint64_t tiles = (uint64_t)g.p * g.p * ((g.n * (uint64_t)elem_bytes / 16 + kA2aLdsTV - 1) / kA2aLdsTV);
  return tiles < (uint64_t{1} << 32);
}

int launch_alltoall_lds(int elem_bytes, const RankPtrs& ptrs, const CopyGeom& g, int max_grid, void* stream) {
  if (!can_stage_alltoall(elem_bytes, g)) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t v = 16 / (uint64_t)elem_bytes;
  const uint64_t head = (uint64_t)(((16 - g.src_mis) & 15) / elem_bytes) < g.n
                            ? (uint64_t)(((16 - g.src_mis) & 15) / elem_bytes)
                            : g.n;
  const uint64_t nvec = (g.n - head) / v;
  const uint64_t tail = g.n - head - nvec * v;
  const uint64_t tiles = (uint64_t)g.p * g.p * ((nvec + kA2aLdsTV - 1) / kA2aLdsTV);
  const uint64_t waves = tiles > (uint64_t)g.p * g.p ? tiles : (uint64_t)g.p * g.p;
  uint64_t grid = (waves + kWavesPerWg - 1) / kWavesPerWg;
  if (grid > (uint64_t)max_grid) grid = (uint64_t)max_grid;
  if (grid == 0) return 0;
  if (elem_bytes == 1)
    hipLaunchKernelGGL((alltoall_lds_kernel<1>), dim3((unsigned)grid), dim3(kBlock), 0, s, ptrs, g, head, nvec, tail);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL((alltoall_lds_kernel<2>), dim3((unsigned)grid), dim3(kBlock), 0, s, ptrs, g, head, nvec, tail);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL((alltoall_lds_kernel<4>), dim3((unsigned)grid), dim3(kBlock), 0, s, ptrs, g, head, nvec, tail);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace coll
