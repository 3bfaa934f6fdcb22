// Direction-mix bandwidth probe: the attainable ceiling of a read:write
// stream mix, measured with the collectives' own tile code.
//
// "集合通信：原语、算法、NCCL 实现与拓扑映射" (hpc/04) section 4.1 models a
// collective's time with separate bandwidths per resource and compares
// bus bandwidth against what the hardware sustains (section 2.5).  With
// every rank in one HBM the resource is the memory system, and what it
// sustains depends on the mix of read and write streams a kernel keeps in
// flight.  This kernel streams NS sources and ND destinations of equal
// length through the same 16-byte vector tiles as the collectives (U
// vectors per lane, every load of a tile issued before its first store,
// the same launch bounds and grid sizing).  The caller sweeps the tile size
// U, the cache policy of the loads and of the stores (plain, non-temporal,
// device scope or both, as the collectives use them) and the grid, and
// takes the best, so a
// collective's throughput can be set against the ceiling of its own mix.  It is a measurement helper: destinations
// receive the XOR of the sources (a fixed pattern when NS = 0).  With no
// destination the loaded words are folded into one value per lane that
// is stored to a sink only if it equals a run-time pattern, so the loads
// cannot be optimised away.
#include <type_traits>

#include "device_common.h"

namespace coll {

// Vectors per lane of a tile: 1, 2, 4 or 8 (the collectives use the same
// range: 32/p or 16/p for reductions, 4 for copies), limited to 32 loads
// in flight per lane so that no variant spills.
constexpr bool probe_unroll_ok(int ns, int u) { return (u == 1 || u == 2 || u == 4 || u == 8) && ns * u <= 32; }

// One tile: U vectors per lane from every source, folded, then stored to
// every destination.  FULL: every vector lies inside the streams (no
// bounds checks, as in the collectives' full tiles).  hook(tok) runs after
// the loads have returned, before the stores (the claimed tiles' hook, as
// in the collectives).
template <int NS, int ND, bool NTL, int SP, int U, bool FULL, typename Hook = NoHook>
__device__ __forceinline__ void probe_tile(const u32x4* const (&src)[NS > 0 ? NS : 1],
                                           u32x4* const (&dst)[ND > 0 ? ND : 1], uint64_t j0, uint64_t nvec,
                                           u32x4* sink, uint32_t pattern, const Hook& hook = Hook{}) {
  constexpr int NSA = NS > 0 ? NS : 1;
  u32x4 v[U][NSA];
#pragma unroll
  for (int k = 0; k < NS; ++k)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t j = j0 + (uint64_t)u * kBlock;
      v[u][k] = (FULL || j < nvec) ? ld16<NTL>(src[k] + j) : u32x4{0, 0, 0, 0};
    }
  __builtin_amdgcn_sched_barrier(0);  // every load of the tile before the first store
  if constexpr (!std::is_same<Hook, NoHook>::value) {
    uint32_t tok = 0;
    if constexpr (NS > 0) asm volatile("" : "+v"(tok) : "v"(v[0][0]), "v"(v[U - 1][NS - 1]));
    hook(tok);
  }
  u32x4 x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (NS == 0) {
      const uint32_t j = (uint32_t)(j0 + (uint64_t)u * kBlock);
      x[u] = u32x4{j, j ^ pattern, j, j ^ pattern};
    } else {
      x[u] = v[u][0];
#pragma unroll
      for (int k = 1; k < NS; ++k) x[u] ^= v[u][k];
    }
  }
  if constexpr (ND == 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t f = x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
      if (f == pattern && x[u][0] == pattern) st16<false>(sink, x[u]);
    }
  } else {
#pragma unroll
    for (int d = 0; d < ND; ++d) store_tile<SP, U, kBlock, FULL>(dst[d], j0, nvec, x);
  }
}

// claim: null to deal out every tile in turn, else a claim slot: about a
// quarter of the tiles dealt out in turn and the rest claimed one at a time
// by workgroups from the slot's kClaimPools pooled counters, as the 1:1
// copies claim theirs (workgroup b from pool claim_pool(b); claim c of pool
// x is tile dealt + x + kClaimPools * c).  Thread 0 claims before a tile's
// loads and publishes after them through LDS.
template <int NS, int ND, bool NTL, int SP, int U>
COLL_STREAM_KERNEL void probe_kernel(RankPtrs ptrs, uint64_t nvec, u32x4* sink, uint32_t pattern,
                                     unsigned long long* claim) {
  constexpr uint64_t TV = (uint64_t)U * kBlock;
  const uint64_t nt = ceil_div(nvec, TV), nfull = nvec / TV;
  const uint64_t per = claim ? (nfull - dealt_tiles(nfull, gridDim.x)) / kClaimPools : 0;
  const uint64_t dealt = claim ? nfull - per * kClaimPools : nt;
  const uint32_t pool = claim_pool(blockIdx.x);
  unsigned long long* ctr = claim ? claim + pool * kClaimPoolWords : nullptr;
  unsigned long long first = 0;
  if (claim) first = issue_claim(ctr, (int)threadIdx.x);
  const u32x4* src[NS > 0 ? NS : 1];
  u32x4* dst[ND > 0 ? ND : 1];
#pragma unroll
  for (int k = 0; k < NS; ++k) src[k] = (const u32x4*)ptrs.src[k];
#pragma unroll
  for (int d = 0; d < ND; ++d) dst[d] = (u32x4*)ptrs.dst[d];
  for (uint64_t t = blockIdx.x; t < dealt; t += gridDim.x) {
    const uint64_t j0 = t * TV + threadIdx.x;
    if (t < nfull) probe_tile<NS, ND, NTL, SP, U, true>(src, dst, j0, nvec, sink, pattern);
    else probe_tile<NS, ND, NTL, SP, U, false>(src, dst, j0, nvec, sink, pattern);
  }
  if (!claim) return;
  // the partial last tile is dealt out; the whole tiles [dealt, nfull) are claimed
  if (nfull < nt && nfull % gridDim.x == blockIdx.x)
    probe_tile<NS, ND, NTL, SP, U, false>(src, dst, nfull * TV + threadIdx.x, nvec, sink, pattern);
  __shared__ uint64_t next_tile[2];
  const uint64_t first_claim = wave_value(first);
  if (threadIdx.x == 0) next_tile[0] = first_claim;
  __syncthreads();
  uint64_t u = next_tile[0];
  int par = 1;
  while (u < per) {
    const unsigned long long next = issue_claim(ctr, (int)threadIdx.x);
    const auto publish = [&](uint32_t tok) {
      const uint64_t v = wave_value(next + tok);
      if (threadIdx.x == 0) next_tile[par] = v;
    };
    const u32x4* gs[NS > 0 ? NS : 1];
    u32x4* gd[ND > 0 ? ND : 1];
#pragma unroll
    for (int k = 0; k < NS; ++k) gs[k] = as_global(src[k]);
#pragma unroll
    for (int d = 0; d < ND; ++d) gd[d] = as_global(dst[d]);
    probe_tile<NS, ND, NTL, SP, U, true>(gs, gd, (dealt + pool + (uint64_t)kClaimPools * u) * TV + threadIdx.x, nvec,
                                         sink, pattern, publish);
    asm volatile("" ::"v"(next));  // keep the claim's register out of the stores' reach
    __syncthreads();
    u = next_tile[par];
    par ^= 1;
  }
  if (threadIdx.x == 0) claim_last(ctr, u, per, claim_pool_members(gridDim.x, pool));
}

// The (sources, destinations) mixes the benchmark measures.
#define COLL_PROBE_MIXES(X) \
  X(1, 0) X(4, 0) X(8, 0) X(16, 0) X(0, 1) X(0, 4) X(0, 8) X(0, 16) X(1, 1) X(2, 1) X(3, 1) X(4, 1) X(5, 1) \
  X(6, 1) X(7, 1) X(8, 1) X(12, 1) X(16, 1) X(1, 2) X(1, 4) X(1, 8) X(1, 16) X(3, 3) X(4, 4) X(5, 5) X(6, 6) \
  X(7, 7) X(8, 8) X(12, 12) X(16, 16)

bool probe_mix_supported(int ns, int nd) {
#define COLL_PROBE_HAS(A, B) if (ns == A && nd == B) return true;
  COLL_PROBE_MIXES(COLL_PROBE_HAS)
#undef COLL_PROBE_HAS
  return false;
}

template <int NS, int ND, int U>
static int launch_mix_u(const RankPtrs& ptrs, uint64_t nvec, bool ntl, int sp, void* sink, int max_grid,
                        unsigned long long* claim, hipStream_t s) {
  if constexpr (!probe_unroll_ok(NS, U)) {
    return (int)hipErrorInvalidValue;
  } else {
    constexpr uint64_t TV = (uint64_t)U * kBlock;
    const uint64_t nt = (nvec + TV - 1) / TV;
    const int grid = (int)(nt < (uint64_t)max_grid ? nt : (uint64_t)max_grid);
    if (grid == 0) return 0;
    u32x4* sk = (u32x4*)sink;
    const uint32_t pat = 0x9e3779b9u;
    const dim3 g(grid), b(kBlock);
    // claims only with enough whole tiles per workgroup, and a workgroup in
    // every pool
    unsigned long long* cl =
        nvec / TV >= kClaimMinTilesPerWg * (uint64_t)grid && grid >= kClaimPools * kClaimPools ? claim : nullptr;
    if (ntl == false && sp == kStPlain)
      hipLaunchKernelGGL((probe_kernel<NS, ND, false, kStPlain, U>), g, b, 0, s, ptrs, nvec, sk, pat, cl);
    else if (ntl == false && sp == kStNT)
      hipLaunchKernelGGL((probe_kernel<NS, ND, false, kStNT, U>), g, b, 0, s, ptrs, nvec, sk, pat, cl);
    else if (ntl == false && sp == kStDevice)
      hipLaunchKernelGGL((probe_kernel<NS, ND, false, kStDevice, U>), g, b, 0, s, ptrs, nvec, sk, pat, cl);
    else if (ntl == true && sp == kStPlain)
      hipLaunchKernelGGL((probe_kernel<NS, ND, true, kStPlain, U>), g, b, 0, s, ptrs, nvec, sk, pat, cl);
    else if (ntl == true && sp == kStNT)
      hipLaunchKernelGGL((probe_kernel<NS, ND, true, kStNT, U>), g, b, 0, s, ptrs, nvec, sk, pat, cl);
    else if (ntl == true && sp == kStDevice)
      hipLaunchKernelGGL((probe_kernel<NS, ND, true, kStDevice, U>), g, b, 0, s, ptrs, nvec, sk, pat, cl);
    else if (ntl == false && sp == kStNTDevice)
      hipLaunchKernelGGL((probe_kernel<NS, ND, false, kStNTDevice, U>), g, b, 0, s, ptrs, nvec, sk, pat, cl);
    else if (ntl == true && sp == kStNTDevice)
      hipLaunchKernelGGL((probe_kernel<NS, ND, true, kStNTDevice, U>), g, b, 0, s, ptrs, nvec, sk, pat, cl);
    else
      return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
  }
}

template <int NS, int ND>
static int launch_mix(const RankPtrs& ptrs, uint64_t nvec, int unroll, bool ntl, int sp, void* sink,
                      int max_grid, unsigned long long* claim, hipStream_t s) {
  switch (unroll) {
    case 1: return launch_mix_u<NS, ND, 1>(ptrs, nvec, ntl, sp, sink, max_grid, claim, s);
    case 2: return launch_mix_u<NS, ND, 2>(ptrs, nvec, ntl, sp, sink, max_grid, claim, s);
    case 4: return launch_mix_u<NS, ND, 4>(ptrs, nvec, ntl, sp, sink, max_grid, claim, s);
    case 8: return launch_mix_u<NS, ND, 8>(ptrs, nvec, ntl, sp, sink, max_grid, claim, s);
  }
  return (int)hipErrorInvalidValue;
}

bool probe_unroll_supported(int ns, int unroll) { return probe_unroll_ok(ns, unroll); }

int launch_probe(int ns, int nd, const RankPtrs& ptrs, uint64_t nvec, int unroll, bool nt_loads, int store_policy,
                 void* sink, int max_grid, unsigned long long* claim, void* stream) {
  hipStream_t s = (hipStream_t)stream;
#define COLL_PROBE_CASE(A, B) \
  if (ns == A && nd == B) return launch_mix<A, B>(ptrs, nvec, unroll, nt_loads, store_policy, sink, max_grid, claim, s);
  COLL_PROBE_MIXES(COLL_PROBE_CASE)
#undef COLL_PROBE_CASE
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
