// AllReduce, Reduce and ReduceScatter: one kernel family (kernels and their
// launchers; reduce_kernels.hip and reduce_kernels_p*.hip instantiate them
// for the rank counts each covers).
//
// Segment c is chunk c of the operation: for AllReduce and Reduce the
// elements [c*q, (c+1)*q) with q = ceil(n/p); for ReduceScatter block c of
// every rank's [p*n] input.  Every workgroup walks the segments in order
// and takes the tiles whose flat index is congruent to its id modulo the
// grid, so all p segments spread over the whole chip.  The destination
// mode picks where a segment's result goes:
//   all    every rank's buffer at the segment offset (AllReduce: the
//          reduce-scatter result of chunk c and its all-gather to every
//          rank come out of one pass; stores are non-temporal),
//   fixed  the root buffer at the segment offset (Reduce),
//   owner  rank c's buffer from its start (ReduceScatter, block c lands on
//          rank c: "集合通信：原语、算法、NCCL 实现与拓扑映射", section 1.5).
// A segment's sources are read from the kernel arguments with constant
// offsets and put in the schedule's order in registers (list_for_chunk).
#pragma once

#include "reduce_tile.h"

namespace coll {

// Rank listed k-th for chunk c (the order list_for_chunk produces).
template <int ORD, int P>
__device__ __forceinline__ int listed_rank(int c, int k) {
  if constexpr (ORD == kOrdRing) return (c + 1 + k) % P;
  else if constexpr (ORD == kOrdDBT) return c < P / 2 ? k : P - 1 - k;
  else return k;
}

__device__ __forceinline__ void chunk_range(const ReduceGeom& g, int c, uint64_t* lo, uint64_t* len) {
  uint64_t a = (uint64_t)c * g.stride;
  uint64_t b = a + g.stride;
  if (a > g.total) a = g.total;
  if (b > g.total) b = g.total;
  *lo = a;
  *len = b - a;
}

// Operands of chunk c starting lo elements into every buffer: the p
// sources in the schedule's order, the destinations of the mode, and the
// per-operand scales.
template <int DT, int OP, int P, int ORD, int DMODE, int ND>
__device__ __forceinline__ void chunk_operands(const RankPtrs& ptrs, const ReduceGeom& g, int c, uint64_t lo,
                                               const typename Traits<DT>::S* (&src)[P],
                                               typename Traits<DT>::S* (&dst)[ND], Scales<P>& sc) {
  using S = typename Traits<DT>::S;
#pragma unroll
  for (int k = 0; k < P; ++k) src[k] = (const S*)ptrs.src[k];
  list_for_chunk<ORD, P>(src, c);
#pragma unroll
  for (int k = 0; k < P; ++k) src[k] += lo;
  if constexpr (DMODE == kDstAll) {
#pragma unroll
    for (int k = 0; k < P; ++k) dst[k] = (S*)ptrs.dst[k] + lo;
  } else if constexpr (DMODE == kDstOwner) {
    dst[0] = (S*)ptrs.dst[c];
  } else {
    dst[0] = (S*)ptrs.dst[0] + lo;
  }
  // The scales (pre-multiplied sums only) are indexed by the listed rank
  // directly: reordering them in registers as the pointers are left an
  // unused stack reservation in some kernels.
#pragma unroll
  for (int k = 0; k < P; ++k) sc.s[k] = OP == kPreMul ? g.scale[listed_rank<ORD, P>(c, k)] : 1.0f;
}

// Geometry of segment c: its range, the vector/element split and its
// workgroup tile count.
template <int DT, int P, int DMODE>
struct SegGeom {
  uint64_t lo, len, nt;
  int mis, amis;
  SegSpan sp;
  __device__ __forceinline__ SegGeom(const ReduceGeom& g, int c) {
    constexpr int ND = DMODE == kDstAll ? P : 1;
    chunk_range(g, c, &lo, &len);
    const uint64_t doff = (DMODE == kDstOwner) ? 0 : lo;
    mis = seg_mis(g.src_mis, g.dst_mis, lo * Traits<DT>::B, doff * Traits<DT>::B);
    amis = seg_amis(g.src_amis, lo * Traits<DT>::B);
    sp = seg_span_a<Traits<DT>::B>(len, mis, amis);
    nt = segment_tiles<DT, P, ND>(sp, len);
  }
};

// The claimed tiles [dealt, total) of reduce_kernel (AllReduce and
// ReduceScatter), one workgroup tile per claim.
// - Thread 0 claims; the value reaches the other threads through LDS at a
//   barrier (on gfx950 a workgroup barrier waits for LDS operations only,
//   not for the tile's stores).  It goes to one of two LDS words in turn,
//   so a fast wave cannot overwrite it before a slow one has read it.
// - A single counter serves about 83 claims per microsecond (12 ns each,
//   serialized), so claims are per workgroup and per whole tile: claiming
//   quarter tiles per wave made a ReduceScatter (p = 8, 2^26 bf16 per
//   rank) 20% slower.
// - The next claim is issued before the loads of the tile in hand and read
//   after they have returned (the tile's hook), and its register is kept
//   live past the tile's stores, so the loop waits for nothing the dealt
//   loop does not.
// - Claims only grow, so the segment cursor only moves forward.
template <int DT, int OP, int P, int ORD, int DMODE, uint32_t NPOOLS>
__device__ __forceinline__ void reduce_claimed(const RankPtrs& ptrs, const ReduceGeom& g, uint64_t dealt,
                                               uint64_t per, uint32_t pool, unsigned long long* ctr,
                                               unsigned long long first) {
  using T = Traits<DT>;
  using S = typename T::S;
  constexpr bool ALL = DMODE == kDstAll;
  constexpr int ND = ALL ? P : 1;
  constexpr int U = ReduceUnroll<P, ALL>::value;
  constexpr uint64_t TV = (uint64_t)U * kBlock;  // vectors of a tile
  __shared__ uint64_t next_tile[2];
  // every wave reads its `first` (only thread 0's is a claim), so that no
  // path leaves the atomic unread
  const uint64_t first_tile_claimed = wave_value(first);
  if (threadIdx.x == 0) next_tile[0] = first_tile_claimed;
  __syncthreads();
  uint64_t u = next_tile[0];
  int par = 1;
  int c = -1;
  uint64_t cbase = 0, cnt = 0;
  SegSpan sp{};
  const S* src[P];
  S* dst[ND];
  Scales<P> sc;
  while (u < per) {
    // thread 0 claims; every wave reads its own value of `next` in the
    // hook (only thread 0's is a claim), so that no path leaves the atomic
    // unread when the register is set again in the next iteration
    const unsigned long long next = issue_claim(ctr, (int)threadIdx.x);
    const uint64_t f = dealt + pool + (uint64_t)NPOOLS * u;
    if (f >= cbase + cnt) {
      // f < total, the sum of the segments' tile counts, so a segment
      // below P holds it (the bound on c only keeps reads in range)
      uint64_t lo = 0;
      do {
        cbase += cnt;
        ++c;
        const SegGeom<DT, P, DMODE> s(g, c);
        lo = s.lo;
        sp = s.sp;
        cnt = s.nt;
      } while (f >= cbase + cnt && c < P - 1);
      chunk_operands<DT, OP, P, ORD, DMODE, ND>(ptrs, g, c, lo, src, dst, sc);
    }
    const uint64_t t = f - cbase;
    const auto publish = [&](uint32_t tok) {
      const uint64_t v = wave_value(next + tok);
      if (threadIdx.x == 0) next_tile[par] = v;
    };
    // only whole vector tiles are worked here (the partial last tile of a
    // segment is dealt out, and claims are off when a segment is on the
    // element path), so the loop body has one path with loads, whose wait
    // for them covers the claim
    if (t < sp.nvec / TV) {
      // pointers carried across iterations lose their address space:
      // restate it so the tile uses global, not flat, instructions
      const S* gs[P];
      S* gd[ND];
#pragma unroll
      for (int k = 0; k < P; ++k) gs[k] = as_global(src[k] + sp.head);
#pragma unroll
      for (int d = 0; d < ND; ++d) gd[d] = as_global(dst[d] + sp.head);
      reduce_vec_tile<DT, OP, P, ORD, ND, ALL, U, true>(gs, gd, t * TV + threadIdx.x, sp.nvec, sc, P, publish);
    } else {
      publish(0);
    }
    // keep the claim's register live past the tile's stores: reused for
    // their addresses, it would have to wait for them before the next
    // claim could be written into it
    asm volatile("" ::"v"(next));
    __syncthreads();
    u = next_tile[par];
    par ^= 1;
  }
  if (threadIdx.x == 0) claim_last(ctr, u, per, NPOOLS > 1 ? claim_pool_members(gridDim.x, pool) : gridDim.x);
}

template <int DT, int OP, int P, int ORD, int DMODE>
COLL_STREAM_KERNEL void reduce_kernel(RankPtrs ptrs, ReduceGeom g) {
  using T = Traits<DT>;
  using S = typename T::S;
  constexpr bool ALL = DMODE == kDstAll;
  constexpr int ND = ALL ? P : 1;
  // With a claim slot, about a quarter of the tiles are dealt out in turn
  // and the rest claimed (reduce_claimed); the workgroup's first claim is
  // issued now and read after its dealt tiles.  AllReduce at p = 8 claims
  // from the slot's kClaimPools pooled counters (workgroup b from pool
  // claim_pool(b), claim c of pool x being tile dealt + x + kClaimPools * c),
  // the other calls from its first counter.  Same-box A/B, pooled against
  // one counter, AllReduce of 256 MiB fp32 per rank: p = 8 713-714 against
  // 737 us; p = 2 169 against 169, p = 4 354 against 350, p = 12 1132-1136
  // against 1074, p = 16 1544-1580 against 1446-1455 us; ReduceScatter and
  // AllGather within 1% or slower with pools.
  constexpr uint32_t NPOOLS = (ALL && P == 8) ? (uint32_t)kClaimPools : 1u;
  uint64_t dealt = ~0ull, total = 0, per = 0;
  unsigned long long first = 0;
  const uint32_t pool = NPOOLS > 1 ? claim_pool(blockIdx.x) : 0u;
  // AllReduce and ReduceScatter.  Same-box A/Bs against tiles all dealt
  // out: AllReduce 5-7% faster at p = 8 (256 MiB fp32 per rank) and 6-9%
  // at p = 3, 5, 6, 7, 12; ReduceScatter 3-4% faster at p = 8 (2^26 bf16
  // per rank) and within 1% either way at the other counts.
  const bool claims = (ALL || DMODE == kDstOwner) && g.claim;
  unsigned long long* ctr = claims ? g.claim + pool * kClaimPoolWords : nullptr;  // pool 0: the first counter
  if (claims) {
    first = issue_claim(ctr, (int)threadIdx.x);
    // only whole vector tiles are claimed: with a segment on the element
    // path (buffers that disagree modulo 16) every tile is dealt out
    bool vec = true;
    for (int c = 0; c < P; ++c) {
      const SegGeom<DT, P, DMODE> s(g, c);
      total += s.nt;
      vec = vec && (s.sp.vec || s.len == 0);
    }
    per = vec ? (total - dealt_tiles(total, gridDim.x)) / NPOOLS : 0;
    dealt = total - per * NPOOLS;
  }
  uint64_t base = 0;
  for (int c = 0; c < P; ++c) {
    uint64_t lo, len;
    chunk_range(g, c, &lo, &len);
    if (len == 0) continue;
    const uint64_t doff = (DMODE == kDstOwner) ? 0 : lo;
    const int mis = seg_mis(g.src_mis, g.dst_mis, lo * T::B, doff * T::B);
    const int amis = seg_amis(g.src_amis, lo * T::B);
    const uint64_t lim = dealt > base ? dealt - base : 0;
    uint64_t nt;
    if (!segment_owned<DT, P, ND>(len, mis, amis, base, &nt, lim)) {
      base += nt;
      continue;
    }
    const S* src[P];
    S* dst[ND];
    Scales<P> sc;
    chunk_operands<DT, OP, P, ORD, DMODE, ND>(ptrs, g, c, lo, src, dst, sc);
    base += reduce_segment<DT, OP, P, ORD, ND, ALL>(src, dst, len, mis, amis, base, sc, P, lim);
  }
  if constexpr (ALL || DMODE == kDstOwner) {
    if (claims) reduce_claimed<DT, OP, P, ORD, DMODE, NPOOLS>(ptrs, g, dealt, per, pool, ctr, first);
  }
}

// AllReduce, ReduceScatter and Reduce calls whose tiles fit the grid (at
// most one tile per workgroup): workgroup b works tile b % tpc of chunk
// b / tpc, tpc tiles per chunk, and nothing else.  The general kernel gives such calls the
// same tiles but has every workgroup walk all P chunks to find its tile,
// and for small calls that walk (ownership tests, a run-time remainder
// per chunk) outlasts the data movement: at p = 16 a 4 KiB call took
// 8.7 us against 4.3 us, a 64 KiB call 9.3 us against 4.6 us.
template <int DT, int OP, int P, int ORD, int DMODE>
COLL_STREAM_KERNEL void reduce_tile_kernel(RankPtrs ptrs, ReduceGeom g, uint32_t tpc) {
  using T = Traits<DT>;
  using S = typename T::S;
  constexpr bool ALL = DMODE == kDstAll;
  constexpr int ND = ALL ? P : 1;
  constexpr int U = ReduceUnroll<P, ALL>::value;
  constexpr uint64_t TV = (uint64_t)U * kBlock;
  const int c = (int)(blockIdx.x / tpc);
  const uint64_t t = blockIdx.x - (uint64_t)c * tpc;
  uint64_t lo, len;
  chunk_range(g, c, &lo, &len);
  if (len == 0) return;
  const uint64_t doff = (DMODE == kDstOwner) ? 0 : lo;
  const int mis = seg_mis(g.src_mis, g.dst_mis, lo * T::B, doff * T::B);
  const S* src[P];
  S* dst[ND];
  Scales<P> sc;
  chunk_operands<DT, OP, P, ORD, DMODE, ND>(ptrs, g, c, lo, src, dst, sc);
  const SegSpan sp = seg_span_a<T::B>(len, mis, seg_amis(g.src_amis, lo * T::B));
  if (!sp.vec) {
    // element path: tile t covers TV * V elements of the chunk
    const uint64_t from = t * TV * T::V;
    if (from < len)
      reduce_elems<DT, OP, P, ORD, ND, ALL>(src, dst, from, (len - from) < TV * T::V ? (len - from) : TV * T::V,
                                            sc, P);
    return;
  }
  if (t * TV < sp.nvec) {
    const S* vs[P];
    S* vd[ND];
#pragma unroll
    for (int k = 0; k < P; ++k) vs[k] = src[k] + sp.head;
#pragma unroll
    for (int d = 0; d < ND; ++d) vd[d] = dst[d] + sp.head;
    reduce_vec_tile<DT, OP, P, ORD, ND, ALL, U, false>(vs, vd, t * TV + threadIdx.x, sp.nvec, sc, P);
  }
  if (t == 0 && (sp.head || sp.tail))
    reduce_edges<DT, OP, P, ORD, ND, ALL>(src, dst, sp.head, sp.head + sp.nvec * T::V, sp.tail, sc, P,
                                          (int)threadIdx.x);
}

// Any rank count (the slow general path): one vector per lane per tile,
// operands in groups of 8 loads, pointers read from the kernel arguments.
// TILE: at most one tile per workgroup (AllReduce only): workgroup b works
// tile b % tpc of chunk b / tpc instead of walking every chunk, as
// reduce_tile_kernel does for the specialised rank counts.
template <int DT, int OP, int DMODE, bool TILE = false>
COLL_STREAM_KERNEL void reduce_kernel_any(RankPtrs ptrs, ReduceGeom g, uint32_t tpc = 0) {
#pragma clang fp contract(off)
  using T = Traits<DT>;
  using S = typename T::S;
  using A = typename T::A;
  constexpr int V = T::V;
  constexpr bool ALL = DMODE == kDstAll;
  const int p = g.p;
  const uint64_t grid = gridDim.x, wg = blockIdx.x;
  const int c_first = TILE ? (int)(blockIdx.x / tpc) : 0;
  const int c_end = TILE ? c_first + 1 : p;
  const uint64_t my_tile = TILE ? blockIdx.x - (uint64_t)c_first * tpc : 0;
  // first tile and stride of this workgroup in a segment of nt tiles
  auto tile0 = [&](uint64_t base) -> uint64_t { return TILE ? my_tile : first_tile(base, wg, grid); };
  auto tstep = [&](uint64_t nt) -> uint64_t { return TILE ? nt : grid; };
  uint64_t base = 0;
  for (int c = c_first; c < c_end; ++c) {
    uint64_t lo, len;
    chunk_range(g, c, &lo, &len);
    if (len == 0) continue;
    const uint64_t doff = (DMODE == kDstOwner) ? 0 : lo;
    auto sp_src = [&](int k) -> const S* { return (const S*)ptrs.src[(c + 1 + k) % p] + lo; };
    auto sp_dst = [&](int k) -> S* {
      if constexpr (ALL) return (S*)ptrs.dst[k] + lo;
      else if constexpr (DMODE == kDstOwner) return (S*)ptrs.dst[c];
      else return (S*)ptrs.dst[0] + lo;
    };
    const int nd = ALL ? p : 1;
    const SegSpan sp = seg_span<T::B>(len, seg_mis(g.src_mis, g.dst_mis, lo * T::B, doff * T::B));
    auto scale_of = [&](int k) -> float { return g.scale[(c + 1 + k) % p]; };
    auto elem_at = [&](uint64_t e) {
#pragma clang fp contract(off)
      A acc = widen1<DT>(ld1<true>(sp_src(0) + e));
      if constexpr (OP == kPreMul) acc = scale_of(0) * acc;
      for (int k = 1; k < p; ++k) {
        A v = widen1<DT>(ld1<true>(sp_src(k) + e));
        if constexpr (OP == kPreMul) v = scale_of(k) * v;
        acc = combine<OP>(acc, v);
      }
      const auto out = narrow1<DT>(finish<OP>(acc, p));
      for (int d = 0; d < nd; ++d) st1<ALL>(sp_dst(d) + e, out);
    };
    auto elems = [&](uint64_t from, uint64_t cnt) {
      for (uint64_t i = threadIdx.x; i < cnt; i += kBlock) elem_at(from + i);
    };
    if (!sp.vec) {
      constexpr uint64_t TE = (uint64_t)kBlock * 4;
      const uint64_t nt = ceil_div(len, TE);
      for (uint64_t t = tile0(base); t < nt; t += tstep(nt)) {
        const uint64_t from = t * TE;
        elems(from, (len - from) < TE ? (len - from) : TE);
      }
      base += nt;
      continue;
    }
    const uint64_t nt = ceil_div(sp.nvec, (uint64_t)kBlock);
    for (uint64_t t = tile0(base); t < nt; t += tstep(nt)) {
      const uint64_t j = t * kBlock + threadIdx.x;
      if (j >= sp.nvec) continue;
      const uint64_t e = sp.head + j * V;
      A acc[V];
      widen<DT>(ld16<true>(sp_src(0) + e), acc);
      if constexpr (OP == kPreMul) {
#pragma unroll
        for (int x = 0; x < V; ++x) acc[x] = scale_of(0) * acc[x];
      }
      for (int k0 = 1; k0 < p; k0 += 8) {
        u32x4 r[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (k0 + q < p) r[q] = ld16<true>(sp_src(k0 + q) + e);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (k0 + q < p) {
            A t2[V];
            widen<DT>(r[q], t2);
            if constexpr (OP == kPreMul) {
#pragma unroll
              for (int x = 0; x < V; ++x) t2[x] = scale_of(k0 + q) * t2[x];
            }
            combine_vec<OP, DT>(acc, t2);
          }
      }
#pragma unroll
      for (int x = 0; x < V; ++x) acc[x] = finish<OP>(acc[x], p);
      const u32x4 out = narrow<DT>(acc);
      for (int d = 0; d < nd; ++d) st16<ALL>(sp_dst(d) + e, out);
    }
    if ((sp.head || sp.tail) && tile0(base) == 0) {
      // head and tail in one pass (each is shorter than a vector)
      const uint64_t i = threadIdx.x;
      if (i < sp.head + sp.tail) elem_at(i < sp.head ? i : sp.head + sp.nvec * V + (i - sp.head));
    }
    base += nt;
  }
}

// ---------------------------------------------------------------------------
// Host-side launch
// ---------------------------------------------------------------------------
template <int DT, int P, bool ALL>
static uint64_t tile_elems() {
  return (uint64_t)ReduceUnroll<P, ALL>::value * kBlock * Traits<DT>::V;
}

// Upper bound on the tiles of all segments (vector tiles plus one for a
// misaligned head), used only to size the grid.
template <int DT, int P, bool ALL>
static uint64_t count_tiles(const ReduceGeom& g) {
  const uint64_t te = P ? tile_elems<DT, P, ALL>() : (uint64_t)kBlock * Traits<DT>::V;
  uint64_t total = 0;
  for (int c = 0; c < g.p; ++c) {
    uint64_t lo = (uint64_t)c * g.stride, hi = lo + g.stride;
    if (lo > g.total) lo = g.total;
    if (hi > g.total) hi = g.total;
    if (hi > lo) total += (hi - lo + te - 1) / te + 1;
  }
  return total;
}

static int clamp_grid(uint64_t tiles, int max_grid) {
  if (tiles == 0) return 0;
  return (int)(tiles < (uint64_t)max_grid ? tiles : (uint64_t)max_grid);
}

template <int DT, int OP, int P, int ORD>
static int launch_p(const RankPtrs& ptrs, const ReduceGeom& g, int max_grid, hipStream_t s) {
  if (g.dst_mode == kDstAll) {
    // at most one tile per workgroup: each workgroup goes straight to its
    // tile (for the default grid of one workgroup per CU on 256 CUs: up to
    // 1 MiB per rank at p = 16, 2 MiB at 8, 4 MiB at 4)
    const uint64_t te = tile_elems<DT, P, true>();
    const uint64_t tpc = (g.stride + te - 1) / te;
    if (tpc * P <= (uint64_t)max_grid) {
      if (tpc)
        hipLaunchKernelGGL((reduce_tile_kernel<DT, OP, P, ORD, kDstAll>), dim3((unsigned)(tpc * P)), dim3(kBlock),
                           0, s, ptrs, g, (uint32_t)tpc);
      return (int)hipGetLastError();
    }
  }
  if constexpr (ORD == kOrdRing) {
    // ReduceScatter and Reduce (ring order only) likewise
    if (g.dst_mode == kDstOwner || g.dst_mode == kDstFixed) {
      const uint64_t te = tile_elems<DT, P, false>();
      const uint64_t tpc = (g.stride + te - 1) / te;
      if (tpc * P <= (uint64_t)max_grid) {
        if (tpc && g.dst_mode == kDstOwner)
          hipLaunchKernelGGL((reduce_tile_kernel<DT, OP, P, ORD, kDstOwner>), dim3((unsigned)(tpc * P)),
                             dim3(kBlock), 0, s, ptrs, g, (uint32_t)tpc);
        else if (tpc)
          hipLaunchKernelGGL((reduce_tile_kernel<DT, OP, P, ORD, kDstFixed>), dim3((unsigned)(tpc * P)),
                             dim3(kBlock), 0, s, ptrs, g, (uint32_t)tpc);
        return (int)hipGetLastError();
      }
    }
  }
  // claimed tails only for calls with many tiles per workgroup, where the
  // spread between XCDs outweighs the claims
  if (g.dst_mode == kDstAll) {
    const uint64_t tiles = count_tiles<DT, P, true>(g);
    const int grid = clamp_grid(tiles, max_grid);
    ReduceGeom gk = g;
    if (tiles < kClaimMinTilesPerWg * (uint64_t)grid || grid < kClaimPools * kClaimPools) gk.claim = nullptr;
    if (grid)
      hipLaunchKernelGGL((reduce_kernel<DT, OP, P, ORD, kDstAll>), dim3(grid), dim3(kBlock), 0, s, ptrs, gk);
    return (int)hipGetLastError();
  }
  if constexpr (ORD != kOrdRing) {
    // the schedules other than the ring exist for AllReduce only
    return (int)hipErrorInvalidValue;
  } else {
    const int grid = clamp_grid(count_tiles<DT, P, false>(g), max_grid);
    if (!grid) return 0;
    ReduceGeom gk = g;
    if (g.dst_mode != kDstOwner || count_tiles<DT, P, false>(g) < kClaimMinTilesPerWg * (uint64_t)grid ||
        grid < kClaimPools * kClaimPools)
      gk.claim = nullptr;  // claimed tails are for AllReduce and ReduceScatter
    if (g.dst_mode == kDstOwner)
      hipLaunchKernelGGL((reduce_kernel<DT, OP, P, ORD, kDstOwner>), dim3(grid), dim3(kBlock), 0, s, ptrs, gk);
    else
      hipLaunchKernelGGL((reduce_kernel<DT, OP, P, ORD, kDstFixed>), dim3(grid), dim3(kBlock), 0, s, ptrs, gk);
    return (int)hipGetLastError();
  }
}

template <int DT, int OP>
static int launch_any(const RankPtrs& ptrs, const ReduceGeom& g, int max_grid, hipStream_t s) {
  if (g.dst_mode == kDstAll) {
    // at most one tile per workgroup: no chunk walk.  Tiles of kBlock * 4
    // elements (the element path's) also bound the vector path's tiles of
    // kBlock vectors.
    const uint64_t te = (uint64_t)kBlock * 4;
    const uint64_t tpc = (g.stride + te - 1) / te;
    if (tpc * (uint64_t)g.p <= (uint64_t)max_grid) {
      if (tpc)
        hipLaunchKernelGGL((reduce_kernel_any<DT, OP, kDstAll, true>), dim3((unsigned)(tpc * g.p)), dim3(kBlock),
                           0, s, ptrs, g, (uint32_t)tpc);
      return (int)hipGetLastError();
    }
  }
  const int grid = clamp_grid(count_tiles<DT, 0, false>(g), max_grid);
  if (!grid) return 0;
  if (g.dst_mode == kDstAll)
    hipLaunchKernelGGL((reduce_kernel_any<DT, OP, kDstAll>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
  else if (g.dst_mode == kDstOwner)
    hipLaunchKernelGGL((reduce_kernel_any<DT, OP, kDstOwner>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
  else
    hipLaunchKernelGGL((reduce_kernel_any<DT, OP, kDstFixed>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
  return (int)hipGetLastError();
}

// Ring order at compile-time rank count P, for every dtype and op.
template <int P>
static int launch_ring_fixed(int dtype, int op, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                             hipStream_t s) {
#define COLL_RING_CASE(DTV, OPV) \
  if (dtype == DTV && op == OPV) return launch_p<DTV, OPV, P, kOrdRing>(ptrs, g, max_grid, s);
  COLL_RING_CASE(kF32, kSum) COLL_RING_CASE(kF32, kMin) COLL_RING_CASE(kF32, kMax) COLL_RING_CASE(kF32, kAvg)
  COLL_RING_CASE(kF32, kPreMul)
  COLL_RING_CASE(kBF16, kSum) COLL_RING_CASE(kBF16, kMin) COLL_RING_CASE(kBF16, kMax) COLL_RING_CASE(kBF16, kAvg)
  COLL_RING_CASE(kBF16, kPreMul)
  COLL_RING_CASE(kI32, kSum) COLL_RING_CASE(kI32, kMin) COLL_RING_CASE(kI32, kMax) COLL_RING_CASE(kI32, kAvg)
#undef COLL_RING_CASE
  return (int)hipErrorInvalidValue;
}

// The binary tree and the double binary tree at compile-time rank count P.
// Both are defined for any rank count (heap order over P ranks; the second
// tree of the double binary tree mirrors the first), and only change the
// bits of floating-point sums: the caller sends integer sums and min/max
// to the ring-order kernels.
template <int P>
static int launch_tree_fixed(int dtype, int op, int order, const RankPtrs& ptrs, const ReduceGeom& g,
                             int max_grid, hipStream_t s) {
#define COLL_TREE_CASE(DTV, OPV)                                                        \
  if (dtype == DTV && op == OPV) {                                                      \
    if (order == kOrdTree) return launch_p<DTV, OPV, P, kOrdTree>(ptrs, g, max_grid, s); \
    if (order == kOrdDBT) return launch_p<DTV, OPV, P, kOrdDBT>(ptrs, g, max_grid, s);   \
  }
  COLL_TREE_CASE(kF32, kSum) COLL_TREE_CASE(kF32, kAvg) COLL_TREE_CASE(kF32, kPreMul)
  COLL_TREE_CASE(kBF16, kSum) COLL_TREE_CASE(kBF16, kAvg) COLL_TREE_CASE(kBF16, kPreMul)
#undef COLL_TREE_CASE
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
