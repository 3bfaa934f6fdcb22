// Data re-placement without arithmetic: AllGather, Broadcast, All-to-All,
// variable-split All-to-All, Gather and Scatter.
//
// All six are block copies between rank buffers; they differ only in how
// a segment (source range -> destination range(s)) is derived:
//   AllGather  segment s: send[s] -> recv[r] + s*n for every r, rank-order
//              concatenation ("集合通信：原语、算法、NCCL 实现与拓扑映射",
//              section 1.2);
//   Broadcast  one segment: send_root -> recv[r] for every r (section 1.1);
//   AllToAll   segment (i,j): send[i] + j*n -> recv[j] + i*n, the block
//              transpose of section 1.6;
//   Gather     segment s: send[s] -> recv_root + s*n;
//   Scatter    segment r: send_root + r*n -> recv[r];
//   Alltoallv  segment (i,j) of counts[i][j] elements, offsets from the
//              prefix sums of the count matrix ("Collective Communication：
//              AllReduce、AllGather、ReduceScatter 与 All-to-All", ragged
//              All-to-All).
// Fan-out copies (one source, p destinations) load through the cache and
// store non-temporally; 1:1 copies are non-temporal both ways.
#include "copy_tile.h"

namespace coll {

// Destination misalignment of fan-out segment s.
template <int B, int KIND>
__device__ __forceinline__ int fanout_mis(const CopyGeom& g, int s) {
  const uint64_t dst_off = KIND == kCopyAllGather ? (uint64_t)s * g.n : 0;
  return g.dst_mis < 0 ? -1 : (int)((g.dst_mis + dst_off * B) & 15);
}
// ... and their common address modulo kLineAlign (-1: unknown).
template <int B, int KIND>
__device__ __forceinline__ int fanout_amis(const CopyGeom& g, int s) {
  const uint64_t dst_off = KIND == kCopyAllGather ? (uint64_t)s * g.n : 0;
  return seg_amis(g.dst_amis, dst_off * B);
}

// The claimed tiles of fanout_kernel (tiles of FU vectors per lane), one
// workgroup tile per claim from the workgroup's pool (claim c of pool x is
// tile dealt + x + kClaimPools * c), as reduce_claimed does for the
// reductions (thread 0 claims before the tile's loads and publishes after
// them through LDS; only whole vector tiles are claimed).
template <int B, int KIND, int P, int FU>
__device__ __forceinline__ void fanout_claimed(const RankPtrs& ptrs, const CopyGeom& g, uint64_t dealt,
                                               uint64_t per, uint32_t pool, unsigned long long* ctr,
                                               unsigned long long first) {
  using W = typename Word<B>::T;
  constexpr int NSEG = KIND == kCopyAllGather ? P : 1;
  __shared__ uint64_t next_tile[2];
  const uint64_t first_claim = wave_value(first);
  if (threadIdx.x == 0) next_tile[0] = first_claim;
  __syncthreads();
  constexpr uint64_t TVF = (uint64_t)FU * kBlock;  // vectors of a tile
  uint64_t u = next_tile[0];
  int par = 1;
  int s = -1;
  uint64_t sbase = 0, cnt = 0;
  SegSpan sp{};
  const W* src = nullptr;
  W* dst[P];
  while (u < per) {
    const unsigned long long next = issue_claim(ctr, (int)threadIdx.x);
    const uint64_t f = dealt + pool + (uint64_t)kClaimPools * u;
    if (f >= sbase + cnt) {
      do {
        sbase += cnt;
        ++s;
        sp = seg_span_a<B>(g.n, fanout_mis<B, KIND>(g, s), fanout_amis<B, KIND>(g, s));
        cnt = copy_segment_tiles<B, FU>(sp, g.n);
      } while (f >= sbase + cnt && s < NSEG - 1);  // the bound only keeps reads in range
      const uint64_t dst_off = KIND == kCopyAllGather ? (uint64_t)s * g.n : 0;
      src = (const W*)ptrs.src[KIND == kCopyAllGather ? s : 0] + sp.head;
#pragma unroll
      for (int k = 0; k < P; ++k) dst[k] = (W*)ptrs.dst[k] + dst_off + sp.head;
    }
    const uint64_t t = f - sbase;
    const auto publish = [&](uint32_t tok) {
      const uint64_t v = wave_value(next + tok);
      if (threadIdx.x == 0) next_tile[par] = v;
    };
    if (t < sp.nvec / TVF) {
      // pointers carried across iterations lose their address space:
      // restate it so the tile uses global, not flat, instructions
      const u32x4* vs = reinterpret_cast<const u32x4*>(as_global(src));
      u32x4* vd[P];
#pragma unroll
      for (int k = 0; k < P; ++k) vd[k] = reinterpret_cast<u32x4*>(as_global(dst[k]));
      auto gdst = [&](int d) -> u32x4* { return vd[d]; };
      copy_vec_tile<P == 1, true, P, FU>(vs, gdst, P, t * TVF + threadIdx.x, sp.nvec, publish);
    } else {
      publish(0);
    }
    asm volatile("" ::"v"(next));  // keep the claim's register out of the stores' reach
    __syncthreads();
    u = next_tile[par];
    par ^= 1;
  }
  if (threadIdx.x == 0) claim_last(ctr, u, per, claim_pool_members(gridDim.x, pool));
}

// Fan-outs claim tiles at compile-time rank counts of 8 and 16 only, where
// a tile moves (1 + p) * 8 KiB >= 72 KiB (tiles of kFanoutUnroll vectors
// per lane), from the pooled counters.  At p = 1 (a 32 KiB tile) claiming
// every tile from one counter (about 83 claims per microsecond, 12 ns
// each) capped a 1 GiB copy at about 3 TB/s.
template <int P>
constexpr bool kFanoutClaims = P >= 8;
// Vectors per lane of a claiming fan-out's tile, with claims from the
// pooled counters.  AllGather p = 8, 16 MiB bf16 shards, same-box A/B:
// 4 per lane and one counter 171-172 us; with pools, 4 per lane 174-175,
// 2 per lane 163-164, 1 per lane 177-185 us.  (The other copies keep 4:
// at 2, All-to-All took 153 against 146 us and Alltoallv 183-186 against
// 155-156 us.)
constexpr int kFanoutUnroll = 2;

// AllGather / Broadcast with a compile-time rank count P (0: any).
// Destination pointers of a segment are read once into registers.  With
// one rank the fan-out is a 1:1 copy and loads non-temporally too.  With a
// claim slot (P of 8 or 16, sources and destinations agreeing modulo 16),
// a quarter of the tiles are dealt out in turn and the rest claimed
// (fanout_claimed): its workgroups otherwise finish far apart (an
// AllGather at p = 8 with 16 MiB shards: from 80 to 193 us, median 140).
template <int B, int KIND, int P, bool SHIFT>
COLL_STREAM_KERNEL void fanout_kernel(RankPtrs ptrs, CopyGeom g) {
  using W = typename Word<B>::T;
  constexpr bool CLAIMS = kFanoutClaims<P> && !SHIFT;
  const int p = P ? P : g.p;
  const int nseg = KIND == kCopyAllGather ? p : 1;
  constexpr int FU = CLAIMS ? kFanoutUnroll : kCopyU;  // vectors per lane of a tile
  uint64_t dealt = ~0ull, total = 0, per = 0;
  unsigned long long first = 0;
  const bool claims = CLAIMS && g.claim;
  const uint32_t pool = claim_pool(blockIdx.x);
  unsigned long long* ctr = claims ? g.claim + pool * kClaimPoolWords : nullptr;
  if (claims) {
    first = issue_claim(ctr, (int)threadIdx.x);
    bool vec = true;
    for (int s = 0; s < nseg; ++s) {
      const SegSpan sp = seg_span_a<B>(g.n, fanout_mis<B, KIND>(g, s), fanout_amis<B, KIND>(g, s));
      total += copy_segment_tiles<B, FU>(sp, g.n);
      vec = vec && (sp.vec || g.n == 0);
    }
    per = vec ? (total - total / 8 * kCopyDealtEighths / gridDim.x * gridDim.x) / kClaimPools : 0;
    dealt = total - per * kClaimPools;
  }
  uint64_t base = 0;
  for (int s = 0; s < nseg; ++s) {
    const uint64_t dst_off = KIND == kCopyAllGather ? (uint64_t)s * g.n : 0;
    const int mis = fanout_mis<B, KIND>(g, s), amis = fanout_amis<B, KIND>(g, s);
    const uint64_t lim = dealt > base ? dealt - base : 0;
    uint64_t nt;
    if (!copy_segment_owned<B, FU>(g.n, mis, amis, base, &nt, lim)) {
      base += nt;
      continue;
    }
    const W* src = (const W*)ptrs.src[s];
    if constexpr (P > 0) {
      W* dst[P];
#pragma unroll
      for (int k = 0; k < P; ++k) dst[k] = (W*)ptrs.dst[k] + dst_off;
      auto gdst = [&](int d) -> W* { return dst[d]; };
      base += copy_segment<B, P == 1, P, SHIFT, FU>(src, gdst, P, g.n, mis, amis, base, lim);
    } else {
      auto gdst = [&](int d) -> W* { return (W*)ptrs.dst[d] + dst_off; };
      base += copy_segment<B, false, 0, SHIFT>(src, gdst, p, g.n, mis, amis, base);
    }
  }
  if constexpr (CLAIMS) {
    if (claims) fanout_claimed<B, KIND, P, FU>(ptrs, g, dealt, per, pool, ctr, first);
  }
}

// 1:1 block copies, one destination per segment:
//   All-to-All  p*p segments (i, j): send[i] + j*n -> recv[j] + i*n;
//   Gather      p segments s: send[s] -> recv_root + s*n (AllGather with one
//               receiver, "详解分布式训练8大集合通信原语" section 4.3);
//   Scatter     p segments r: send_root + r*n -> recv[r] (section 3.3).
// The in-place forms copy the root's own block onto itself.
template <int B, int KIND, bool SHIFT>
COLL_STREAM_KERNEL void pair_copy_kernel(RankPtrs ptrs, CopyGeom g) {
  using W = typename Word<B>::T;
  const int p = g.p;
  const int nseg = KIND == kCopyAllToAll ? p * p : p;
  uint64_t base = 0;
  for (int sgi = 0; sgi < nseg; ++sgi) {
    uint64_t src_off = 0, dst_off = 0;
    const W* src;
    W* dst;
    if constexpr (KIND == kCopyAllToAll) {
      const int i = sgi / p, j = sgi - (sgi / p) * p;
      src_off = (uint64_t)j * g.n;
      dst_off = (uint64_t)i * g.n;
      src = (const W*)ptrs.src[i] + src_off;
      dst = (W*)ptrs.dst[j] + dst_off;
    } else if constexpr (KIND == kCopyGather) {
      dst_off = (uint64_t)sgi * g.n;
      src = (const W*)ptrs.src[sgi];
      dst = (W*)ptrs.dst[0] + dst_off;
    } else {
      src_off = (uint64_t)sgi * g.n;
      src = (const W*)ptrs.src[0] + src_off;
      dst = (W*)ptrs.dst[sgi];
    }
    (void)src_off;
    const int mis = (int)((uintptr_t)dst & 15), amis = (int)((uintptr_t)dst & (kLineAlign - 1));
    uint64_t nt;
    if (!copy_segment_owned<B>(g.n, mis, amis, base, &nt)) {
      base += nt;
      continue;
    }
    auto gdst = [&](int) -> W* { return dst; };
    base += copy_segment<B, true, 1, SHIFT>(src, gdst, 1, g.n, mis, amis, base);
  }
}

// AllGather calls with at most one tile per workgroup likewise, when
// every segment shares one 16-byte misalignment (common source and
// destination misalignment, n * B a multiple of 16): flat tile f is tile
// f mod tps of segment f / tps (rank s's block, stored to every
// destination at s * n), instead of a walk over the p segments (p = 16,
// 4 KiB per rank: 6.4 -> 3.5 us).  Loads through the cache, non-temporal
// stores, as the walking kernel.
template <int B, int P>
COLL_STREAM_KERNEL void allgather_flat_kernel(RankPtrs ptrs, CopyGeom g, uint64_t head, uint64_t nvec, uint64_t tail,
                                              uint32_t tps) {
  using W = typename Word<B>::T;
  constexpr uint64_t V = 16 / B;
  const uint32_t total = (uint32_t)P * tps;
  for (uint32_t f = blockIdx.x; f < total; f += gridDim.x) {
    const uint32_t sgi = f / tps, t = f - sgi * tps;
    const W* src = (const W*)ptrs.src[sgi];
    W* dst[P];
#pragma unroll
    for (int k = 0; k < P; ++k) dst[k] = (W*)ptrs.dst[k] + (uint64_t)sgi * g.n;
    const u32x4* vs = reinterpret_cast<const u32x4*>(src + head);
    auto gdst = [&](int d) -> u32x4* { return reinterpret_cast<u32x4*>(dst[d] + head); };
    const uint64_t j0 = (uint64_t)t * kCopyTV + threadIdx.x;
    if ((uint64_t)(t + 1) * kCopyTV <= nvec) copy_vec_tile<false, true, P>(vs, gdst, P, j0, nvec);
    else if ((uint64_t)t * kCopyTV < nvec) copy_vec_tile<false, false, P>(vs, gdst, P, j0, nvec);
    if (t == 0 && (head || tail)) {
      const uint64_t i = threadIdx.x;
      if (i < head + tail) {
        const uint64_t x = i < head ? i : head + nvec * V + (i - head);
        const W w = ld1<false>(src + x);
#pragma unroll
        for (int k = 0; k < P; ++k) st1<true>(dst[k] + x, w);
      }
    }
  }
}

// The same 1:1 block copies when every segment shares one 16-byte
// misalignment (common source and destination misalignment, n * B a
// multiple of 16), so every segment has the same head, vector count and
// tail and the same number of tiles, tps.  A workgroup then computes the
// segment and tile of its flat tile f (f / tps, f mod tps) instead of
// walking every segment to find its tiles, and sets up a segment's
// pointers only when the segment changes.  The walk costs every
// workgroup p^2 ownership tests for All-to-All: a 4 KiB-per-rank call took
// 15.7 us at p = 8 and 88 us at p = 16.
template <int B, int KIND>
__device__ __forceinline__ void pair_segment(const RankPtrs& ptrs, const CopyGeom& g, uint32_t sgi,
                                             const typename Word<B>::T** src, typename Word<B>::T** dst) {
  using W = typename Word<B>::T;
  if constexpr (KIND == kCopyAllToAll) {
    const uint32_t i = sgi / (uint32_t)g.p, j = sgi - i * (uint32_t)g.p;
    *src = (const W*)ptrs.src[i] + (uint64_t)j * g.n;
    *dst = (W*)ptrs.dst[j] + (uint64_t)i * g.n;
  } else if constexpr (KIND == kCopyGather) {
    *src = (const W*)ptrs.src[sgi];
    *dst = (W*)ptrs.dst[0] + (uint64_t)sgi * g.n;
  } else {
    *src = (const W*)ptrs.src[0] + (uint64_t)sgi * g.n;
    *dst = (W*)ptrs.dst[sgi];
  }
}

// The uniform 1:1 copies deal out kPairDealtEighths of their flat tiles in
// turn and claim the rest one tile at a time.  Dealt out alone, the
// workgroups of an All-to-All (p = 8, 56 MiB per rank, 512 workgroups)
// finished between 140 and 153 us and those of a Gather or Scatter (p = 8,
// 16 MiB blocks) between 35 and 43 us.  One counter serves about 83 claims
// per microsecond, fewer than these copies make (a tile moves 32 KiB), so
// the claimed tiles are split into kClaimPools pools: workgroup b claims
// from the counter of pool claim_pool(b), and claim c of pool x is flat tile
// dealt + x + kClaimPools * c, so the pools advance through the same
// region together.  (Claiming runs of 8 consecutive tiles from one counter
// had been 10% slower for All-to-All and 27% for Gather and Scatter.)
template <int B, int KIND>
COLL_STREAM_KERNEL void pair_copy_flat_kernel(RankPtrs ptrs, CopyGeom g, uint64_t head, uint64_t nvec,
                                              uint64_t tail, uint32_t tps) {
  using W = typename Word<B>::T;
  constexpr uint64_t V = 16 / B;
  const uint32_t nseg = KIND == kCopyAllToAll ? (uint32_t)g.p * (uint32_t)g.p : (uint32_t)g.p;
  const uint32_t total = nseg * tps;
  // claims: per tiles from each pool, the first `dealt` tiles dealt out
  const uint32_t per = g.claim ? total / 8 * (8 - kPairDealtEighths) / kClaimPools : 0;
  const uint32_t dealt = total - per * kClaimPools;
  const uint32_t pool = claim_pool(blockIdx.x);
  unsigned long long* ctr = g.claim ? g.claim + pool * kClaimPoolWords : nullptr;
  unsigned long long first = 0;
  if (per) first = issue_claim(ctr, (int)threadIdx.x);
  uint32_t cur = 0xffffffffu;
  const W* src = nullptr;
  W* dst = nullptr;
  for (uint32_t f = blockIdx.x; f < dealt; f += gridDim.x) {
    const uint32_t sgi = f / tps, t = f - sgi * tps;
    if (sgi != cur) {
      cur = sgi;
      pair_segment<B, KIND>(ptrs, g, sgi, &src, &dst);
    }
    const u32x4* vs = reinterpret_cast<const u32x4*>(src + head);
    u32x4* vd = reinterpret_cast<u32x4*>(dst + head);
    auto gdst = [&](int) -> u32x4* { return vd; };
    const uint64_t j0 = (uint64_t)t * kCopyTV + threadIdx.x;
    if ((uint64_t)(t + 1) * kCopyTV <= nvec) copy_vec_tile<true, true, 1>(vs, gdst, 1, j0, nvec);
    else if ((uint64_t)t * kCopyTV < nvec) copy_vec_tile<true, false, 1>(vs, gdst, 1, j0, nvec);
    if (t == 0 && (head || tail)) {
      // head and tail in one pass (each is shorter than a vector)
      const uint64_t i = threadIdx.x;
      if (i < head + tail) {
        const uint64_t x = i < head ? i : head + nvec * V + (i - head);
        st1<true>(dst + x, ld1<true>(src + x));
      }
    }
  }
  if (!per) return;
  // claimed tiles: thread 0 claims the next tile before the current tile's
  // loads and publishes it through LDS once they have returned
  __shared__ uint64_t next_tile[2];
  const uint64_t first_claim = wave_value(first);
  if (threadIdx.x == 0) next_tile[0] = first_claim;
  __syncthreads();
  uint64_t c = next_tile[0];
  int par = 1;
  while (c < per) {
    const unsigned long long next = issue_claim(ctr, (int)threadIdx.x);
    const uint32_t f = dealt + pool + kClaimPools * (uint32_t)c;
    const uint32_t sgi = f / tps, t = f - sgi * tps;
    if (sgi != cur) {
      cur = sgi;
      pair_segment<B, KIND>(ptrs, g, sgi, &src, &dst);
    }
    const auto publish = [&](uint32_t tok) {
      const uint64_t v = wave_value(next + tok);
      if (threadIdx.x == 0) next_tile[par] = v;
    };
    // pointers carried across iterations lose their address space:
    // restate it so the tile uses global, not flat, instructions
    const W* gs = as_global(src);
    W* gd = as_global(dst);
    const u32x4* vs = reinterpret_cast<const u32x4*>(gs + head);
    u32x4* vd = reinterpret_cast<u32x4*>(gd + head);
    auto gdst = [&](int) -> u32x4* { return vd; };
    const uint64_t j0 = (uint64_t)t * kCopyTV + threadIdx.x;
    if ((uint64_t)(t + 1) * kCopyTV <= nvec) copy_vec_tile<true, true, 1>(vs, gdst, 1, j0, nvec, publish);
    else if ((uint64_t)t * kCopyTV < nvec) copy_vec_tile<true, false, 1>(vs, gdst, 1, j0, nvec, publish);
    else publish(0);
    if (t == 0 && (head || tail)) {
      const uint64_t i = threadIdx.x;
      if (i < head + tail) {
        const uint64_t x = i < head ? i : head + nvec * V + (i - head);
        st1<true>(gd + x, ld1<true>(gs + x));
      }
    }
    asm volatile("" ::"v"(next));  // keep the claim's register out of the stores' reach
    __syncthreads();
    c = next_tile[par];
    par ^= 1;
  }
  if (threadIdx.x == 0) claim_last(ctr, c, per, claim_pool_members(gridDim.x, pool));
}

// ---------------------------------------------------------------------------
// Alltoallv.  Every workgroup stages the p x p count matrix in LDS, checks
// it against the buffer capacities, and derives the send offsets (row
// exclusive prefix sums) and receive offsets (column exclusive prefix sums
// in source order).  Invalid counts make every workgroup return before any
// payload is written.  Then the segments (i, j) are copied: by flat tile
// index for p <= 16, else walked like the equal split.
// ---------------------------------------------------------------------------
// Stages the p x p count matrix in LDS (cnt), with the send offsets (soff,
// row exclusive prefix sums) and receive offsets (roff, column exclusive
// prefix sums in source order), and checks it against the capacities.
// Returns true when the call is rejected (every workgroup then returns
// before any payload is written); workgroup 0 reports the status.
__device__ __forceinline__ bool stage_a2av_counts(const A2avArgs& a, int64_t* lds, int* bad) {
  const int p = a.p;
  const int pp = p * p;
  int64_t* cnt = lds;
  int64_t* soff = lds + pp;
  int64_t* roff = lds + 2 * pp;
  const int tid = threadIdx.x;
  if (tid == 0) *bad = 0;
  for (int i = tid; i < pp; i += kBlock) {
    const int src = i / p, dst = i - (i / p) * p;
    cnt[i] = a.transposed ? a.counts[dst * p + src] : a.counts[i];
  }
  __syncthreads();
  if (tid < p) {
    const int i = tid;
    int64_t s = 0;
    bool ok = true;
    for (int j = 0; j < p; ++j) {
      const int64_t c = cnt[i * p + j];
      if (c < 0 || c > a.send_cap[i]) ok = false;
      soff[i * p + j] = s;
      s += (c < 0 ? 0 : c);
    }
    if (s > a.send_cap[i]) ok = false;
    if (!ok) *bad = 1;
  } else if (tid >= 64 && tid < 64 + p) {
    const int j = tid - 64;
    int64_t s = 0;
    bool ok = true;
    for (int i = 0; i < p; ++i) {
      const int64_t c = cnt[i * p + j];
      if (c < 0 || c > a.recv_cap[j]) ok = false;
      roff[i * p + j] = s;
      s += (c < 0 ? 0 : c);
    }
    if (s > a.recv_cap[j]) ok = false;
    if (!ok) *bad = 1;
  }
  __syncthreads();
  const bool reject = *bad != 0;
  if (blockIdx.x == 0 && tid == 0 && a.status) *a.status = reject ? 1 : 0;
  return reject;
}

template <int B>
COLL_STREAM_KERNEL void alltoallv_kernel(RankPtrs ptrs, A2avArgs a) {
  using W = typename Word<B>::T;
  extern __shared__ int64_t lds[];
  __shared__ int bad;
  if (stage_a2av_counts(a, lds, &bad)) return;
  const int p = a.p;
  const int pp = p * p;
  const int64_t* cnt = lds;
  const int64_t* soff = lds + pp;
  const int64_t* roff = lds + 2 * pp;
  uint64_t base = 0;
  for (int sgi = 0; sgi < pp; ++sgi) {
    const int i = sgi / p, j = sgi - (sgi / p) * p;
    const uint64_t len = (uint64_t)cnt[sgi];
    if (len == 0) continue;
    const uint64_t so = (uint64_t)soff[sgi];
    const uint64_t ro = (uint64_t)roff[sgi];
    const W* src = (const W*)ptrs.src[i] + so;
    W* dst = (W*)ptrs.dst[j] + ro;
    const int mis = (int)((uintptr_t)dst & 15), amis = (int)((uintptr_t)dst & (kLineAlign - 1));
    auto gdst = [&](int) -> W* { return dst; };
    base += copy_segment<B, true, 1, true>(src, gdst, 1, len, mis, amis, base);
  }
}

// Alltoallv for p <= 16 (p^2 <= kBlock segments): after staging the
// counts, thread s computes segment s's geometry from its pointers (a head
// up to the receive buffer's next 256-byte line, aligned destination
// vectors, a tail) and its tile count (a segment with only a head or tail
// gets one tile); workgroup-wide scans turn the counts into tile starts,
// and each flat tile finds its segment by binary search over the starts.  The
// walking kernel above has every workgroup run the segment routine for
// all p^2 segments, which made small calls take 40 us at p = 8 and 149 us
// at p = 16.  With a claim slot and at least kClaimMinTilesPerWg aligned
// tiles per workgroup, the aligned tiles are split as in
// pair_copy_flat_kernel: kPairDealtEighths of them dealt out in turn, the
// rest claimed one at a time from kClaimPools pooled counters (every
// workgroup computes the same tile counts, so all agree on the split).
template <int B>
COLL_STREAM_KERNEL void alltoallv_flat_kernel(RankPtrs ptrs, A2avArgs a) {
  using W = typename Word<B>::T;
  constexpr uint64_t V = 16 / B;
  extern __shared__ int64_t lds[];
  __shared__ int bad;
  // tile starts of the segments whose sources share the destinations'
  // 16-byte alignment (plain vector tiles) and of the others (byte-shifted
  // tiles): two separate loops below, so the common aligned loop keeps its
  // own waits (one loop holding both paths cost the aligned case 4%)
  __shared__ uint64_t tstart[2][kBlock + 1];
  if (stage_a2av_counts(a, lds, &bad)) return;
  const int p = a.p;
  const int pp = p * p;
  const int64_t* cnt = lds;
  const int64_t* soff = lds + pp;
  const int64_t* roff = lds + 2 * pp;
  const int tid = threadIdx.x;
  uint64_t nt[2] = {0, 0};
  if (tid < pp && cnt[tid] > 0) {
    const uint64_t len = (uint64_t)cnt[tid];
    const int si = tid / p, sj = tid - (tid / p) * p;
    const ShiftSpan sp = shift_span<B>((const W*)ptrs.src[si] + soff[tid], (W*)ptrs.dst[sj] + roff[tid], len);
    const uint64_t n = sp.nvec ? ceil_div(sp.nvec, kCopyTV) : 1;
    nt[(sp.m != 0 && sp.nvec != 0) ? 1 : 0] = n;
  }
  // inclusive scans: tstart[c][s + 1] = tiles of class c among segments 0..s
  for (int c = 0; c < 2; ++c) {
    tstart[c][tid + 1] = nt[c];
    if (tid == 0) tstart[c][0] = 0;
  }
  __syncthreads();
  for (int off = 1; off < kBlock; off <<= 1) {
    const uint64_t v0 = tid >= off ? tstart[0][tid + 1 - off] : 0;
    const uint64_t v1 = tid >= off ? tstart[1][tid + 1 - off] : 0;
    __syncthreads();
    tstart[0][tid + 1] += v0;
    tstart[1][tid + 1] += v1;
    __syncthreads();
  }
  // segment of class c holding that class's tile f, and the tile's index in it
  auto find = [&](int c, uint64_t f, int* sgi, uint64_t* t) {
    int lo = 0, hi = pp;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tstart[c][mid] <= f) lo = mid;
      else hi = mid;
    }
    *sgi = lo;
    *t = f - tstart[c][lo];
  };
  auto edges = [&](const W* src, W* dst, const ShiftSpan& sp) {
    // the head (up to the next 256-byte line of the receive buffer) and
    // the tail (under one vector)
    for (uint64_t e = tid; e < sp.head + sp.tail; e += kBlock) {
      const uint64_t x = e < sp.head ? e : sp.head + sp.nvec * V + (e - sp.head);
      st1<true>(dst + x, ld1<true>(src + x));
    }
  };
  const uint64_t total0 = tstart[0][pp], total = total0 + tstart[1][pp];
  const bool claims =
      a.claim && total0 >= kClaimMinTilesPerWg * gridDim.x && gridDim.x >= (uint32_t)(kClaimPools * kClaimPools);
  const uint64_t per = claims ? total0 / 8 * (8 - kPairDealtEighths) / kClaimPools : 0;
  const uint64_t dealt0 = total0 - per * kClaimPools;
  const uint32_t pool = claim_pool(blockIdx.x);
  unsigned long long* ctr = per ? a.claim + pool * kClaimPoolWords : nullptr;
  unsigned long long first = 0;
  if (per) first = issue_claim(ctr, tid);
  for (uint64_t f = blockIdx.x; f < dealt0; f += gridDim.x) {
    int sgi;
    uint64_t t;
    find(0, f, &sgi, &t);
    const int i = sgi / p, j = sgi - (sgi / p) * p;
    const W* src = (const W*)ptrs.src[i] + soff[sgi];
    W* dst = (W*)ptrs.dst[j] + roff[sgi];
    const ShiftSpan sp = shift_span<B>(src, dst, (uint64_t)cnt[sgi]);
    const u32x4* vs = reinterpret_cast<const u32x4*>(src + sp.head);
    u32x4* vd = reinterpret_cast<u32x4*>(dst + sp.head);
    auto gdst = [&](int) -> u32x4* { return vd; };
    const uint64_t j0 = t * kCopyTV + tid;
    if ((t + 1) * kCopyTV <= sp.nvec) copy_vec_tile<true, true, 1>(vs, gdst, 1, j0, sp.nvec);
    else if (t * kCopyTV < sp.nvec) copy_vec_tile<true, false, 1>(vs, gdst, 1, j0, sp.nvec);
    if (t == 0 && (sp.head || sp.tail)) edges(src, dst, sp);
  }
  for (uint64_t f = total0 + blockIdx.x; f < total; f += gridDim.x) {
    int sgi;
    uint64_t t;
    find(1, f - total0, &sgi, &t);
    const int i = sgi / p, j = sgi - (sgi / p) * p;
    const W* src = (const W*)ptrs.src[i] + soff[sgi];
    W* dst = (W*)ptrs.dst[j] + roff[sgi];
    const ShiftSpan sp = shift_span<B>(src, dst, (uint64_t)cnt[sgi]);
    const u32x4* vs = reinterpret_cast<const u32x4*>((uintptr_t)(src + sp.head) & ~(uintptr_t)15);
    u32x4* vd = reinterpret_cast<u32x4*>(dst + sp.head);
    auto gdst = [&](int) -> u32x4* { return vd; };
    const uint64_t j0 = t * kCopyTV + tid;
    if ((t + 1) * kCopyTV <= sp.nvec) copy_shift_tile<true, 1>(vs, gdst, 1, j0, sp.nvec, sp.m);
    else if (t * kCopyTV < sp.nvec) copy_shift_tile<false, 1>(vs, gdst, 1, j0, sp.nvec, sp.m);
    if (t == 0 && (sp.head || sp.tail)) edges(src, dst, sp);
  }
  if (!per) return;
  // claimed aligned tiles (thread 0 claims before a tile's loads and
  // publishes after them, as in pair_copy_flat_kernel)
  __shared__ uint64_t next_tile[2];
  const uint64_t first_claim = wave_value(first);
  if (tid == 0) next_tile[0] = first_claim;
  __syncthreads();
  uint64_t c = next_tile[0];
  int par = 1;
  while (c < per) {
    const unsigned long long next = issue_claim(ctr, tid);
    int sgi;
    uint64_t t;
    find(0, dealt0 + pool + (uint64_t)kClaimPools * c, &sgi, &t);
    const int i = sgi / p, j = sgi - (sgi / p) * p;
    const W* src = as_global((const W*)ptrs.src[i] + soff[sgi]);
    W* dst = as_global((W*)ptrs.dst[j] + roff[sgi]);
    const ShiftSpan sp = shift_span<B>(src, dst, (uint64_t)cnt[sgi]);
    const auto publish = [&](uint32_t tok) {
      const uint64_t v = wave_value(next + tok);
      if (tid == 0) next_tile[par] = v;
    };
    const u32x4* vs = reinterpret_cast<const u32x4*>(src + sp.head);
    u32x4* vd = reinterpret_cast<u32x4*>(dst + sp.head);
    auto gdst = [&](int) -> u32x4* { return vd; };
    const uint64_t j0 = t * kCopyTV + tid;
    if ((t + 1) * kCopyTV <= sp.nvec) copy_vec_tile<true, true, 1>(vs, gdst, 1, j0, sp.nvec, publish);
    else if (t * kCopyTV < sp.nvec) copy_vec_tile<true, false, 1>(vs, gdst, 1, j0, sp.nvec, publish);
    else publish(0);
    if (t == 0 && (sp.head || sp.tail)) edges(src, dst, sp);
    asm volatile("" ::"v"(next));  // keep the claim's register out of the stores' reach
    __syncthreads();
    c = next_tile[par];
    par ^= 1;
  }
  if (tid == 0) claim_last(ctr, c, per, claim_pool_members(gridDim.x, pool));
}

// ---------------------------------------------------------------------------
// Host-side launch
// ---------------------------------------------------------------------------
static int clamp_grid(uint64_t tiles, int max_grid) {
  if (tiles == 0) return 0;
  return (int)(tiles < (uint64_t)max_grid ? tiles : (uint64_t)max_grid);
}

template <int B, int KIND, bool SHIFT>
static void launch_fanout(int p, int grid, const RankPtrs& ptrs, const CopyGeom& g, hipStream_t s) {
  switch (p) {
    case 1: hipLaunchKernelGGL((fanout_kernel<B, KIND, 1, SHIFT>), dim3(grid), dim3(kBlock), 0, s, ptrs, g); break;
    case 2: hipLaunchKernelGGL((fanout_kernel<B, KIND, 2, SHIFT>), dim3(grid), dim3(kBlock), 0, s, ptrs, g); break;
    case 4: hipLaunchKernelGGL((fanout_kernel<B, KIND, 4, SHIFT>), dim3(grid), dim3(kBlock), 0, s, ptrs, g); break;
    case 8: hipLaunchKernelGGL((fanout_kernel<B, KIND, 8, SHIFT>), dim3(grid), dim3(kBlock), 0, s, ptrs, g); break;
    case 16: hipLaunchKernelGGL((fanout_kernel<B, KIND, 16, SHIFT>), dim3(grid), dim3(kBlock), 0, s, ptrs, g); break;
    default: hipLaunchKernelGGL((fanout_kernel<B, KIND, 0, SHIFT>), dim3(grid), dim3(kBlock), 0, s, ptrs, g); break;
  }
}

// Whether some segment's source disagrees modulo 16 with its destinations
// (the walking kernels then compile the byte-shift path).  Segment
// offsets are multiples of n elements: s * n for AllGather destinations,
// Gather destinations and Scatter sources, (j * n, i * n) for All-to-All.
template <int B>
static bool copy_needs_shift(const CopyGeom& g) {
  if (g.src_mis < 0 || g.dst_mis < 0) return true;
  if (g.src_mis != g.dst_mis) return true;
  if (g.kind == kCopyBroadcast || g.p == 1) return false;
  return ((g.n * (uint64_t)B) & 15) != 0;
}

// Uniform segments (see pair_copy_flat_kernel): the common head, vector
// count and tail, and the tiles per segment; false if the layout does not
// qualify or the flat tile count does not fit 32 bits.
template <int B>
static bool uniform_pair_layout(const CopyGeom& g, uint64_t nseg, uint64_t* head, uint64_t* nvec, uint64_t* tail,
                                uint64_t* tps) {
  if (!(g.src_mis >= 0 && g.src_mis == g.dst_mis && g.src_mis % B == 0 && (g.n * (uint64_t)B) % 16 == 0))
    return false;
  constexpr uint64_t V = 16 / B;
  uint64_t h = (uint64_t)(((16 - g.src_mis) & 15) / B);
  if (h > g.n) h = g.n;
  *head = h;
  *nvec = (g.n - h) / V;
  *tail = g.n - h - *nvec * V;
  const uint64_t t = (*nvec + kCopyTV - 1) / kCopyTV;
  *tps = t ? t : 1;
  return nseg * *tps < (uint64_t{1} << 32);
}

template <int B, bool SHIFT>
static void launch_walking(const RankPtrs& ptrs, const CopyGeom& g0, int grid, hipStream_t s) {
  // claimed tails for fan-outs with many tiles per workgroup
  CopyGeom g = g0;
  const uint64_t te = kCopyTV * (16 / B);
  const uint64_t nseg = g.kind == kCopyAllGather ? (uint64_t)g.p : 1;
  if (g.kind != kCopyAllGather && g.kind != kCopyBroadcast) g.claim = nullptr;
  if (nseg * ((g.n + te - 1) / te) < kClaimMinTilesPerWg * (uint64_t)grid || grid < kClaimPools * kClaimPools)
    g.claim = nullptr;
  if (g.kind == kCopyAllToAll)
    hipLaunchKernelGGL((pair_copy_kernel<B, kCopyAllToAll, SHIFT>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
  else if (g.kind == kCopyGather)
    hipLaunchKernelGGL((pair_copy_kernel<B, kCopyGather, SHIFT>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
  else if (g.kind == kCopyScatter)
    hipLaunchKernelGGL((pair_copy_kernel<B, kCopyScatter, SHIFT>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
  else if (g.kind == kCopyAllGather)
    launch_fanout<B, kCopyAllGather, SHIFT>(g.p, grid, ptrs, g, s);
  else
    launch_fanout<B, kCopyBroadcast, SHIFT>(g.p, grid, ptrs, g, s);
}

template <int B>
static int launch_copy_b(const RankPtrs& ptrs, const CopyGeom& g, int max_grid, hipStream_t s, int fanout_grid) {
  const uint64_t nseg = g.kind == kCopyBroadcast ? 1 : (g.kind == kCopyAllToAll ? (uint64_t)g.p * g.p : g.p);
  if (g.kind == kCopyAllGather && (g.p == 2 || g.p == 4 || g.p == 8 || g.p == 16)) {
    uint64_t head, nvec, tail, tps;
    // only while every workgroup has at most one tile: larger AllGathers
    // keep the walking kernel, whose cost there is spread over many tiles
    if (uniform_pair_layout<B>(g, nseg, &head, &nvec, &tail, &tps) && nseg * tps <= (uint64_t)max_grid) {
      const int grid = clamp_grid(nseg * tps, max_grid);
      if (!grid) return 0;
      const uint32_t t32 = (uint32_t)tps;
      switch (g.p) {
        case 2: hipLaunchKernelGGL((allgather_flat_kernel<B, 2>), dim3(grid), dim3(kBlock), 0, s, ptrs, g, head, nvec, tail, t32); break;
        case 4: hipLaunchKernelGGL((allgather_flat_kernel<B, 4>), dim3(grid), dim3(kBlock), 0, s, ptrs, g, head, nvec, tail, t32); break;
        case 8: hipLaunchKernelGGL((allgather_flat_kernel<B, 8>), dim3(grid), dim3(kBlock), 0, s, ptrs, g, head, nvec, tail, t32); break;
        default: hipLaunchKernelGGL((allgather_flat_kernel<B, 16>), dim3(grid), dim3(kBlock), 0, s, ptrs, g, head, nvec, tail, t32); break;
      }
      return (int)hipGetLastError();
    }
  }
  if (g.kind == kCopyAllToAll || g.kind == kCopyGather || g.kind == kCopyScatter) {
    uint64_t head, nvec, tail, tps;
    if (uniform_pair_layout<B>(g, nseg, &head, &nvec, &tail, &tps)) {
      const uint64_t tiles = nseg * tps;
      const int grid = clamp_grid(tiles, max_grid);
      if (!grid) return 0;
      const uint32_t t32 = (uint32_t)tps;
      // claims only with enough whole tiles per workgroup and every pool
      // served by several workgroups
      CopyGeom gc = g;
      if (tiles < kClaimMinTilesPerWg * (uint64_t)grid || grid < kClaimPools * kClaimPools) gc.claim = nullptr;
      if (g.kind == kCopyAllToAll)
        hipLaunchKernelGGL((pair_copy_flat_kernel<B, kCopyAllToAll>), dim3(grid), dim3(kBlock), 0, s, ptrs, gc, head,
                           nvec, tail, t32);
      else if (g.kind == kCopyGather)
        hipLaunchKernelGGL((pair_copy_flat_kernel<B, kCopyGather>), dim3(grid), dim3(kBlock), 0, s, ptrs, gc, head,
                           nvec, tail, t32);
      else
        hipLaunchKernelGGL((pair_copy_flat_kernel<B, kCopyScatter>), dim3(grid), dim3(kBlock), 0, s, ptrs, gc, head,
                           nvec, tail, t32);
      return (int)hipGetLastError();
    }
  }
  const uint64_t te = kCopyTV * (16 / B);
  // fan-outs that may claim tiles take fanout_grid
  const bool fan = (g.kind == kCopyAllGather || g.kind == kCopyBroadcast) && (g.p == 8 || g.p == 16) && g.claim;
  const int grid = clamp_grid(nseg * ((g.n + te - 1) / te + 1), fan && fanout_grid > 0 ? fanout_grid : max_grid);
  if (!grid) return 0;
  if (copy_needs_shift<B>(g)) launch_walking<B, true>(ptrs, g, grid, s);
  else launch_walking<B, false>(ptrs, g, grid, s);
  return (int)hipGetLastError();
}

int launch_copy(int elem_bytes, const RankPtrs& ptrs, const CopyGeom& g, int max_grid, void* stream,
                int fanout_grid) {
  hipStream_t s = (hipStream_t)stream;
  if (elem_bytes == 1) return launch_copy_b<1>(ptrs, g, max_grid, s, fanout_grid);
  if (elem_bytes == 2) return launch_copy_b<2>(ptrs, g, max_grid, s, fanout_grid);
  if (elem_bytes == 4) return launch_copy_b<4>(ptrs, g, max_grid, s, fanout_grid);
  return (int)hipErrorInvalidValue;
}

int launch_alltoallv(int elem_bytes, const RankPtrs& ptrs, const A2avArgs& a, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const size_t shm = (size_t)3 * a.p * a.p * sizeof(int64_t);
  const bool flat = a.p * a.p <= kBlock;
  if (elem_bytes == 1) {
    if (flat) hipLaunchKernelGGL((alltoallv_flat_kernel<1>), dim3(grid), dim3(kBlock), shm, s, ptrs, a);
    else hipLaunchKernelGGL((alltoallv_kernel<1>), dim3(grid), dim3(kBlock), shm, s, ptrs, a);
  } else if (elem_bytes == 2) {
    if (flat) hipLaunchKernelGGL((alltoallv_flat_kernel<2>), dim3(grid), dim3(kBlock), shm, s, ptrs, a);
    else hipLaunchKernelGGL((alltoallv_kernel<2>), dim3(grid), dim3(kBlock), shm, s, ptrs, a);
  } else if (elem_bytes == 4) {
    if (flat) hipLaunchKernelGGL((alltoallv_flat_kernel<4>), dim3(grid), dim3(kBlock), shm, s, ptrs, a);
    else hipLaunchKernelGGL((alltoallv_kernel<4>), dim3(grid), dim3(kBlock), shm, s, ptrs, a);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace coll
