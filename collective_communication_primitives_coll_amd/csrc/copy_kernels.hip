// Data re-placement without arithmetic: AllGather, Broadcast, All-to-All
// and variable-split All-to-All.
//
// All four are block copies between rank buffers; they differ only in how
// a segment (source range -> destination range(s)) is derived:
//   AllGather  segment s: send[s] -> recv[r] + s*n for every r, rank-order
//              concatenation ("集合通信：原语、算法、NCCL 实现与拓扑映射",
//              section 1.2);
//   Broadcast  one segment: send_root -> recv[r] for every r (section 1.1);
//   AllToAll   segment (i,j): send[i] + j*n -> recv[j] + i*n, the block
//              transpose of section 1.6;
//   Alltoallv  segment (i,j) of counts[i][j] elements, offsets from the
//              prefix sums of the count matrix ("Collective Communication：
//              AllReduce、AllGather、ReduceScatter 与 All-to-All", ragged
//              All-to-All).
// A lane loads kCopyUnroll 16-byte vectors, then stores each to every
// destination of the segment; the copy is type-blind apart from the
// element width used for misaligned heads and tails.
#include "device_common.h"

namespace coll {

template <int B>
struct Word;
template <>
struct Word<2> {
  using T = uint16_t;
};
template <>
struct Word<4> {
  using T = uint32_t;
};

template <int B>
constexpr uint64_t copy_tile_elems() {
  return kCopyUnroll * kBlock * (16 / B);
}

// Copy one tile of a segment.  src and dst(k) point at the segment start.
template <int B, bool DSTALL, typename GD>
__device__ __forceinline__ void copy_tile(const typename Word<B>::T* src, const GD& gdst, int ndst,
                                          const TileSpan& sp) {
  using W = typename Word<B>::T;
  constexpr int V = 16 / B;
  constexpr int U = (int)kCopyUnroll;
  const uint64_t tid = threadIdx.x;
  auto elems = [&](uint64_t from, uint64_t cnt) {
    for (uint64_t i = tid; i < cnt; i += kBlock) {
      const uint64_t e = from + i;
      const W w = ld1(src + e);
      if constexpr (DSTALL) {
        for (int k = 0; k < ndst; ++k) st1(gdst(k) + e, w);
      } else {
        st1(gdst(0) + e, w);
      }
    }
  };
  if (!sp.vec) {
    elems(sp.begin, sp.head);
    return;
  }
  if (sp.nvec) {
    const uint64_t v0 = sp.begin + sp.head;
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t vi = (uint64_t)u * kBlock + tid;
      if (vi < sp.nvec) r[u] = ld16(src + v0 + vi * V);
    }
    if constexpr (DSTALL) {
      for (int k = 0; k < ndst; ++k) {
        W* d = gdst(k);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint64_t vi = (uint64_t)u * kBlock + tid;
          if (vi < sp.nvec) st16(d + v0 + vi * V, r[u]);
        }
      }
    } else {
      W* d = gdst(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t vi = (uint64_t)u * kBlock + tid;
        if (vi < sp.nvec) st16(d + v0 + vi * V, r[u]);
      }
    }
  }
  if (sp.head) elems(sp.begin, sp.head);
  if (sp.tail) elems(sp.begin + sp.head + sp.nvec * V, sp.tail);
}

__device__ __forceinline__ int seg_mis(int src_mis, int dst_mis, uint64_t src_byte_off,
                                       uint64_t dst_byte_off) {
  if (src_mis < 0 || dst_mis < 0) return -1;
  const int sm = (int)((src_mis + src_byte_off) & 15);
  const int dm = (int)((dst_mis + dst_byte_off) & 15);
  return sm == dm ? sm : -1;
}

template <int B, bool DSTALL>
__global__ __launch_bounds__(kBlock) void copy_kernel(RankPtrs ptrs, CopyGeom g) {
  using W = typename Word<B>::T;
  constexpr uint64_t TE = copy_tile_elems<B>();
  const int p = g.p;
  const uint64_t grid = gridDim.x, wg = blockIdx.x;
  const int nseg = g.kind == kCopyAllGather ? p : (g.kind == kCopyBroadcast ? 1 : p * p);
  const uint64_t ntiles = ceil_div(g.n, TE);
  uint64_t base = 0;
  for (int sgi = 0; sgi < nseg; ++sgi, base += ntiles) {
    const W* src;
    uint64_t src_off = 0, dst_off = 0;
    int dj = 0;
    if (g.kind == kCopyAllGather) {
      src = (const W*)ptrs.src[sgi];
      dst_off = (uint64_t)sgi * g.n;
    } else if (g.kind == kCopyBroadcast) {
      src = (const W*)ptrs.src[0];
    } else {
      const int i = sgi / p, j = sgi - (sgi / p) * p;
      src_off = (uint64_t)j * g.n;
      dst_off = (uint64_t)i * g.n;
      src = (const W*)ptrs.src[i] + src_off;
      dj = j;
    }
    const int mis = seg_mis(g.src_mis, g.dst_mis, src_off * B, dst_off * B);
    auto gdst = [&](int k) -> W* {
      if constexpr (DSTALL) return (W*)ptrs.dst[k] + dst_off;
      else return (W*)ptrs.dst[dj] + dst_off;
    };
    for (uint64_t t = first_tile(base, wg, grid); t < ntiles; t += grid) {
      const TileSpan sp = tile_span<B, 16 / B>(g.n, TE, t, mis);
      copy_tile<B, DSTALL>(src, gdst, p, sp);
    }
  }
}

// ---------------------------------------------------------------------------
// Alltoallv.  Every workgroup stages the p x p count matrix in LDS, checks
// it against the buffer capacities, and derives the send offsets (row
// exclusive prefix sums) and receive offsets (column exclusive prefix sums
// in source order).  Then the segments (i, j) are walked like the equal
// split.  Invalid counts make every workgroup return before any payload
// is written.
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(kBlock) void alltoallv_kernel(RankPtrs ptrs, A2avArgs a) {
  using W = typename Word<B>::T;
  constexpr uint64_t TE = copy_tile_elems<B>();
  extern __shared__ int64_t lds[];
  __shared__ int bad;
  const int p = a.p;
  const int pp = p * p;
  int64_t* cnt = lds;
  int64_t* soff = lds + pp;
  int64_t* roff = lds + 2 * pp;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  for (int i = tid; i < pp; i += kBlock) cnt[i] = a.counts[i];
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
    if (!ok) bad = 1;
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
    if (!ok) bad = 1;
  }
  __syncthreads();
  const bool reject = bad != 0;
  if (blockIdx.x == 0 && tid == 0 && a.status) *a.status = reject ? 1 : 0;
  if (reject) return;

  const uint64_t grid = gridDim.x, wg = blockIdx.x;
  uint64_t base = 0;
  for (int sgi = 0; sgi < pp; ++sgi) {
    const int i = sgi / p, j = sgi - (sgi / p) * p;
    const uint64_t len = (uint64_t)cnt[sgi];
    if (len == 0) continue;
    const uint64_t ntiles = ceil_div(len, TE);
    const uint64_t so = (uint64_t)soff[sgi];
    const uint64_t ro = (uint64_t)roff[sgi];
    const W* src = (const W*)ptrs.src[i] + so;
    W* dst = (W*)ptrs.dst[j] + ro;
    const int mis = seg_mis(a.src_mis, a.dst_mis, so * B, ro * B);
    auto gdst = [&](int) -> W* { return dst; };
    for (uint64_t t = first_tile(base, wg, grid); t < ntiles; t += grid) {
      const TileSpan sp = tile_span<B, 16 / B>(len, TE, t, mis);
      copy_tile<B, false>(src, gdst, 1, sp);
    }
    base += ntiles;
  }
}

static int clamp_grid(uint64_t tiles, int max_grid) {
  if (tiles == 0) return 0;
  return (int)(tiles < (uint64_t)max_grid ? tiles : (uint64_t)max_grid);
}

template <int B>
static int launch_copy_b(const RankPtrs& ptrs, const CopyGeom& g, int max_grid, hipStream_t s) {
  const uint64_t nseg = g.kind == kCopyAllGather ? g.p : (g.kind == kCopyBroadcast ? 1 : (uint64_t)g.p * g.p);
  const int grid = clamp_grid(nseg * ((g.n + copy_tile_elems<B>() - 1) / copy_tile_elems<B>()), max_grid);
  if (!grid) return 0;
  if (g.kind == kCopyAllToAll)
    hipLaunchKernelGGL((copy_kernel<B, false>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
  else
    hipLaunchKernelGGL((copy_kernel<B, true>), dim3(grid), dim3(kBlock), 0, s, ptrs, g);
  return (int)hipGetLastError();
}

int launch_copy(int elem_bytes, const RankPtrs& ptrs, const CopyGeom& g, int max_grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (elem_bytes == 2) return launch_copy_b<2>(ptrs, g, max_grid, s);
  if (elem_bytes == 4) return launch_copy_b<4>(ptrs, g, max_grid, s);
  return (int)hipErrorInvalidValue;
}

int launch_alltoallv(int elem_bytes, const RankPtrs& ptrs, const A2avArgs& a, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const size_t shm = (size_t)3 * a.p * a.p * sizeof(int64_t);
  if (elem_bytes == 2)
    hipLaunchKernelGGL((alltoallv_kernel<2>), dim3(grid), dim3(kBlock), shm, s, ptrs, a);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL((alltoallv_kernel<4>), dim3(grid), dim3(kBlock), shm, s, ptrs, a);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace coll
