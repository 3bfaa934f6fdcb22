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
// Each wave (64 lanes) is an independent worker that takes short runs of
// the flat tile range, finds a run's first call by binary search and then
// walks forward call by call and chunk by chunk, so descriptors, rotated
// pointers and chunk geometry are read once per chunk of a run.
// Wave-sized tiles keep lanes busy on the many chunks of a few hundred
// elements that small calls produce.
// Within a tile the work is the single-call AllReduce's: ring order,
// partial in registers, p stores; the wave that holds tile 0 of a chunk
// also does the chunk's misaligned head and tail.
#include "reduce_tile.h"

namespace coll {

// Vectors per lane of a batch tile: 64 / P, at most 8 (4 at p = 16, 278
// VGPRs, no spills).  A wave tile is small (64 lanes), so its fixed cost
// (2P 64-bit addresses, the bounds and the loop) is paid per few hundred
// bytes; larger tiles amortise it.  The 10,000-call p = 16 plan took
// 14.56 ms at 1 vector per lane (the single-call AllReduce's 16 / P),
// 13.65 ms at 2 and 13.21 ms at 4; 8 spills.
template <int P>
struct BatchUnroll {
  static constexpr int raw = P == 0 ? 1 : 64 / P;
  static constexpr int value = raw < 1 ? 1 : (raw > 8 ? 8 : raw);
};

// Elements of a batch tile: one wave's share, U vectors per lane.
template <int DT, int P>
__host__ __device__ constexpr uint64_t batch_tile_elems() {
  return (uint64_t)BatchUnroll<P>::value * kWave * Traits<DT>::V;
}

// Tiles [from, to) of one call (tile indices local to the call), walked
// chunk by chunk by one wave: a chunk's rotated pointers and geometry are
// set up once for all of its tiles in the run.
template <int DT, int OP, int P>
__device__ __forceinline__ void batch_run(const BatchCall& bc, const void* const* pt, uint64_t from,
                                          uint64_t to, int lane) {
  using T = Traits<DT>;
  using S = typename T::S;
  constexpr int U = BatchUnroll<P>::value;
  constexpr uint64_t TV = (uint64_t)U * kWave;
  constexpr int V = T::V;
  const uint64_t tpc = bc.tiles_per_chunk;
  const uint64_t q = (bc.n + P - 1) / P;
  const Scales<P> sc{};  // unused: the batch has no pre-multiplied sums
  int c = (int)(from / tpc);
  uint64_t t = from - (uint64_t)c * tpc;
  uint64_t left = to - from;
  while (left) {
    const uint64_t cnt = (tpc - t) < left ? (tpc - t) : left;
    uint64_t lo = (uint64_t)c * q, hi = lo + q;
    if (lo > bc.n) lo = bc.n;
    if (hi > bc.n) hi = bc.n;
    const uint64_t len = hi - lo;
    if (len) {
      // the call's pointers at constant offsets, then the ring rotation
      // of chunk c in registers
      const S* src[P];
      S* dst[P];
#pragma unroll
      for (int k = 0; k < P; ++k) {
        src[k] = (const S*)ld_const(&pt[k]);
        dst[k] = as_global((S*)ld_const(&pt[P + k])) + lo;
      }
      rotate_left<P>(src, (c + 1) % P);
#pragma unroll
      for (int k = 0; k < P; ++k) src[k] = as_global(src[k]) + lo;
      const int mis = bc.mis < 0 ? -1 : (int)(((bc.mis & 255) + lo * T::B) & 15);
      const int amis = (bc.mis < 0 || bc.mis >= 256) ? -1 : seg_amis(bc.mis, lo * T::B);
      const SegSpan sp = seg_span_a<T::B>(len, mis, amis);
      if (!sp.vec) {
        for (uint64_t i = t; i < t + cnt; ++i) {
          const uint64_t e0 = i * TV * V;
          if (e0 < len)
            reduce_elems<DT, OP, P, kOrdRing, P, true, kWave>(src, dst, e0,
                                                          (len - e0) < TV * V ? (len - e0) : TV * V, sc, P,
                                                          lane);
        }
      } else {
        const S* vs[P];
        S* vd[P];
#pragma unroll
        for (int k = 0; k < P; ++k) {
          vs[k] = src[k] + sp.head;
          vd[k] = dst[k] + sp.head;
        }
        const uint64_t nfull = sp.nvec / TV;
        for (uint64_t i = t; i < t + cnt; ++i) {
          const uint64_t j0 = i * TV + lane;
          if (i < nfull)
            reduce_vec_tile<DT, OP, P, kOrdRing, P, true, U, true, kWave>(vs, vd, j0, sp.nvec, sc, P);
          else if (i * TV < sp.nvec)
            reduce_vec_tile<DT, OP, P, kOrdRing, P, true, U, false, kWave>(vs, vd, j0, sp.nvec, sc, P);
        }
        if (t == 0 && (sp.head || sp.tail))
          reduce_edges<DT, OP, P, kOrdRing, P, true, kWave>(src, dst, sp.head, sp.head + sp.nvec * V, sp.tail,
                                                            sc, P, lane);
      }
    }
    left -= cnt;
    ++c;
    t = 0;
  }
}

// Any rank count: element path with pointers read from the table.
template <int DT, int OP>
__device__ __forceinline__ void batch_run_any(const BatchCall& bc, const void* const* pt, int p, uint64_t from,
                                              uint64_t to, int lane) {
  using T = Traits<DT>;
  using S = typename T::S;
  using A = typename T::A;
  constexpr uint64_t TE = (uint64_t)kWave * T::V;
  const uint64_t tpc = bc.tiles_per_chunk;
  const uint64_t q = (bc.n + p - 1) / p;
  for (uint64_t local = from; local < to; ++local) {
    const int c = (int)(local / tpc);
    const uint64_t t = local - (uint64_t)c * tpc;
    uint64_t lo = (uint64_t)c * q, hi = lo + q;
    if (lo > bc.n) lo = bc.n;
    if (hi > bc.n) hi = bc.n;
    const uint64_t len = hi - lo;
    for (uint64_t e = t * TE + lane; e < len && e < (t + 1) * TE; e += kWave) {
      A acc = widen1<DT>(ld1<true>(as_global((const S*)ld_const(&pt[(c + 1) % p])) + lo + e));
      for (int k = 1; k < p; ++k)
        acc = combine<OP>(acc, widen1<DT>(ld1<true>(as_global((const S*)ld_const(&pt[(c + 1 + k) % p])) + lo + e)));
      const S out = narrow1<DT>(finish<OP>(acc, p));
      for (int k = 0; k < p; ++k) st1<true>(as_global((S*)ld_const(&pt[p + k])) + lo + e, out);
    }
  }
}

template <int P>
__device__ __forceinline__ void batch_dispatch(const BatchCall& bc, const void* const* pt, int p, uint64_t from,
                                               uint64_t to, int lane) {
#define COLL_BATCH_CASE(DTV, OPV)                                          \
  case DTV * 4 + OPV:                                                      \
    if constexpr (P > 0) batch_run<DTV, OPV, P>(bc, pt, from, to, lane);   \
    else batch_run_any<DTV, OPV>(bc, pt, p, from, to, lane);               \
    break;
  switch (bc.dtype * 4 + bc.op) {
    COLL_BATCH_CASE(kF32, kSum)
    COLL_BATCH_CASE(kF32, kMin)
    COLL_BATCH_CASE(kF32, kMax)
    COLL_BATCH_CASE(kF32, kAvg)
    COLL_BATCH_CASE(kBF16, kSum)
    COLL_BATCH_CASE(kBF16, kMin)
    COLL_BATCH_CASE(kBF16, kMax)
    COLL_BATCH_CASE(kBF16, kAvg)
    COLL_BATCH_CASE(kI32, kSum)
    COLL_BATCH_CASE(kI32, kMin)
    COLL_BATCH_CASE(kI32, kMax)
    COLL_BATCH_CASE(kI32, kAvg)
    default: break;
  }
#undef COLL_BATCH_CASE
}

// A call record, read with scalar loads (the table is not written while
// the kernel runs).
__device__ __forceinline__ BatchCall load_call(const BatchCall* c) {
  BatchCall b;
  b.n = ld_const(&c->n);
  b.first_tile = ld_const(&c->first_tile);
  b.dtype = ld_const(&c->dtype);
  b.op = ld_const(&c->op);
  b.tiles_per_chunk = ld_const(&c->tiles_per_chunk);
  b.mis = ld_const(&c->mis);
  return b;
}

// Every wave is an independent worker.  The flat tile range is cut into
// runs of kBatchRun tiles.  The first quarter of the runs are dealt out in
// turn (wave w takes runs w, w + W, ... for W waves in the grid), so the
// waves work on one window of the range and move through it front to back
// together.  Waves do not all stream at the same rate (dealt out to the
// end, the 10,000-call p = 16 plan's waves finished over a spread of 1.2
// ms, those of the odd-numbered XCDs last), so the remaining runs are
// claimed one at a time from a counter in the descriptor table (zero at
// launch), and a wave that runs ahead claims more of them; claims come in
// increasing order, so the window stays narrow.  Same-box A/B of the plan:
// 11.86 ms with 7/8 of the runs dealt out, 11.72 with 5/8, 11.53 with 2/8.
// A claim is issued before the run in hand and read at its end (gfx9
// counts loads, stores and atomics on one in-order counter, so that read
// also waits for the run's stores).  A wave finds a run's first call by
// binary search (from its previous run's call onward, as its runs only
// grow) and walks forward call by call.  Short runs keep the window
// narrow: with 4-vector tiles the plan took 13.2 ms with runs of 32 tiles,
// 13.0 with 8 and 12.9 with 2 (1: 13.1, a search per tile; all dealt out).
constexpr uint64_t kBatchRun = 2;

template <int P>
COLL_STREAM_KERNEL void batch_kernel(BatchArgs a) {
  const int p = P ? P : a.p;
  const int lane = (int)(threadIdx.x % kWave);
  const uint64_t waves = (uint64_t)gridDim.x * (kBlock / kWave);
  const uint64_t wid =
      (uint64_t)blockIdx.x * (kBlock / kWave) + (uint64_t)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint64_t total = ld_const(&a.calls[a.ncalls].first_tile);
  const uint64_t nruns = (total + kBatchRun - 1) / kBatchRun;
  const uint64_t nfixed = nruns / 8 * 2 / waves * waves;  // runs dealt out in turn
  int from_call = 0;
  uint64_t run = wid < nfixed ? wid : nfixed + wave_value(issue_claim(a.next_run, lane));
  // every claim returns a distinct, larger value, so each wave leaves the
  // loop after at most nruns / W + 1 dealt runs and nruns + 1 claims
  while (run < nruns) {
    const bool dealt = run + waves < nfixed;  // the next run is dealt, not claimed
    unsigned long long pending = 0;
    if (!dealt) pending = issue_claim(a.next_run, lane);
    uint64_t t = run * kBatchRun;
    const uint64_t end = t + kBatchRun < total ? t + kBatchRun : total;
    // last call whose first tile is <= t
    int lo = from_call, hi = a.ncalls;  // answer in [lo, hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ld_const(&a.calls[mid].first_tile) <= t) lo = mid;
      else hi = mid;
    }
    from_call = lo;
    // calls[ncalls].first_tile == total >= end, so k stays below ncalls
    for (int k = lo; t < end; ++k) {
      const BatchCall bc = load_call(a.calls + k);
      const uint64_t next = ld_const(&a.calls[k + 1].first_tile);
      const uint64_t stop = next < end ? next : end;
      if (stop > t)
        batch_dispatch<P>(bc, a.ptrs + (size_t)k * 2 * p, p, t - bc.first_tile, stop - bc.first_tile, lane);
      t = stop > t ? stop : t;
    }
    if (dealt) run += waves;
    else run = nfixed + wave_value(pending);
  }
}

uint64_t batch_tile_elems_host(int dtype, int p) {
  const bool bf = dtype == kBF16;
  switch (p) {
    case 2: return bf ? batch_tile_elems<kBF16, 2>() : batch_tile_elems<kF32, 2>();
    case 4: return bf ? batch_tile_elems<kBF16, 4>() : batch_tile_elems<kF32, 4>();
    case 8: return bf ? batch_tile_elems<kBF16, 8>() : batch_tile_elems<kF32, 8>();
    case 16: return bf ? batch_tile_elems<kBF16, 16>() : batch_tile_elems<kF32, 16>();
    default: return (uint64_t)kWave * (bf ? 8 : 4);
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
