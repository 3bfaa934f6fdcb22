// Device-side building blocks shared by the collective kernels (gfx950).
//
// Data moves in 16-byte vectors (global_load/store_dwordx4).  Each kernel
// picks the cache policy per direction from what the direction mix of the
// collective sustains on MI355X HBM3E:
//   * reductions (p loads per store) stream their loads non-temporally and
//     store through the cache;
//   * fan-out copies (one load per p stores: AllGather, Broadcast) load
//     through the cache and store non-temporally;
//   * AllReduce (p loads, p stores) and 1:1 copies are non-temporal both
//     ways.
// A segment is a run of elements that starts at one offset in every
// source and at one offset in every destination.  Its 16-byte aligned
// middle goes through vector tiles; the misaligned head and tail (fewer
// than one vector each) go element by element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_args.h"

namespace coll {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;  // threads per workgroup (4 wave64s)

// Launch attributes of the streaming kernels.  They run one or two
// workgroups per CU and rely on many loads in flight per lane, so the
// compiler is told to target at most two waves per SIMD: it may then keep
// every operand of a tile in registers instead of serialising loads to
// fit a high-occupancy register budget.
#define COLL_STREAM_KERNEL __global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 2)))

template <int DT> struct Traits;
template <> struct Traits<kF32> {
  using S = float;     // storage type
  using A = float;     // accumulation type
  static constexpr int V = 4;  // elements per 16-byte vector
  static constexpr int B = 4;  // bytes per element
};
template <> struct Traits<kBF16> {
  using S = uint16_t;
  using A = float;
  static constexpr int V = 8;
  static constexpr int B = 2;
};
template <> struct Traits<kI32> {
  using S = int32_t;
  using A = int32_t;
  static constexpr int V = 4;
  static constexpr int B = 4;
};

// ---------------------------------------------------------------------------
// Loads and stores.  NT selects the non-temporal (streaming) hint.
// ---------------------------------------------------------------------------
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else *reinterpret_cast<u32x4*>(p) = v;
}
template <bool NT, typename S>
__device__ __forceinline__ S ld1(const S* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename S>
__device__ __forceinline__ void st1(S* p, S v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// A pointer that a kernel reads from device memory (not from its
// arguments) has no known address space, so accesses through it compile to
// FLAT instructions.  Those also count against the scalar-memory counter:
// a later scalar load then waits for every outstanding FLAT store.  Every
// buffer here is device-visible global memory, so such pointers are
// declared global, which gives GLOBAL loads and stores.
template <typename T>
__device__ __forceinline__ T* as_global(T* p) {
  return (T*)(__attribute__((address_space(1))) T*)(uintptr_t)p;
}

// Load from memory that no thread writes during the kernel (descriptor
// tables uploaded before the launch): read through the constant address
// space, a uniform address becomes a scalar load.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(uintptr_t)p;
}

// ---------------------------------------------------------------------------
// Widening and narrowing.  bf16 widens exactly (the pattern is the upper
// half of the fp32 pattern) and narrows with round-to-nearest-even through
// the gfx950 conversion instruction (v_cvt_pk_bf16_f32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

template <int DT>
__device__ __forceinline__ void widen(u32x4 v, typename Traits<DT>::A (&a)[Traits<DT>::V]) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = __uint_as_float(v[e]);
  } else if constexpr (DT == kI32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = (int32_t)v[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[2 * e] = bf16_lo(v[e]);
      a[2 * e + 1] = bf16_hi(v[e]);
    }
  }
}

template <int DT>
__device__ __forceinline__ u32x4 narrow(const typename Traits<DT>::A (&a)[Traits<DT>::V]) {
  u32x4 v;
  if constexpr (DT == kF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(a[e]);
  } else if constexpr (DT == kI32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (uint32_t)a[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = bf16_pack(a[2 * e], a[2 * e + 1]);
  }
  return v;
}

template <int DT>
__device__ __forceinline__ typename Traits<DT>::A widen1(typename Traits<DT>::S s) {
  if constexpr (DT == kBF16) return __uint_as_float((uint32_t)s << 16);
  else return s;
}
template <int DT>
__device__ __forceinline__ typename Traits<DT>::S narrow1(typename Traits<DT>::A a) {
  if constexpr (DT == kBF16) return (uint16_t)bf16_bits(a);
  else return a;
}

// ---------------------------------------------------------------------------
// The elementwise operation.  acc is the running partial, v the next
// rank's value; min/max are compare-selects that keep acc on ties and when
// either operand is NaN (the comparison is then false); avg and
// pre-multiplied sums add.  int32 sums add through uint32_t, so they wrap
// modulo 2^32 by definition rather than by signed overflow.
// ---------------------------------------------------------------------------
template <int OP, typename A>
__device__ __forceinline__ A combine(A acc, A v) {
  if constexpr (OP == kSum || OP == kAvg || OP == kPreMul) {
    if constexpr (__is_same(A, int32_t)) return (int32_t)((uint32_t)acc + (uint32_t)v);
    else return acc + v;
  } else if constexpr (OP == kMin) {
    return (v < acc) ? v : acc;
  } else {
    return (v > acc) ? v : acc;
  }
}

template <int OP, int DT>
__device__ __forceinline__ void combine_vec(typename Traits<DT>::A (&acc)[Traits<DT>::V],
                                            const typename Traits<DT>::A (&v)[Traits<DT>::V]) {
#pragma unroll
  for (int e = 0; e < Traits<DT>::V; ++e) acc[e] = combine<OP>(acc[e], v[e]);
}

// ---------------------------------------------------------------------------
// Segment geometry.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// Split of a segment of `len` elements of B bytes whose start sits `mis`
// bytes past a 16-byte boundary in every source and destination (mis < 0:
// they disagree, so nothing can be vectorised).
struct SegSpan {
  uint64_t head;  // elements before the first aligned vector
  uint64_t nvec;  // aligned 16-byte vectors
  uint64_t tail;  // elements after the last vector
  bool vec;
};

template <int B>
__device__ __forceinline__ SegSpan seg_span(uint64_t len, int mis) {
  constexpr uint64_t V = 16 / B;
  SegSpan s;
  if (mis < 0 || mis % B != 0) {
    s.vec = false;
    s.head = len;
    s.nvec = 0;
    s.tail = 0;
    return s;
  }
  s.vec = true;
  uint64_t h = (uint64_t)(((16 - mis) & 15) / B);
  if (h > len) h = len;
  s.head = h;
  s.nvec = (len - h) / V;
  s.tail = len - h - s.nvec * V;
  return s;
}

// Vector tiles start at this byte alignment of the sources when the
// segment allows it: a wave's 1 KiB access then covers exactly eight
// 128-byte cache lines instead of nine (AllReduce p = 8 at 256 MiB per
// rank ran at 4.5-4.8 TB/s with chunks a few bytes off a 256-byte
// boundary, 5.5 TB/s on it).
constexpr int kLineAlign = 256;

// seg_span with the element-wise head extended until one side (the
// reductions' sources, the copies' destinations) reaches a kLineAlign
// boundary.  amis is that side's common address modulo kLineAlign at the
// segment start, or -1 if unknown (then as seg_span).  The head stays
// below kLineAlign / B elements; after it that side is kLineAlign-aligned
// and the other 16-byte aligned whenever they agree modulo 16 (mis >= 0).
template <int B>
__device__ __forceinline__ SegSpan seg_span_a(uint64_t len, int mis, int amis) {
  SegSpan s = seg_span<B>(len, mis);
  if (!s.vec || amis < 0) return s;
  constexpr uint64_t V = 16 / B;
  uint64_t h = (uint64_t)(((kLineAlign - amis) & (kLineAlign - 1)) / B);
  if (h > len) h = len;
  s.head = h;
  s.nvec = (len - h) / V;
  s.tail = len - h - s.nvec * V;
  return s;
}

// Address modulo kLineAlign of a segment starting byte_off bytes past
// bases whose common misalignment modulo kLineAlign is amis (-1: none).
__device__ __forceinline__ int seg_amis(int amis, uint64_t byte_off) {
  return amis < 0 ? -1 : (int)((amis + byte_off) & (kLineAlign - 1));
}

// Misalignment of a segment whose sources start src_byte_off bytes past
// bases with common misalignment src_mis (and likewise for destinations).
__device__ __forceinline__ int seg_mis(int src_mis, int dst_mis, uint64_t src_byte_off,
                                       uint64_t dst_byte_off) {
  if (src_mis < 0 || dst_mis < 0) return -1;
  const int sm = (int)((src_mis + src_byte_off) & 15);
  const int dm = (int)((dst_mis + dst_byte_off) & 15);
  return sm == dm ? sm : -1;
}

// First tile index t >= 0 of a segment whose flat index base + t is
// congruent to the workgroup id modulo the grid size.  The workgroup for
// which this is 0 also owns the segment's element-wise head and tail.
__device__ __forceinline__ uint64_t first_tile(uint64_t base, uint64_t wg, uint64_t grid) {
  const uint64_t r = base % grid;
  return (wg + grid - r) % grid;
}

// The same with one 32-bit remainder, for the per-segment ownership
// checks that every workgroup makes for every segment: tile counts of a
// call stay below 2^32 (a tile covers at least 1 KiB and a call at most
// the device's memory), and 64-bit division is a long software sequence.
// (The tile loops keep the 64-bit form: their code measured faster so.)
__device__ __forceinline__ uint32_t first_tile32(uint64_t base, uint32_t wg, uint32_t grid) {
  const uint32_t r = (uint32_t)base % grid;
  const uint32_t t = wg + grid - r;
  return t >= grid ? t - grid : t;
}

// ---------------------------------------------------------------------------
// Claimed work.  Workgroups do not all stream at the same rate: with tiles
// dealt out in turn, those of the odd-numbered XCDs finish a large
// ReduceScatter or AllReduce 3-5% after the others, and an AllGather's
// workgroups finish anywhere between 40% and 100% of the kernel's time.
// So the streaming kernels deal out part of their tiles in turn and let
// the workers (workgroups, or waves) claim the rest, one at a time, from a
// counter: a worker that runs ahead claims more.  Each launch gets a
// counter slot, zero at launch; the copies, Alltoallv, the MoE token
// copies and AllReduce at p = 8 split their claimed work over the slot's
// kClaimPools counters (claim_pool), the other kernels use one counter.  Every worker claims until a claim comes back past the last
// unit of its counter, so a counter with `units` claimable units and W
// workers takes exactly units + W claims; the worker whose claim returns
// units + W - 1 makes the last one and zeroes the counter for the next
// launch that uses the slot (claim_last), without waiting for the other
// workers to finish their tiles.
// ---------------------------------------------------------------------------
constexpr int kWave = 64;  // lanes of a wave

// Tiles of a reduction dealt out in turn when `tiles` tiles are shared by
// a grid of `grid` workgroups: a quarter, rounded down to whole rounds of
// the grid; the rest are claimed.  Same-box A/B against 7/8 and 4/8 dealt:
// AllReduce p = 8 (2^26 fp32 per rank) 755, 741, 737 us; at p = 3 and 12
// 274, 263, 256 us and 1147, 1097, 1076 us; ReduceScatter p = 8 (2^26
// bf16 per rank) 203, 200, 199 us, other rank counts within 1%.
__device__ __forceinline__ uint64_t dealt_tiles(uint64_t tiles, uint64_t grid) {
  return tiles / 8 * 2 / grid * grid;
}

// Lane 0's claim of one unit (the other lanes get 0).  Read its result
// with wave_value only after a wait that covers it: gfx9 counts loads,
// stores and atomics on one in-order counter, so the wait for the loads
// of the work issued after the claim also covers the claim, whereas
// reading the result at the end of that work would also wait for its
// stores.  (Sources using this are built without LLVM's atomic
// optimizer, which would read the result right after the atomic.)
__device__ __forceinline__ unsigned long long issue_claim(unsigned long long* slot, int lane) {
  unsigned long long r = 0;
  if (lane == 0) r = atomicAdd(as_global(slot), 1ull);
  return r;
}

__device__ __forceinline__ uint64_t wave_value(unsigned long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// Store policy of a tile's 16-byte vectors (kStPlain, kStNT, kStDevice in
// kernel_args.h).  A CDNA3/CDNA4 store carries a
// coherence scope (its sc0 and sc1 bits) and a non-temporal hint (nt):
//   kStPlain   plain store: the line stays dirty in the XCD's L2 and is
//              written back when evicted;
//   kStNT      non-temporal: streams past the caches;
//   kStDevice  device scope (sc1): written through the L2 at once, into the
//              memory-side Infinity Cache;
//   kStNTDevice  both (nt and sc1).
// Measured on MI355X with a ReduceScatter (p = 8, 2^26 bf16 per rank)
// followed by the AllGather of its shards: plain 199-203 us, then 175 us;
// non-temporal 187-191 us, but the AllGather took 210-211 us because its
// 128 MiB of shards no longer came from the Infinity Cache; device scope
// 187-190 us and 174-175 us.  The same store of device scope made an
// AllReduce (p = 8, 256 MiB fp32 per rank) slower than non-temporal stores
// (756 against 737 us).  AllGather's fan-out (1 GiB written) took 172-173 us
// with non-temporal stores of device scope against 174-175 us with
// non-temporal ones.  Stores that leave dirty lines in the Infinity Cache
// move part of their cost to whichever later kernel evicts them (a MoE
// pack with device-scope stores was 8 us faster but made the exchange after
// it 26 us slower), so each kernel takes the policy that measured best
// over the path it sits in, not alone.
// ---------------------------------------------------------------------------

// HIP's global stores cannot carry sc1, so device-scope stores go through a
// buffer resource over one wave-uniform range [base, base + bytes):
// offsets are bytes from base, and a store past the range is dropped by the
// hardware's range check.  Word 3 of a gfx9 buffer descriptor: 32-bit data
// format, no swizzle or index stride (a raw byte range).
constexpr int kBufferWord3 = 0x00020000;
// the builtin's cache-policy operand: bit 1 nt, bit 4 sc1
constexpr int kCachePolicySc1 = 16, kCachePolicyNtSc1 = 18;

template <int CPOL>
struct DeviceScopeStores {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ DeviceScopeStores(uint64_t base, uint32_t bytes)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(wave_value(base)), 0, (int)bytes,
                                               kBufferWord3)) {}
  __device__ __forceinline__ void put(uint32_t off, u32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)off, 0, CPOL);
  }
};

// The stores of one tile: vector u of this lane goes to dst[j0 + u * LANES],
// where j0 = tile start + lane and lane = threadIdx.x % LANES (so j0 - lane
// is the same on every lane of the tile).  FULL: every vector lies below
// nvec (else those at or past nvec are skipped).
template <int SP, int U, int LANES, bool FULL>
__device__ __forceinline__ void store_tile(u32x4* dst, uint64_t j0, uint64_t nvec, const u32x4 (&v)[U]) {
  if constexpr (SP == kStDevice || SP == kStNTDevice) {
    const uint32_t lane = threadIdx.x % LANES;
    const DeviceScopeStores<SP == kStDevice ? kCachePolicySc1 : kCachePolicyNtSc1> st(
        (uint64_t)(dst + (j0 - lane)), (uint32_t)U * LANES * 16);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (FULL || j0 + (uint64_t)u * LANES < nvec) st.put(((uint32_t)u * LANES + lane) * 16, v[u]);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t j = j0 + (uint64_t)u * LANES;
      if (FULL || j < nvec) st16<SP == kStNT>(dst + j, v[u]);
    }
  }
}

// Pooled claims: the pool of workgroup b.  Runs of kClaimPools consecutive
// workgroups share a pool, so that every pool draws its workgroups from
// all XCDs (workgroups are dispatched to the XCDs in turn, and some XCDs
// stream a few percent slower than others).  Needs at least
// kClaimPools^2 workgroups for every pool to have one.
__device__ __forceinline__ uint32_t claim_pool(uint32_t b) { return (b / kClaimPools) % kClaimPools; }
// The number of workgroups among the first n in pool x.
__device__ __forceinline__ uint64_t claim_pool_members(uint64_t n, uint32_t x) {
  constexpr uint64_t span = (uint64_t)kClaimPools * kClaimPools;
  const uint64_t rem = n % span, lo = (uint64_t)x * kClaimPools;
  const uint64_t extra = rem > lo ? (rem - lo < (uint64_t)kClaimPools ? rem - lo : (uint64_t)kClaimPools) : 0;
  return n / span * kClaimPools + extra;
}

// A worker whose claim v came back past the last of `units` units: if it
// was the launch's last claim, zero the counter.
__device__ __forceinline__ void claim_last(unsigned long long* slot, uint64_t v, uint64_t units,
                                           uint64_t nworkers) {
  if (v == units + nworkers - 1) atomicExch(as_global(slot), 0ull);
}

// A callable that does nothing: the default mid-tile hook.
struct NoHook {
  __device__ __forceinline__ void operator()(uint32_t) const {}
};

}  // namespace coll
