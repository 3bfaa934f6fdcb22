// MoE dispatch pack and weighted combine around the ragged exchange.
//
// "Collective Communication：AllReduce、AllGather、ReduceScatter 与
// All-to-All" lists the expert-parallel flow (Ragged All-to-All and Expert
// Parallel sections): router output -> count assignments per destination
// -> prefix-sum offsets -> pack/permute payload -> variable-split
// All-to-All -> expert compute -> reverse variable-split All-to-All ->
// unpermute and weighted combine.  The exchanges are the Alltoallv
// kernels; this file holds the steps either side of them.
//
// Index pass (one 1024-thread workgroup per source rank): every wave owns
// a contiguous run of the rank's assignments.  It counts destinations 64
// assignments at a time with ballots (one per destination for rank counts
// 2, 4, 8 and 16; otherwise one per distinct destination of the group,
// lane d counting destination d).  The per-wave counts are turned into
// exclusive offsets (by destination, then by wave); a second walk gives
// every assignment its packed row, stable in assignment order.
// Destinations outside [0, p) reject the rank: its counts are 0 and every
// pos is -1.
//
// Payload copy and combine: one wave per token row, rows spread over every
// wave of the grid, so a workgroup keeps four rows in flight.  The copy
// reads a token once and writes it to each of its k slots: rows of the
// rank's packed buffer (the pack) or rows of the destinations' receive
// buffers (the direct dispatch, which replaces pack + exchange).
#include "copy_tile.h"
#include "moe_direct.h"

namespace coll {

constexpr int kIdxThreads = 1024;
constexpr int kIdxWaves = kIdxThreads / 64;
constexpr int kIdxBatch = 8;  // groups of 64 assignments whose destinations a wave loads together

// PC: the rank count when it is 2, 4, 8 or 16 (0: any).  With a known,
// small rank count a group of 64 assignments is counted and placed with
// one compare-and-ballot per destination, the per-destination counts and
// running offsets in scalar registers.  Otherwise the wave elects one
// destination of the group at a time (a chain of dependent lane reads and
// ballots) and lane d keeps destination d's count.
template <int PC>
__global__ __launch_bounds__(kIdxThreads) void moe_index_kernel(MoeIndexArgs a) {
  __shared__ int wofs[kIdxWaves][kMaxRanks];  // per-wave counts, then offsets
  __shared__ int total[kMaxRanks];
  __shared__ int base[kMaxRanks];
  __shared__ int bad;
  const int rank = blockIdx.x;
  const int p = a.p;
  const uint64_t A = a.assignments;
  const int32_t* dest = as_global(a.dest[rank]);
  int32_t* pos = as_global(a.pos[rank]);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  if (tid == 0) bad = 0;
  __syncthreads();
  const uint64_t per = ((A + kIdxWaves - 1) / kIdxWaves + 63) / 64 * 64;
  uint64_t lo = (uint64_t)w * per, hi = lo + per;
  if (lo > A) lo = A;
  if (hi > A) hi = A;
  // pass 1: per-wave destination counts (kIdxBatch groups of 64 loaded
  // together).  p <= 64, so lane d keeps the wave's count for destination
  // d in a register.
  int cnt = 0;
  int cntd[PC > 0 ? PC : 1];
#pragma unroll
  for (int dd = 0; dd < (PC > 0 ? PC : 1); ++dd) cntd[dd] = 0;
  for (uint64_t b0 = lo; b0 < hi; b0 += 64 * kIdxBatch) {
    int dv[kIdxBatch];
#pragma unroll
    for (int i = 0; i < kIdxBatch; ++i) {
      const uint64_t x = b0 + (uint64_t)i * 64 + lane;
      dv[i] = x < hi ? dest[x] : -1;
    }
#pragma unroll
    for (int i = 0; i < kIdxBatch; ++i) {
      int d = dv[i];
      if (b0 + (uint64_t)i * 64 + lane < hi && (d < 0 || d >= p)) {
        bad = 1;
        d = -1;
      }
      if constexpr (PC > 0) {
#pragma unroll
        for (int dd = 0; dd < PC; ++dd) cntd[dd] += __popcll(__ballot(d == dd));
      } else {
        uint64_t rem = __ballot(d >= 0);
        while (rem) {
          const int leader = __ffsll((unsigned long long)rem) - 1;
          const int dl = __builtin_amdgcn_readlane(d, leader);
          const uint64_t m = __ballot(d == dl) & rem;
          if (lane == dl) cnt += __popcll(m);
          rem &= ~m;
        }
      }
    }
  }
  if constexpr (PC > 0) {
#pragma unroll
    for (int dd = 0; dd < PC; ++dd)
      if (lane == dd) cnt = cntd[dd];
  }
  if (lane < p) wofs[w][lane] = cnt;
  __syncthreads();
  if (tid < p) {
    int t = 0;
    for (int ww = 0; ww < kIdxWaves; ++ww) {
      const int c = wofs[ww][tid];
      wofs[ww][tid] = t;
      t += c;
    }
    total[tid] = t;
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int d = 0; d < p; ++d) {
      base[d] = s;
      s += total[d];
    }
  }
  __syncthreads();
  const bool reject = bad != 0;
  if (tid < p) {
    a.counts[(uint64_t)rank * p + tid] = reject ? 0 : (int64_t)total[tid] * (int64_t)a.hidden;
    if (a.counts2) a.counts2[(uint64_t)rank * p + tid] = reject ? 0 : (int64_t)total[tid] * (int64_t)a.hidden2;
    for (int ww = 0; ww < kIdxWaves; ++ww) wofs[ww][tid] += base[tid];
  }
  if (tid == 0 && a.status) a.status[rank] = reject ? 1 : 0;
  __syncthreads();
  if (reject) {
    for (uint64_t x = tid; x < A; x += kIdxThreads) pos[x << a.pos_shift] = -1;
    return;
  }
  // pass 2: packed row of every assignment; lane d (or, with a known rank
  // count, scalar register d) holds the wave's next row for destination d
  int next = lane < p ? wofs[w][lane] : 0;
  int nextd[PC > 0 ? PC : 1];
#pragma unroll
  for (int dd = 0; dd < (PC > 0 ? PC : 1); ++dd) nextd[dd] = PC > 0 ? wofs[w][dd] : 0;
  for (uint64_t b0 = lo; b0 < hi; b0 += 64 * kIdxBatch) {
    int dv[kIdxBatch];
#pragma unroll
    for (int i = 0; i < kIdxBatch; ++i) {
      const uint64_t x = b0 + (uint64_t)i * 64 + lane;
      dv[i] = x < hi ? dest[x] : -1;
    }
#pragma unroll
    for (int i = 0; i < kIdxBatch; ++i) {
      const uint64_t x = b0 + (uint64_t)i * 64 + lane;
      const int d = dv[i];
      int mine = 0;
      if constexpr (PC > 0) {
#pragma unroll
        for (int dd = 0; dd < PC; ++dd) {
          const uint64_t m = __ballot(d == dd);
          if (d == dd) mine = nextd[dd] + __popcll(m & below);
          nextd[dd] += __popcll(m);
        }
      } else {
        uint64_t rem = __ballot(d >= 0);
        while (rem) {
          const int leader = __ffsll((unsigned long long)rem) - 1;
          const int dl = __builtin_amdgcn_readlane(d, leader);
          const uint64_t m = __ballot(d == dl) & rem;
          const int at = __builtin_amdgcn_readlane(next, dl);
          if (d == dl) mine = at + __popcll(m & below);
          if (lane == dl) next += __popcll(m);
          rem &= ~m;
        }
      }
      if (d >= 0) pos[x << a.pos_shift] = mine;
    }
  }
}

constexpr int kWaveLanes = 64;
constexpr int kRowBatch = 16;  // 16-byte vectors per lane issued together in a row copy

// Global index of this wave (uniform across its lanes) and the wave count.
__device__ __forceinline__ uint64_t wave_id() {
  return (uint64_t)blockIdx.x * (kBlock / kWaveLanes) +
         (uint64_t)__builtin_amdgcn_readfirstlane(threadIdx.x / kWaveLanes);
}
__device__ __forceinline__ uint64_t wave_count() { return (uint64_t)gridDim.x * (kBlock / kWaveLanes); }

// Copy one row of len elements with one wave: every lane issues up to
// kRowBatch vector loads before its first store.
template <int B>
__device__ __forceinline__ void copy_row_wave(const typename Word<B>::T* src, typename Word<B>::T* dst,
                                              uint64_t len, int mis, int lane) {
  const SegSpan sp = seg_span<B>(len, mis);
  if (sp.vec && sp.nvec) {
    const u32x4* vs = reinterpret_cast<const u32x4*>(src + sp.head);
    u32x4* vd = reinterpret_cast<u32x4*>(dst + sp.head);
    for (uint64_t j0 = 0; j0 < sp.nvec; j0 += (uint64_t)kRowBatch * kWaveLanes) {
      u32x4 r[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const uint64_t j = j0 + (uint64_t)u * kWaveLanes + lane;
        if (j < sp.nvec) r[u] = ld16<false>(vs + j);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const uint64_t j = j0 + (uint64_t)u * kWaveLanes + lane;
        if (j < sp.nvec) st16<true>(vd + j, r[u]);
      }
    }
  }
  const uint64_t head = sp.vec ? sp.head : len;
  for (uint64_t e = lane; e < head; e += kWaveLanes) st1<true>(dst + e, ld1<false>(src + e));
  if (sp.vec) {
    const uint64_t t0 = sp.head + sp.nvec * (16 / B);
    for (uint64_t e = t0 + lane; e < len; e += kWaveLanes) st1<true>(dst + e, ld1<false>(src + e));
  }
}

// Where a token's slot rows go.  SlotRows<MoeRowArgs>: the rank's packed
// buffer at row pos (the pack).  SlotRows<MoeDirectArgs>: the destination's
// receive buffer at row roff[i][j] + ps - soff[i][j] (the direct dispatch,
// ps = the index pass's packed row, kept in the low word of the location),
// with loc[i][x] = (j << 32) | row written back once the token is done.
template <class Args> struct SlotRows;

template <> struct SlotRows<MoeRowArgs> {
  const MoeRowArgs& a;
  __device__ void* row(int rank, uint64_t x, uint64_t row_bytes, int64_t& loc, uint64_t& off) const {
    loc = -1;
    const int32_t ps = as_global(a.pos[rank])[x];
    if (ps < 0 || (uint64_t)ps >= a.tokens * (uint64_t)a.k) return nullptr;
    off = (uint64_t)ps * row_bytes;
    return as_global((uint8_t*)a.dst[rank]) + off;
  }
  __device__ void finish(int, uint64_t, const int64_t (&)[kMaxTopK], int) const {}
};

template <> struct SlotRows<MoeDirectArgs> {
  const MoeDirectArgs& a;
  const int32_t* soff;
  const int32_t* roff;
  bool reject;
  __device__ void* row(int rank, uint64_t x, uint64_t row_bytes, int64_t& loc, uint64_t& off) const {
    loc = -1;
    if (reject) return nullptr;
    // every lane reads the same words: keep them in scalar registers
    const int32_t ps = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(uint64_t)as_global(a.loc[rank])[x]);
    if (ps < 0 || (uint64_t)ps >= a.tokens * (uint64_t)a.k) return nullptr;
    const int j = __builtin_amdgcn_readfirstlane(as_global(a.dest[rank])[x]);
    if (j < 0 || j >= a.p) return nullptr;
    const int64_t rw = (int64_t)roff[rank * a.p + j] + (ps - soff[rank * a.p + j]);
    loc = direct_loc(j, rw);
    off = (uint64_t)rw * row_bytes;
    return as_global((uint8_t*)a.dst[j]) + off;
  }
  // after every read of the token's locations
  __device__ void finish(int rank, uint64_t x0, const int64_t (&loc)[kMaxTopK], int lane) const {
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
      if (s < a.k && lane == 0) as_global(a.loc[rank])[x0 + s] = loc[s];
  }
};

__device__ __forceinline__ SlotRows<MoeRowArgs> make_slot_rows(const MoeRowArgs& a, int32_t*, int*) {
  return SlotRows<MoeRowArgs>{a};
}
__device__ __forceinline__ SlotRows<MoeDirectArgs> make_slot_rows(const MoeDirectArgs& a, int32_t* tabs, int* flag) {
  const bool reject = direct_tables(a, tabs, tabs + a.p * a.p, flag);
  return SlotRows<MoeDirectArgs>{a, tabs, tabs + a.p * a.p, reject};
}

// Token rows copied to their k slots, one token per wave: the row is read
// once, kRowBatch 16-byte vectors per lane at a time, and each batch is
// stored to every slot.  Rows that are not all 16-byte aligned (row bytes
// not a multiple of 16, or a base off a 16-byte boundary) go slot by slot
// through copy_row_wave, which handles heads and tails.
// Stores: the pack's are non-temporal of device scope (4096 x 7168 bf16
// per rank, p = 8, top-2: 282-284 us against 290-293 us non-temporal, the
// exchange after it unchanged); the direct dispatch keeps non-temporal
// ones (290-292 us against 297-303 us with either device-scope policy).
// Rows: with a claim slot, kRowDealtEighths of them are dealt out to the
// waves in turn and the rest claimed one row at a time from kClaimPools
// pooled counters (the waves of workgroup b claim from pool claim_pool(b);
// claim c of pool x is row dealt + x + kClaimPools * c), at two workgroups per CU so
// that every wave is resident from the start.  Dealt out alone at two per
// CU, the waves of the pack above ended between 239 and 268 us.  Same-box
// A/B: pack 276-277 us against 284 us (eight workgroups per CU, dealt),
// direct dispatch 282-283 against 286 us.  The combines gained nothing
// from the same claims (328-330 us either way) and deal out every row.
template <int B, class Args>
COLL_STREAM_KERNEL void moe_token_copy_kernel(Args a) {
  using W = typename Word<B>::T;
  extern __shared__ int32_t tabs[];  // direct dispatch: placement tables
  __shared__ int flag;
  const SlotRows<Args> tgt = make_slot_rows(a, tabs, &flag);
  const int lane = (int)(threadIdx.x % kWaveLanes);
  const uint64_t H = a.hidden;
  const uint64_t RB = H * B;
  const bool aligned = RB % 16 == 0 && a.src_mis == 0 && a.dst_mis == 0;
  const uint64_t nvec = RB / 16;
  const uint64_t rows = a.tokens * (uint64_t)a.p;
  const uint64_t nw = wave_count(), w = wave_id();
  // claimed rows: `per` from each of kClaimPools pools, after `dealt` rows
  // dealt out in turn (see kRowDealtEighths)
  const uint32_t pool = claim_pool(blockIdx.x);
  const uint64_t per = a.claim && rows >= kClaimMinRowsPerWave * nw && gridDim.x >= (uint32_t)(kClaimPools * kClaimPools)
                           ? rows / 8 * (8 - kRowDealtEighths) / kClaimPools
                           : 0;
  const uint64_t dealt = rows - per * kClaimPools;
  unsigned long long* ctr = per ? a.claim + pool * kClaimPoolWords : nullptr;
  const unsigned long long first = per ? issue_claim(ctr, lane) : 0;
  // one row; after_loads(tok) runs once the row's first batch of loads has
  // returned (tok: an opaque zero produced after them), if there are loads
  auto copy_row = [&](uint64_t r, auto&& after_loads) {
    const int rank = (int)(r / a.tokens);
    const uint64_t t = r - (uint64_t)rank * a.tokens;
    void* drow[kMaxTopK];
    int64_t loc[kMaxTopK];
    uint64_t off[kMaxTopK];
    bool any = false;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
      drow[s] = nullptr;
      loc[s] = -1;
      off[s] = 0;
      if (s < a.k) {
        drow[s] = tgt.row(rank, t * (uint64_t)a.k + s, RB, loc[s], off[s]);
        any |= drow[s] != nullptr;
      }
    }
    if (any) {
      const W* src = as_global((const W*)a.src[rank]) + t * H;
      if (aligned) {
        const u32x4* vs = reinterpret_cast<const u32x4*>(src);
        for (uint64_t j0 = 0; j0 < nvec; j0 += (uint64_t)kRowBatch * kWaveLanes) {
          u32x4 v[kRowBatch];
#pragma unroll
          for (int u = 0; u < kRowBatch; ++u) {
            const uint64_t j = j0 + (uint64_t)u * kWaveLanes + lane;
            if (j < nvec) v[u] = ld16<true>(vs + j);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (j0 == 0) {
            uint32_t tok = 0;
            asm volatile("" : "+v"(tok) : "v"(v[0]));
            after_loads(tok);
          }
#pragma unroll
          for (int s = 0; s < kMaxTopK; ++s) {
            if (!drow[s]) continue;
            u32x4* vd = as_global(reinterpret_cast<u32x4*>(drow[s]));
            if constexpr (std::is_same<Args, MoeRowArgs>::value) {
              store_tile<kStNTDevice, kRowBatch, kWaveLanes, false>(vd, j0 + lane, nvec, v);
            } else {
#pragma unroll
              for (int u = 0; u < kRowBatch; ++u) {
                const uint64_t j = j0 + (uint64_t)u * kWaveLanes + lane;
                if (j < nvec) st16<true>(vd + j, v[u]);
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s) {
          if (!drow[s]) continue;
          const int mis = seg_mis(a.src_mis, a.dst_mis, t * RB, off[s]);
          copy_row_wave<B>(src, as_global((W*)drow[s]), H, mis, lane);
        }
      }
    }
    tgt.finish(rank, t * (uint64_t)a.k, loc, lane);
  };
  for (uint64_t r = w; r < dealt; r += nw) copy_row(r, [](uint32_t) {});
  if (!per) return;
  // the next claim is issued before a row's loads and read once they have
  // returned (or after the row, when it had none)
  uint64_t c = wave_value(first);
  while (c < per) {
    const unsigned long long next = issue_claim(ctr, lane);
    uint64_t cn = 0;
    bool got = false;
    copy_row(dealt + pool + (uint64_t)kClaimPools * c, [&](uint32_t tok) {
      cn = wave_value(next + tok);
      got = true;
    });
    if (!got) cn = wave_value(next);
    asm volatile("" ::"v"(next));  // keep the claim's register out of the stores' reach
    c = cn;
  }
  if (lane == 0) claim_last(ctr, c, per, (kBlock / kWaveLanes) * claim_pool_members(gridDim.x, pool));
}

// out[rank][t] = residual[rank][t] (or +0) + sum_s w[t*k+s] * back[rank][pos[t*k+s]],
// accumulated in fp32 in slot order with every product and sum rounded on
// its own; slots whose pos lies outside [0, T*k) are skipped.  One token
// row per wave, CombBatch<K> vectors per lane per step.
//
// A step issues all its loads (residual and every slot) before its stores,
// and gfx9 counts loads and stores on one counter, so each step's load
// wait also drains the previous step's stores: fewer, larger steps cost
// fewer round trips.  With one or two slots a step covers a whole bf16
// row of 7168 (14 vectors per lane, 194 VGPRs, no spills): 355 us against
// 365 us with 4-vector steps for 4096 tokens x 7168, p = 8, top-2.  More
// slots keep 4-vector steps to stay within the register budget.
template <int K>
struct CombBatch {
  static constexpr int value = K <= 2 ? 14 : 4;
};

// DIRECT: pos[rank] is an int64 location array from the direct dispatch;
// slot s reads row (loc & 0xffffffff) of src[loc >> 32] (skipped when the
// location is -1 or outside the rank count or the row capacity cap[j]).
// Vector stores are non-temporal of device scope.  Same-box A/B, 4096 x
// 7168 bf16 per rank, p = 8, top-2, timed as a stage of the whole path
// (pack, exchange, reverse exchange, combine): combine 332-333 us against
// 339 us with device-scope stores and 355 us with plain ones (path 1256-1259
// against 1270 and 1294-1296 us); DIRECT 330-333 us against 339-343 and
// 354 us.  Device-scope stores alone had made the combine faster still
// when measured after a pack that stored the same way (304 us), but that
// pack then slowed the exchange after it by 26 us: dirty lines left in the
// Infinity Cache are written back during a later kernel.
// K: slots held in registers, the smallest power of two >= k.
template <int DT, bool DIRECT, int K>
COLL_STREAM_KERNEL void moe_combine_kernel(MoeRowArgs a) {
#pragma clang fp contract(off)
  using T = Traits<DT>;
  using S = typename T::S;
  using A = typename T::A;
  constexpr int V = T::V;
  const int lane = (int)(threadIdx.x % kWaveLanes);
  const uint64_t Aa = a.tokens * (uint64_t)a.k;
  const uint64_t rows = a.tokens * (uint64_t)a.p;
  const int k = a.k;
  const uint64_t H = a.hidden;
  for (uint64_t r = wave_id(); r < rows; r += wave_count()) {
    const int rank = (int)(r / a.tokens);
    const uint64_t t = r - (uint64_t)rank * a.tokens;
    const S* yrow[K];
    float wt[K];
    bool ok[K];
    int mis = a.dst_mis < 0 ? -1 : (int)((a.dst_mis + t * H * T::B) & 15);
    if (a.has_residual) mis = seg_mis(mis, a.res_mis, 0, t * H * T::B);
#pragma unroll
    for (int s = 0; s < K; ++s) {
      ok[s] = false;
      wt[s] = 0.0f;
      yrow[s] = nullptr;
      if (s < k) {
        int j = rank;
        int64_t row;
        if constexpr (DIRECT) {
          // the same location in every lane: read it into scalar registers
          const uint64_t lw = as_global(reinterpret_cast<const uint64_t*>(a.pos[rank]))[t * k + s];
          const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)lw);
          const int32_t hi = __builtin_amdgcn_readfirstlane((int32_t)(lw >> 32));
          j = hi;
          row = lo;
          ok[s] = hi >= 0 && hi < a.p && row < a.cap[hi];
        } else {
          row = as_global(a.pos[rank])[t * k + s];
          ok[s] = row >= 0 && (uint64_t)row < Aa;
        }
        if (ok[s]) {
          wt[s] = as_global(a.weights[rank])[t * k + s];
          yrow[s] = as_global((const S*)a.src[j]) + (uint64_t)row * H;
          mis = seg_mis(mis, a.src_mis, 0, (uint64_t)row * H * T::B);
        }
      }
    }
    const S* res = a.has_residual ? as_global((const S*)a.residual[rank]) + t * H : nullptr;
    S* out = as_global((S*)a.dst[rank]) + t * H;
    auto elems = [&](uint64_t from, uint64_t cnt) {
      for (uint64_t e = from + lane; e < from + cnt; e += kWaveLanes) {
        A acc = res ? widen1<DT>(ld1<true>(res + e)) : A(0.0f);
#pragma unroll
        for (int s = 0; s < K; ++s)
          if (ok[s]) {
            const A prod = wt[s] * widen1<DT>(ld1<true>(yrow[s] + e));
            acc = acc + prod;
          }
        st1<false>(out + e, narrow1<DT>(acc));
      }
    };
    const SegSpan sp = seg_span<T::B>(H, mis);
    if (!sp.vec) {
      elems(0, H);
      continue;
    }
    constexpr int kCB = CombBatch<K>::value;
    for (uint64_t j0 = 0; j0 < sp.nvec; j0 += (uint64_t)kCB * kWaveLanes) {
      // every load of the batch (residual and all slots) before any arithmetic
      u32x4 rr[kCB];
      u32x4 y[K][kCB];
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
        const uint64_t j = j0 + (uint64_t)u * kWaveLanes + lane;
        rr[u] = u32x4{0, 0, 0, 0};
        if (res && j < sp.nvec) rr[u] = ld16<true>(res + sp.head + j * V);
      }
#pragma unroll
      for (int s = 0; s < K; ++s)
#pragma unroll
        for (int u = 0; u < kCB; ++u) {
          const uint64_t j = j0 + (uint64_t)u * kWaveLanes + lane;
          y[s][u] = u32x4{0, 0, 0, 0};
          if (ok[s] && j < sp.nvec) y[s][u] = ld16<true>(yrow[s] + sp.head + j * V);
        }
      const DeviceScopeStores<kCachePolicyNtSc1> st(
          (uint64_t)(out + sp.head) + j0 * 16, (uint32_t)kCB * kWaveLanes * 16);
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
        A acc[V];
        if (res) {
          widen<DT>(rr[u], acc);
        } else {
#pragma unroll
          for (int x = 0; x < V; ++x) acc[x] = 0.0f;
        }
#pragma unroll
        for (int s = 0; s < K; ++s) {
          if (!ok[s]) continue;
          A v[V];
          widen<DT>(y[s][u], v);
#pragma unroll
          for (int x = 0; x < V; ++x) {
            const A prod = wt[s] * v[x];
            acc[x] = acc[x] + prod;
          }
        }
        const uint64_t j = j0 + (uint64_t)u * kWaveLanes + lane;
        if (j < sp.nvec) st.put(((uint32_t)u * kWaveLanes + lane) * 16, narrow<DT>(acc));
      }
    }
    if (sp.head) elems(0, sp.head);
    if (sp.tail) elems(sp.head + sp.nvec * V, sp.tail);
  }
}

// ---------------------------------------------------------------------------
// Host-side launch
// ---------------------------------------------------------------------------
int launch_moe_index(const MoeIndexArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (a.p) {
    case 2: hipLaunchKernelGGL(moe_index_kernel<2>, dim3(a.p), dim3(kIdxThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL(moe_index_kernel<4>, dim3(a.p), dim3(kIdxThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL(moe_index_kernel<8>, dim3(a.p), dim3(kIdxThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL(moe_index_kernel<16>, dim3(a.p), dim3(kIdxThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(moe_index_kernel<0>, dim3(a.p), dim3(kIdxThreads), 0, s, a); break;
  }
  return (int)hipGetLastError();
}

template <class Args>
static int launch_token_copy(int elem_bytes, const Args& a, int max_grid, size_t shm, hipStream_t s) {
  const uint64_t rows = a.tokens * (uint64_t)a.p;
  if (!rows) return 0;
  const uint64_t wgs = (rows + (kBlock / kWaveLanes) - 1) / (kBlock / kWaveLanes);
  const int grid = (int)(wgs < (uint64_t)max_grid ? wgs : (uint64_t)max_grid);
  if (elem_bytes == 1)
    hipLaunchKernelGGL((moe_token_copy_kernel<1, Args>), dim3(grid), dim3(kBlock), shm, s, a);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL((moe_token_copy_kernel<2, Args>), dim3(grid), dim3(kBlock), shm, s, a);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL((moe_token_copy_kernel<4, Args>), dim3(grid), dim3(kBlock), shm, s, a);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_moe_pack(int elem_bytes, const MoeRowArgs& a, int max_grid, void* stream) {
  return launch_token_copy(elem_bytes, a, max_grid, 0, (hipStream_t)stream);
}

template <int DT, bool DIRECT>
static void launch_combine_k(const MoeRowArgs& a, int grid, hipStream_t s) {
  if (a.k <= 1) hipLaunchKernelGGL((moe_combine_kernel<DT, DIRECT, 1>), dim3(grid), dim3(kBlock), 0, s, a);
  else if (a.k <= 2) hipLaunchKernelGGL((moe_combine_kernel<DT, DIRECT, 2>), dim3(grid), dim3(kBlock), 0, s, a);
  else if (a.k <= 4) hipLaunchKernelGGL((moe_combine_kernel<DT, DIRECT, 4>), dim3(grid), dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL((moe_combine_kernel<DT, DIRECT, kMaxTopK>), dim3(grid), dim3(kBlock), 0, s, a);
}

template <bool DIRECT>
static int launch_combine(int dtype, const MoeRowArgs& a, int max_grid, hipStream_t s) {
  const uint64_t rows = a.tokens * (uint64_t)a.p;
  if (!rows) return 0;
  const int grid = (int)(rows < (uint64_t)max_grid ? rows : (uint64_t)max_grid);
  if (dtype == kF32) launch_combine_k<kF32, DIRECT>(a, grid, s);
  else if (dtype == kBF16) launch_combine_k<kBF16, DIRECT>(a, grid, s);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_moe_combine(int dtype, const MoeRowArgs& a, int max_grid, void* stream) {
  return launch_combine<false>(dtype, a, max_grid, (hipStream_t)stream);
}

int launch_moe_combine_direct(int dtype, const MoeRowArgs& a, int max_grid, void* stream) {
  return launch_combine<true>(dtype, a, max_grid, (hipStream_t)stream);
}

int launch_moe_dispatch(int elem_bytes, const MoeDirectArgs& a, int max_grid, void* stream) {
  return launch_token_copy(elem_bytes, a, max_grid, direct_tables_bytes(a.p), (hipStream_t)stream);
}

}  // namespace coll
