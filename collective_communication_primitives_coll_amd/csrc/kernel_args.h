// Kernel argument blocks and launcher declarations (host and device).
//
// Rank pointer arrays travel in the kernel-argument segment, so a launch
// needs no device-side descriptor and nothing is allocated per call.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace coll {

constexpr int kMaxRanks = 64;

enum DType : int { kF32 = 0, kBF16 = 1, kI32 = 2 };

// Summation order of a reduction.
enum Order : int {
  kOrdRing = 0,  // left fold over the rotated ring order x_{c+1}, ..., x_c
  kOrdRD = 1,    // balanced tree pairing ranks (0,1), (2,3), ... first (recursive doubling)
  kOrdHD = 2,    // balanced tree pairing ranks (k, k + p/2) first (halving-doubling)
  kOrdTree = 3,  // binary tree in heap order: node v = (x_v + subtree 2v+1) + subtree 2v+2
  kOrdDBT = 4    // double binary tree: chunks c < p/2 on the heap tree, the others on its mirror
};
// Reductions.  kAvg: the sum, then divided by the rank count; kPreMul:
// every operand times its rank's scale, then the sum.
enum Op : int { kSum = 0, kMin = 1, kMax = 2, kAvg = 3, kPreMul = 4 };

// Destination selection of the reduction kernels.
enum DstMode : int {
  kDstAll = 0,    // every rank r: dst[r] + segment offset      (AllReduce)
  kDstFixed = 1,  // dst[0] + segment offset                     (Reduce: root buffer)
  kDstOwner = 2   // dst[c] + 0 for segment c                    (ReduceScatter)
};

struct RankPtrs {
  const void* src[kMaxRanks];
  void* dst[kMaxRanks];
};

// Reduction geometry: segment c covers source elements
// [min(total, c*stride), min(total, (c+1)*stride)).
struct ReduceGeom {
  uint64_t stride;
  uint64_t total;
  int p;
  int dst_mode;
  int src_mis;  // common byte misalignment of the source bases, or -1
  int dst_mis;  // common byte misalignment of the destination bases, or -1
  int src_amis; // common source base address modulo kLineAlign (256), or -1
  float scale[kMaxRanks];  // kPreMul: scale of rank r's operand
  // Claim slot (a zeroed counter) for the claimed tail of reduce_kernel
  // (AllReduce, ReduceScatter), or null to deal out every tile in turn.
  unsigned long long* claim;
};

// Copy kinds.
enum CopyKind : int {
  kCopyAllGather = 0,  // segment s: src[s] -> dst[r] + s*n, every r
  kCopyBroadcast = 1,  // one segment: src[0] -> dst[r], every r
  kCopyAllToAll = 2,   // segment (i,j): src[i] + j*n -> dst[j] + i*n
  kCopyGather = 3,     // segment s: src[s] -> dst[0] + s*n (root buffer)
  kCopyScatter = 4     // segment r: src[0] + r*n -> dst[r]
};

struct CopyGeom {
  uint64_t n;  // elements per segment
  int p;
  int kind;
  int src_mis;
  int dst_mis;
  // Claim slot for the claimed tails of fanout_kernel (AllGather,
  // Broadcast) and pair_copy_flat_kernel (All-to-All, Gather, Scatter), or
  // null to deal out every tile in turn.
  unsigned long long* claim;
  // Fan-outs: the destinations' common address modulo kLineAlign, or -1
  // (vector tiles then start on their 16-byte alignment only).
  int dst_amis = -1;
};

struct A2avArgs {
  const int64_t* counts;         // device, p*p, row = source (column = source if transposed)
  int32_t* status;               // device, optional
  int64_t send_cap[kMaxRanks];   // elements
  int64_t recv_cap[kMaxRanks];
  int p;
  int src_mis;
  int dst_mis;
  int transposed;                // elements from i to j are counts[j*p + i]
  unsigned long long* claim;     // claim slot (pooled claims of the flat kernel), or null
};

// MoE dispatch pack and combine.
constexpr int kMaxTopK = 8;

struct MoeIndexArgs {
  const int32_t* dest[kMaxRanks];  // per rank: destination rank of each assignment
  int32_t* pos[kMaxRanks];         // per rank: packed row of each assignment, at pos[x << pos_shift]
  int64_t* counts;                 // [p][p]: rows * hidden
  int64_t* counts2;                // optional [p][p]: rows * hidden2
  int32_t* status;                 // optional
  uint64_t assignments;            // T * k per rank
  uint64_t hidden;
  uint64_t hidden2;
  int p;
  int pos_shift;                   // 1: pos goes to the low words of an int64 array
};

struct MoeRowArgs {
  const void* src[kMaxRanks];      // pack: tokens; combine: returned rows
  void* dst[kMaxRanks];            // pack: packed rows; combine: output tokens
  const int32_t* pos[kMaxRanks];
  const float* weights[kMaxRanks];  // combine only
  const void* residual[kMaxRanks];  // combine only, optional
  uint64_t tokens;                 // T per rank
  uint64_t hidden;
  int k;
  int p;
  int has_residual;
  int src_mis;                     // common misalignment of the src bases, or -1
  int dst_mis;
  int res_mis;
  int32_t cap[kMaxRanks];          // direct combine: rows each src[j] holds
  unsigned long long* claim;       // pack: claim slot (pooled row claims), or null
};

// Direct dispatch: token rows written straight into the destinations'
// receive buffers.  loc[i][a] holds the packed row (low word, from the
// index pass) on entry and (dest << 32) | row inside recv[dest] on exit,
// or -1 for an assignment that is not delivered.
struct MoeDirectArgs {
  const void* src[kMaxRanks];      // tokens
  void* dst[kMaxRanks];            // receive buffers
  int64_t* loc[kMaxRanks];
  const int32_t* dest[kMaxRanks];
  int64_t cap[kMaxRanks];          // rows each receive buffer holds
  const int64_t* counts;           // [p][p]: rows * count_unit
  int32_t* status;                 // optional [p + 1]; entry p: 1 if a receive buffer is too small
  uint64_t tokens;                 // T per rank
  uint64_t hidden;                 // elements per token
  uint64_t count_unit;             // counts per row
  uint64_t group;                  // FP8 only
  uint64_t row_bytes;              // FP8 only
  int k;
  int p;
  int src_mis;
  int dst_mis;
  unsigned long long* claim;       // bf16 dispatch: claim slot (pooled row claims), or null
};

// Quantized dispatch: FP8 e4m3 rows with one fp32 scale per group of
// `group` elements.  Row layout: hidden code bytes, hidden/group scales,
// zero bytes up to row_bytes (a multiple of 16).
constexpr uint64_t kFp8MaxHidden = 16384;  // row-wide groups: 16 units of 16 elements per lane
struct Fp8Args {
  const void* src[kMaxRanks];      // pack: bf16 tokens; dequant: received rows
  void* dst[kMaxRanks];            // pack: packed rows; dequant: bf16 rows
  const int32_t* pos[kMaxRanks];   // pack: packed row of each assignment
  int64_t rows_cap[kMaxRanks];     // dequant: rows each output holds
  const int64_t* counts;           // dequant: [p][p] bytes, row = source
  int32_t* status;                 // dequant: optional
  uint64_t tokens;                 // pack: T per rank
  uint64_t hidden;
  uint64_t group;
  uint64_t row_bytes;
  int k;
  int p;
};

// Literal ring: one neighbour step per launch.
struct RingStepGeom {
  uint64_t n;
  uint64_t q;    // chunk length ceil(n/p)
  int p;
  int phase;     // 0 reduce-scatter, 1 all-gather
  int step;      // 1..p-1 (kAvg divides by p in the last reduce-scatter step)
  int mis;       // common misalignment of all send and recv bases, or -1
};

// Batched AllReduce descriptors (device resident).
struct BatchCall {
  uint64_t n;
  uint64_t first_tile;   // flat index of the call's first tile
  uint32_t dtype;
  uint32_t op;
  uint32_t tiles_per_chunk;
  // -1: the buffers disagree modulo 16 (element path); 0..255: every
  // source base's address modulo 256 (destinations agree modulo 16);
  // 256 + m: only a common misalignment m modulo 16.
  int32_t mis;
};

struct BatchArgs {
  const BatchCall* calls;   // ncalls + 1 entries; the last holds the total tile count
  const void* const* ptrs;  // per call: p sources then p destinations
  unsigned long long* next_run;  // zero at launch; waves claim runs of tiles from it
  int ncalls;
  int p;
};

// Launchers (return a hipError_t as int).
// max_grid bounds the number of workgroups; launchers shrink it to the
// number of tiles.  launch_alltoallv and launch_batch take the grid as is.
int launch_reduce(int dtype, int op, int order, const RankPtrs& ptrs, const ReduceGeom& g,
                  int max_grid, void* stream);
// fanout_grid (> 0): the grid bound for AllGather and Broadcast calls at
// p = 8 or 16 that walk their segments (their claimed tails balance best
// at one workgroup per CU); 0: max_grid.
int launch_copy(int elem_bytes, const RankPtrs& ptrs, const CopyGeom& g, int max_grid, void* stream,
                int fanout_grid = 0);
int launch_alltoallv(int elem_bytes, const RankPtrs& ptrs, const A2avArgs& a, int grid, void* stream);
// All-to-All staged through LDS; only for layouts where every block shares
// one 16-byte misalignment (can_stage_alltoall).
bool can_stage_alltoall(int elem_bytes, const CopyGeom& g);
int launch_alltoall_lds(int elem_bytes, const RankPtrs& ptrs, const CopyGeom& g, int max_grid, void* stream);
int launch_ring_step(int dtype, int op, const RankPtrs& ptrs, const RingStepGeom& g, int max_grid,
                     void* stream);
int launch_batch(const BatchArgs& a, int grid, void* stream);

// Elements of one batch tile for a dtype and rank count (the host cuts
// each call's chunks into tiles of this size).
uint64_t batch_tile_elems_host(int dtype, int p);

// The batch descriptor table of the entry point that allocates nothing: a
// static device array of kNoAllocScratchBytes per GPU.  noalloc_scratch
// returns its address on device `dev` (which must be current), looked up
// once per device.
constexpr size_t kNoAllocScratchBytes = size_t{4} << 20;
int noalloc_scratch(int dev, void** out);

// Claim slots (claim_slots.hip): kClaimSlots slots in a static device
// array per GPU, each of kClaimPools counters kClaimPoolWords 64-bit words
// apart (one 128-byte line each).  claim_slots_base gives device dev's
// array (dev current).  Launches with at least kClaimMinTilesPerWg tiles
// per workgroup use their slot: the uniform 1:1 copies, Alltoallv, the MoE
// token copies, AllGather and Broadcast at p >= 8 and AllReduce at p = 8
// all kClaimPools counters of it, the other reductions the first.
constexpr int kClaimSlots = 1024;
constexpr int kClaimPools = 8;
constexpr int kClaimPoolWords = 16;
constexpr int kClaimSlotWords = kClaimPools * kClaimPoolWords;
constexpr uint64_t kClaimMinTilesPerWg = 8;
int claim_slots_base(int dev, unsigned long long** out);

// MoE: the index pass (one workgroup per rank), the payload pack and the
// weighted combine.
int launch_moe_index(const MoeIndexArgs& a, void* stream);
int launch_moe_pack(int elem_bytes, const MoeRowArgs& a, int max_grid, void* stream);
int launch_moe_combine(int dtype, const MoeRowArgs& a, int max_grid, void* stream);

// FP8 dispatch: quantizing pack (after launch_moe_index with counts in
// bytes) and the bf16 dequantization of received rows.
int launch_moe_pack_fp8(const Fp8Args& a, int max_grid, void* stream);
int launch_moe_dequant_fp8(const Fp8Args& a, int max_grid, void* stream);

// Direct dispatch (after launch_moe_index with pos_shift 1) and the
// combine reading expert outputs through the locations.
int launch_moe_dispatch(int elem_bytes, const MoeDirectArgs& a, int max_grid, void* stream);
int launch_moe_dispatch_fp8(const MoeDirectArgs& a, int max_grid, void* stream);
int launch_moe_combine_direct(int dtype, const MoeRowArgs& a, int max_grid, void* stream);

// Direction-mix bandwidth probe: ns source and nd destination streams of
// nvec 16-byte vectors each, `unroll` vectors per lane per tile
// (probe_mix_supported and probe_unroll_supported list what is built).
bool probe_mix_supported(int ns, int nd);
bool probe_unroll_supported(int ns, int unroll);
// Store policies of 16-byte vector stores: plain, non-temporal, device
// scope, non-temporal of device scope (device_common.h describes each).
constexpr int kStPlain = 0, kStNT = 1, kStDevice = 2, kStNTDevice = 3;

// store_policy: one of the kSt* policies.
int launch_probe(int ns, int nd, const RankPtrs& ptrs, uint64_t nvec, int unroll, bool nt_loads, int store_policy,
                 void* sink, int max_grid, unsigned long long* claim, void* stream);

// 16-byte vectors each lane of a copy kernel keeps in flight.
constexpr uint64_t kCopyUnroll = 4;
// Eighths of a fan-out's tiles dealt out in turn when it claims the rest.
// AllGather at p = 8, 16 MiB bf16 shards, same-box A/B: 193-199 us all
// dealt out (two workgroups per CU); with claims, one workgroup per CU,
// 7/8 dealt ~190, 4/8 178-180, 2/8 175-176, 0/8 175-176 (at two per CU
// 2/8 gave 186-187 and 0/8 193-194).
constexpr uint64_t kCopyDealtEighths = 2;
// The uniform 1:1 copies (pair_copy_flat_kernel) deal out this many
// eighths of their tiles and claim the rest from kClaimPools counters.
constexpr uint32_t kPairDealtEighths = 4;
// The MoE token copies (pack, direct dispatch) deal out this many eighths
// of their rows to the waves in turn and claim the rest one row at a time
// from kClaimPools counters, given at least kClaimMinRowsPerWave rows per
// wave.
constexpr uint64_t kRowDealtEighths = 4;
constexpr uint64_t kClaimMinRowsPerWave = 4;

}  // namespace coll
