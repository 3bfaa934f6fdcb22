// Host side of the C ABI: argument validation, aliasing rules, grid sizing
// and dispatch to the kernel launchers.  Everything that can be checked on
// the host is checked before any HIP call, so an invalid call has no side
// effect on the device.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "coll.h"
#include "kernel_args.h"

#define COLL_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using coll::kMaxRanks;
static_assert(COLL_MAX_RANKS == coll::kMaxRanks, "rank limit mismatch");

thread_local int g_last_hip = 0;

coll_status_t hip_fail(int err) {
  g_last_hip = err;
  return COLL_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Device facts, cached per device.
// ---------------------------------------------------------------------------
struct DevInfo {
  std::atomic<int> cus{0};
  std::atomic<int> lds_per_block{0};
};
DevInfo g_dev[64];
std::atomic<int> g_wg_per_cu{0};

// Default workgroups (of 256 threads) per compute unit, per kernel family.
// Reductions keep 16-32 loads in flight per lane and run best with one
// workgroup per CU; copies with two.  Row kernels (MoE pack and combine)
// move one token row (a few KiB) per workgroup step and need more
// workgroups to keep enough bytes in flight; the FP8 pack and dequant,
// with a short conversion step between their loads and stores, gain a
// few percent more at sixteen.  The direct FP8 dispatch (quantizing
// straight into the receive buffers, placement tables staged per
// workgroup) measured best at two: 221 us against 237 us at sixteen for
// 4096 x 7168 tokens, p = 8, top-2.
// AllGather and Broadcast calls that walk their segments claim their last
// tiles dynamically and balance best at one workgroup per CU (kFamFanout).
// The bf16 MoE token copies, which claim rows, run two per CU
// (kFamRowClaim): all their workgroups are then resident at once (the row
// kernels hold at most two waves per SIMD), so the dealt rows start
// together.
enum Family {
  kFamReduce = 0,
  kFamCopy = 1,
  kFamRow = 2,
  kFamFp8 = 3,
  kFamFp8Direct = 4,
  kFamFanout = 5,
  kFamRowClaim = 6
};
constexpr int kDefaultWgPerCu[7] = {1, 2, 8, 16, 2, 1, 2};
// Largest accepted override (coll_set_grid_limit clamps to it).  A CU
// holds far fewer 256-thread workgroups at once, so larger values would
// only queue workgroups; the clamp also keeps CUs * limit within int.
constexpr int kMaxWgPerCu = 64;

int current_device(int* dev) { return (int)hipGetDevice(dev); }

// Claim slot of a stream on the current device.  Streams get slots in
// order of first use, one each, so that the launches that share a slot are
// ordered by their stream and each finds it zeroed by the one before.
// Null (every tile dealt out in turn) for the per-thread default stream,
// whose handle names a different stream in every thread, once all slots
// are taken, or on any error.
std::mutex g_claim_mu;
std::vector<std::pair<void*, int>> g_claim_map[64];

unsigned long long* stream_claim_slot(void* stream) {
  if ((hipStream_t)stream == hipStreamPerThread) return nullptr;
  int dev = 0;
  if (current_device(&dev) || dev < 0 || dev >= 64) return nullptr;
  unsigned long long* base = nullptr;
  if (coll::claim_slots_base(dev, &base)) return nullptr;
  std::lock_guard<std::mutex> lock(g_claim_mu);
  std::vector<std::pair<void*, int>>& m = g_claim_map[dev];
  int idx = -1;
  for (const auto& e : m)
    if (e.first == stream) {
      idx = e.second;
      break;
    }
  if (idx < 0) {
    if ((int)m.size() >= coll::kClaimSlots) return nullptr;
    idx = (int)m.size();
    m.emplace_back(stream, idx);
  }
  return base + (size_t)idx * coll::kClaimSlotWords;
}

int device_cus(int dev, int* out) {
  if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
  int c = g_dev[dev].cus.load(std::memory_order_relaxed);
  if (!c) {
    hipError_t e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    int l = 0;
    e = hipDeviceGetAttribute(&l, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return (int)e;
    g_dev[dev].lds_per_block.store(l, std::memory_order_relaxed);
    g_dev[dev].cus.store(c, std::memory_order_relaxed);
  }
  *out = c;
  return 0;
}

// Grid limit: workgroups per CU times CUs of the current device.
int max_grid(int* out, Family fam) {
  int dev = 0, cus = 0;
  int e = current_device(&dev);
  if (e) return e;
  e = device_cus(dev, &cus);
  if (e) return e;
  int w = g_wg_per_cu.load(std::memory_order_relaxed);
  if (w <= 0) w = kDefaultWgPerCu[fam];
  const int64_t g = (int64_t)cus * w;  // w <= kMaxWgPerCu: no overflow
  if (g <= 0) return (int)hipErrorInvalidConfiguration;
  *out = (int)g;
  return 0;
}

// ---------------------------------------------------------------------------
// Argument checks
// ---------------------------------------------------------------------------
// Types with arithmetic (reductions, combine) and all types (data movement).
bool arith_dtype_ok(int d) { return d == COLL_F32 || d == COLL_BF16 || d == COLL_I32; }
bool dtype_ok(int d) { return arith_dtype_ok(d) || d == COLL_U8; }
bool op_ok(int o) { return o == COLL_SUM || o == COLL_MIN || o == COLL_MAX || o == COLL_AVG; }
size_t dsize(int d) { return d == COLL_BF16 ? 2 : d == COLL_U8 ? 1 : 4; }

// bytes = a * b * c without overflow, and below 2^62 so that every derived
// offset stays representable.
bool mul_ok(size_t a, size_t b, size_t c, size_t* out) {
  size_t t;
  if (__builtin_mul_overflow(a, b, &t)) return false;
  if (__builtin_mul_overflow(t, c, &t)) return false;
  if (t >= (size_t{1} << 62)) return false;
  *out = t;
  return true;
}

template <typename PtrT>
bool all_non_null(PtrT const* arr, int p) {
  if (!arr) return false;
  for (int r = 0; r < p; ++r)
    if (!arr[r]) return false;
  return true;
}

// Every pointer aligned to the element size (the vector path relies on it).
template <typename PtrT>
bool elem_aligned(PtrT const* arr, int p, size_t d) {
  for (int r = 0; r < p; ++r)
    if ((uintptr_t)arr[r] % d) return false;
  return true;
}
bool elem_aligned1(const void* ptr, size_t d) { return (uintptr_t)ptr % d == 0; }

// Common byte misalignment (address mod 16) of a set of pointers, or -1.
int common_mis(const void* const* arr, int p) {
  const int m = (int)((uintptr_t)arr[0] & 15);
  for (int r = 1; r < p; ++r)
    if ((int)((uintptr_t)arr[r] & 15) != m) return -1;
  return m;
}
int common_mis2(int a, int b) { return (a < 0 || b < 0 || a != b) ? -1 : a; }

// Common address modulo 256 of a set of pointers, or -1: the reductions
// start their vector tiles on 256-byte lines of the sources when known.
int common_amis(const void* const* arr, int p) {
  const int m = (int)((uintptr_t)arr[0] & 255);
  for (int r = 1; r < p; ++r)
    if ((int)((uintptr_t)arr[r] & 255) != m) return -1;
  return m;
}

// ---------------------------------------------------------------------------
// Aliasing.  Every buffer becomes a byte range tagged (input|output, rank).
// Outputs must not overlap anything, except pairs the operation allows
// (its in-place forms).  Inputs may overlap each other.
// ---------------------------------------------------------------------------
struct Range {
  uintptr_t b, e;
  bool out;
  int rank;
};

template <typename Allowed>
coll_status_t check_alias(const std::vector<Range>& rs, Allowed allowed) {
  const size_t m = rs.size();
  for (size_t i = 0; i < m; ++i) {
    if (!rs[i].out || rs[i].b == rs[i].e) continue;
    for (size_t j = 0; j < m; ++j) {
      if (i == j || rs[j].b == rs[j].e) continue;
      if (rs[j].out && j < i) continue;  // output pairs checked once
      const bool overlap = rs[i].b < rs[j].e && rs[j].b < rs[i].e;
      if (overlap && !allowed(rs[i], rs[j])) return COLL_ERR_ALIAS;
    }
  }
  return COLL_OK;
}

Range rng(const void* p, size_t bytes, bool out, int rank) {
  const uintptr_t b = (uintptr_t)p;
  return Range{b, b + bytes, out, rank};
}

coll::RankPtrs make_ptrs(const void* const* src, int ns, void* const* dst, int nd) {
  coll::RankPtrs P;
  std::memset(&P, 0, sizeof(P));
  for (int r = 0; r < ns; ++r) P.src[r] = src[r];
  for (int r = 0; r < nd; ++r) P.dst[r] = dst[r];
  return P;
}

coll_status_t finish(int err) { return err ? hip_fail(err) : COLL_OK; }

// Summation order of an AllReduce schedule (RING_LITERAL has its own kernels).
// Rank counts each schedule is built for: the ring at any count; recursive
// doubling and halving-doubling pair ranks by powers of two, so p in
// {2, 4, 8, 16}; the heap-ordered trees at any count from 2 to 16.
bool schedule_supported(coll_algo_t algo, int p) {
  switch (algo) {
    case COLL_ALGO_RING:
    case COLL_ALGO_RING_LITERAL: return true;
    case COLL_ALGO_TREE:
    case COLL_ALGO_DOUBLE_BINARY_TREE: return p >= 2 && p <= 16;
    default: return p == 2 || p == 4 || p == 8 || p == 16;
  }
}

int order_of(coll_algo_t algo) {
  switch (algo) {
    case COLL_ALGO_RECURSIVE_DOUBLING: return coll::kOrdRD;
    case COLL_ALGO_HALVING_DOUBLING: return coll::kOrdHD;
    case COLL_ALGO_TREE: return coll::kOrdTree;
    case COLL_ALGO_DOUBLE_BINARY_TREE: return coll::kOrdDBT;
    default: return coll::kOrdRing;
  }
}

// AllReduce validation shared by the single and the batched entry points.
coll_status_t check_allreduce(const void* const* send, void* const* recv, int p, size_t n, int dtype,
                              int op) {
  if (p < 1 || p > kMaxRanks || !arith_dtype_ok(dtype) || !op_ok(op)) return COLL_ERR_INVALID_ARG;
  if (n == 0) return COLL_OK;
  size_t bytes;
  if (!mul_ok(n, dsize(dtype), (size_t)p, &bytes)) return COLL_ERR_INVALID_ARG;
  if (!all_non_null(send, p) || !all_non_null(recv, p)) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned(send, p, dsize(dtype)) || !elem_aligned(recv, p, dsize(dtype))) return COLL_ERR_INVALID_ARG;
  const size_t nb = n * dsize(dtype);
  std::vector<Range> rs;
  rs.reserve(2 * p);
  for (int r = 0; r < p; ++r) rs.push_back(rng(send[r], nb, false, r));
  for (int r = 0; r < p; ++r) rs.push_back(rng(recv[r], nb, true, r));
  return check_alias(rs, [](const Range& o, const Range& x) {
    return !x.out && x.rank == o.rank && x.b == o.b;  // recv[r] == send[r]
  });
}

}  // namespace

// ===========================================================================
// Entry points
// ===========================================================================

COLL_EXPORT coll_status_t coll_allreduce_algo(const void* const* send, void* const* recv, int p, size_t n,
                                              coll_dtype_t dtype, coll_op_t op, coll_algo_t algo,
                                              void* stream) {
  if ((int)algo < COLL_ALGO_RING || (int)algo > COLL_ALGO_DOUBLE_BINARY_TREE) return COLL_ERR_INVALID_ARG;
  coll_status_t st = check_allreduce(send, recv, p, n, dtype, op);
  if (st != COLL_OK || n == 0) return st;
  if (!schedule_supported(algo, p)) return COLL_ERR_UNSUPPORTED;
  if (algo == COLL_ALGO_RING_LITERAL && dtype == COLL_BF16) return COLL_ERR_UNSUPPORTED;
  int grid;
  int e = max_grid(&grid, algo == COLL_ALGO_RING_LITERAL ? kFamCopy : kFamReduce);
  if (e) return hip_fail(e);
  const int smis = common_mis(send, p), dmis = common_mis((const void* const*)recv, p);
  if (algo == COLL_ALGO_RING_LITERAL) {
    if (p == 1) {
      if (send[0] == recv[0]) return COLL_OK;
      coll::RankPtrs P = make_ptrs(send, 1, recv, 1);
      coll::CopyGeom g{n, 1, coll::kCopyBroadcast, smis, dmis};
      return finish(coll::launch_copy((int)dsize(dtype), P, g, grid, stream));
    }
    coll::RankPtrs P = make_ptrs(send, p, recv, p);
    coll::RingStepGeom g{};
    g.n = n;
    g.q = (n + p - 1) / p;
    g.p = p;
    g.mis = common_mis2(smis, dmis);
    for (int phase = 0; phase < 2; ++phase)
      for (int s = 1; s < p; ++s) {
        g.phase = phase;
        g.step = s;
        e = coll::launch_ring_step(dtype, op, P, g, grid, stream);
        if (e) return hip_fail(e);
      }
    return COLL_OK;
  }
  coll::RankPtrs P = make_ptrs(send, p, recv, p);
  coll::ReduceGeom g{};
  g.stride = (n + p - 1) / p;
  g.total = n;
  g.p = p;
  g.dst_mode = coll::kDstAll;
  g.src_mis = smis;
  g.dst_mis = dmis;
  g.src_amis = common_amis(send, p);
  g.claim = stream_claim_slot(stream);
  const int order = order_of(algo);
  return finish(coll::launch_reduce(dtype, op, order, P, g, grid, stream));
}

COLL_EXPORT coll_status_t coll_allreduce(const void* const* send, void* const* recv, int p, size_t n,
                                         coll_dtype_t dtype, coll_op_t op, void* stream) {
  return coll_allreduce_algo(send, recv, p, n, dtype, op, COLL_ALGO_RING, stream);
}

COLL_EXPORT coll_status_t coll_allreduce_premul(const void* const* send, void* const* recv, int p, size_t n,
                                                coll_dtype_t dtype, const float* scale, coll_algo_t algo,
                                                void* stream) {
  if ((int)algo < COLL_ALGO_RING || (int)algo > COLL_ALGO_DOUBLE_BINARY_TREE) return COLL_ERR_INVALID_ARG;
  coll_status_t st = check_allreduce(send, recv, p, n, dtype, COLL_SUM);
  if (st != COLL_OK || n == 0) return st;
  if (!scale) return COLL_ERR_INVALID_ARG;
  if (dtype == COLL_I32 || algo == COLL_ALGO_RING_LITERAL) return COLL_ERR_UNSUPPORTED;
  if (!schedule_supported(algo, p)) return COLL_ERR_UNSUPPORTED;
  int grid;
  int e = max_grid(&grid, kFamReduce);
  if (e) return hip_fail(e);
  coll::RankPtrs P = make_ptrs(send, p, recv, p);
  coll::ReduceGeom g{};
  g.stride = (n + p - 1) / p;
  g.total = n;
  g.p = p;
  g.dst_mode = coll::kDstAll;
  g.src_mis = common_mis(send, p);
  g.dst_mis = common_mis((const void* const*)recv, p);
  g.src_amis = common_amis(send, p);
  g.claim = stream_claim_slot(stream);
  for (int r = 0; r < p; ++r) g.scale[r] = scale[r];
  const int order = order_of(algo);
  return finish(coll::launch_reduce(dtype, coll::kPreMul, order, P, g, grid, stream));
}

COLL_EXPORT coll_status_t coll_reduce(const void* const* send, void* recv_root, int p, size_t n,
                                      coll_dtype_t dtype, coll_op_t op, int root, void* stream) {
  if (p < 1 || p > kMaxRanks || !arith_dtype_ok(dtype) || !op_ok(op) || root < 0 || root >= p)
    return COLL_ERR_INVALID_ARG;
  if (n == 0) return COLL_OK;
  size_t bytes;
  if (!mul_ok(n, dsize(dtype), (size_t)p, &bytes)) return COLL_ERR_INVALID_ARG;
  if (!all_non_null(send, p) || !recv_root) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned(send, p, dsize(dtype)) || !elem_aligned1(recv_root, dsize(dtype))) return COLL_ERR_INVALID_ARG;
  const size_t nb = n * dsize(dtype);
  std::vector<Range> rs;
  for (int r = 0; r < p; ++r) rs.push_back(rng(send[r], nb, false, r));
  rs.push_back(rng(recv_root, nb, true, root));
  coll_status_t st = check_alias(rs, [](const Range& o, const Range& x) {
    return !x.out && x.rank == o.rank && x.b == o.b;  // recv_root == send[root]
  });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamReduce);
  if (e) return hip_fail(e);
  void* dst[1] = {recv_root};
  coll::RankPtrs P = make_ptrs(send, p, dst, 1);
  coll::ReduceGeom g{};
  g.stride = (n + p - 1) / p;
  g.total = n;
  g.p = p;
  g.dst_mode = coll::kDstFixed;
  g.src_mis = common_mis(send, p);
  g.dst_mis = (int)((uintptr_t)recv_root & 15);
  g.src_amis = common_amis(send, p);
  g.claim = stream_claim_slot(stream);
  return finish(coll::launch_reduce(dtype, op, coll::kOrdRing, P, g, grid, stream));
}

COLL_EXPORT coll_status_t coll_broadcast(const void* send_root, void* const* recv, int p, size_t n,
                                         coll_dtype_t dtype, int root, void* stream) {
  if (p < 1 || p > kMaxRanks || !dtype_ok(dtype) || root < 0 || root >= p) return COLL_ERR_INVALID_ARG;
  if (n == 0) return COLL_OK;
  size_t bytes;
  if (!mul_ok(n, dsize(dtype), (size_t)p, &bytes)) return COLL_ERR_INVALID_ARG;
  if (!send_root || !all_non_null(recv, p)) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned1(send_root, dsize(dtype)) || !elem_aligned(recv, p, dsize(dtype))) return COLL_ERR_INVALID_ARG;
  const size_t nb = n * dsize(dtype);
  std::vector<Range> rs;
  rs.push_back(rng(send_root, nb, false, root));
  for (int r = 0; r < p; ++r) rs.push_back(rng(recv[r], nb, true, r));
  coll_status_t st = check_alias(rs, [](const Range& o, const Range& x) {
    return !x.out && x.rank == o.rank && x.b == o.b;  // recv[root] == send_root
  });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamCopy);
  if (e) return hip_fail(e);
  const void* src[1] = {send_root};
  coll::RankPtrs P = make_ptrs(src, 1, recv, p);
  coll::CopyGeom g{n, p, coll::kCopyBroadcast, (int)((uintptr_t)send_root & 15),
                   common_mis((const void* const*)recv, p), nullptr};
  g.claim = stream_claim_slot(stream);
  g.dst_amis = common_amis((const void* const*)recv, p);
  int fgrid;
  e = max_grid(&fgrid, kFamFanout);
  if (e) return hip_fail(e);
  return finish(coll::launch_copy((int)dsize(dtype), P, g, grid, stream, fgrid));
}

namespace {
coll_status_t reduce_scatter_impl(const void* const* send, void* const* recv, int p, size_t n, coll_dtype_t dtype,
                                  int op, const float* scale, void* stream) {
  if (p < 1 || p > kMaxRanks || !arith_dtype_ok(dtype) || !(op_ok(op) || op == coll::kPreMul)) return COLL_ERR_INVALID_ARG;
  if (n == 0) return COLL_OK;
  size_t bytes;
  if (!mul_ok(n, dsize(dtype), (size_t)p * p, &bytes)) return COLL_ERR_INVALID_ARG;
  if (!all_non_null(send, p) || !all_non_null(recv, p)) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned(send, p, dsize(dtype)) || !elem_aligned(recv, p, dsize(dtype))) return COLL_ERR_INVALID_ARG;
  const size_t nb = n * dsize(dtype);
  std::vector<Range> rs;
  for (int r = 0; r < p; ++r) rs.push_back(rng(send[r], nb * p, false, r));
  for (int r = 0; r < p; ++r) rs.push_back(rng(recv[r], nb, true, r));
  coll_status_t st = check_alias(rs, [nb](const Range& o, const Range& x) {
    // recv[r] == send[r] + r*n elements (the rank's own output block)
    return !x.out && x.rank == o.rank && o.b == x.b + (uintptr_t)o.rank * nb;
  });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamReduce);
  if (e) return hip_fail(e);
  coll::RankPtrs P = make_ptrs(send, p, recv, p);
  coll::ReduceGeom g{};
  g.stride = n;
  g.total = n * (uint64_t)p;
  g.p = p;
  g.dst_mode = coll::kDstOwner;
  g.src_mis = common_mis(send, p);
  g.dst_mis = common_mis((const void* const*)recv, p);
  g.src_amis = common_amis(send, p);
  g.claim = stream_claim_slot(stream);
  if (scale)
    for (int r = 0; r < p; ++r) g.scale[r] = scale[r];
  return finish(coll::launch_reduce(dtype, op, coll::kOrdRing, P, g, grid, stream));
}
}  // namespace

COLL_EXPORT coll_status_t coll_reduce_scatter(const void* const* send, void* const* recv, int p, size_t n,
                                              coll_dtype_t dtype, coll_op_t op, void* stream) {
  if (!op_ok(op)) return COLL_ERR_INVALID_ARG;
  return reduce_scatter_impl(send, recv, p, n, dtype, op, nullptr, stream);
}

COLL_EXPORT coll_status_t coll_reduce_scatter_premul(const void* const* send, void* const* recv, int p,
                                                     size_t n, coll_dtype_t dtype, const float* scale,
                                                     void* stream) {
  if (p < 1 || p > kMaxRanks || !arith_dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (n == 0) return COLL_OK;
  if (!scale) return COLL_ERR_INVALID_ARG;
  if (dtype == COLL_I32) return COLL_ERR_UNSUPPORTED;
  return reduce_scatter_impl(send, recv, p, n, dtype, coll::kPreMul, scale, stream);
}

COLL_EXPORT coll_status_t coll_allgather(const void* const* send, void* const* recv, int p, size_t n,
                                         coll_dtype_t dtype, void* stream) {
  if (p < 1 || p > kMaxRanks || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (n == 0) return COLL_OK;
  size_t bytes;
  if (!mul_ok(n, dsize(dtype), (size_t)p * p, &bytes)) return COLL_ERR_INVALID_ARG;
  if (!all_non_null(send, p) || !all_non_null(recv, p)) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned(send, p, dsize(dtype)) || !elem_aligned(recv, p, dsize(dtype))) return COLL_ERR_INVALID_ARG;
  const size_t nb = n * dsize(dtype);
  std::vector<Range> rs;
  for (int r = 0; r < p; ++r) rs.push_back(rng(send[r], nb, false, r));
  for (int r = 0; r < p; ++r) rs.push_back(rng(recv[r], nb * p, true, r));
  coll_status_t st = check_alias(rs, [nb](const Range& o, const Range& x) {
    // send[r] == recv[r] + r*n elements (the rank's own block of the output)
    return !x.out && x.rank == o.rank && x.b == o.b + (uintptr_t)o.rank * nb;
  });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamCopy);
  if (e) return hip_fail(e);
  coll::RankPtrs P = make_ptrs(send, p, recv, p);
  coll::CopyGeom g{n, p, coll::kCopyAllGather, common_mis(send, p), common_mis((const void* const*)recv, p),
                   nullptr};
  g.claim = stream_claim_slot(stream);
  g.dst_amis = common_amis((const void* const*)recv, p);
  int fgrid;
  e = max_grid(&fgrid, kFamFanout);
  if (e) return hip_fail(e);
  return finish(coll::launch_copy((int)dsize(dtype), P, g, grid, stream, fgrid));
}

COLL_EXPORT coll_status_t coll_alltoall(const void* const* send, void* const* recv, int p, size_t n_block,
                                        coll_dtype_t dtype, void* stream) {
  return coll_alltoall_algo(send, recv, p, n_block, dtype, COLL_A2A_DIRECT, stream);
}

COLL_EXPORT coll_status_t coll_alltoall_algo(const void* const* send, void* const* recv, int p, size_t n_block,
                                             coll_dtype_t dtype, coll_a2a_algo_t algo, void* stream) {
  if (p < 1 || p > kMaxRanks || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (algo != COLL_A2A_DIRECT && algo != COLL_A2A_LDS_STAGED) return COLL_ERR_INVALID_ARG;
  if (n_block == 0) return COLL_OK;
  size_t bytes;
  if (!mul_ok(n_block, dsize(dtype), (size_t)p * p, &bytes)) return COLL_ERR_INVALID_ARG;
  if (!all_non_null(send, p) || !all_non_null(recv, p)) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned(send, p, dsize(dtype)) || !elem_aligned(recv, p, dsize(dtype))) return COLL_ERR_INVALID_ARG;
  const size_t nb = n_block * dsize(dtype) * p;
  std::vector<Range> rs;
  for (int r = 0; r < p; ++r) rs.push_back(rng(send[r], nb, false, r));
  for (int r = 0; r < p; ++r) rs.push_back(rng(recv[r], nb, true, r));
  coll_status_t st = check_alias(rs, [](const Range&, const Range&) { return false; });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamCopy);
  if (e) return hip_fail(e);
  coll::RankPtrs P = make_ptrs(send, p, recv, p);
  coll::CopyGeom g{n_block, p, coll::kCopyAllToAll, common_mis(send, p),
                   common_mis((const void* const*)recv, p)};
  g.claim = stream_claim_slot(stream);
  if (algo == COLL_A2A_LDS_STAGED && coll::can_stage_alltoall((int)dsize(dtype), g))
    return finish(coll::launch_alltoall_lds((int)dsize(dtype), P, g, grid, stream));
  return finish(coll::launch_copy((int)dsize(dtype), P, g, grid, stream));
}

COLL_EXPORT coll_status_t coll_gather(const void* const* send, void* recv_root, int p, size_t n,
                                      coll_dtype_t dtype, int root, void* stream) {
  if (p < 1 || p > kMaxRanks || !dtype_ok(dtype) || root < 0 || root >= p) return COLL_ERR_INVALID_ARG;
  if (n == 0) return COLL_OK;
  size_t bytes;
  if (!mul_ok(n, dsize(dtype), (size_t)p, &bytes)) return COLL_ERR_INVALID_ARG;
  if (!all_non_null(send, p) || !recv_root) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned(send, p, dsize(dtype)) || !elem_aligned1(recv_root, dsize(dtype))) return COLL_ERR_INVALID_ARG;
  const size_t nb = n * dsize(dtype);
  std::vector<Range> rs;
  for (int r = 0; r < p; ++r) rs.push_back(rng(send[r], nb, false, r));
  rs.push_back(rng(recv_root, nb * p, true, root));
  coll_status_t st = check_alias(rs, [nb](const Range& o, const Range& x) {
    // send[root] == recv_root + root*n elements (the root's own block)
    return !x.out && x.rank == o.rank && x.b == o.b + (uintptr_t)o.rank * nb;
  });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamCopy);
  if (e) return hip_fail(e);
  void* dst[1] = {recv_root};
  coll::RankPtrs P = make_ptrs(send, p, dst, 1);
  coll::CopyGeom g{n, p, coll::kCopyGather, common_mis(send, p), (int)((uintptr_t)recv_root & 15)};
  g.claim = stream_claim_slot(stream);
  return finish(coll::launch_copy((int)dsize(dtype), P, g, grid, stream));
}

COLL_EXPORT coll_status_t coll_scatter(const void* send_root, void* const* recv, int p, size_t n,
                                       coll_dtype_t dtype, int root, void* stream) {
  if (p < 1 || p > kMaxRanks || !dtype_ok(dtype) || root < 0 || root >= p) return COLL_ERR_INVALID_ARG;
  if (n == 0) return COLL_OK;
  size_t bytes;
  if (!mul_ok(n, dsize(dtype), (size_t)p, &bytes)) return COLL_ERR_INVALID_ARG;
  if (!send_root || !all_non_null(recv, p)) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned1(send_root, dsize(dtype)) || !elem_aligned(recv, p, dsize(dtype))) return COLL_ERR_INVALID_ARG;
  const size_t nb = n * dsize(dtype);
  std::vector<Range> rs;
  rs.push_back(rng(send_root, nb * p, false, root));
  for (int r = 0; r < p; ++r) rs.push_back(rng(recv[r], nb, true, r));
  coll_status_t st = check_alias(rs, [nb](const Range& o, const Range& x) {
    // recv[root] == send_root + root*n elements (the root's own block)
    return !x.out && x.rank == o.rank && o.b == x.b + (uintptr_t)o.rank * nb;
  });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamCopy);
  if (e) return hip_fail(e);
  const void* src[1] = {send_root};
  coll::RankPtrs P = make_ptrs(src, 1, recv, p);
  coll::CopyGeom g{n, p, coll::kCopyScatter, (int)((uintptr_t)send_root & 15),
                   common_mis((const void* const*)recv, p)};
  g.claim = stream_claim_slot(stream);
  return finish(coll::launch_copy((int)dsize(dtype), P, g, grid, stream));
}

namespace {
coll_status_t alltoallv_impl(const void* const* send, void* const* recv, int p, const int64_t* counts_dev,
                             const int64_t* send_cap, const int64_t* recv_cap, int32_t* status_dev,
                             coll_dtype_t dtype, int transposed, void* stream) {
  if (p < 1 || p > kMaxRanks || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (!counts_dev || !send_cap || !recv_cap) return COLL_ERR_INVALID_ARG;
  if (!all_non_null(send, p) || !all_non_null(recv, p)) return COLL_ERR_INVALID_ARG;
  const size_t d = dsize(dtype);
  if (!elem_aligned(send, p, d) || !elem_aligned(recv, p, d)) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned1(counts_dev, sizeof(int64_t)) || (status_dev && !elem_aligned1(status_dev, sizeof(int32_t))))
    return COLL_ERR_INVALID_ARG;
  std::vector<Range> rs;
  for (int r = 0; r < p; ++r) {
    size_t b;
    if (send_cap[r] < 0 || recv_cap[r] < 0) return COLL_ERR_INVALID_ARG;
    // p counts of at most a capacity each must sum without int64 overflow
    // on the device: cap * d * 64 < 2^62.
    if (!mul_ok((size_t)send_cap[r], d, kMaxRanks, &b) || !mul_ok((size_t)recv_cap[r], d, kMaxRanks, &b))
      return COLL_ERR_INVALID_ARG;
    rs.push_back(rng(send[r], (size_t)send_cap[r] * d, false, r));
    rs.push_back(rng(recv[r], (size_t)recv_cap[r] * d, true, r));
  }
  rs.push_back(rng(counts_dev, (size_t)p * p * sizeof(int64_t), false, -1));
  if (status_dev) rs.push_back(rng(status_dev, sizeof(int32_t), true, -1));
  coll_status_t st = check_alias(rs, [](const Range&, const Range&) { return false; });
  if (st != COLL_OK) return st;
  int dev = 0, cus = 0;
  int e = current_device(&dev);
  if (!e) e = device_cus(dev, &cus);
  if (e) return hip_fail(e);
  const size_t lds = (size_t)3 * p * p * sizeof(int64_t) + 64;
  if (lds > (size_t)g_dev[dev].lds_per_block.load()) return COLL_ERR_UNSUPPORTED;
  int grid;
  e = max_grid(&grid, kFamCopy);
  if (e) return hip_fail(e);
  coll::RankPtrs P = make_ptrs(send, p, recv, p);
  coll::A2avArgs a;
  std::memset(&a, 0, sizeof(a));
  a.counts = counts_dev;
  a.status = status_dev;
  for (int r = 0; r < p; ++r) {
    a.send_cap[r] = send_cap[r];
    a.recv_cap[r] = recv_cap[r];
  }
  a.p = p;
  a.src_mis = common_mis(send, p);
  a.dst_mis = common_mis((const void* const*)recv, p);
  a.transposed = transposed;
  a.claim = stream_claim_slot(stream);
  return finish(coll::launch_alltoallv((int)d, P, a, grid, stream));
}
}  // namespace

COLL_EXPORT coll_status_t coll_alltoallv(const void* const* send, void* const* recv, int p,
                                         const int64_t* counts_dev, const int64_t* send_cap,
                                         const int64_t* recv_cap, int32_t* status_dev, coll_dtype_t dtype,
                                         void* stream) {
  return alltoallv_impl(send, recv, p, counts_dev, send_cap, recv_cap, status_dev, dtype, 0, stream);
}

COLL_EXPORT coll_status_t coll_alltoallv_transposed(const void* const* send, void* const* recv, int p,
                                                    const int64_t* counts_dev, const int64_t* send_cap,
                                                    const int64_t* recv_cap, int32_t* status_dev,
                                                    coll_dtype_t dtype, void* stream) {
  return alltoallv_impl(send, recv, p, counts_dev, send_cap, recv_cap, status_dev, dtype, 1, stream);
}

// ---------------------------------------------------------------------------
// MoE dispatch pack and combine
// ---------------------------------------------------------------------------
COLL_EXPORT coll_status_t coll_moe_pack(const void* const* tokens, const int32_t* const* dest,
                                        void* const* packed, int32_t* const* pos, int64_t* counts_dev,
                                        int32_t* status_dev, int p, size_t tokens_per_rank, int k,
                                        size_t hidden, coll_dtype_t dtype, void* stream) {
  if (p < 1 || p > kMaxRanks || !dtype_ok(dtype) || k < 1 || k > coll::kMaxTopK || hidden == 0)
    return COLL_ERR_INVALID_ARG;
  if (!counts_dev || !elem_aligned1(counts_dev, sizeof(int64_t))) return COLL_ERR_INVALID_ARG;
  if (status_dev && !elem_aligned1(status_dev, sizeof(int32_t))) return COLL_ERR_INVALID_ARG;
  const size_t d = dsize(dtype);
  size_t A, rowbytes, tb, pb;
  if (!mul_ok(tokens_per_rank, (size_t)k, 1, &A) || A > 0x7fffffffull) return COLL_ERR_INVALID_ARG;
  if (!mul_ok(hidden, d, 1, &rowbytes) || !mul_ok(tokens_per_rank, rowbytes, 1, &tb) ||
      !mul_ok(A, rowbytes, (size_t)kMaxRanks, &pb))
    return COLL_ERR_INVALID_ARG;
  pb = A * rowbytes;
  std::vector<Range> rs;
  if (A > 0) {
    if (!all_non_null(tokens, p) || !all_non_null(dest, p) || !all_non_null(packed, p) || !all_non_null(pos, p))
      return COLL_ERR_INVALID_ARG;
    if (!elem_aligned(tokens, p, d) || !elem_aligned(packed, p, d) || !elem_aligned(dest, p, 4) ||
        !elem_aligned(pos, p, 4))
      return COLL_ERR_INVALID_ARG;
    for (int r = 0; r < p; ++r) {
      rs.push_back(rng(tokens[r], tb, false, r));
      rs.push_back(rng(dest[r], A * 4, false, r));
      rs.push_back(rng(packed[r], pb, true, r));
      rs.push_back(rng(pos[r], A * 4, true, r));
    }
  }
  rs.push_back(rng(counts_dev, (size_t)p * p * sizeof(int64_t), true, -1));
  if (status_dev) rs.push_back(rng(status_dev, (size_t)p * sizeof(int32_t), true, -1));
  coll_status_t st = check_alias(rs, [](const Range&, const Range&) { return false; });
  if (st != COLL_OK) return st;
  coll::MoeIndexArgs ia;
  std::memset(&ia, 0, sizeof(ia));
  for (int r = 0; r < p && A > 0; ++r) {
    ia.dest[r] = dest[r];
    ia.pos[r] = pos[r];
  }
  ia.counts = counts_dev;
  ia.status = status_dev;
  ia.assignments = A;
  ia.hidden = hidden;
  ia.p = p;
  int e = coll::launch_moe_index(ia, stream);
  if (e) return hip_fail(e);
  if (A == 0) return COLL_OK;
  int grid;
  e = max_grid(&grid, kFamRow);
  if (e) return hip_fail(e);
  coll::MoeRowArgs ra;
  std::memset(&ra, 0, sizeof(ra));
  for (int r = 0; r < p; ++r) {
    ra.src[r] = tokens[r];
    ra.dst[r] = packed[r];
    ra.pos[r] = pos[r];
  }
  ra.tokens = tokens_per_rank;
  ra.hidden = hidden;
  ra.k = k;
  ra.p = p;
  ra.src_mis = common_mis(tokens, p);
  ra.dst_mis = common_mis((const void* const*)packed, p);
  ra.claim = stream_claim_slot(stream);
  if (ra.claim) {
    e = max_grid(&grid, kFamRowClaim);
    if (e) return hip_fail(e);
  }
  return finish(coll::launch_moe_pack((int)d, ra, grid, stream));
}

// Range tag of residual buffers (kept apart from the back rows of the same rank).
constexpr int kResidualTag = 4 * kMaxRanks;

COLL_EXPORT coll_status_t coll_moe_combine(const void* const* back, const int32_t* const* pos,
                                           const float* const* weights, const void* const* residual,
                                           void* const* out, int p, size_t tokens_per_rank, int k,
                                           size_t hidden, coll_dtype_t dtype, void* stream) {
  if (p < 1 || p > kMaxRanks || !arith_dtype_ok(dtype) || k < 1 || k > coll::kMaxTopK || hidden == 0)
    return COLL_ERR_INVALID_ARG;
  if (dtype == COLL_I32) return COLL_ERR_UNSUPPORTED;
  const size_t d = dsize(dtype);
  size_t A, rowbytes, tb, pb;
  if (!mul_ok(tokens_per_rank, (size_t)k, 1, &A) || A > 0x7fffffffull) return COLL_ERR_INVALID_ARG;
  if (!mul_ok(hidden, d, 1, &rowbytes) || !mul_ok(tokens_per_rank, rowbytes, 1, &tb) ||
      !mul_ok(A, rowbytes, (size_t)kMaxRanks, &pb))
    return COLL_ERR_INVALID_ARG;
  pb = A * rowbytes;
  if (A == 0) return COLL_OK;
  if (!all_non_null(back, p) || !all_non_null(pos, p) || !all_non_null(weights, p) || !all_non_null(out, p))
    return COLL_ERR_INVALID_ARG;
  if (residual && !all_non_null(residual, p)) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned(back, p, d) || !elem_aligned(out, p, d) || !elem_aligned(pos, p, 4) ||
      !elem_aligned(weights, p, 4) || (residual && !elem_aligned(residual, p, d)))
    return COLL_ERR_INVALID_ARG;
  std::vector<Range> rs;
  for (int r = 0; r < p; ++r) {
    rs.push_back(rng(back[r], pb, false, r));
    rs.push_back(rng(pos[r], A * 4, false, r));
    rs.push_back(rng(weights[r], A * 4, false, r));
    if (residual) rs.push_back(rng(residual[r], tb, false, kResidualTag + r));
    rs.push_back(rng(out[r], tb, true, r));
  }
  coll_status_t st = check_alias(rs, [](const Range& o, const Range& x) {
    // in place: out[r] is exactly residual[r] (the residual add)
    return !x.out && x.rank == kResidualTag + o.rank && x.b == o.b && x.e == o.e;
  });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamRow);
  if (e) return hip_fail(e);
  coll::MoeRowArgs ra;
  std::memset(&ra, 0, sizeof(ra));
  for (int r = 0; r < p; ++r) {
    ra.src[r] = back[r];
    ra.dst[r] = out[r];
    ra.pos[r] = pos[r];
    ra.weights[r] = weights[r];
    if (residual) ra.residual[r] = residual[r];
  }
  ra.tokens = tokens_per_rank;
  ra.hidden = hidden;
  ra.k = k;
  ra.p = p;
  ra.has_residual = residual ? 1 : 0;
  ra.src_mis = common_mis(back, p);
  ra.dst_mis = common_mis((const void* const*)out, p);
  ra.res_mis = residual ? common_mis(residual, p) : 0;
  return finish(coll::launch_moe_combine(dtype, ra, grid, stream));
}

// ---------------------------------------------------------------------------
// FP8 e4m3 dispatch
// ---------------------------------------------------------------------------
namespace {
// 0: accepted; otherwise the status to return.
coll_status_t fp8_shape(size_t hidden, size_t group) {
  if (hidden == 0 || group == 0 || hidden % group) return COLL_ERR_INVALID_ARG;
  if (group < 16 || hidden >= (size_t{1} << 31)) return COLL_ERR_UNSUPPORTED;
  if (group <= 1024 ? (group & (group - 1)) != 0 : group % 1024 != 0) return COLL_ERR_UNSUPPORTED;
  // groups wider than 1024 elements keep the whole row in registers
  if (group > 1024 && hidden > coll::kFp8MaxHidden) return COLL_ERR_UNSUPPORTED;
  return COLL_OK;
}
size_t fp8_row_bytes(size_t hidden, size_t group) { return hidden + 16 * ((4 * (hidden / group) + 15) / 16); }
bool aligned16(const void* const* arr, int p) {
  for (int r = 0; r < p; ++r)
    if ((uintptr_t)arr[r] & 15) return false;
  return true;
}
}  // namespace

COLL_EXPORT size_t coll_moe_fp8_row_bytes(size_t hidden, size_t group) {
  return fp8_shape(hidden, group) == COLL_OK ? fp8_row_bytes(hidden, group) : 0;
}

COLL_EXPORT coll_status_t coll_moe_pack_fp8(const void* const* tokens, const int32_t* const* dest,
                                            void* const* packed, int32_t* const* pos, int64_t* counts_dev,
                                            int64_t* counts_hidden_dev, int32_t* status_dev, int p,
                                            size_t tokens_per_rank, int k, size_t hidden, size_t group,
                                            void* stream) {
  if (p < 1 || p > kMaxRanks || k < 1 || k > coll::kMaxTopK) return COLL_ERR_INVALID_ARG;
  coll_status_t st = fp8_shape(hidden, group);
  if (st != COLL_OK) return st;
  if (!counts_dev || !elem_aligned1(counts_dev, sizeof(int64_t))) return COLL_ERR_INVALID_ARG;
  if (counts_hidden_dev && !elem_aligned1(counts_hidden_dev, sizeof(int64_t))) return COLL_ERR_INVALID_ARG;
  if (status_dev && !elem_aligned1(status_dev, sizeof(int32_t))) return COLL_ERR_INVALID_ARG;
  const size_t R = fp8_row_bytes(hidden, group);
  size_t A, tb, pb;
  if (!mul_ok(tokens_per_rank, (size_t)k, 1, &A) || A > 0x7fffffffull) return COLL_ERR_INVALID_ARG;
  if (!mul_ok(tokens_per_rank, hidden * 2, 1, &tb) || !mul_ok(A, R, (size_t)kMaxRanks, &pb))
    return COLL_ERR_INVALID_ARG;
  pb = A * R;
  std::vector<Range> rs;
  if (A > 0) {
    if (!all_non_null(tokens, p) || !all_non_null(dest, p) || !all_non_null(packed, p) || !all_non_null(pos, p))
      return COLL_ERR_INVALID_ARG;
    if (!aligned16(tokens, p) || !aligned16((const void* const*)packed, p) || !elem_aligned(dest, p, 4) ||
        !elem_aligned(pos, p, 4))
      return COLL_ERR_INVALID_ARG;
    for (int r = 0; r < p; ++r) {
      rs.push_back(rng(tokens[r], tb, false, r));
      rs.push_back(rng(dest[r], A * 4, false, r));
      rs.push_back(rng(packed[r], pb, true, r));
      rs.push_back(rng(pos[r], A * 4, true, r));
    }
  }
  rs.push_back(rng(counts_dev, (size_t)p * p * sizeof(int64_t), true, -1));
  if (counts_hidden_dev) rs.push_back(rng(counts_hidden_dev, (size_t)p * p * sizeof(int64_t), true, -1));
  if (status_dev) rs.push_back(rng(status_dev, (size_t)p * sizeof(int32_t), true, -1));
  st = check_alias(rs, [](const Range&, const Range&) { return false; });
  if (st != COLL_OK) return st;
  coll::MoeIndexArgs ia;
  std::memset(&ia, 0, sizeof(ia));
  for (int r = 0; r < p && A > 0; ++r) {
    ia.dest[r] = dest[r];
    ia.pos[r] = pos[r];
  }
  ia.counts = counts_dev;
  ia.counts2 = counts_hidden_dev;
  ia.status = status_dev;
  ia.assignments = A;
  ia.hidden = R;  // counts in bytes
  ia.hidden2 = hidden;
  ia.p = p;
  int e = coll::launch_moe_index(ia, stream);
  if (e) return hip_fail(e);
  if (A == 0) return COLL_OK;
  int grid;
  e = max_grid(&grid, kFamFp8);
  if (e) return hip_fail(e);
  coll::Fp8Args fa;
  std::memset(&fa, 0, sizeof(fa));
  for (int r = 0; r < p; ++r) {
    fa.src[r] = tokens[r];
    fa.dst[r] = packed[r];
    fa.pos[r] = pos[r];
  }
  fa.tokens = tokens_per_rank;
  fa.hidden = hidden;
  fa.group = group;
  fa.row_bytes = R;
  fa.k = k;
  fa.p = p;
  return finish(coll::launch_moe_pack_fp8(fa, grid, stream));
}

COLL_EXPORT coll_status_t coll_moe_dequant_fp8(const void* const* recv, void* const* out, int p,
                                               const int64_t* counts_dev, const int64_t* rows_cap,
                                               int32_t* status_dev, size_t hidden, size_t group, void* stream) {
  if (p < 1 || p > kMaxRanks || !rows_cap) return COLL_ERR_INVALID_ARG;
  coll_status_t st = fp8_shape(hidden, group);
  if (st != COLL_OK) return st;
  if (!counts_dev || !elem_aligned1(counts_dev, sizeof(int64_t))) return COLL_ERR_INVALID_ARG;
  if (status_dev && !elem_aligned1(status_dev, sizeof(int32_t))) return COLL_ERR_INVALID_ARG;
  if (!all_non_null(recv, p) || !all_non_null(out, p)) return COLL_ERR_INVALID_ARG;
  if (!aligned16(recv, p) || !aligned16((const void* const*)out, p)) return COLL_ERR_INVALID_ARG;
  const size_t R = fp8_row_bytes(hidden, group);
  std::vector<Range> rs;
  for (int r = 0; r < p; ++r) {
    size_t b;
    if (rows_cap[r] < 0) return COLL_ERR_INVALID_ARG;
    // p counts of at most a capacity each must sum without int64 overflow
    // on the device
    if (!mul_ok((size_t)rows_cap[r], R, kMaxRanks, &b) || !mul_ok((size_t)rows_cap[r], hidden * 2, 1, &b))
      return COLL_ERR_INVALID_ARG;
    rs.push_back(rng(recv[r], (size_t)rows_cap[r] * R, false, r));
    rs.push_back(rng(out[r], (size_t)rows_cap[r] * hidden * 2, true, r));
  }
  rs.push_back(rng(counts_dev, (size_t)p * p * sizeof(int64_t), false, -1));
  if (status_dev) rs.push_back(rng(status_dev, sizeof(int32_t), true, -1));
  st = check_alias(rs, [](const Range&, const Range&) { return false; });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamFp8);
  if (e) return hip_fail(e);
  coll::Fp8Args fa;
  std::memset(&fa, 0, sizeof(fa));
  for (int r = 0; r < p; ++r) {
    fa.src[r] = recv[r];
    fa.dst[r] = out[r];
    fa.rows_cap[r] = rows_cap[r];
  }
  fa.counts = counts_dev;
  fa.status = status_dev;
  fa.hidden = hidden;
  fa.group = group;
  fa.row_bytes = R;
  fa.p = p;
  return finish(coll::launch_moe_dequant_fp8(fa, grid, stream));
}

// ---------------------------------------------------------------------------
// Direct MoE dispatch and combine
// ---------------------------------------------------------------------------
namespace {
// Dynamic LDS of the direct dispatch kernels: the row counts and the two
// placement tables, p x p int32 each.
size_t direct_lds_bytes(int p) { return (size_t)3 * p * p * sizeof(int32_t); }

// Shared validation of the direct dispatches.  elem: payload bytes per
// token element (tokens); row_bytes: bytes per delivered row (recv).
coll_status_t check_direct(const void* const* tokens, const int32_t* const* dest, void* const* recv,
                           int64_t* const* loc, int64_t* counts_dev, int64_t* counts2_dev, int32_t* status_dev,
                           int p, size_t T, int k, size_t hidden, const int64_t* recv_cap, size_t elem,
                           size_t row_bytes, size_t align, size_t* A_out) {
  if (p < 1 || p > kMaxRanks || k < 1 || k > coll::kMaxTopK || hidden == 0 || !recv_cap)
    return COLL_ERR_INVALID_ARG;
  if (!counts_dev || !elem_aligned1(counts_dev, sizeof(int64_t))) return COLL_ERR_INVALID_ARG;
  if (counts2_dev && !elem_aligned1(counts2_dev, sizeof(int64_t))) return COLL_ERR_INVALID_ARG;
  if (status_dev && !elem_aligned1(status_dev, sizeof(int32_t))) return COLL_ERR_INVALID_ARG;
  size_t A, tb, b;
  if (!mul_ok(T, (size_t)k, 1, &A) || A > 0x7fffffffull) return COLL_ERR_INVALID_ARG;
  if (!mul_ok(hidden, elem, 1, &b) || !mul_ok(T, hidden * elem, 1, &tb) || !mul_ok(A, row_bytes, kMaxRanks, &b))
    return COLL_ERR_INVALID_ARG;
  for (int r = 0; r < p; ++r)
    if (recv_cap[r] < 0 || recv_cap[r] > 0x7fffffffll || !mul_ok((size_t)recv_cap[r], row_bytes, kMaxRanks, &b))
      return COLL_ERR_INVALID_ARG;
  std::vector<Range> rs;
  if (A > 0) {
    if (!all_non_null(tokens, p) || !all_non_null(dest, p) || !all_non_null(recv, p) || !all_non_null(loc, p))
      return COLL_ERR_INVALID_ARG;
    if (!elem_aligned(tokens, p, align) || !elem_aligned(recv, p, align) || !elem_aligned(dest, p, 4) ||
        !elem_aligned(loc, p, 8))
      return COLL_ERR_INVALID_ARG;
    for (int r = 0; r < p; ++r) {
      rs.push_back(rng(tokens[r], tb, false, r));
      rs.push_back(rng(dest[r], A * 4, false, r));
      rs.push_back(rng(loc[r], A * 8, true, r));
      rs.push_back(rng(recv[r], (size_t)recv_cap[r] * row_bytes, true, r));
    }
  }
  rs.push_back(rng(counts_dev, (size_t)p * p * sizeof(int64_t), true, -1));
  if (counts2_dev) rs.push_back(rng(counts2_dev, (size_t)p * p * sizeof(int64_t), true, -1));
  if (status_dev) rs.push_back(rng(status_dev, (size_t)(p + 1) * sizeof(int32_t), true, -1));
  coll_status_t st = check_alias(rs, [](const Range&, const Range&) { return false; });
  if (st != COLL_OK) return st;
  *A_out = A;
  return COLL_OK;
}

// Index pass writing each assignment's packed row into the low word of its
// location (the dispatch kernels turn it into the location).
int launch_direct_index(const int32_t* const* dest, int64_t* const* loc, int64_t* counts, int64_t* counts2,
                        int32_t* status, int p, size_t A, size_t unit, size_t unit2, void* stream) {
  coll::MoeIndexArgs ia;
  std::memset(&ia, 0, sizeof(ia));
  for (int r = 0; r < p && A > 0; ++r) {
    ia.dest[r] = dest[r];
    ia.pos[r] = reinterpret_cast<int32_t*>(loc[r]);
  }
  ia.counts = counts;
  ia.counts2 = counts2;
  ia.status = status;
  ia.assignments = A;
  ia.hidden = unit;
  ia.hidden2 = unit2;
  ia.p = p;
  ia.pos_shift = 1;
  return coll::launch_moe_index(ia, stream);
}

coll::MoeDirectArgs direct_args(const void* const* tokens, const int32_t* const* dest, void* const* recv,
                                int64_t* const* loc, const int64_t* counts, int32_t* status, int p, size_t T,
                                int k, size_t hidden, const int64_t* recv_cap, size_t unit) {
  coll::MoeDirectArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int r = 0; r < p; ++r) {
    a.src[r] = tokens[r];
    a.dst[r] = recv[r];
    a.loc[r] = loc[r];
    a.dest[r] = dest[r];
    a.cap[r] = recv_cap[r];
  }
  a.counts = counts;
  a.status = status;
  a.tokens = T;
  a.hidden = hidden;
  a.count_unit = unit;
  a.k = k;
  a.p = p;
  a.src_mis = common_mis(tokens, p);
  a.dst_mis = common_mis((const void* const*)recv, p);
  return a;
}
}  // namespace

COLL_EXPORT coll_status_t coll_moe_dispatch(const void* const* tokens, const int32_t* const* dest,
                                            void* const* recv, int64_t* const* loc, int64_t* counts_dev,
                                            int32_t* status_dev, int p, size_t tokens_per_rank, int k,
                                            size_t hidden, const int64_t* recv_cap, coll_dtype_t dtype,
                                            void* stream) {
  if (!dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  const size_t d = dsize(dtype);
  size_t A = 0;
  coll_status_t st = check_direct(tokens, dest, recv, loc, counts_dev, nullptr, status_dev, p, tokens_per_rank, k,
                                  hidden, recv_cap, d, hidden * d, d, &A);
  if (st != COLL_OK) return st;
  int e = launch_direct_index(dest, loc, counts_dev, nullptr, status_dev, p, A, hidden, 0, stream);
  if (e) return hip_fail(e);
  if (A == 0) return COLL_OK;
  int dev = 0, cus = 0;
  e = current_device(&dev);
  if (!e) e = device_cus(dev, &cus);
  if (e) return hip_fail(e);
  if (direct_lds_bytes(p) > (size_t)g_dev[dev].lds_per_block.load()) return COLL_ERR_UNSUPPORTED;
  int grid;
  e = max_grid(&grid, kFamRow);
  if (e) return hip_fail(e);
  coll::MoeDirectArgs a =
      direct_args(tokens, dest, recv, loc, counts_dev, status_dev, p, tokens_per_rank, k, hidden, recv_cap, hidden);
  a.claim = stream_claim_slot(stream);
  if (a.claim) {
    e = max_grid(&grid, kFamRowClaim);
    if (e) return hip_fail(e);
  }
  return finish(coll::launch_moe_dispatch((int)d, a, grid, stream));
}

COLL_EXPORT coll_status_t coll_moe_dispatch_fp8(const void* const* tokens, const int32_t* const* dest,
                                                void* const* recv, int64_t* const* loc, int64_t* counts_dev,
                                                int64_t* counts_hidden_dev, int32_t* status_dev, int p,
                                                size_t tokens_per_rank, int k, size_t hidden, size_t group,
                                                const int64_t* recv_cap, void* stream) {
  coll_status_t st = fp8_shape(hidden, group);
  if (st != COLL_OK) return st;
  const size_t R = fp8_row_bytes(hidden, group);
  size_t A = 0;
  st = check_direct(tokens, dest, recv, loc, counts_dev, counts_hidden_dev, status_dev, p, tokens_per_rank, k,
                    hidden, recv_cap, 2, R, 16, &A);
  if (st != COLL_OK) return st;
  int e = launch_direct_index(dest, loc, counts_dev, counts_hidden_dev, status_dev, p, A, R, hidden, stream);
  if (e) return hip_fail(e);
  if (A == 0) return COLL_OK;
  int dev = 0, cus = 0;
  e = current_device(&dev);
  if (!e) e = device_cus(dev, &cus);
  if (e) return hip_fail(e);
  if (direct_lds_bytes(p) > (size_t)g_dev[dev].lds_per_block.load()) return COLL_ERR_UNSUPPORTED;
  int grid;
  e = max_grid(&grid, kFamFp8Direct);
  if (e) return hip_fail(e);
  coll::MoeDirectArgs a =
      direct_args(tokens, dest, recv, loc, counts_dev, status_dev, p, tokens_per_rank, k, hidden, recv_cap, R);
  a.group = group;
  a.row_bytes = R;
  return finish(coll::launch_moe_dispatch_fp8(a, grid, stream));
}

COLL_EXPORT coll_status_t coll_moe_combine_direct(const void* const* y, const int64_t* const* loc,
                                                  const float* const* weights, const void* const* residual,
                                                  void* const* out, int p, size_t tokens_per_rank, int k,
                                                  size_t hidden, const int64_t* y_rows, coll_dtype_t dtype,
                                                  void* stream) {
  if (p < 1 || p > kMaxRanks || !arith_dtype_ok(dtype) || k < 1 || k > coll::kMaxTopK || hidden == 0 || !y_rows)
    return COLL_ERR_INVALID_ARG;
  if (dtype == COLL_I32) return COLL_ERR_UNSUPPORTED;
  const size_t d = dsize(dtype);
  size_t A, tb, b;
  if (!mul_ok(tokens_per_rank, (size_t)k, 1, &A) || A > 0x7fffffffull) return COLL_ERR_INVALID_ARG;
  if (!mul_ok(hidden, d, 1, &b) || !mul_ok(tokens_per_rank, hidden * d, 1, &tb)) return COLL_ERR_INVALID_ARG;
  for (int r = 0; r < p; ++r)
    if (y_rows[r] < 0 || y_rows[r] > 0x7fffffffll || !mul_ok((size_t)y_rows[r], hidden * d, 1, &b))
      return COLL_ERR_INVALID_ARG;
  if (A == 0) return COLL_OK;
  if (!all_non_null(y, p) || !all_non_null(loc, p) || !all_non_null(weights, p) || !all_non_null(out, p))
    return COLL_ERR_INVALID_ARG;
  if (residual && !all_non_null(residual, p)) return COLL_ERR_INVALID_ARG;
  if (!elem_aligned(y, p, d) || !elem_aligned(out, p, d) || !elem_aligned(loc, p, 8) ||
      !elem_aligned(weights, p, 4) || (residual && !elem_aligned(residual, p, d)))
    return COLL_ERR_INVALID_ARG;
  std::vector<Range> rs;
  for (int r = 0; r < p; ++r) {
    rs.push_back(rng(y[r], (size_t)y_rows[r] * hidden * d, false, r));
    rs.push_back(rng(loc[r], A * 8, false, r));
    rs.push_back(rng(weights[r], A * 4, false, r));
    if (residual) rs.push_back(rng(residual[r], tb, false, kResidualTag + r));
    rs.push_back(rng(out[r], tb, true, r));
  }
  coll_status_t st = check_alias(rs, [](const Range& o, const Range& x) {
    // in place: out[r] is exactly residual[r] (the residual add)
    return !x.out && x.rank == kResidualTag + o.rank && x.b == o.b && x.e == o.e;
  });
  if (st != COLL_OK) return st;
  int grid;
  int e = max_grid(&grid, kFamRow);
  if (e) return hip_fail(e);
  coll::MoeRowArgs ra;
  std::memset(&ra, 0, sizeof(ra));
  for (int r = 0; r < p; ++r) {
    ra.src[r] = y[r];
    ra.dst[r] = out[r];
    ra.pos[r] = reinterpret_cast<const int32_t*>(loc[r]);
    ra.weights[r] = weights[r];
    if (residual) ra.residual[r] = residual[r];
    ra.cap[r] = (int32_t)y_rows[r];
  }
  ra.tokens = tokens_per_rank;
  ra.hidden = hidden;
  ra.k = k;
  ra.p = p;
  ra.has_residual = residual ? 1 : 0;
  ra.src_mis = common_mis(y, p);
  ra.dst_mis = common_mis((const void* const*)out, p);
  ra.res_mis = residual ? common_mis(residual, p) : 0;
  return finish(coll::launch_moe_combine_direct(dtype, ra, grid, stream));
}

// ---------------------------------------------------------------------------
// Batched AllReduce
// ---------------------------------------------------------------------------
namespace {

// One descriptor table: a device buffer, its pinned staging buffer, and an
// event recorded after the batch kernel that reads them.
struct BatchSlot {
  void* dev_buf = nullptr;
  size_t dev_cap = 0;
  void* host_buf = nullptr;
  size_t host_cap = 0;
  hipEvent_t done = nullptr;
};

// Two slots used in turn: a batch waits only for the batch two calls
// before it (which used the same slot), so the host validates and packs
// the next batch while the previous kernel runs.
struct BatchState {
  std::mutex mu;
  BatchSlot slot[2];
  int next = 0;
  int device = -1;
};
BatchState g_batch;

// Release everything; caller holds the mutex.
void batch_release() {
  for (BatchSlot& b : g_batch.slot) {
    if (b.done) {
      hipEventSynchronize(b.done);
      hipEventDestroy(b.done);
    }
    if (b.dev_buf) hipFree(b.dev_buf);
    if (b.host_buf) hipHostFree(b.host_buf);
    b = BatchSlot{};
  }
  g_batch.next = 0;
  g_batch.device = -1;
}

bool ranges_disjoint_sorted(std::vector<Range>& rs) {
  std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.b < b.b; });
  // any overlap that involves an output is an error, except identical
  // (in-place) input/output pairs of the same call, which were checked per
  // call and are excluded by the caller.
  uintptr_t max_end_out = 0, max_end_any = 0;
  for (const Range& r : rs) {
    if (r.b == r.e) continue;
    if (r.b < max_end_out) return false;               // starts inside an output
    if (r.out && r.b < max_end_any) return false;      // output starts inside anything
    max_end_any = std::max(max_end_any, r.e);
    if (r.out) max_end_out = std::max(max_end_out, r.e);
  }
  return true;
}

}  // namespace

namespace {

// Descriptor table of a batch: (ncalls + 1) BatchCall records (the last
// holds the total tile count); then, 256-byte aligned, a 256-byte block
// whose first 8 bytes are the kernel's run counter (uploaded as zero with
// the table); then ncalls * 2p pointers (per call: p sources, then p
// destinations).
struct BatchLayout {
  size_t rec_bytes = 0;
  size_t ctr_off = 0;  // the kernel's run counter (64-bit, zero on upload)
  size_t ptr_off = 0;
  size_t total = 0;
  uint64_t tiles = 0;
};

// Checks every call (and, with COLL_BATCH_CHECK_ALIAS, overlaps between
// calls) and sizes the descriptor table.  Touches no device state.
coll_status_t batch_validate(const coll_call_t* calls, int ncalls, int p, unsigned flags, BatchLayout* L) {
  if (p < 1 || p > kMaxRanks || ncalls < 0 || (ncalls > 0 && !calls)) return COLL_ERR_INVALID_ARG;
  if (flags & ~COLL_BATCH_CHECK_ALIAS) return COLL_ERR_INVALID_ARG;
  uint64_t tiles = 0;
  for (int k = 0; k < ncalls; ++k) {
    const coll_call_t& c = calls[k];
    coll_status_t st = check_allreduce(c.send, c.recv, p, c.n, c.dtype, c.op);
    if (st != COLL_OK) return st;
    if (!c.n) continue;
    const uint64_t te = coll::batch_tile_elems_host(c.dtype, p);
    const uint64_t q = (c.n + p - 1) / p;
    const uint64_t tpc = std::max<uint64_t>(1, (q + te - 1) / te);
    if (tpc > 0xffffffffull) return COLL_ERR_INVALID_ARG;
    tiles += (uint64_t)p * tpc;
  }
  if (flags & COLL_BATCH_CHECK_ALIAS) {
    std::vector<Range> rs;
    rs.reserve((size_t)ncalls * 2 * p);
    for (int k = 0; k < ncalls; ++k) {
      const coll_call_t& c = calls[k];
      if (c.n == 0) continue;
      const size_t nb = c.n * dsize(c.dtype);
      for (int r = 0; r < p; ++r) {
        // an in-place pair (validated above) is one output range
        if (c.send[r] != c.recv[r]) rs.push_back(rng(c.send[r], nb, false, r));
        rs.push_back(rng(c.recv[r], nb, true, r));
      }
    }
    if (!ranges_disjoint_sorted(rs)) return COLL_ERR_ALIAS;
  }
  L->rec_bytes = ((size_t)ncalls + 1) * sizeof(coll::BatchCall);
  L->ctr_off = (L->rec_bytes + 255) & ~size_t(255);
  L->ptr_off = L->ctr_off + 256;
  L->total = L->ptr_off + (size_t)ncalls * 2 * p * sizeof(void*);
  L->tiles = tiles;
  return COLL_OK;
}

// Writes the descriptor table of validated calls into host memory h
// (L.total bytes).
void batch_pack(const coll_call_t* calls, int ncalls, int p, const BatchLayout& L, char* h) {
  coll::BatchCall* recs = (coll::BatchCall*)h;
  uint64_t tiles = 0;
  for (int k = 0; k < ncalls; ++k) {
    const coll_call_t& c = calls[k];
    coll::BatchCall b{};
    b.n = c.n;
    b.first_tile = tiles;
    b.dtype = (uint32_t)c.dtype;
    b.op = (uint32_t)c.op;
    // BatchCall::mis: -1, the sources' common address mod 256, or 256 + the
    // common misalignment mod 16
    const int m16 = c.n ? common_mis2(common_mis(c.send, p), common_mis((const void* const*)c.recv, p)) : -1;
    const int m256 = m16 < 0 ? -1 : common_amis(c.send, p);
    b.mis = m16 < 0 ? -1 : (m256 >= 0 ? m256 : 256 + m16);
    const uint64_t te = coll::batch_tile_elems_host(c.dtype, p);
    const uint64_t q = (c.n + p - 1) / p;
    b.tiles_per_chunk = c.n ? (uint32_t)std::max<uint64_t>(1, (q + te - 1) / te) : 0;
    tiles += (uint64_t)p * b.tiles_per_chunk;
    std::memcpy(&recs[k], &b, sizeof(b));
  }
  coll::BatchCall last{};
  last.first_tile = tiles;
  std::memcpy(&recs[ncalls], &last, sizeof(last));
  std::memset(h + L.rec_bytes, 0, L.ptr_off - L.rec_bytes);
  const void** hp = (const void**)(h + L.ptr_off);
  for (int k = 0; k < ncalls; ++k) {
    for (int r = 0; r < p; ++r) {
      hp[(size_t)k * 2 * p + r] = calls[k].n ? calls[k].send[r] : nullptr;
      hp[(size_t)k * 2 * p + p + r] = calls[k].n ? (const void*)calls[k].recv[r] : nullptr;
    }
  }
}

// Launches the batch kernel over a descriptor table already in device
// memory (or enqueued to arrive there on `stream` first).
coll_status_t batch_launch(void* table, const BatchLayout& L, int ncalls, int p, void* stream) {
  int grid;
  int e = max_grid(&grid, kFamReduce);
  if (e) return hip_fail(e);
  coll::BatchArgs a;
  a.calls = (const coll::BatchCall*)table;
  a.ptrs = (const void* const*)((char*)table + L.ptr_off);
  a.next_run = (unsigned long long*)((char*)table + L.ctr_off);
  a.ncalls = ncalls;
  a.p = p;
  const int g = (int)std::min<uint64_t>(L.tiles, (uint64_t)grid);
  return finish(coll::launch_batch(a, g, stream));
}

}  // namespace

COLL_EXPORT coll_status_t coll_allreduce_batch(const coll_call_t* calls, int ncalls, int p, unsigned flags,
                                               void* stream) {
  BatchLayout L;
  coll_status_t st = batch_validate(calls, ncalls, p, flags, &L);
  if (st != COLL_OK || ncalls == 0 || L.tiles == 0) return st;

  int dev = 0;
  int e = current_device(&dev);
  if (e) return hip_fail(e);
  std::lock_guard<std::mutex> lock(g_batch.mu);
  if (g_batch.device != -1 && g_batch.device != dev) batch_release();
  g_batch.device = dev;
  BatchSlot& b = g_batch.slot[g_batch.next];
  if (b.done) {
    // the last kernel that used this slot reads its device buffer, and that
    // kernel's upload read its pinned staging buffer: both must be finished
    // before reuse
    e = (int)hipEventSynchronize(b.done);
    if (e) return hip_fail(e);
  } else {
    e = (int)hipEventCreateWithFlags(&b.done, hipEventDisableTiming);
    if (e) return hip_fail(e);
  }
  if (b.dev_cap < L.total) {
    const size_t cap = std::max(L.total, b.dev_cap * 2);
    if (b.dev_buf) hipFree(b.dev_buf);
    b.dev_buf = nullptr;
    b.dev_cap = 0;
    e = (int)hipMalloc(&b.dev_buf, cap);
    if (e) return hip_fail(e);
    b.dev_cap = cap;
  }
  if (b.host_cap < L.total) {
    if (b.host_buf) hipHostFree(b.host_buf);
    b.host_buf = nullptr;
    b.host_cap = 0;
    e = (int)hipHostMalloc(&b.host_buf, b.dev_cap, hipHostMallocDefault);
    if (e) return hip_fail(e);
    b.host_cap = b.dev_cap;
  }
  batch_pack(calls, ncalls, p, L, (char*)b.host_buf);
  hipStream_t s = (hipStream_t)stream;
  e = (int)hipMemcpyAsync(b.dev_buf, b.host_buf, L.total, hipMemcpyHostToDevice, s);
  if (e) return hip_fail(e);
  st = batch_launch(b.dev_buf, L, ncalls, p, stream);
  if (st != COLL_OK) return st;
  e = (int)hipEventRecord(b.done, s);
  if (e) return hip_fail(e);
  g_batch.next ^= 1;
  return COLL_OK;
}

// ---------------------------------------------------------------------------
// Batched AllReduce that allocates nothing: the descriptor table goes to a
// static device array (batch_noalloc.hip), staged through a static host
// buffer with a copy from pageable memory, which HIP has read before the
// copy call returns.
// ---------------------------------------------------------------------------
namespace {
std::mutex g_noalloc_mu;
alignas(256) char g_noalloc_host[coll::kNoAllocScratchBytes];
}  // namespace

COLL_EXPORT coll_status_t coll_allreduce_batch_noalloc(const coll_call_t* calls, int ncalls, int p, unsigned flags,
                                                       void* stream) {
  BatchLayout L;
  coll_status_t st = batch_validate(calls, ncalls, p, flags, &L);
  if (st != COLL_OK || ncalls == 0 || L.tiles == 0) return st;
  if (L.total > coll::kNoAllocScratchBytes) return COLL_ERR_INVALID_ARG;
  int dev = 0;
  int e = current_device(&dev);
  if (e) return hip_fail(e);
  void* table = nullptr;
  e = coll::noalloc_scratch(dev, &table);
  if (e) return hip_fail(e);
  {
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    batch_pack(calls, ncalls, p, L, g_noalloc_host);
    e = (int)hipMemcpyAsync(table, g_noalloc_host, L.total, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e) return hip_fail(e);
  }
  return batch_launch(table, L, ncalls, p, stream);
}

// ---------------------------------------------------------------------------
// Direction-mix bandwidth probe (measurement helper)
// ---------------------------------------------------------------------------
COLL_EXPORT coll_status_t coll_stream_probe(const void* const* src, int nsrc, void* const* dst, int ndst,
                                            size_t bytes, int unroll, unsigned flags, void* sink, void* stream) {
  if (nsrc < 0 || ndst < 0 || nsrc > kMaxRanks || ndst > kMaxRanks || nsrc + ndst == 0) return COLL_ERR_INVALID_ARG;
  if (flags & ~(unsigned)(COLL_PROBE_NT_LOADS | COLL_PROBE_NT_STORES | COLL_PROBE_CLAIM | COLL_PROBE_DEVICE_STORES))
    return COLL_ERR_INVALID_ARG;
  if (bytes % 16 || unroll < 1) return COLL_ERR_INVALID_ARG;
  if (!coll::probe_mix_supported(nsrc, ndst) || !coll::probe_unroll_supported(nsrc, unroll))
    return COLL_ERR_UNSUPPORTED;
  if (bytes == 0) return COLL_OK;
  if (nsrc && !all_non_null(src, nsrc)) return COLL_ERR_INVALID_ARG;
  if (ndst && !all_non_null(dst, ndst)) return COLL_ERR_INVALID_ARG;
  if (ndst == 0 && (!sink || (uintptr_t)sink % 16)) return COLL_ERR_INVALID_ARG;
  for (int k = 0; k < nsrc; ++k)
    if ((uintptr_t)src[k] % 16) return COLL_ERR_INVALID_ARG;
  for (int d = 0; d < ndst; ++d)
    if ((uintptr_t)dst[d] % 16) return COLL_ERR_INVALID_ARG;
  std::vector<Range> rs;
  for (int k = 0; k < nsrc; ++k) rs.push_back(rng(src[k], bytes, false, k));
  for (int d = 0; d < ndst; ++d) rs.push_back(rng(dst[d], bytes, true, d));
  if (!ranges_disjoint_sorted(rs)) return COLL_ERR_ALIAS;
  int grid;
  int e = max_grid(&grid, kFamReduce);
  if (e) return hip_fail(e);
  coll::RankPtrs P = make_ptrs(src, nsrc, dst, ndst);
  unsigned long long* claim = (flags & COLL_PROBE_CLAIM) ? stream_claim_slot(stream) : nullptr;
  const bool nts = flags & COLL_PROBE_NT_STORES, dev = flags & COLL_PROBE_DEVICE_STORES;
  const int sp = nts && dev ? coll::kStNTDevice : nts ? coll::kStNT : dev ? coll::kStDevice : coll::kStPlain;
  return finish(coll::launch_probe(nsrc, ndst, P, bytes / 16, unroll, flags & COLL_PROBE_NT_LOADS, sp, sink, grid,
                                   claim, stream));
}

// ---------------------------------------------------------------------------
// Misc
// ---------------------------------------------------------------------------
COLL_EXPORT const char* coll_status_string(coll_status_t s) {
  switch (s) {
    case COLL_OK: return "COLL_OK";
    case COLL_ERR_INVALID_ARG: return "COLL_ERR_INVALID_ARG: invalid argument";
    case COLL_ERR_UNSUPPORTED: return "COLL_ERR_UNSUPPORTED: valid request this build does not implement";
    case COLL_ERR_ALIAS: return "COLL_ERR_ALIAS: illegal overlap between buffers";
    case COLL_ERR_HIP: return "COLL_ERR_HIP: the HIP runtime reported an error";
  }
  return "unknown coll_status_t";
}

COLL_EXPORT int coll_last_hip_error(void) { return g_last_hip; }

COLL_EXPORT int coll_version(void) { return 200; }

COLL_EXPORT void coll_set_grid_limit(int workgroups_per_cu) {
  int w = workgroups_per_cu > 0 ? workgroups_per_cu : 0;
  if (w > kMaxWgPerCu) w = kMaxWgPerCu;
  g_wg_per_cu.store(w, std::memory_order_relaxed);
}

COLL_EXPORT void coll_finalize(void) {
  std::lock_guard<std::mutex> lock(g_batch.mu);
  batch_release();
}
