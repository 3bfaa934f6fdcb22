// Placement tables of the direct MoE dispatch.
//
// The index pass leaves, per source rank i, the count matrix (rows of i to
// each destination j, times count_unit) and every assignment's row in i's
// packed order (grouped by destination).  Writing rows straight into the
// receive buffers needs two prefix sums of that matrix:
//   soff[i][j] = sum over j' < j of rows[i][j']  (start of block j in i's packed order)
//   roff[i][j] = sum over i' < i of rows[i'][j]  (start of source i's rows in recv[j])
// so that packed row ps of an assignment to j lands on row
// roff[i][j] + ps - soff[i][j] of recv[j]: the receive layout of the
// ragged exchange (sources in rank order, each source's rows in its packed
// order).  Each workgroup builds both tables in dynamic LDS (3 p^2 int32:
// the row counts, loaded by all threads at once, then the two scans) and
// checks every receive buffer's capacity.
#pragma once

#include "device_common.h"

namespace coll {

// LDS bytes the tables need for p ranks.
__host__ __device__ constexpr size_t direct_tables_bytes(int p) { return (size_t)3 * p * p * sizeof(int32_t); }

// Fills soff and roff (each p*p, row-major [i][j]); returns true if some
// receive buffer is too small, in which case nothing may be delivered.
// Workgroup 0 records the outcome in status[p].  Capacities are at most
// 2^31 - 1 rows (checked on the host), so accepted offsets fit in int32.
__device__ __forceinline__ bool direct_tables(const MoeDirectArgs& a, int32_t* soff, int32_t* roff, int* flag) {
  const int p = a.p;
  const int tid = threadIdx.x;
  const int64_t unit = (int64_t)a.count_unit;
  int32_t* rows = roff + p * p;  // third table: the row counts
  if (tid == 0) *flag = 0;
  // one load per thread (a dependent chain of p loads per thread would
  // cost every workgroup p memory latencies before its first row)
  for (int x = tid; x < p * p; x += blockDim.x) rows[x] = (int32_t)(a.counts[x] / unit);
  __syncthreads();
  if (tid < p) {
    int32_t s = 0;
    for (int j = 0; j < p; ++j) {
      soff[tid * p + j] = s;
      s += rows[tid * p + j];
    }
  } else if (tid >= 64 && tid < 64 + p) {
    const int j = tid - 64;
    int64_t s = 0;
    for (int i = 0; i < p; ++i) {
      roff[i * p + j] = (int32_t)(s < 0x7fffffff ? s : 0x7fffffff);
      s += rows[i * p + j];
    }
    if (s > a.cap[j]) *flag = 1;
  }
  __syncthreads();
  const bool bad = *flag != 0;
  if (blockIdx.x == 0 && tid == 0 && a.status) a.status[p] = bad ? 1 : 0;
  return bad;
}

// Location of a delivered assignment: destination rank and row.
__device__ __forceinline__ int64_t direct_loc(int j, int64_t row) { return ((int64_t)j << 32) | row; }

}  // namespace coll
