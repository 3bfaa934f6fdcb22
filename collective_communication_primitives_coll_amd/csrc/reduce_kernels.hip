// Reduction launch for every rank count: the power-of-two counts (every
// schedule) here, the other counts up to 16 in ring order in
// reduce_kernels_p*.hip and in the tree orders in reduce_trees_p*.hip
// (compiled separately so the build runs in parallel), and counts above 16
// with the general any-p kernel.
#include "reduce_impl.h"

namespace coll {

// Ring order at compile-time rank counts that are not powers of two.
int launch_reduce_p3_7(int p, int dtype, int op, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                       void* stream);
int launch_reduce_p9_12(int p, int dtype, int op, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                        void* stream);
int launch_reduce_p13_15(int p, int dtype, int op, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                         void* stream);
// Tree and double-binary-tree orders at the same rank counts.
int launch_tree_p3_7(int p, int dtype, int op, int order, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                     void* stream);
int launch_tree_p9_12(int p, int dtype, int op, int order, const RankPtrs& ptrs, const ReduceGeom& g,
                      int max_grid, void* stream);
int launch_tree_p13_15(int p, int dtype, int op, int order, const RankPtrs& ptrs, const ReduceGeom& g,
                       int max_grid, void* stream);

// Tree orders only change the result of floating-point sums (plain,
// averaged or pre-multiplied); integer sums and min/max give the same bits
// in any order, so they always run the ring-order kernel.
template <int DT, int OP, int ORD>
static int launch_tree(const RankPtrs& ptrs, const ReduceGeom& g, int max_grid, hipStream_t s) {
  switch (g.p) {
    case 2: return launch_p<DT, OP, 2, ORD>(ptrs, g, max_grid, s);
    case 4: return launch_p<DT, OP, 4, ORD>(ptrs, g, max_grid, s);
    case 8: return launch_p<DT, OP, 8, ORD>(ptrs, g, max_grid, s);
    case 16: return launch_p<DT, OP, 16, ORD>(ptrs, g, max_grid, s);
    default: return (int)hipErrorInvalidValue;
  }
}

template <int DT, int OP>
static int launch_dt_op(int order, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid, hipStream_t s) {
  if constexpr ((DT == kF32 || DT == kBF16) && (OP == kSum || OP == kAvg || OP == kPreMul)) {
    if (order == kOrdRD) return launch_tree<DT, OP, kOrdRD>(ptrs, g, max_grid, s);
    if (order == kOrdHD) return launch_tree<DT, OP, kOrdHD>(ptrs, g, max_grid, s);
    if (order == kOrdTree) return launch_tree<DT, OP, kOrdTree>(ptrs, g, max_grid, s);
    if (order == kOrdDBT) return launch_tree<DT, OP, kOrdDBT>(ptrs, g, max_grid, s);
  }
  switch (g.p) {
    case 2: return launch_p<DT, OP, 2, kOrdRing>(ptrs, g, max_grid, s);
    case 4: return launch_p<DT, OP, 4, kOrdRing>(ptrs, g, max_grid, s);
    case 8: return launch_p<DT, OP, 8, kOrdRing>(ptrs, g, max_grid, s);
    case 16: return launch_p<DT, OP, 16, kOrdRing>(ptrs, g, max_grid, s);
    default: return launch_any<DT, OP>(ptrs, g, max_grid, s);
  }
}

template <int DT>
static int launch_dt(int op, int order, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                     hipStream_t s) {
  switch (op) {
    case kSum: return launch_dt_op<DT, kSum>(order, ptrs, g, max_grid, s);
    case kMin: return launch_dt_op<DT, kMin>(order, ptrs, g, max_grid, s);
    case kMax: return launch_dt_op<DT, kMax>(order, ptrs, g, max_grid, s);
    case kAvg: return launch_dt_op<DT, kAvg>(order, ptrs, g, max_grid, s);
    case kPreMul:
      if constexpr (DT != kI32) return launch_dt_op<DT, kPreMul>(order, ptrs, g, max_grid, s);
      break;
  }
  return (int)hipErrorInvalidValue;
}

int launch_reduce(int dtype, int op, int order, const RankPtrs& ptrs, const ReduceGeom& g,
                  int max_grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const bool float_sum = (dtype == kF32 || dtype == kBF16) && (op == kSum || op == kAvg || op == kPreMul);
  if (float_sum && (order == kOrdTree || order == kOrdDBT)) {
    switch (g.p) {
      case 3: case 5: case 6: case 7:
        return launch_tree_p3_7(g.p, dtype, op, order, ptrs, g, max_grid, stream);
      case 9: case 10: case 11: case 12:
        return launch_tree_p9_12(g.p, dtype, op, order, ptrs, g, max_grid, stream);
      case 13: case 14: case 15:
        return launch_tree_p13_15(g.p, dtype, op, order, ptrs, g, max_grid, stream);
    }
  }
  if (order == kOrdRing || !float_sum) {
    switch (g.p) {
      case 3: case 5: case 6: case 7:
        return launch_reduce_p3_7(g.p, dtype, op, ptrs, g, max_grid, stream);
      case 9: case 10: case 11: case 12:
        return launch_reduce_p9_12(g.p, dtype, op, ptrs, g, max_grid, stream);
      case 13: case 14: case 15:
        return launch_reduce_p13_15(g.p, dtype, op, ptrs, g, max_grid, stream);
    }
  }
  switch (dtype) {
    case kF32: return launch_dt<kF32>(op, order, ptrs, g, max_grid, s);
    case kBF16: return launch_dt<kBF16>(op, order, ptrs, g, max_grid, s);
    case kI32: return launch_dt<kI32>(op, order, ptrs, g, max_grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
