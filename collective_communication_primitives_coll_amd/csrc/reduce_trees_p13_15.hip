// Tree and double-binary-tree AllReduce orders at compile-time rank counts
// 13, 14 and 15 (the power-of-two counts are in reduce_kernels.hip).
#include "reduce_impl.h"

namespace coll {

int launch_tree_p13_15(int p, int dtype, int op, int order, const RankPtrs& ptrs, const ReduceGeom& g,
                       int max_grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (p) {
    case 13: return launch_tree_fixed<13>(dtype, op, order, ptrs, g, max_grid, s);
    case 14: return launch_tree_fixed<14>(dtype, op, order, ptrs, g, max_grid, s);
    case 15: return launch_tree_fixed<15>(dtype, op, order, ptrs, g, max_grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
