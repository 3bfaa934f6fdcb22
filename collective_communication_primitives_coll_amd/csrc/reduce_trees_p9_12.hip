// Tree and double-binary-tree AllReduce orders at compile-time rank counts
// 9, 10, 11 and 12 (the power-of-two counts are in reduce_kernels.hip).
#include "reduce_impl.h"

namespace coll {

int launch_tree_p9_12(int p, int dtype, int op, int order, const RankPtrs& ptrs, const ReduceGeom& g,
                      int max_grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (p) {
    case 9: return launch_tree_fixed<9>(dtype, op, order, ptrs, g, max_grid, s);
    case 10: return launch_tree_fixed<10>(dtype, op, order, ptrs, g, max_grid, s);
    case 11: return launch_tree_fixed<11>(dtype, op, order, ptrs, g, max_grid, s);
    case 12: return launch_tree_fixed<12>(dtype, op, order, ptrs, g, max_grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
