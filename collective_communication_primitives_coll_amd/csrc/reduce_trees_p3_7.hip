// Tree and double-binary-tree AllReduce orders at compile-time rank counts
// 3, 5, 6 and 7 (the power-of-two counts are in reduce_kernels.hip).
#include "reduce_impl.h"

namespace coll {

int launch_tree_p3_7(int p, int dtype, int op, int order, const RankPtrs& ptrs, const ReduceGeom& g,
                     int max_grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (p) {
    case 3: return launch_tree_fixed<3>(dtype, op, order, ptrs, g, max_grid, s);
    case 5: return launch_tree_fixed<5>(dtype, op, order, ptrs, g, max_grid, s);
    case 6: return launch_tree_fixed<6>(dtype, op, order, ptrs, g, max_grid, s);
    case 7: return launch_tree_fixed<7>(dtype, op, order, ptrs, g, max_grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
