// Ring-order reductions at compile-time rank counts 13, 14, 15: the
// kernels of reduce_impl.h with the pointer rotation done in registers as
// for the power-of-two counts (rotate_left holds for any count).
#include "reduce_impl.h"

namespace coll {

int launch_reduce_p13_15(int p, int dtype, int op, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                       void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (p) {
    case 13: return launch_ring_fixed<13>(dtype, op, ptrs, g, max_grid, s);
    case 14: return launch_ring_fixed<14>(dtype, op, ptrs, g, max_grid, s);
    case 15: return launch_ring_fixed<15>(dtype, op, ptrs, g, max_grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
