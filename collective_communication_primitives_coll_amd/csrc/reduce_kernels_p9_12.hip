// Ring-order reductions at compile-time rank counts 9, 10, 11, 12: the
// kernels of reduce_impl.h with the pointer rotation done in registers as
// for the power-of-two counts (rotate_left holds for any count).
#include "reduce_impl.h"

namespace coll {

int launch_reduce_p9_12(int p, int dtype, int op, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                       void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (p) {
    case 9: return launch_ring_fixed<9>(dtype, op, ptrs, g, max_grid, s);
    case 10: return launch_ring_fixed<10>(dtype, op, ptrs, g, max_grid, s);
    case 11: return launch_ring_fixed<11>(dtype, op, ptrs, g, max_grid, s);
    case 12: return launch_ring_fixed<12>(dtype, op, ptrs, g, max_grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
