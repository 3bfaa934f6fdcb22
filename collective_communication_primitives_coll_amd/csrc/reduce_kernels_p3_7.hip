// Ring-order reductions at compile-time rank counts 3, 5, 6, 7: the
// kernels of reduce_impl.h with the pointer rotation done in registers as
// for the power-of-two counts (rotate_left holds for any count).
#include "reduce_impl.h"

namespace coll {

int launch_reduce_p3_7(int p, int dtype, int op, const RankPtrs& ptrs, const ReduceGeom& g, int max_grid,
                       void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (p) {
    case 3: return launch_ring_fixed<3>(dtype, op, ptrs, g, max_grid, s);
    case 5: return launch_ring_fixed<5>(dtype, op, ptrs, g, max_grid, s);
    case 6: return launch_ring_fixed<6>(dtype, op, ptrs, g, max_grid, s);
    case 7: return launch_ring_fixed<7>(dtype, op, ptrs, g, max_grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace coll
