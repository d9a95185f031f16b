// hqq_solve_b8.hip -- the 8-bit HQQ solve kernels (every group size and
// axis), in a translation unit of their own so the bit widths compile in
// parallel.
#include "hqq_solve_impl.h"

namespace hqq {
template hipError_t launch_solve_nb<8, false>(int, int, int, const SolveArgs &, hipStream_t);
}  // namespace hqq
