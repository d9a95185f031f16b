// hqq_solve_b4_bf16.hip -- the 4-bit HQQ solve kernels for bf16 weights
// (every group size and axis), in a translation unit of their own so the
// variants compile in parallel.
#include "hqq_solve_impl.h"

namespace hqq {
template hipError_t launch_solve_nb<4, true>(int, int, int, const SolveArgs &, hipStream_t);
}  // namespace hqq
