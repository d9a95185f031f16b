// hqq_solve.hip -- dispatch of the HQQ solve to its per-bit-width kernels.
#include "hqq_internal.h"

namespace hqq {

template <int NB>
hipError_t launch_solve_nb(int group_size, int axis, const SolveArgs &a, hipStream_t st);

hipError_t launch_solve(int nbits, int group_size, int axis, const SolveArgs &a, hipStream_t st)
{
    switch (nbits) {
    case 1: return launch_solve_nb<1>(group_size, axis, a, st);
    case 2: return launch_solve_nb<2>(group_size, axis, a, st);
    case 3: return launch_solve_nb<3>(group_size, axis, a, st);
    case 4: return launch_solve_nb<4>(group_size, axis, a, st);
    case 8: return launch_solve_nb<8>(group_size, axis, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hqq
