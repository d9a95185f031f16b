// hqq_solve.hip -- dispatch of the HQQ solve to its per-bit-width kernels.
#include "hqq_internal.h"

namespace hqq {

template <int NB, bool BF>
hipError_t launch_solve_nb(int group_size, int axis, const SolveArgs &a, hipStream_t st);

template <bool BF>
hipError_t launch_solve_dt(int nbits, int group_size, int axis, const SolveArgs &a, hipStream_t st)
{
    switch (nbits) {
    case 1: return launch_solve_nb<1, BF>(group_size, axis, a, st);
    case 2: return launch_solve_nb<2, BF>(group_size, axis, a, st);
    case 3: return launch_solve_nb<3, BF>(group_size, axis, a, st);
    case 4: return launch_solve_nb<4, BF>(group_size, axis, a, st);
    case 8: return launch_solve_nb<8, BF>(group_size, axis, a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_solve(int nbits, int group_size, int axis, bool bf16, const SolveArgs &a, hipStream_t st)
{
    return bf16 ? launch_solve_dt<true>(nbits, group_size, axis, a, st)
                : launch_solve_dt<false>(nbits, group_size, axis, a, st);
}

}  // namespace hqq
