// xent.hip -- instantiates the cross-entropy kernels of the configuration menu and
// launches the one the plan names.
#include "launch_util.hpp"
#include "xent_kernel.hpp"

namespace rr {
namespace {

template <class E, int P, int R, bool VEC>
hipError_t launch_cfg(const void *x, const int32_t *labels, float *loss, float *lse, int64_t M,
                      int64_t N, const LaunchArgs &a) {
    unsigned blocks;
    hipError_t e = blocks_for_rows(M, rows_per_block_for(R), &blocks);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((xent_kernel<E, P, R, VEC>), dim3(blocks), dim3(block_threads_for(R)), 0,
                       a.stream, static_cast<const char *>(x), labels, loss, lse, M, (int)N);
    return hipGetLastError();
}

template <class E, bool VEC>
hipError_t dispatch(const Plan &p, const void *x, const int32_t *labels, float *loss, float *lse,
                    int64_t M, int64_t N, const LaunchArgs &a) {
#define RR_X(P_, R_)                   \
    if (p.P == P_ && p.R == R_)        \
        return launch_cfg<E, P_, R_, VEC>(x, labels, loss, lse, M, N, a);
    RR_XENT_CONFIGS(RR_X)
#undef RR_X
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_xent(const Plan &p, int dtype, const void *x, const int32_t *labels,
                       float *loss, float *lse, int64_t M, int64_t N, const LaunchArgs &a) {
    if (dtype == kF32)
        return p.vec ? dispatch<F32, true>(p, x, labels, loss, lse, M, N, a)
                     : dispatch<F32, false>(p, x, labels, loss, lse, M, N, a);
    return p.vec ? dispatch<BF16, true>(p, x, labels, loss, lse, M, N, a)
                 : dispatch<BF16, false>(p, x, labels, loss, lse, M, N, a);
}

}  // namespace rr
