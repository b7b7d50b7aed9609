// softmax_bwd.hip -- instantiates the softmax backward kernels of the configuration
// menu and launches the one the plan names.
#include "launch_util.hpp"
#include "softmax_bwd.hpp"

namespace rr {
namespace {

template <class E, int P, int R, bool VEC>
hipError_t launch_block(const void *y, const void *dy, void *dx, int64_t M, int64_t N,
                        const LaunchArgs &a) {
    unsigned blocks;
    hipError_t e = blocks_for_rows(M, rows_per_block_for(R), &blocks);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((softmax_bwd_block_kernel<E, P, R, VEC>), dim3(blocks),
                       dim3(block_threads_for(R)), 0, a.stream, static_cast<const char *>(y),
                       static_cast<const char *>(dy), static_cast<char *>(dx), M, (int)N);
    return hipGetLastError();
}

template <class E, int P, int R, int G, bool VEC>
hipError_t launch_stream(const void *y, const void *dy, void *dx, int64_t M, int64_t N, void *ws,
                         const LaunchArgs &a) {
    auto kernel = softmax_bwd_stream_kernel<E, P, R, G, VEC>;
    int groups;
    hipError_t e = resident_groups(kernel, R, G, M, a, &groups);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(groups * G), dim3(R), 0, a.stream,
                       static_cast<const char *>(y), static_cast<const char *>(dy),
                       static_cast<char *>(dx), M, (int)N, static_cast<uint8_t *>(ws), groups,
                       a.spin_limit);
    return hipGetLastError();
}

template <class E, bool VEC>
hipError_t dispatch(const Plan &p, const void *y, const void *dy, void *dx, int64_t M, int64_t N,
                    void *ws, const LaunchArgs &a) {
    if (!p.stream) {
#define RR_X(P_, R_)                                                               \
    if constexpr (block_config_enabled(kCfgSoftmaxBwd, E::BYTES, VEC, P_, R_))     \
        if (p.P == P_ && p.R == R_) return launch_block<E, P_, R_, VEC>(y, dy, dx, M, N, a);
        RR_BLOCK_CONFIGS(RR_X)
#undef RR_X
    } else {
#define RR_X(P_, R_, G_)                                                                \
    if constexpr (stream_config_enabled(kCfgSoftmaxBwd, E::BYTES, VEC, P_, R_, G_))     \
        if (p.P == P_ && p.R == R_ && p.G == G_)                                        \
            return launch_stream<E, P_, R_, G_, VEC>(y, dy, dx, M, N, ws, a);
        RR_STREAM_CONFIGS(RR_X)
#undef RR_X
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_softmax_bwd(const Plan &p, int dtype, const void *y, const void *dy, void *dx,
                              int64_t M, int64_t N, void *ws, const LaunchArgs &a) {
    if (dtype == kF32)
        return p.vec ? dispatch<F32, true>(p, y, dy, dx, M, N, ws, a)
                     : dispatch<F32, false>(p, y, dy, dx, M, N, ws, a);
    return p.vec ? dispatch<BF16, true>(p, y, dy, dx, M, N, ws, a)
                 : dispatch<BF16, false>(p, y, dy, dx, M, N, ws, a);
}

}  // namespace rr
