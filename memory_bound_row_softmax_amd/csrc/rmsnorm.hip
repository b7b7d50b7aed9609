// rmsnorm.hip -- instantiates the RMSNorm kernels of the configuration menu and
// launches the one the plan names.
#include "launch_util.hpp"
#include "row_kernels.hpp"

namespace rr {
namespace {

template <class E, int P, int R, bool VEC>
hipError_t launch_block(const void *x, const void *w, void *y, float *rstd, int64_t M,
                        int64_t N, float eps, const LaunchArgs &a) {
    unsigned blocks;
    hipError_t e = blocks_for_rows(M, rows_per_block_for(R), &blocks);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((rmsnorm_block_kernel<E, P, R, VEC>), dim3(blocks),
                       dim3(block_threads_for(R)), 0, a.stream, static_cast<const char *>(x),
                       static_cast<const char *>(w), static_cast<char *>(y), rstd, M, (int)N,
                       eps);
    return hipGetLastError();
}

template <class E, int P, int R, int G, bool VEC>
hipError_t launch_stream(const void *x, const void *w, void *y, float *rstd, int64_t M,
                         int64_t N, float eps, void *ws, const LaunchArgs &a) {
    auto kernel = rmsnorm_stream_kernel<E, P, R, G, VEC>;
    int groups;
    hipError_t e = resident_groups(kernel, R, G, M, a, &groups);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(groups * G), dim3(R), 0, a.stream,
                       static_cast<const char *>(x), static_cast<const char *>(w),
                       static_cast<char *>(y), rstd, M, (int)N, eps, static_cast<uint8_t *>(ws),
                       groups, a.spin_limit);
    return hipGetLastError();
}

template <class E, bool VEC>
hipError_t dispatch(const Plan &p, const void *x, const void *w, void *y, float *rstd, int64_t M,
                    int64_t N, float eps, void *ws, const LaunchArgs &a) {
    if (!p.stream) {
#define RR_X(P_, R_)                                                               \
    if constexpr (block_config_enabled(kCfgRmsnorm, E::BYTES, VEC, P_, R_))        \
        if (p.P == P_ && p.R == R_)                                                \
            return launch_block<E, P_, R_, VEC>(x, w, y, rstd, M, N, eps, a);
        RR_BLOCK_CONFIGS(RR_X)
#undef RR_X
    } else {
#define RR_X(P_, R_, G_)                                                                \
    if constexpr (stream_config_enabled(kCfgRmsnorm, E::BYTES, VEC, P_, R_, G_))        \
        if (p.P == P_ && p.R == R_ && p.G == G_)                                        \
            return launch_stream<E, P_, R_, G_, VEC>(x, w, y, rstd, M, N, eps, ws, a);
        RR_STREAM_CONFIGS(RR_X)
#undef RR_X
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rmsnorm(const Plan &p, int dtype, const void *x, const void *w, void *y,
                          float *rstd, int64_t M, int64_t N, float eps, void *ws,
                          const LaunchArgs &a) {
    if (p.P == kPackedP)  // packed bf16 rows (packed.hip)
        return launch_rmsnorm_packed(p, x, w, y, rstd, M, N, eps, ws, a);
    if (dtype == kF32)
        return p.vec ? dispatch<F32, true>(p, x, w, y, rstd, M, N, eps, ws, a)
                     : dispatch<F32, false>(p, x, w, y, rstd, M, N, eps, ws, a);
    return p.vec ? dispatch<BF16, true>(p, x, w, y, rstd, M, N, eps, ws, a)
                 : dispatch<BF16, false>(p, x, w, y, rstd, M, N, eps, ws, a);
}

}  // namespace rr
