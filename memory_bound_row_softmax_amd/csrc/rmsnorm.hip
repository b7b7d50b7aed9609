// rmsnorm.hip -- instantiates the RMSNorm kernels of the configuration menu and
// launches the one the plan names.
#include "launch_util.hpp"
#include "row_kernels.hpp"

namespace rr {
namespace {

template <class E, int P, int R, int G, bool VEC>
hipError_t launch_cfg(const void *x, const void *w, void *y, float *rstd, int64_t M, int64_t N,
                      float eps, void *ws, const LaunchArgs &a) {
    auto kernel = rmsnorm_kernel<E, P, R, G, VEC>;
    constexpr int B = block_threads_for(R);
    const char *xp = static_cast<const char *>(x);
    const char *wp = static_cast<const char *>(w);
    char *yp = static_cast<char *>(y);
    int n = (int)N;
    int spin = a.spin_limit;
    if constexpr (G == 1) {
        unsigned blocks;
        hipError_t e = blocks_for_rows(M, rows_per_block_for(R), &blocks);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kernel, dim3(blocks), dim3(B), 0, a.stream, xp, wp, yp, rstd, M, n, eps,
                           (uint8_t *)nullptr, 0, spin);
        return hipGetLastError();
    } else {
        int groups;
        hipError_t e = cooperative_groups(kernel, B, G, M, a, &groups);
        if (e != hipSuccess) return e;
        uint8_t *wsp = static_cast<uint8_t *>(ws);
        void *args[] = {&xp, &wp, &yp, &rstd, &M, &n, &eps, &wsp, &groups, &spin};
        return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(kernel),
                                          dim3(groups * G), dim3(B), args, 0, a.stream);
    }
}

template <class E, bool VEC>
hipError_t dispatch(const Plan &p, const void *x, const void *w, void *y, float *rstd, int64_t M,
                    int64_t N, float eps, void *ws, const LaunchArgs &a) {
#define RR_X(P_, R_, G_)                                                      \
    if constexpr (row_config_enabled(kCfgRmsnorm, E::BYTES, VEC, P_, R_, G_))        \
        if (p.P == P_ && p.R == R_ && p.G == G_)                              \
        return launch_cfg<E, P_, R_, G_, VEC>(x, w, y, rstd, M, N, eps, ws, a);
    RR_ROW_CONFIGS(RR_X)
#undef RR_X
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rmsnorm(const Plan &p, int dtype, const void *x, const void *w, void *y,
                          float *rstd, int64_t M, int64_t N, float eps, void *ws,
                          const LaunchArgs &a) {
    if (dtype == kF32)
        return p.vec ? dispatch<F32, true>(p, x, w, y, rstd, M, N, eps, ws, a)
                     : dispatch<F32, false>(p, x, w, y, rstd, M, N, eps, ws, a);
    return p.vec ? dispatch<BF16, true>(p, x, w, y, rstd, M, N, eps, ws, a)
                 : dispatch<BF16, false>(p, x, w, y, rstd, M, N, eps, ws, a);
}

}  // namespace rr
