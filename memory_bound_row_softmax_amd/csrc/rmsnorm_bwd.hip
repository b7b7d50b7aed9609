// rmsnorm_bwd.hip -- instantiates the RMSNorm backward kernels of the configuration
// menu and launches the one the plan names, then the dw column reduction.
#include "launch_util.hpp"
#include "rmsnorm_bwd.hpp"

namespace rr {
namespace {

template <class E, int P, int R, int G, bool VEC>
hipError_t launch_cfg(const Plan &p, const void *x, const void *w, const void *dy,
                      const float *rstd, void *dx, int64_t M, int64_t N, uint8_t *ws,
                      int *parts, const LaunchArgs &a) {
    auto kernel = rmsnorm_bwd_kernel<E, P, R, G, VEC>;
    const int threads = bwd_threads(R, G);
    int groups;
    if constexpr (G == 1) {
        // no workgroup waits for another: one per CU (measured best or within a few
        // percent of two or four), at most one per row block and at most the
        // workspace's partial rows
        int64_t g = a.num_cus;
        // test override of the number of persistent workgroups (rr_set_test_overrides)
        if (a.forced_groups > 0) g = a.forced_groups;
        if (g > p.max_parts) g = p.max_parts;
        groups = (int)g;
    } else {
        hipError_t e = resident_groups(kernel, threads, G, M, a, &groups);
        if (e != hipSuccess) return e;
        if (groups > p.max_parts) groups = p.max_parts;
    }
    *parts = groups;
    const char *xp = static_cast<const char *>(x);
    const char *wp = static_cast<const char *>(w);
    const char *dyp = static_cast<const char *>(dy);
    char *dxp = static_cast<char *>(dx);
    float *part = reinterpret_cast<float *>(ws + p.part_off);
    int n = (int)N;
    int spin = a.spin_limit;
    hipLaunchKernelGGL(kernel, dim3(groups * G), dim3(threads), 0, a.stream, xp, wp, dyp, rstd,
                       dxp, part, M, n, ws, groups, spin);
    return hipGetLastError();
}

template <class E, bool VEC>
hipError_t dispatch(const Plan &p, const void *x, const void *w, const void *dy,
                    const float *rstd, void *dx, int64_t M, int64_t N, uint8_t *ws, int *parts,
                    const LaunchArgs &a) {
#define RR_X(P_, R_, G_)                                                                 \
    if constexpr (rmsbwd_config_enabled(VEC, P_, E::BYTES))                              \
        if (p.P == P_ && p.R == R_ && p.G == G_)                                         \
            return launch_cfg<E, P_, R_, G_, VEC>(p, x, w, dy, rstd, dx, M, N, ws, parts, a);
    RR_RMSBWD_CONFIGS(RR_X)
#undef RR_X
    return hipErrorInvalidValue;
}

// dw = the sum of `parts` partial rows (one pass, see rmsnorm_dw_reduce).
hipError_t reduce_dw(const Plan &p, uint8_t *ws, int parts, int64_t N, float *dw,
                     const LaunchArgs &a) {
    const float *part = reinterpret_cast<const float *>(ws + p.part_off);
    const unsigned tiles = (unsigned)((N + 4 * kDwTileQuads - 1) / (4 * kDwTileQuads));
    if (N % 4 == 0)
        hipLaunchKernelGGL(rmsnorm_dw_reduce<true>, dim3(tiles), dim3(256), 0, a.stream, part,
                           parts, (int)N, dw);
    else
        hipLaunchKernelGGL(rmsnorm_dw_reduce<false>, dim3(tiles), dim3(256), 0, a.stream, part,
                           parts, (int)N, dw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_bwd(const Plan &p, int dtype, const void *x, const void *w,
                              const void *dy, const float *rstd, void *dx, float *dw, int64_t M,
                              int64_t N, void *ws, const LaunchArgs &a) {
    uint8_t *wsb = static_cast<uint8_t *>(ws);
    int parts = 0;
    if (M > 0) {
        hipError_t e;
        if (dtype == kF32)
            e = p.vec ? dispatch<F32, true>(p, x, w, dy, rstd, dx, M, N, wsb, &parts, a)
                      : dispatch<F32, false>(p, x, w, dy, rstd, dx, M, N, wsb, &parts, a);
        else
            e = p.vec ? dispatch<BF16, true>(p, x, w, dy, rstd, dx, M, N, wsb, &parts, a)
                      : dispatch<BF16, false>(p, x, w, dy, rstd, dx, M, N, wsb, &parts, a);
        if (e != hipSuccess) return e;
    }
    return reduce_dw(p, wsb, parts, N, dw, a);
}

}  // namespace rr
