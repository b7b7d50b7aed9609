// long_row.hip -- instantiates the two-pass long-row kernels (softmax and RMSNorm
// forward, the softmax backward and the cross-entropy gradient past the on-chip
// capacity) and launches the one the plan names.
#include "launch_util.hpp"
#include "long_row.hpp"

namespace rr {
namespace {

template <class E, int OP, int P, int G, bool VEC>
hipError_t launch_cfg(const void *x, const void *w, void *y, float *rstd, int64_t M, int64_t N,
                      float eps, void *ws, const LaunchArgs &a, XentRows xr) {
    constexpr int R = kLongR;
    auto kernel = long_row_kernel<E, OP, P, R, G, VEC>;
    int groups;
    hipError_t e = resident_groups(kernel, R, G, M, a, &groups);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(groups * G), dim3(R), 0, a.stream,
                       static_cast<const char *>(x), static_cast<const char *>(w),
                       static_cast<char *>(y), rstd, M, (int)N, eps, static_cast<uint8_t *>(ws),
                       groups, a.spin_limit, xr);
    return hipGetLastError();
}

template <class E, int OP>
hipError_t dispatch(const Plan &p, const void *x, const void *w, void *y, float *rstd, int64_t M,
                    int64_t N, float eps, void *ws, const LaunchArgs &a, XentRows xr) {
    // 16, 32 or 64 workgroups per row (long_row_groups)
    {
        if (p.G == 32)
            return p.vec ? launch_cfg<E, OP, kLongP, 32, true>(x, w, y, rstd, M, N, eps, ws, a, xr)
                         : launch_cfg<E, OP, kLongPElem, 32, false>(x, w, y, rstd, M, N, eps, ws, a, xr);
        if (p.G == 64)
            return p.vec ? launch_cfg<E, OP, kLongP, 64, true>(x, w, y, rstd, M, N, eps, ws, a, xr)
                         : launch_cfg<E, OP, kLongPElem, 64, false>(x, w, y, rstd, M, N, eps, ws, a, xr);
    }
    if (p.G != kLongG) return hipErrorInvalidValue;
    if (p.vec) return launch_cfg<E, OP, kLongP, kLongG, true>(x, w, y, rstd, M, N, eps, ws, a, xr);
    return launch_cfg<E, OP, kLongPElem, kLongG, false>(x, w, y, rstd, M, N, eps, ws, a, xr);
}

}  // namespace

hipError_t launch_long_row(const Plan &p, int op, int dtype, const void *x, const void *w,
                           void *y, float *rstd, int64_t M, int64_t N, float eps, void *ws,
                           const LaunchArgs &a, XentRows xr) {
    if (op == kOpSoftmax)
        return dtype == kF32 ? dispatch<F32, kLongSoftmax>(p, x, w, y, rstd, M, N, eps, ws, a, xr)
                             : dispatch<BF16, kLongSoftmax>(p, x, w, y, rstd, M, N, eps, ws, a, xr);
    if (op == kOpSoftmaxBwd)
        return dtype == kF32 ? dispatch<F32, kLongSoftmaxBwd>(p, x, w, y, rstd, M, N, eps, ws, a, xr)
                             : dispatch<BF16, kLongSoftmaxBwd>(p, x, w, y, rstd, M, N, eps, ws, a, xr);
    if (op == kOpXentGrad) {
        if (!xr.labels || !xr.dloss || !xr.loss) return hipErrorInvalidValue;
        return dtype == kF32 ? dispatch<F32, kLongXentGrad>(p, x, w, y, rstd, M, N, eps, ws, a, xr)
                             : dispatch<BF16, kLongXentGrad>(p, x, w, y, rstd, M, N, eps, ws, a, xr);
    }
    if (op != kOpRmsnorm) return hipErrorInvalidValue;
    return dtype == kF32 ? dispatch<F32, kLongRmsnorm>(p, x, w, y, rstd, M, N, eps, ws, a, xr)
                         : dispatch<BF16, kLongRmsnorm>(p, x, w, y, rstd, M, N, eps, ws, a, xr);
}

}  // namespace rr
