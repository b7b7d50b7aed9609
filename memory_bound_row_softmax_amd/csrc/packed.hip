// packed.hip -- instantiates the packed bf16 RMSNorm stream kernels and launches the
// one the plan names (P = kPackedP; 16-byte aligned bf16 rows).
#include "launch_util.hpp"
#include "packed_bf16.hpp"

namespace rr {
namespace {

template <int R, int G>
hipError_t launch_cfg(const void *x, const void *w, void *y, float *rstd, int64_t M, int64_t N,
                      float eps, void *ws, const LaunchArgs &a) {
    auto kernel = rmsnorm_packed_kernel<R, G>;
    int groups;
    hipError_t e = resident_groups(kernel, R, G, M, a, &groups);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(groups * G), dim3(R), 0, a.stream,
                       static_cast<const char *>(x), static_cast<const char *>(w),
                       static_cast<char *>(y), rstd, M, (int)N, eps, static_cast<uint8_t *>(ws),
                       groups, a.spin_limit);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_packed(const Plan &p, const void *x, const void *w, void *y, float *rstd,
                                 int64_t M, int64_t N, float eps, void *ws, const LaunchArgs &a) {
    if (p.P != kPackedP || !p.vec) return hipErrorInvalidValue;
#define RR_X(R_, G_) \
    if (p.R == R_ && p.G == G_) return launch_cfg<R_, G_>(x, w, y, rstd, M, N, eps, ws, a);
    RR_PACKED_CONFIGS(RR_X)
#undef RR_X
    return hipErrorInvalidValue;
}

}  // namespace rr
