// xent_grad.hip -- instantiates the softmax kernels of the configuration menu with
// the fused cross-entropy gradient epilogue and launches the one the plan names.
#include "softmax_launch.hpp"
#include "xent_grad.hpp"

namespace rr {

hipError_t launch_xent_grad(const Plan &p, int dtype, const void *x, const int32_t *labels,
                            const float *dloss, float *loss, float *lse, void *dx, int64_t M,
                            int64_t N, void *ws, const LaunchArgs &a) {
    return softmax_launch::launch(p, dtype, x, dx, M, N, ws,
                                  XentGradOut{labels, dloss, loss, lse, M}, a);
}

}  // namespace rr
