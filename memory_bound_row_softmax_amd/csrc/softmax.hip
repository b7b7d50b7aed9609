// softmax.hip -- instantiates the softmax kernels of the configuration menu and
// launches the one the plan names.
#include "softmax_launch.hpp"

namespace rr {

hipError_t launch_softmax(const Plan &p, int dtype, const void *x, void *y, int64_t M, int64_t N,
                          void *ws, const LaunchArgs &a) {
    return softmax_launch::launch(p, dtype, x, y, M, N, ws, SoftmaxOut{}, a);
}

}  // namespace rr
