// softmax.hip -- instantiates the softmax kernels of the configuration menu and
// launches the one the plan names; holds the workspace of rr_softmax_fwd_static.
#include <mutex>

#include "softmax_launch.hpp"

// The split-row workspace of rr_softmax_fwd_static, for callers that cannot allocate:
// one array on each GPU the library runs on, held until the process ends.  It is zero
// when the code object loads, and every launch that completes leaves its exchange area
// zero again (grid_exchange.hpp), so calls need not clear it; a wait that gave up
// leaves only the header's error word set, which no kernel reads.  Calls that overlap
// on one GPU share it and race.  In host code `scratch` names a host-side stand-in:
// the device address comes from hipGetSymbolAddress (static_scratch below).
static __device__ __align__(256) uint8_t scratch[rr::kStaticScratchBytes];

namespace rr {

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t static_scratch(int dev, void **ptr) {
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;  // the array's address on the current device (`dev`)
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_softmax(const Plan &p, int dtype, const void *x, void *y, int64_t M, int64_t N,
                          void *ws, const LaunchArgs &a) {
    return softmax_launch::launch(p, dtype, x, y, M, N, ws, SoftmaxOut{}, a);
}

}  // namespace rr
