// launch.hpp -- host-side launchers of the HIP kernels (one per op).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

namespace rr {

struct LaunchArgs {
    hipStream_t stream;
    int num_cus;     // compute units of the current device
    int spin_limit;     // bound on each grid-exchange wait (polls); <= 0: a wait gives up at once
    int forced_groups;  // row groups of a persistent grid (0: from the occupancy query)
};

hipError_t launch_softmax(const Plan &p, int dtype, const void *x, void *y, int64_t M, int64_t N,
                          void *ws, const LaunchArgs &a);
hipError_t launch_rmsnorm(const Plan &p, int dtype, const void *x, const void *w, void *y,
                          float *rstd, int64_t M, int64_t N, float eps, void *ws,
                          const LaunchArgs &a);
hipError_t launch_xent(const Plan &p, int dtype, const void *x, const int32_t *labels,
                       float *loss, float *lse, int64_t M, int64_t N, const LaunchArgs &a);
hipError_t launch_xent_grad(const Plan &p, int dtype, const void *x, const int32_t *labels,
                            const float *dloss, float *loss, float *lse, void *dx, int64_t M,
                            int64_t N, void *ws, const LaunchArgs &a);
hipError_t launch_softmax_bwd(const Plan &p, int dtype, const void *y, const void *dy, void *dx,
                              int64_t M, int64_t N, void *ws, const LaunchArgs &a);
hipError_t launch_rmsnorm_bwd(const Plan &p, int dtype, const void *x, const void *w,
                              const void *dy, const float *rstd, void *dx, float *dw, int64_t M,
                              int64_t N, void *ws, const LaunchArgs &a);
// Per-row inputs and outputs of the cross-entropy gradient on the long-row kernel
// (unused by the other ops).
struct XentRows {
    const int32_t *labels = nullptr;
    const float *dloss = nullptr;
    float *loss = nullptr;
};

// op kOpSoftmax or kOpRmsnorm: x, w (RMSNorm), y, rstd (RMSNorm, may be NULL);
// kOpSoftmaxBwd: x = the forward's y, w = dy (M x N), y = dx;
// kOpXentGrad: x = logits, y = dlogits, rstd = lse (may be NULL), and xr.
hipError_t launch_long_row(const Plan &p, int op, int dtype, const void *x, const void *w,
                           void *y, float *rstd, int64_t M, int64_t N, float eps, void *ws,
                           const LaunchArgs &a, XentRows xr = {});
hipError_t launch_rmsnorm_packed(const Plan &p, const void *x, const void *w, void *y, float *rstd,
                                 int64_t M, int64_t N, float eps, void *ws, const LaunchArgs &a);
hipError_t launch_copy(const void *src, void *dst, size_t bytes, const LaunchArgs &a);

// Bytes of the library-held softmax workspace on each GPU (rr_softmax_fwd_static): the
// largest a softmax plan needs, 256 + 1024 * (64 + 64 * 128) = 8454400 (on 256
// workgroups per row at most 512 row groups: 8421632), rounded up.
constexpr size_t kStaticScratchBytes = (size_t)(8u << 20) + (256u << 10);
// Its device address on device `dev`, which must be the current device (found with
// hipGetSymbolAddress on the first call for each device, then kept).
hipError_t static_scratch(int dev, void **ptr);
hipError_t launch_read(const void *src, size_t bytes, uint32_t *sink, const LaunchArgs &a);
hipError_t launch_fill(void *dst, size_t bytes, uint32_t value, const LaunchArgs &a);
// Bytes of the per-block checksums launch_read writes for `bytes` of input.
size_t stream_read_sink_bytes(size_t bytes);

}  // namespace rr
