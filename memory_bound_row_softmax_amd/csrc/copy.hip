// copy.hip -- 128-bit streaming copy: the same-run HBM ceiling for one read plus one
// write per byte, against which the three row kernels are reported.
#include "launch_util.hpp"
#include "vec_io.hpp"

namespace rr {
namespace {

constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 8;  // 16-byte chunks per lane, all loads issued before the stores

__global__ void __launch_bounds__(kCopyBlock) copy_kernel(const u32x4 *src, u32x4 *dst,
                                                          int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * kCopyBlock * kCopyUnroll + threadIdx.x;
    u32x4 t[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kCopyBlock;
        t[u] = src[i < n ? i : n - 1];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kCopyBlock;
        if (i < n) dst[i] = t[u];
    }
}

}  // namespace

hipError_t launch_copy(const void *src, void *dst, size_t bytes, const LaunchArgs &a) {
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return hipSuccess;
    const int64_t per_block = (int64_t)kCopyBlock * kCopyUnroll;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyBlock), 0, a.stream,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace rr
