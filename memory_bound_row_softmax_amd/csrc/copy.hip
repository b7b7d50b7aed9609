// copy.hip -- 128-bit streaming copy: the same-run HBM ceiling for one read plus one
// write per byte, against which the three row kernels are reported.  Each block
// copies 256 * kCopyUnroll chunks of 16 bytes through buffer resources that span
// exactly its own range, with the same cache policies as the row kernels' streams.
#include "launch_util.hpp"
#include "vec_io.hpp"

namespace rr {
namespace {

constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 4;  // chunks per lane; all loads issued before the stores

__global__ void __launch_bounds__(kCopyBlock) copy_kernel(const char *src, char *dst, int64_t n) {
    const int64_t first = (int64_t)blockIdx.x * kCopyBlock * kCopyUnroll;
    int64_t left = n - first;
    if (left > kCopyBlock * kCopyUnroll) left = kCopyBlock * kCopyUnroll;
    const uint32_t bytes = (uint32_t)left * 16u;
    const Buf s = make_buf(src + first * 16, bytes);
    const Buf d = make_buf(dst + first * 16, bytes);
    u32x4 t[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
        t[u] = buf_load16<kStreamLoad>(s, (uint32_t)(threadIdx.x + u * kCopyBlock) * 16u);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
        buf_store16(d, (uint32_t)(threadIdx.x + u * kCopyBlock) * 16u, t[u]);
}

}  // namespace

hipError_t launch_copy(const void *src, void *dst, size_t bytes, const LaunchArgs &a) {
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return hipSuccess;
    const int64_t per_block = (int64_t)kCopyBlock * kCopyUnroll;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyBlock), 0, a.stream,
                       static_cast<const char *>(src), static_cast<char *>(dst), n);
    return hipGetLastError();
}

}  // namespace rr
