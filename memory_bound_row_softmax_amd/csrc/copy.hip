// copy.hip -- streaming ceilings the row kernels are reported against: a 128-bit copy
// (one read plus one write per byte, the shape of softmax and RMSNorm), a read-only
// stream and a write-only stream, each with the row kernels' non-temporal policies.
//
// Block b moves 16 units of 1 KiB (one wave-wide 16-byte access each) out of the
// 128 KiB region b / 8.  The eight blocks of a region run on the eight XCDs (block b
// on XCD b mod 8), and block b takes the units whose index has bits 2..4 equal to
// b mod 8: each XCD then touches only the 4 KiB granules of one address class
// (address bits 12..14).  Which address bits an XCD's traffic fixes changes what
// HBM delivers for writes.  Measured on MI355X (GB/s, 16 GiB each way):
//   XCD's fixed address bits   10-12  12-14  14-16 (16 KiB per block)  17-19  18-20
//   write-only                  6662   6417   5865                     6199   6543
//   copy (read + write)         6307   6334   5845                     5729   5993
// Reads measured 7.0-7.2 TB/s whatever the mapping.  Bits 12..14 gave the best copy
// from 4 to 16 GiB (6.3-6.5 TB/s; 16 KiB of contiguous bytes per block, the usual
// copy, 5.7-5.9).  Any bijection of blocks onto units copies correctly; the mapping
// only decides which XCD moves which bytes.
#include "launch_util.hpp"
#include "vec_io.hpp"

namespace rr {
namespace {

constexpr int kCopyBlock = 256;        // 4 waves
constexpr int kUnitsPerBlock = 16;     // 4 per wave, all loads issued before any store
constexpr uint32_t kUnit = 1024;       // bytes
constexpr uint32_t kRegion = 8 * kUnitsPerBlock * kUnit;  // 128 KiB: one block per XCD
constexpr int kClassShift = 2;         // unit-index bits 2..4 = address bits 12..14

// Unit (0..127 inside the region) of the j-th access of block class c (0..7).
__device__ __forceinline__ uint32_t unit_in_region(uint32_t c, uint32_t j) {
    const uint32_t low = j & ((1u << kClassShift) - 1);
    const uint32_t high = j >> kClassShift;
    return (((high << 3) | c) << kClassShift) | low;
}

// The region of block b as a buffer resource (the last region may be partial: the
// range check then drops what lies past the end).
__device__ __forceinline__ Buf region_buf(const char *base, int64_t bytes) {
    const int64_t off = (int64_t)(blockIdx.x >> 3) * kRegion;
    int64_t left = bytes - off;
    if (left > kRegion) left = kRegion;
    return make_buf(base + off, (uint32_t)left);
}

__global__ void __launch_bounds__(kCopyBlock) copy_kernel(const char *src, char *dst, int64_t bytes) {
    const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63, c = blockIdx.x & 7;
    const Buf s = region_buf(src, bytes);
    const Buf d = region_buf(dst, bytes);
    u32x4 t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        t[i] = buf_load16<kStreamLoad>(s, unit_in_region(c, i * 4 + w) * kUnit + lane * 16u);
#pragma unroll
    for (int i = 0; i < 4; ++i) buf_store16(d, unit_in_region(c, i * 4 + w) * kUnit + lane * 16u, t[i]);
}

// Reads every byte once; each block writes the XOR of its 32-bit words to sink[b]
// (4 bytes per 16 KiB read), so that the loads cannot be dropped.
__global__ void __launch_bounds__(kCopyBlock) read_kernel(const char *src, int64_t bytes,
                                                          uint32_t *sink) {
    const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63, c = blockIdx.x & 7;
    const Buf s = region_buf(src, bytes);
    u32x4 t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        t[i] = buf_load16<kStreamLoad>(s, unit_in_region(c, i * 4 + w) * kUnit + lane * 16u);
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc ^= t[i][0] ^ t[i][1] ^ t[i][2] ^ t[i][3];
    // XOR over the wave, then over the 4 waves through LDS
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, 64);
    __shared__ uint32_t part[kCopyBlock / 64];
    if (lane == 0) part[w] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Writes every byte once with a 32-bit pattern.
__global__ void __launch_bounds__(kCopyBlock) fill_kernel(char *dst, int64_t bytes, uint32_t v) {
    const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63, c = blockIdx.x & 7;
    const Buf d = region_buf(dst, bytes);
    const u32x4 t = {v, v, v, v};
#pragma unroll
    for (int i = 0; i < 4; ++i) buf_store16(d, unit_in_region(c, i * 4 + w) * kUnit + lane * 16u, t);
}

hipError_t blocks_for_bytes(size_t bytes, unsigned *blocks) {
    const uint64_t regions = (bytes + kRegion - 1) / kRegion;
    if (regions * 8 > 0x7FFFFFFFull) return hipErrorInvalidValue;
    *blocks = (unsigned)(regions * 8);
    return hipSuccess;
}

}  // namespace

size_t stream_read_sink_bytes(size_t bytes) { return (bytes + kRegion - 1) / kRegion * 8 * 4; }

hipError_t launch_copy(const void *src, void *dst, size_t bytes, const LaunchArgs &a) {
    unsigned blocks;
    hipError_t e = blocks_for_bytes(bytes, &blocks);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(kCopyBlock), 0, a.stream,
                       static_cast<const char *>(src), static_cast<char *>(dst), (int64_t)bytes);
    return hipGetLastError();
}

hipError_t launch_read(const void *src, size_t bytes, uint32_t *sink, const LaunchArgs &a) {
    unsigned blocks;
    hipError_t e = blocks_for_bytes(bytes, &blocks);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kCopyBlock), 0, a.stream,
                       static_cast<const char *>(src), (int64_t)bytes, sink);
    return hipGetLastError();
}

hipError_t launch_fill(void *dst, size_t bytes, uint32_t value, const LaunchArgs &a) {
    unsigned blocks;
    hipError_t e = blocks_for_bytes(bytes, &blocks);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(kCopyBlock), 0, a.stream,
                       static_cast<char *>(dst), (int64_t)bytes, value);
    return hipGetLastError();
}

}  // namespace rr
