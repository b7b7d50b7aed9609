// softmax_launch.hpp -- host launchers of the softmax-shaped kernels (plain softmax
// and the fused cross-entropy gradient), templated on the kernels' output policy.
#pragma once

#include "launch_util.hpp"
#include "row_kernels.hpp"

namespace rr {
namespace softmax_launch {

template <class E, int P, int R, bool VEC, class Out>
hipError_t block(const void *x, void *y, int64_t M, int64_t N, const Out &out,
                 const LaunchArgs &a) {
    unsigned blocks;
    hipError_t e = blocks_for_rows(M, rows_per_block_for(R), &blocks);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((softmax_block_kernel<E, P, R, VEC, Out>), dim3(blocks),
                       dim3(block_threads_for(R)), 0, a.stream, static_cast<const char *>(x),
                       static_cast<char *>(y), M, (int)N, out);
    return hipGetLastError();
}

template <class E, int P, int R, int G, bool VEC, class Out>
hipError_t stream(const void *x, void *y, int64_t M, int64_t N, void *ws, const Out &out,
                  const LaunchArgs &a) {
    auto kernel = softmax_stream_kernel<E, P, R, G, VEC, Out>;
    int groups;
    hipError_t e = resident_groups(kernel, R, G, M, a, &groups);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(groups * G), dim3(R), 0, a.stream,
                       static_cast<const char *>(x), static_cast<char *>(y), M, (int)N,
                       static_cast<uint8_t *>(ws), groups, a.spin_limit, out);
    return hipGetLastError();
}

template <class E, bool VEC, class Out>
hipError_t dispatch(const Plan &p, const void *x, void *y, int64_t M, int64_t N, void *ws,
                    const Out &out, const LaunchArgs &a) {
    if (!p.stream) {
#define RR_X(P_, R_)                                                               \
    if constexpr (block_config_enabled(Out::kCfg, E::BYTES, VEC, P_, R_))           \
        if (p.P == P_ && p.R == R_) return block<E, P_, R_, VEC>(x, y, M, N, out, a);
        RR_BLOCK_CONFIGS(RR_X)
#undef RR_X
    } else {
#define RR_X(P_, R_, G_)                                                                \
    if constexpr (stream_config_enabled(Out::kCfg, E::BYTES, VEC, P_, R_, G_))           \
        if (p.P == P_ && p.R == R_ && p.G == G_)                                        \
            return stream<E, P_, R_, G_, VEC>(x, y, M, N, ws, out, a);
        RR_STREAM_CONFIGS(RR_X)
#undef RR_X
    }
    return hipErrorInvalidValue;
}

template <class Out>
hipError_t launch(const Plan &p, int dtype, const void *x, void *y, int64_t M, int64_t N,
                  void *ws, const Out &out, const LaunchArgs &a) {
    if (dtype == kF32)
        return p.vec ? dispatch<F32, true>(p, x, y, M, N, ws, out, a)
                     : dispatch<F32, false>(p, x, y, M, N, ws, out, a);
    return p.vec ? dispatch<BF16, true>(p, x, y, M, N, ws, out, a)
                 : dispatch<BF16, false>(p, x, y, M, N, ws, out, a);
}

}  // namespace softmax_launch
}  // namespace rr
