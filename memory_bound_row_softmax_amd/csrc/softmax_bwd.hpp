// softmax_bwd.hpp -- softmax backward from the forward output: per row
//     c = sum_k y_k * dy_k,   dx_j = y_j * (dy_j - c).
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%), section 让内存密集型内核达到"光速",
// presents its memory-bound kernels as building blocks of training as well as
// inference; the softmax backward is the textbook derivative of the softmax it
// describes (sections NCU 性能分析（Softmax 内核） and 内存吞吐量).  It is again one
// row reduction between a load and a store: y and dy are read once, dx written once
// (two reads and one write per element).  Each lane keeps its part of both input
// rows, so a lane holds 2P values and the menu is narrower than the forward's.
// Rows split over G workgroups exchange the partial dot product like RMSNorm's sum
// of squares.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "configs.hpp"
#include "grid_exchange.hpp"
#include "reduce.hpp"
#include "row_io.hpp"
#include "row_kernels.hpp"
#include "vec_io.hpp"

namespace rr {

// The row's dot product c over this workgroup's part (a: y, b: dy).  Registers past
// the row are zeroed in both operands where lane groups of fewer than 64 lanes share
// one buffer resource: there they hold the next row's values, and an Inf or NaN in
// them must not reach this row's sum through 0 * Inf.  (With a buffer per row or per
// split-row part, loads past its end return 0.)
template <class E, int P, int R, bool STREAM>
__device__ __forceinline__ float softmax_bwd_local(float *a, float *b, RowCtx &c) {
    constexpr int C = P / E::VPC;
    if (!c.full) {
        mask_part<E, C, R, STREAM>(c.ln, c.N, 0.0f, a);
        if constexpr (R < 64) mask_part<E, C, R, STREAM>(c.ln, c.N, 0.0f, b);
    }
    const float t = tree_dot<P>(a, b);
    return row_reduce<R>(t, c.one_reduction_slots(), c.l, OpSum{});
}

// dx = y * (dy - c) into a, then the store.
template <class E, int P, int R, bool VEC, bool STREAM>
__device__ __forceinline__ void softmax_bwd_apply(float *a, const float *b, float t,
                                                  RowView dxv, bool valid, const RowCtx &c) {
    constexpr int C = P / E::VPC;
#pragma unroll
    for (int j = 0; j < P; ++j) a[j] = a[j] * (b[j] - t);
    store_part<E, C, R, VEC, STREAM>(dxv, c.ln, c.N, valid, c.full, a);
}

// a: the lane's part of y, b: of dy; a becomes dx.
template <class E, int P, int R, int G, bool VEC, bool STREAM>
__device__ __forceinline__ void softmax_bwd_finish(float *a, float *b, RowView dxv, bool valid,
                                                   RowCtx &c) {
    float t = softmax_bwd_local<E, P, R, STREAM>(a, b, c);
    if constexpr (G > 1) {
        exchange_pairs<G>(c.g, c.member, c.it, t, 0.0f, c.spin_limit, c.bcast, MergeSum{});
        t = c.bcast[0];
    }
    softmax_bwd_apply<E, P, R, VEC, STREAM>(a, b, t, dxv, valid, c);
}

template <class E, int P, int R, bool VEC>
__global__ void __launch_bounds__(block_threads_for(R))
    softmax_bwd_block_kernel(const char *y, const char *dy, char *dx, int64_t M, int N) {
    constexpr int C = P / E::VPC;
    constexpr int RPB = rows_per_block_for(R);
    constexpr int W = R > 64 ? R / 64 : 1;
    __shared__ float red[RPB * W];
    const int sub = lane_group<R>();
    const uint32_t row_bytes = (uint32_t)N * E::BYTES;
    RowCtx c{N, (int)(threadIdx.x % R), 0, 0, part_full<kCfgSoftmaxBwd, E, C, R, 1>(0, N),
             red + sub * W, nullptr, nullptr, GroupRef{}, 0};
    const bool valid = (int64_t)blockIdx.x * RPB + sub < M;
    float a[P], b[P];
    c.ln = lane_of<kCfgSoftmaxBwd, E, C, R, 1>(0, c.l);
    load_part<E, C, R, VEC>(block_row_view<R>(y, M, sub, row_bytes), c.ln, a);
    load_part<E, C, R, VEC>(block_row_view<R>(dy, M, sub, row_bytes), c.ln, b);
    softmax_bwd_finish<E, P, R, 1, VEC, false>(a, b, block_row_view<R>(dx, M, sub, row_bytes), valid,
                                               c);
}

// Persistent stream kernel: each buffer holds a row of y (first P values) and of
// dy (next P), the next row's loads in flight while the current one is finished.
template <class E, int P, int R, int G, bool VEC>
__global__ void __launch_bounds__(R)
    __attribute__((amdgpu_waves_per_eu(stream_waves(kCfgSoftmaxBwd, E::BYTES, VEC, P, R, G))))
    softmax_bwd_stream_kernel(const char *y, const char *dy, char *dx, int64_t M, int N,
                              uint8_t *ws, int groups, int spin_limit) {
    static_assert(R >= 64, "one row per workgroup");
    constexpr int C = P / E::VPC;
    constexpr int W = R / 64;
    __shared__ float red[2][W];
    __shared__ float bcast[3];
    RowCtx c{N, (int)threadIdx.x, 0, 0, true, red[0], red[1], bcast, GroupRef{}, spin_limit};
    int group = blockIdx.x;
    if constexpr (G > 1) {
        member_of<G>(&group, &c.member);
        c.g = group_ref<G>(ws, group);
        if (threadIdx.x == 0) bcast[2] = 0.0f;  // read only after later barriers
    }
    c.ln = lane_of<kCfgSoftmaxBwd, E, C, R, G>(c.member, (int)threadIdx.x);
    c.full = part_full<kCfgSoftmaxBwd, E, C, R, G>(c.member, N);
    const uint32_t rb = (uint32_t)N * E::BYTES;

    if constexpr (kDeferredExchange && defer_split(kCfgSoftmaxBwd, E::BYTES, VEC, P, R, G)) {
        // Split rows, deferred exchange (see the softmax stream kernel): row k's
        // partial dot product is published before the wait for row k - 1's; rows in
        // flight are kept as raw chunks.
        float buf[3][2 * P];
        int64_t row = group;
        auto load = [&](float *v, int64_t r) {
            if constexpr (VEC) {
                load_part_raw<E, C, R>(stream_row_view(y, r, M, rb), c.ln, v);
                load_part_raw<E, C, R>(stream_row_view(dy, r, M, rb), c.ln, v + P);
            } else {
                load_part<E, C, R, VEC>(stream_row_view(y, r, M, rb), c.ln, v);
                load_part<E, C, R, VEC>(stream_row_view(dy, r, M, rb), c.ln, v + P);
            }
        };
        load(buf[0], row);
        load(buf[1], row + groups);
        auto step = [&](auto Kc) -> bool {
            constexpr int K = decltype(Kc)::value, KP = (K + 2) % 3;
            const bool more = row < M;
            if (more) {
                if constexpr (VEC) {
                    widen_part<E, C>(buf[K]);
                    widen_part<E, C>(buf[K] + P);
                }
                const float t = softmax_bwd_local<E, P, R, true>(buf[K], buf[K] + P, c);
                publish_pair<G>(c.g, c.member, c.it, t, 0.0f);
            } else {
                __syncthreads();  // as in the softmax kernel: the merged c is read
            }
            if (c.it > 0) {  // complete the previous row
                wait_pairs<G>(c.g, c.it - 1, c.spin_limit, c.bcast, MergeSum{});
                softmax_bwd_apply<E, P, R, VEC, true>(buf[KP], buf[KP] + P, c.bcast[0],
                                                stream_row_view(dx, row - groups, M, rb), true, c);
            }
            if (!more) return false;
            load(buf[KP], row + 2 * (int64_t)groups);
            ++c.it;
            row += groups;
            return true;
        };
        while (stream_steps<0, 3>(step)) {
        }
    } else {
        float buf[2][2 * P];
        stream_rows<2>(
            (int64_t)group, M, groups, buf,
            [&](float *v, int64_t r) {
                load_part<E, C, R, VEC>(stream_row_view(y, r, M, rb), c.ln, v);
                load_part<E, C, R, VEC>(stream_row_view(dy, r, M, rb), c.ln, v + P);
            },
            [&](float *v, int64_t r) {
                softmax_bwd_finish<E, P, R, G, VEC, true>(v, v + P, stream_row_view(dx, r, M, rb), true,
                                                    c);
                ++c.it;
            });
    }
    if constexpr (G > 1) {
        if (c.it > 0) depart_group<G>(c.g);
    }
}

}  // namespace rr
