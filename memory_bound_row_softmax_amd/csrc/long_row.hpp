// long_row.hpp -- softmax and RMSNorm forward, the softmax backward and the
// cross-entropy forward fused with its gradient, for rows longer than the split-row
// stream kernels hold in registers or run faster.
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%), section 内存吞吐量, names the
// alternative to reducing a long row across a cluster: an online algorithm that reads
// the row twice.  Here the G workgroups of a row group own every G-th tile of T = P * R
// elements of the row:
//   pass 1: stream the owned tiles, keeping a running (max, sum of exp) pair (softmax
//           and cross-entropy, the online-softmax rescaling), the sum of squares
//           (RMSNorm) or the dot product of y and dy (softmax backward);
//   merge:  reduce over the workgroup, then over the G workgroups through the
//           workspace (grid_exchange.hpp);
//   pass 2: read the owned tiles again and write y (dx, dlogits).
// A workgroup's tiles were read a moment before, so the second read is served in large
// part by the caches between the CUs and HBM (the 256 MB last-level cache holds the
// few hundred KB each of the resident workgroups reads per row) rather than by HBM.
// Each pass keeps the next tile's loads in flight while the current one is used, and
// the wait for the row group's partials overlaps the second pass's first loads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "configs.hpp"
#include "grid_exchange.hpp"
#include "launch.hpp"
#include "reduce.hpp"
#include "row_io.hpp"
#include "row_kernels.hpp"
#include "vec_io.hpp"

namespace rr {

constexpr int kLongSoftmax = 0;
constexpr int kLongRmsnorm = 1;
constexpr int kLongSoftmaxBwd = 2;  // x: y of the forward, w: dy (M x N), y: dx
constexpr int kLongXentGrad = 3;    // x: logits, y: dlogits, rstd: lse (or null), and XentRows


// Cache policy of the first read of a tile: it is read again shortly, so it must
// not carry the non-temporal hint of the other streams.  The second read is the
// last use and streams.
#ifndef RR_LONG_PASS1_POLICY
#define RR_LONG_PASS1_POLICY 0
#endif
constexpr int kLongPass1Load = RR_LONG_PASS1_POLICY;

// Walks the tiles t = first, first + step, ... that lie in [0, tiles), with two
// register buffers of B values: the next tile's loads are issued before the current
// tile is used.  `step` may be negative (the second pass walks backwards, so that it
// first reads the tiles the first pass read last, the ones most likely still cached).
// `pre` runs once, after the first tile's loads are issued and before it is used (the
// second pass waits there for the row group's merged partials, so the wait overlaps
// the loads).  `t` is the same for the whole workgroup, so the branches are uniform.
template <int B, class Load, class Use, class Pre>
__device__ __forceinline__ void walk_tiles(int first, int step, int tiles, Load load, Use use,
                                           Pre pre) {
    auto in = [&](int t) { return t >= 0 && t < tiles; };
    float a[B], b[B];
    int t = first;
    if (in(t)) load(a, t);
    pre();
    while (in(t)) {
        int tn = t + step;
        if (in(tn)) load(b, tn);
        use(a, t);
        t = tn;
        if (!in(t)) break;
        tn = t + step;
        if (in(tn)) load(a, tn);
        use(b, t);
        t = tn;
    }
}

// The last of the tiles first, first + step, ... below `tiles` (or `first` if none).
__device__ __forceinline__ int last_tile(int first, int step, int tiles) {
    return first < tiles ? first + ((tiles - 1 - first) / step) * step : first;
}

template <class E, int OP, int P, int R, int G, bool VEC>
__global__ void __launch_bounds__(R)
    long_row_kernel(const char *x, const char *w, char *y, float *rstd, int64_t M, int N,
                    float eps, uint8_t *ws, int groups, int spin_limit, XentRows xr) {
    static_assert(R >= 64 && G > 1, "whole waves, several workgroups per row");
    constexpr int C = P / E::VPC;
    constexpr int W = R / 64;
    constexpr int T = P * R;  // elements per tile
    __shared__ MaxSum red_ms[2][W];
    __shared__ float red_q[2][W];
    __shared__ float bcast[3];
    RowCtx c{N, (int)threadIdx.x, 0, 0, true, nullptr, nullptr, bcast, GroupRef{}, spin_limit};
    int group;
    member_of<G>(&group, &c.member);
    c.g = group_ref<G>(ws, group);
    if (threadIdx.x == 0) bcast[2] = 0.0f;  // read only after later barriers
    const int l = threadIdx.x;
    const uint32_t rb = (uint32_t)N * E::BYTES;
    const int tiles = (N + T - 1) / T;
    const Buf wb = make_buf(w, rb);

    for (int64_t row = group; row < M; row += groups) {
        const RowView xv = stream_row_view(x, row, M, rb);
        const RowView yv = stream_row_view(y, row, M, rb);
        auto tile = [&](int t) { return Lane{t * C * R + l, R}; };  // lane l's chunks of tile t
        // dy's row (softmax backward; the other ops do not use it)
        const RowView dv = OP == kLongSoftmaxBwd ? stream_row_view(w, row, M, rb) : xv;
        auto load1 = [&](float *v, int t) {
            load_part<E, C, R, VEC, kLongPass1Load>(xv, tile(t), v);
            if constexpr (OP == kLongSoftmaxBwd)
                load_part<E, C, R, VEC, kLongPass1Load>(dv, tile(t), v + P);
        };

        // Cross-entropy: the row's label, dloss and x[label], read before this
        // workgroup publishes its partial (so before any workgroup of the row group
        // writes dlogits, which may be the logits themselves).  A label outside
        // [0, N) is never used as an address: loss and dlogits are then NaN.
        int label = 0;
        bool ok = false;
        float ge = 0.0f, x_label = 0.0f;
        if constexpr (OP == kLongXentGrad) {
            label = xr.labels[row];
            ok = label >= 0 && label < N;
            ge = ok ? xr.dloss[row] : __builtin_nanf("");
            if (ok) x_label = buf_load_elem<E, 0>(xv.buf, xv.base + (uint32_t)label * E::BYTES);
        }

        // pass 1
        MaxSum acc = {-INFINITY, 0.0f};
        float q = 0.0f;
        constexpr int B1 = OP == kLongSoftmaxBwd ? 2 * P : P;
        walk_tiles<B1>(
            c.member, G, tiles, load1,
            [&](float *v, int t) {
                const bool full = part_full_at<E, C, R>(t * C * R, N);
                if constexpr (OP == kLongSoftmaxBwd) {
                    if (!full) {  // both operands: padding adds nothing to the dot product
                        mask_part<E, C, R>(tile(t), N, 0.0f, v);
                        mask_part<E, C, R>(tile(t), N, 0.0f, v + P);
                    }
                    q += tree_dot<P>(v, v + P);
                } else if constexpr (OP == kLongSoftmax || OP == kLongXentGrad) {
                    if (!full) mask_part<E, C, R>(tile(t), N, -INFINITY, v);
                    const float mnew = fmaxf(acc.m, tree_reduce<P>(v, OpMax{}));
                    const float mu = safe_max(mnew);
#pragma unroll
                    for (int j = 0; j < P; ++j) v[j] = exp_shift(v[j], mu);
                    acc.s = acc.s * exp_shift(acc.m, mu) + tree_reduce<P>(v, OpSum{});
                    acc.m = mnew;
                } else {
                    if (!full) mask_part<E, C, R>(tile(t), N, 0.0f, v);
                    q += tree_sum_squares<P>(v);
                }
            },
            [] {});

        // merge over the workgroup and publish; the row group's merged partials are
        // waited for once the second pass has its first tile's loads in flight
        if constexpr (OP == kLongSoftmax || OP == kLongXentGrad) {
            acc = row_reduce<R>(acc, red_ms[c.it & 1], l, OpMerge{});
            publish_pair<G>(c.g, c.member, c.it, acc.m, acc.s);
        } else {
            q = row_reduce<R>(q, red_q[c.it & 1], l, OpSum{});
            publish_pair<G>(c.g, c.member, c.it, q, 0.0f);
        }
        float m_row = 0.0f, s_row = 0.0f, r = 0.0f;
        auto wait = [&] {
            if constexpr (OP == kLongSoftmaxBwd) {
                wait_pairs<G>(c.g, c.it, c.spin_limit, c.bcast, MergeSum{});
                r = c.bcast[0];  // the row's sum of y * dy
            } else if constexpr (OP == kLongSoftmax || OP == kLongXentGrad) {
                wait_pairs<G>(c.g, c.it, c.spin_limit, c.bcast, MergeMaxSum{});
                m_row = safe_max(c.bcast[0]);
                s_row = __builtin_amdgcn_rcpf(c.bcast[1]);
                if constexpr (OP == kLongXentGrad) {
                    if (c.member == 0 && l == 0) {
                        const float row_lse = c.bcast[0] + __builtin_amdgcn_logf(c.bcast[1]) * kLn2;
                        if (rstd) rstd[row] = row_lse;
                        xr.loss[row] = ok ? row_lse - x_label : __builtin_nanf("");
                    }
                    s_row *= ge;  // dlogits = p * g - [j == label] * g
                }
            } else {
                wait_pairs<G>(c.g, c.it, c.spin_limit, c.bcast, MergeSum{});
                r = __builtin_amdgcn_rsqf(c.bcast[0] / (float)N + eps);
                if (rstd && c.member == 0 && l == 0) rstd[row] = r;
            }
        };

        // pass 2, backwards (RMSNorm: the tile of w is loaded with the tile of x;
        // softmax backward: the tile of dy with the tile of y)
        constexpr int B2 = (OP == kLongSoftmax || OP == kLongXentGrad) ? P : 2 * P;
        walk_tiles<B2>(
            last_tile(c.member, G, tiles), -G, tiles,
            [&](float *v, int t) {
                load_part<E, C, R, VEC>(xv, tile(t), v);
                if constexpr (OP == kLongRmsnorm)
                    load_part<E, C, R, VEC, kReuseLoad>(RowView{wb, 0u, rb}, tile(t), v + P);
                if constexpr (OP == kLongSoftmaxBwd) load_part<E, C, R, VEC>(dv, tile(t), v + P);
            },
            [&](float *v, int t) {
                const bool full = part_full_at<E, C, R>(t * C * R, N);
                if constexpr (OP == kLongSoftmaxBwd) {
#pragma unroll
                    for (int j = 0; j < P; ++j) v[j] = v[j] * (v[P + j] - r);
                } else if constexpr (OP == kLongSoftmax || OP == kLongXentGrad) {
#pragma unroll
                    for (int j = 0; j < P; ++j) v[j] = exp_shift(v[j], m_row) * s_row;
                    if constexpr (OP == kLongXentGrad) {
                        if (ok) {
                            constexpr int VPC = E::VPC;
                            const Lane ln = tile(t);
#pragma unroll
                            for (int i = 0; i < C; ++i) {
                                const int d = label - ln.chunk(i) * VPC;
                                if ((unsigned)d < (unsigned)VPC) {
#pragma unroll
                                    for (int e = 0; e < VPC; ++e) v[i * VPC + e] -= (d == e) ? ge : 0.0f;
                                }
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < P; ++j) v[j] = v[j] * v[P + j] * r;
                }
                store_part<E, C, R, VEC>(yv, tile(t), N, true, full, v);
            },
            wait);
        ++c.it;
    }
    if (c.it > 0) depart_group<G>(c.g);
}

}  // namespace rr
