// row_kernels.hpp -- softmax and RMSNorm forward with the row held in registers.
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%): the closing paragraph of
// section 内存吞吐量 describes softmax as the conventional three passes (row max,
// exponential sum, normalise) over data already on chip, so each element is read
// from HBM once and written once (section NCU 性能分析（Softmax 内核）: one extra
// global load costs a third of the effective bandwidth).  RMSNorm reuses the same
// layout, load/store and reduction helpers (section 总结).
//
// One kernel template per op, parameterised by
//   E  element type (F32 / BF16),  P  fp32 values per lane,  R  lanes per row,
//   G  workgroups per row,  VEC  128-bit path or per-element path.
// With G == 1 each workgroup handles rows_per_block_for(R) rows, one per lane
// group, and the grid has one workgroup per such set of rows.  With G > 1 the
// grid is cooperative and persistent: each row group of G workgroups loops over
// rows group, group + groups, ... and meets its peers in the workspace.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "configs.hpp"
#include "grid_exchange.hpp"
#include "reduce.hpp"
#include "row_io.hpp"
#include "vec_io.hpp"

namespace rr {

// Lane-group index inside the block.  For R >= 64 it is the same for the whole
// wave, which lets the compiler keep row addresses in scalar registers.
template <int R>
__device__ __forceinline__ int lane_group() {
    const int t = threadIdx.x / R;
    if constexpr (R >= 64) return __builtin_amdgcn_readfirstlane(t);
    return t;
}

// The row of lane group `sub` of this block (G == 1).  Rows past M are clamped
// (R >= 64) or lie past the end of the block's buffer (R < 64); either way they
// are only read, never written.
template <int R>
__device__ __forceinline__ RowView block_row_view(const char *base, int64_t M, int sub,
                                                  uint32_t row_bytes) {
    constexpr int RPB = rows_per_block_for(R);
    const int64_t first = (int64_t)blockIdx.x * RPB;
    if constexpr (R >= 64) {
        int64_t row = first + sub;
        if (row >= M) row = M - 1;
        return {make_buf(base + row * row_bytes, row_bytes), 0u};
    } else {
        const int64_t left = M - first;
        const uint32_t nrows = (uint32_t)(left < RPB ? left : RPB);
        return {make_buf(base + first * row_bytes, nrows * row_bytes), (uint32_t)sub * row_bytes};
    }
}

// Everything a row body needs besides the row buffers.
struct RowCtx {
    int N;
    int l;          // lane within the row's lane group
    int member;     // workgroup index within the row (0 when G == 1)
    int it;         // row iteration of this workgroup (grid path)
    bool full;      // this lane group's part of the row has no padding
    float *red_a;   // LDS slots of this row, first reduction
    float *red_b;   // LDS slots of this row, second reduction
    float *bcast;   // LDS: merged grid partials [0..1], "a wait timed out" flag [2]
    GroupRef g;
    int spin_limit;
};

// ---------------------------------------------------------------- softmax

struct MergeMaxSum {
    __device__ __forceinline__ void operator()(float &m, float &s, float mj, float sj) const {
        MaxSum r = merge(MaxSum{m, s}, MaxSum{mj, sj});
        m = r.m;
        s = r.s;
    }
};

template <class E, int P, int R, int G, bool VEC>
__device__ __forceinline__ void softmax_row(RowView xv, RowView yv, bool valid, RowCtx &c) {
    constexpr int C = P / E::VPC;
    const int chunk0 = c.member * C * R;
    float v[P];
    load_part<E, C, R, VEC>(xv, chunk0, c.l, v);
    if (!c.full) mask_part<E, C, R>(chunk0, c.l, c.N, -INFINITY, v);

    // pass 1: row max
    float m = tree_reduce<P>(v, OpMax{});
    m = row_reduce<R>(m, c.red_a, c.l, OpMax{});

    // pass 2: e = exp(x - m) kept in place (padding: exp(-inf) = 0), and its sum
    const float mu = safe_max(m);
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] = exp_shift(v[j], mu);
    float s = tree_reduce<P>(v, OpSum{});
    s = row_reduce<R>(s, c.red_b, c.l, OpSum{});

    // pass 3: normalise (a split row first merges the G partial (max, sum) pairs)
    float scale;
    if constexpr (G == 1) {
        scale = __builtin_amdgcn_rcpf(s);
    } else {
        exchange_pairs<G>(c.g, c.member, c.it, m, s, c.spin_limit, c.bcast, MergeMaxSum{});
        const float M = c.bcast[0], S = c.bcast[1];
        scale = exp_shift(m, safe_max(M)) * __builtin_amdgcn_rcpf(S);
    }
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] *= scale;
    store_part<E, C, R, VEC>(yv, chunk0, c.l, c.N, valid, c.full, v);
}

template <class E, int P, int R, int G, bool VEC>
__global__ void __launch_bounds__(block_threads_for(R))
    softmax_kernel(const char *x, char *y, int64_t M, int N, uint8_t *ws, int groups,
                   int spin_limit) {
    constexpr int C = P / E::VPC;
    constexpr int RPB = rows_per_block_for(R);
    constexpr int W = R > 64 ? R / 64 : 1;
    __shared__ float red_max[RPB * W];
    __shared__ float red_sum[RPB * W];
    __shared__ float bcast[3];
    const int sub = lane_group<R>();
    const uint32_t row_bytes = (uint32_t)N * E::BYTES;
    RowCtx c{N, (int)(threadIdx.x % R), 0, 0, true, red_max + sub * W, red_sum + sub * W, bcast,
             GroupRef{}, spin_limit};

    if constexpr (G == 1) {
        c.full = part_full<E, C, R>(0, N);
        const bool valid = (int64_t)blockIdx.x * RPB + sub < M;
        softmax_row<E, P, R, 1, VEC>(block_row_view<R>(x, M, sub, row_bytes),
                                     block_row_view<R>(y, M, sub, row_bytes), valid, c);
    } else {
        static_assert(RPB == 1, "split rows use one row per workgroup");
        int group;
        group_of_block<G>(groups, &group, &c.member);
        c.g = group_ref<G>(ws, group);
        c.full = part_full<E, C, R>(c.member * C * R, N);
        if (threadIdx.x == 0) bcast[2] = 0.0f;  // ordered before its first read by two barriers
        for (int64_t row = group; row < M; row += groups, ++c.it) {
            const RowView xv{make_buf(x + row * row_bytes, row_bytes), 0u};
            const RowView yv{make_buf(y + row * row_bytes, row_bytes), 0u};
            softmax_row<E, P, R, G, VEC>(xv, yv, true, c);
        }
        if (c.it > 0) depart_group<G>(c.g);
    }
}

// ---------------------------------------------------------------- RMSNorm

struct MergeSum {
    __device__ __forceinline__ void operator()(float &q, float &unused, float qj, float) const {
        q = q + qj;
        unused = 0.0f;
    }
};

template <class E, int P, int R, int G, bool VEC>
__device__ __forceinline__ void rmsnorm_row(RowView xv, RowView wview, RowView yv,
                                            float *rstd_out, float eps, bool valid,
                                            RowCtx &c) {
    constexpr int C = P / E::VPC;
    const int chunk0 = c.member * C * R;
    float v[P];
    load_part<E, C, R, VEC>(xv, chunk0, c.l, v);
    float wv[P];
    load_part<E, C, R, VEC>(wview, chunk0, c.l, wv);
    if (!c.full) mask_part<E, C, R>(chunk0, c.l, c.N, 0.0f, v);

    // sum of squares, then t = x * w in place; y = t * r once r is known
    float sq[P];
#pragma unroll
    for (int j = 0; j < P; ++j) sq[j] = v[j] * v[j];
    float q = tree_reduce<P>(sq, OpSum{});
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] *= wv[j];
    q = row_reduce<R>(q, c.red_a, c.l, OpSum{});
    if constexpr (G > 1) {
        exchange_pairs<G>(c.g, c.member, c.it, q, 0.0f, c.spin_limit, c.bcast, MergeSum{});
        q = c.bcast[0];
    }
    const float r = __builtin_amdgcn_rsqf(q / (float)c.N + eps);
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] *= r;
    store_part<E, C, R, VEC>(yv, chunk0, c.l, c.N, valid, c.full, v);
    if (rstd_out && valid && c.l == 0 && c.member == 0) *rstd_out = r;
}

template <class E, int P, int R, int G, bool VEC>
__global__ void __launch_bounds__(block_threads_for(R))
    rmsnorm_kernel(const char *x, const char *w, char *y, float *rstd, int64_t M, int N,
                   float eps, uint8_t *ws, int groups, int spin_limit) {
    constexpr int C = P / E::VPC;
    constexpr int RPB = rows_per_block_for(R);
    constexpr int W = R > 64 ? R / 64 : 1;
    __shared__ float red[RPB * W];
    __shared__ float bcast[3];
    const int sub = lane_group<R>();
    const uint32_t row_bytes = (uint32_t)N * E::BYTES;
    const RowView wview{make_buf(w, row_bytes), 0u};
    RowCtx c{N, (int)(threadIdx.x % R), 0, 0, true, red + sub * W, nullptr, bcast, GroupRef{},
             spin_limit};

    if constexpr (G == 1) {
        c.full = part_full<E, C, R>(0, N);
        const int64_t row = (int64_t)blockIdx.x * RPB + sub;
        const bool valid = row < M;
        rmsnorm_row<E, P, R, 1, VEC>(block_row_view<R>(x, M, sub, row_bytes), wview,
                                     block_row_view<R>(y, M, sub, row_bytes),
                                     rstd ? rstd + row : nullptr, eps, valid, c);
    } else {
        static_assert(RPB == 1, "split rows use one row per workgroup");
        int group;
        group_of_block<G>(groups, &group, &c.member);
        c.g = group_ref<G>(ws, group);
        c.full = part_full<E, C, R>(c.member * C * R, N);
        if (threadIdx.x == 0) bcast[2] = 0.0f;  // ordered before its first read by a barrier
        // `red` and `bcast` are rewritten every row; each write comes after a
        // barrier that all readers of the previous row have passed.
        for (int64_t row = group; row < M; row += groups, ++c.it) {
            const RowView xv{make_buf(x + row * row_bytes, row_bytes), 0u};
            const RowView yv{make_buf(y + row * row_bytes, row_bytes), 0u};
            rmsnorm_row<E, P, R, G, VEC>(xv, wview, yv, rstd ? rstd + row : nullptr, eps, true, c);
        }
        if (c.it > 0) depart_group<G>(c.g);
    }
}

}  // namespace rr
