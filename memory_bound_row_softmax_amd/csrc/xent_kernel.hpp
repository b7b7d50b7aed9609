// xent_kernel.hpp -- cross-entropy forward: lse = logsumexp(row), loss = lse - row[label].
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%), section 让内存密集型内核达到"光速",
// lists the cross-entropy loss among its three memory-bound kernels.  It writes
// no per-element output, so the row need not stay on chip: the R lanes of a row
// stream it P values per lane per step, each lane keeping a running (max, sum of
// exp) pair (the online-softmax rescaling), and the pairs are merged across lanes
// at the end.  The lane that loads the label's column keeps that value (no extra
// read), and writes the loss once the merged lse is known.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "configs.hpp"
#include "reduce.hpp"
#include "row_io.hpp"
#include "row_kernels.hpp"
#include "vec_io.hpp"

namespace rr {

template <class E, int P, int R, bool VEC>
__global__ void __launch_bounds__(block_threads_for(R))
    xent_kernel(const char *x, const int32_t *labels, float *loss, float *lse, int64_t M, int N) {
    constexpr int VPC = E::VPC;
    constexpr int C = P / VPC;
    constexpr int RPB = rows_per_block_for(R);
    constexpr int W = R > 64 ? R / 64 : 1;
    __shared__ MaxSum red[RPB * W];

    const int sub = lane_group<R>();
    const int l = threadIdx.x % R;
    const int64_t r0 = (int64_t)blockIdx.x * RPB + sub;
    const bool valid = r0 < M;
    const int64_t row = valid ? r0 : M - 1;
    const RowView xv = block_row_view<R>(x, M, sub, (uint32_t)N * E::BYTES);
    const int label = labels[row];

    const int step = C * R;  // chunks per step for the whole lane group
    const int steps = (int)(((int64_t)N + (int64_t)step * VPC - 1) / ((int64_t)step * VPC));

    MaxSum acc = {-INFINITY, 0.0f};
    float x_label = 0.0f;
    bool has_label = false;
    for (int k = 0; k < steps; ++k) {
        float v[P];
        const Lane ln = {k * step + l, R};
        load_part<E, C, R, VEC>(xv, ln, v);
        if (!part_full_at<E, C, R>(k * step, N)) mask_part<E, C, R>(ln, N, -INFINITY, v);
        // keep row[label] if this lane loaded it
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int d = label - ln.chunk(i) * VPC;
            if ((unsigned)d < (unsigned)VPC) {
#pragma unroll
                for (int e = 0; e < VPC; ++e)
                    if (d == e) x_label = v[i * VPC + e];
                has_label = true;
            }
        }
        const float mnew = fmaxf(acc.m, tree_reduce<P>(v, OpMax{}));
        const float mu = safe_max(mnew);
#pragma unroll
        for (int j = 0; j < P; ++j) v[j] = exp_shift(v[j], mu);
        acc.s = acc.s * exp_shift(acc.m, mu) + tree_reduce<P>(v, OpSum{});
        acc.m = mnew;
    }
    acc = row_reduce<R>(acc, red + sub * W, l, OpMerge{});

    const float row_lse = acc.m + __builtin_amdgcn_logf(acc.s) * kLn2;
    if (valid) {
        const bool label_ok = label >= 0 && label < N;
        if (l == 0) {
            if (lse) lse[row] = row_lse;
            if (!label_ok) loss[row] = __builtin_nanf("");
        }
        if (label_ok && has_label) loss[row] = row_lse - x_label;
    }
}

}  // namespace rr
