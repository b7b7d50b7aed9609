// packed_bf16.hpp -- RMSNorm stream kernel for bf16 rows kept packed.
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%), sections 硬件感知的加载与存储策略
// and 内存吞吐量, keeps a row in registers so that it is read from HBM once, and
// splits a row over more blocks only when one block cannot hold it.  The other
// stream kernels widen a bf16 row to fp32 as it arrives: P values per lane cost P
// VGPRs, so a 512-lane workgroup holds 64 KiB of a bf16 row against 128 KiB of an
// fp32 one, and a bf16 row needs twice the workgroups (and twice the exchanges per
// byte) of an fp32 row of the same bytes.  Here a lane keeps its part of the row
// as the raw 16-byte chunks it loaded, two bf16 values per VGPR, and unpacks a
// value where it is used (a 16-bit shift or a mask, exact):
//   * 128 values per lane, 65536 per 512-lane workgroup: a bf16 row of 262144
//     elements takes four workgroups instead of eight, one of 1048576 sixteen;
//   * the workgroup's slice of w stays packed in LDS (128 KiB).
// RMSNorm touches each value three times (square, scale, weight), so unpacking
// where used is cheap.  A softmax built the same way has to compute exp(x - M)
// twice (for the sum and for the output), since e = exp(x - m) no longer fits in
// fp32 registers; on MI355X that measured 0.4-8.5 % slower than the widened
// kernels at every length from 65536 to 1048576, so the softmax has no packed
// kernel.
// Only the 128-bit path (16-byte aligned rows) has this kernel.
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

constexpr int kPackedC = kPackedP / 8;  // 16-byte chunks per lane
constexpr int kPackedW = kPackedP / 2;  // 32-bit words per lane

__device__ __forceinline__ float bf16_lo(float w) { return __uint_as_float(__float_as_uint(w) << 16); }
__device__ __forceinline__ float bf16_hi(float w) {
    return __uint_as_float(__float_as_uint(w) & 0xFFFF0000u);
}
// Element j of a lane's packed part (word j / 2, low half first).
template <int J>
__device__ __forceinline__ float packed_elem(const float *raw) {
    return (J & 1) ? bf16_hi(raw[J / 2]) : bf16_lo(raw[J / 2]);
}

// Balanced pairwise combination of f(K0) .. f(K0 + N - 1), each leaf computed where
// it is used (so only about log2(N) partial results are live at once).
template <int N, int K0, class F, class Op>
__device__ __forceinline__ float tree_map(F f, Op op) {
    if constexpr (N == 1) {
        return f(std::integral_constant<int, K0>{});
    } else {
        constexpr int H = N / 2;
        return op(tree_map<H, K0>(f, op), tree_map<N - H, K0 + H>(f, op));
    }
}

// Sum of squares of this workgroup's packed part (chunks past the end of the row
// were read past the end of its buffer: zeros, which add nothing).
template <int R>
__device__ __forceinline__ float rmsnorm_packed_local(const float *raw, RowCtx &c) {
    const float q = tree_map<kPackedP, 0>(
        [&](auto J) {
            const float v = packed_elem<decltype(J)::value>(raw);
            return v * v;
        },
        OpSum{});
    return row_reduce<R>(q, c.one_reduction_slots(), c.l, OpSum{});
}

// y = (x * w) * r with r = rsqrt(Q / N + eps), w from the packed slice in LDS.
template <int R>
__device__ __forceinline__ void rmsnorm_packed_apply(const float *raw, const u32x4 *wslot, float Q,
                                                     RowView yv, float *rstd_out, float eps,
                                                     const RowCtx &c) {
    const float r = __builtin_amdgcn_rsqf(Q / (float)c.N + eps);
#pragma unroll
    for (int i = 0; i < kPackedC; ++i) {
        const int ch = c.ln.chunk(i);
        const u32x4 wq = wslot[i * R + c.l];
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float xw = raw[4 * i + q];
            const float ww = __uint_as_float(wq[q]);
            o[q] = pack_bf16x2((bf16_lo(xw) * bf16_lo(ww)) * r, (bf16_hi(xw) * bf16_hi(ww)) * r);
        }
        // yv ends where the row ends: the range check drops chunks past it
        buf_store16(yv.buf, yv.base + (uint32_t)ch * 16u, o);
    }
    if (rstd_out && c.l == 0 && c.member == 0) *rstd_out = r;
}

template <int R, int G>
__global__ void __launch_bounds__(R)
    rmsnorm_packed_kernel(const char *x, const char *w, char *y, float *rstd, int64_t M, int N,
                          float eps, uint8_t *ws, int groups, int spin_limit) {
    static_assert(R >= 64, "one row per workgroup");
    constexpr int W = R / 64;
    __shared__ float red[2][W];
    __shared__ float bcast[3];
    __shared__ u32x4 wslot[kPackedC * R];
    RowCtx c{N, (int)threadIdx.x, 0, 0, true, red[0], red[1], bcast, GroupRef{}, spin_limit};
    int group = blockIdx.x;
    if constexpr (G > 1) {
        member_of<G>(&group, &c.member);
        c.g = group_ref<G>(ws, group);
        if (threadIdx.x == 0) bcast[2] = 0.0f;  // read only after later barriers
    }
    c.ln = lane_of<kCfgRmsnorm, BF16, kPackedC, R, G>(c.member, c.l);
    const uint32_t rb = (uint32_t)N * 2u;

    // This workgroup's slice of w, packed, once; each lane later reads back only
    // the slots it wrote, so no barrier is needed.
    {
        const Buf wb = make_buf(w, rb);
#pragma unroll
        for (int i = 0; i < kPackedC; ++i)
            wslot[i * R + c.l] =
                buf_load16<kReuseLoad>(wb, (uint32_t)(c.ln.chunk(i)) * 16u);
    }

    if constexpr (kDeferredExchange && G >= kPackedDeferMinG) {
        // Split rows, deferred exchange (as in the other stream kernels): row k is
        // reduced and published before the workgroup waits for row k - 1's peers
        // and writes row k - 1, with the loads of row k + 1 in flight meanwhile.
        float buf[3][kPackedW];
        int64_t row = group;
        auto load = [&](float *v, int64_t r) {
            load_part_raw<BF16, kPackedC, R>(stream_row_view(x, r, M, rb), c.ln, v);
        };
        load(buf[0], row);
        load(buf[1], row + groups);
        auto step = [&](auto Kc) -> bool {
            constexpr int K = decltype(Kc)::value, KP = (K + 2) % 3;
            const bool more = row < M;
            if (more) {
                const float q = rmsnorm_packed_local<R>(buf[K], c);
                publish_pair<G>(c.g, c.member, c.it, q, 0.0f);
            } else {
                // no reduction (and its barriers) in this step: every wave has read
                // the previous row's merged sum before wave 0 writes the next one
                __syncthreads();
            }
            if (c.it > 0) {  // complete the previous row
                wait_pairs<G>(c.g, c.it - 1, c.spin_limit, c.bcast, MergeSum{});
                const int64_t rp = row - groups;
                rmsnorm_packed_apply<R>(buf[KP], wslot, c.bcast[0], stream_row_view(y, rp, M, rb),
                                        rstd ? rstd + rp : nullptr, eps, c);
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
    float buf[2][kPackedW];
    stream_rows<2>(
        (int64_t)group, M, groups, buf,
        [&](float *v, int64_t r) {
            load_part_raw<BF16, kPackedC, R>(stream_row_view(x, r, M, rb), c.ln, v);
        },
        [&](float *v, int64_t r) {
            float q = rmsnorm_packed_local<R>(v, c);
            if constexpr (G > 1) {
                exchange_pairs<G>(c.g, c.member, c.it, q, 0.0f, c.spin_limit, c.bcast, MergeSum{});
                q = c.bcast[0];
            }
            rmsnorm_packed_apply<R>(v, wslot, q, stream_row_view(y, r, M, rb),
                                    rstd ? rstd + r : nullptr, eps, c);
            ++c.it;
        });
    }
    if constexpr (G > 1) {
        if (c.it > 0) depart_group<G>(c.g);
    }
}

}  // namespace rr
