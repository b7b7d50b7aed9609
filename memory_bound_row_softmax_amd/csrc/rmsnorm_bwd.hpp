// rmsnorm_bwd.hpp -- RMSNorm backward from x, w, the upstream gradient dy and the
// forward's rstd r (per row):
//     c = sum_k dy_k w_k x_k,   dx_j = r (w_j dy_j - x_j r^2 c / N),
//     dw_j = sum_i dy_ij x_ij r_i   (over all rows).
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%), section 让内存密集型内核达到"光速",
// names RMSNorm among its memory-bound kernels and presents them as building blocks
// of training as well as inference; the gradient is the textbook derivative of the
// forward (eps inside the root, weight, no bias).  dx is a row reduction of the
// forward's shape: x and dy read once, dx written once.  dw is a reduction down the
// columns, over all M rows: every persistent workgroup keeps the partial sums of its
// columns in registers across the rows it processes, combines its lane groups
// through LDS and writes one fp32 partial row to the workspace; one small pass
// (rmsnorm_dw_reduce) then adds the partial rows in a fixed order, so dw is the
// same bits on every run.  A workgroup's running sums over its M / 256 rows do not
// round once per row (DwAcc below), so the error of dw does not grow with M: the
// steps after them (the fp32 partial row, the lane-group combine and the reduce
// pass) round a bounded number of times.
//
// Kernel: a persistent grid; with G = 1 a workgroup holds rows_per_block_for(R)
// rows at a time (R lanes each) and walks the row blocks group, group + groups,
// ...; with G > 1 the G workgroups of a row group split each row and exchange the
// partial c through the workspace (as RMSNorm's sum of squares).  Each workgroup
// keeps two row buffers (x, dy and r of the next rows in flight while the current
// ones are finished) and its dw partials in registers, and its slice of w in LDS.
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

// Row block `blk` (rows blk * RPB ...) of a persistent kernel, lane group `sub`.
// Rows past M read 0 (past the end of the buffer) and are never written.
template <int R>
__device__ __forceinline__ RowView rows_view(const char *base, int64_t M, int64_t blk, int sub,
                                             uint32_t row_bytes) {
    constexpr int RPB = rows_per_block_for(R);
    const int64_t first = blk * RPB;
    if (first >= M) return {make_buf(base, 0u), 0u, 0u};
    if constexpr (R >= 64) {
        // the buffer holds only this row: the range check drops what lies past its end
        if constexpr (RPB == 1)
            return {make_buf(base + first * row_bytes, row_bytes), 0u, row_bytes};
        int64_t row = first + sub;
        const bool ok = row < M;
        return {make_buf(base + (ok ? row : 0) * row_bytes, ok ? row_bytes : 0u), 0u, row_bytes};
    } else {
        const int64_t left = M - first;
        const uint32_t nrows = (uint32_t)(left < RPB ? left : RPB);
        return {make_buf(base + first * row_bytes, nrows * row_bytes), (uint32_t)sub * row_bytes,
                (uint32_t)(sub + 1) * row_bytes};
    }
}

// Stores P fp32 values of a lane (the element layout of E) into an fp32 row.
template <class E, int C, int R>
__device__ __forceinline__ void store_part_f32(Buf b, Lane ln, int N, const float *v) {
    constexpr int VPC = E::VPC;
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int first = ln.chunk(i) * VPC;
#pragma unroll
        for (int q = 0; q < VPC / 4; ++q) {
            const int e0 = first + 4 * q;
            if (e0 + 4 <= N) {
                u32x4 u = {__float_as_uint(v[i * VPC + 4 * q]), __float_as_uint(v[i * VPC + 4 * q + 1]),
                           __float_as_uint(v[i * VPC + 4 * q + 2]), __float_as_uint(v[i * VPC + 4 * q + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(u, b.rsrc, e0 * 4, 0, 0);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e0 + e < N)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            __float_as_uint(v[i * VPC + 4 * q + e]), b.rsrc, (e0 + e) * 4, 0, 0);
            }
        }
    }
}

// The dw running sums of a lane's P columns.  Each term dy * x * r is formed in fp32.
// Wide: the sums are fp64 registers, so adding a term rounds at 2^-53 and n terms
// stay within n * 2^-53 of the exact sum of the fp32 terms.  Compensated (for the
// kernels whose registers cannot hold P more): fp32 sums with Kahan compensation,
// the compensation terms in LDS (P * T floats); the sum of n terms is then within
// about 2^-23 of the exact sum, whatever n is.
template <int P, bool WIDE>
struct DwAcc;

template <int P>
struct DwAcc<P, true> {
    double s[P];
    __device__ __forceinline__ void init(float *) {
#pragma unroll
        for (int j = 0; j < P; ++j) s[j] = 0.0;
    }
    __device__ __forceinline__ void add(int j, float t) { s[j] += (double)t; }
    __device__ __forceinline__ float get(int j) const { return (float)s[j]; }
};

template <int P>
struct DwAcc<P, false> {
    float s[P];
    float *comp;  // this thread's compensation terms: comp[j * T]
    int stride;
    __device__ __forceinline__ void init(float *c) {
        comp = c;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            s[j] = 0.0f;
            comp[j * stride] = 0.0f;
        }
    }
    __device__ __forceinline__ void add(int j, float t) {
        const float y = t - comp[j * stride];
        const float n = s[j] + y;
        comp[j * stride] = (n - s[j]) - y;
        s[j] = n;
    }
    __device__ __forceinline__ float get(int j) const { return s[j]; }
};

// fp64 sums need P more registers than fp32 ones; the kernels with 32 values on 512
// lanes (1 workgroup per CU, 256 registers a lane) whose other registers already fill
// most of that budget take the compensated sums instead: fp32 rows, and bf16 rows
// on the per-element path.
template <class E, int P, int R, bool VEC>
constexpr bool dw_wide() {
    return !(P == 32 && R >= 512 && (E::BYTES == 4 || !VEC));
}

// a: x, b: dy of the lane's part of a row (b is reused); wsrc: w; acc: dw partials.
template <class E, int P, int R, int G, bool VEC, class Acc>
__device__ __forceinline__ void rmsnorm_bwd_finish(float *a, float *b, float r,
                                                   const WeightLds<P, R> &wsrc, Acc &acc,
                                                   RowView dxv, bool valid, RowCtx &c) {
    constexpr int C = P / E::VPC;
    if (!c.full) {
        mask_part<E, C, R, true>(c.ln, c.N, 0.0f, a);
        mask_part<E, C, R, true>(c.ln, c.N, 0.0f, b);
    }
    // dw partial first (before b is overwritten): dy * x * r
#pragma unroll
    for (int j = 0; j < P; ++j) acc.add(j, (b[j] * a[j]) * r);
    // b <- w * dy, then c = sum (w dy) x
    wsrc.apply(b, c.l);
    float t = tree_dot<P>(b, a);
    t = row_reduce<R>(t, c.one_reduction_slots(), c.l, OpSum{});
    if constexpr (G > 1) {
        exchange_pairs<G>(c.g, c.member, c.it, t, 0.0f, c.spin_limit, c.bcast, MergeSum{});
        t = c.bcast[0];
    }
    const float k = r * r * t / (float)c.N;
#pragma unroll
    for (int j = 0; j < P; ++j) a[j] = r * (b[j] - a[j] * k);
    store_part<E, C, R, VEC, true>(dxv, c.ln, c.N, valid, c.full, a);
}

constexpr int bwd_threads(int R, int G) { return G == 1 ? block_threads_for(R) : R; }

template <class E, int P, int R, int G, bool VEC>
__global__ void __launch_bounds__(bwd_threads(R, G))
    __attribute__((amdgpu_waves_per_eu(stream_waves(kCfgRmsnormBwd, E::BYTES, VEC, P, R, G))))
    rmsnorm_bwd_kernel(const char *x, const char *w, const char *dy, const float *rstd, char *dx,
                       float *partial, int64_t M, int N, uint8_t *ws, int groups,
                       int spin_limit) {
    static_assert(G == 1 || R >= 64, "split rows take whole waves");
    constexpr int C = P / E::VPC;
    constexpr int RPB = G == 1 ? rows_per_block_for(R) : 1;
    constexpr int W = R > 64 ? R / 64 : 1;
    constexpr int T = bwd_threads(R, G);
    __shared__ float red[2][RPB * W];
    __shared__ float bcast[3];
    const int sub = G == 1 ? lane_group<R>() : 0;
    const int l = threadIdx.x % R;
    RowCtx c{N, l, 0, 0, true, red[0] + sub * W, red[1] + sub * W, bcast, GroupRef{}, spin_limit};
    int group = blockIdx.x;
    if constexpr (G > 1) {
        member_of<G>(&group, &c.member);
        c.g = group_ref<G>(ws, group);
        if (threadIdx.x == 0) bcast[2] = 0.0f;  // read only after later barriers
    }
    c.ln = lane_of<kCfgRmsnorm, E, C, R, G>(c.member, l);
    c.full = part_full<kCfgRmsnorm, E, C, R, G>(c.member, N);
    const uint32_t rb = (uint32_t)N * E::BYTES;
    const int64_t nblk = (M + RPB - 1) / RPB;

    // The workgroup's slice of w, once, decoded to fp32 in LDS (the lane groups of a
    // workgroup share its columns).
    __shared__ float4 wslot[(P / 4) * R];
    if (sub == 0) {
        float t[P];
        load_part<E, C, R, VEC, kReuseLoad>(RowView{make_buf(w, rb), 0u, rb}, c.ln, t);
#pragma unroll
        for (int q = 0; q < P / 4; ++q)
            wslot[q * R + l] = make_float4(t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]);
    }
    if constexpr (RPB > 1) __syncthreads();
    const WeightLds<P, R> wsrc{wslot};
    constexpr bool kWide = dw_wide<E, P, R, VEC>();
    __shared__ float dw_comp[kWide ? 1 : P * T];
    DwAcc<P, kWide> acc;
    if constexpr (!kWide) acc.stride = T;
    acc.init(dw_comp + threadIdx.x);  // each thread reads back only what it wrote

    // buffer: x (P), dy (P), r (1)
    float buf[2][2 * P + 1];
    stream_rows<2>(
        (int64_t)group, nblk, groups, buf,
        [&](float *v, int64_t blk) {
            load_part<E, C, R, VEC>(rows_view<R>(x, M, blk, sub, rb), c.ln, v);
            load_part<E, C, R, VEC>(rows_view<R>(dy, M, blk, sub, rb), c.ln, v + P);
            const int64_t row = blk * RPB + sub;
            v[2 * P] = (blk < nblk) ? rstd[row < M ? row : M - 1] : 0.0f;
        },
        [&](float *v, int64_t blk) {
            const int64_t row = blk * RPB + sub;
            rmsnorm_bwd_finish<E, P, R, G, VEC>(v, v + P, v[2 * P], wsrc, acc,
                                                rows_view<R>(dx, M, blk, sub, rb), row < M, c);
            ++c.it;
        });
    if constexpr (G > 1) {
        if (c.it > 0) depart_group<G>(c.g);
    }

    // One partial row per workgroup (its lane groups summed in order through LDS,
    // in fp32).
    float part[P];
#pragma unroll
    for (int j = 0; j < P; ++j) part[j] = acc.get(j);
    if constexpr (RPB > 1) {
        __shared__ float comb[T * P];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < P; ++j) comb[j * T + threadIdx.x] = part[j];
        __syncthreads();
        if (sub == 0) {
#pragma unroll
            for (int j = 0; j < P; ++j) {
                float s = comb[j * T + l];
#pragma unroll
                for (int q = 1; q < RPB; ++q) s += comb[j * T + q * R + l];
                part[j] = s;
            }
        }
    }
    if (sub == 0) {
        const Buf pb = make_buf(partial + (int64_t)group * N, (uint32_t)N * 4u);
        store_part_f32<E, C, R>(pb, c.ln, N, part);  // this member's columns only
    }
}

// dw = the sum of the `rows` partial rows of `in` (rows x N fp32), one pass.  A
// workgroup owns a tile of kDwTileQuads * 4 columns; its thread (g, q) adds column
// quad q of rows g, g + kDwRowGroups, ... in row order (eight loads in flight), and
// the kDwRowGroups sums of a quad are then added pairwise through LDS.  The order
// of the additions is fixed, so dw is the same bits on every run.  `in` is
// 16-byte aligned and N is a multiple of 4 when VEC4.
constexpr int kDwTileQuads = 8;
constexpr int kDwRowGroups = 256 / kDwTileQuads;

template <bool VEC4>
__device__ __forceinline__ float4 dw_load4(const float *p, int col, int N) {
    if constexpr (VEC4) {
        return *reinterpret_cast<const float4 *>(p);
    } else {
        return make_float4(col < N ? p[0] : 0.0f, col + 1 < N ? p[1] : 0.0f,
                           col + 2 < N ? p[2] : 0.0f, col + 3 < N ? p[3] : 0.0f);
    }
}

template <bool VEC4>
__global__ void __launch_bounds__(256) rmsnorm_dw_reduce(const float *in, int rows, int N, float *dw) {
    constexpr int U = 8;
    __shared__ float4 sums[kDwRowGroups][kDwTileQuads];
    const int q = threadIdx.x % kDwTileQuads, g = threadIdx.x / kDwTileQuads;
    const int col = (blockIdx.x * kDwTileQuads + q) * 4;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (col < N) {
        int r = g;
        for (; r + (U - 1) * kDwRowGroups < rows; r += U * kDwRowGroups) {
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = dw_load4<VEC4>(in + (int64_t)(r + u * kDwRowGroups) * N + col, col, N);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                acc.x += v[u].x;
                acc.y += v[u].y;
                acc.z += v[u].z;
                acc.w += v[u].w;
            }
        }
        for (; r < rows; r += kDwRowGroups) {
            const float4 v = dw_load4<VEC4>(in + (int64_t)r * N + col, col, N);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
    }
    // the row groups' sums, added pairwise (a tree of log2(kDwRowGroups) levels)
    sums[g][q] = acc;
    __syncthreads();
#pragma unroll
    for (int h = kDwRowGroups / 2; h >= 1; h /= 2) {
        if (g < h) {
            const float4 v = sums[g + h][q];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
            sums[g][q] = acc;
        }
        __syncthreads();
    }
    if (g == 0 && col < N) {
        const float o[4] = {acc.x, acc.y, acc.z, acc.w};  // dw need not be 16-byte aligned
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (col + e < N) dw[col + e] = o[e];
    }
}

}  // namespace rr
