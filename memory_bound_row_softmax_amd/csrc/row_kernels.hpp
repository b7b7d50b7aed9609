// row_kernels.hpp -- softmax and RMSNorm forward with the row held in registers.
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%): the closing paragraph of
// section 内存吞吐量 describes softmax as the conventional three passes (row max,
// exponential sum, normalise) over data already on chip, so each element is read
// from HBM once and written once (section NCU 性能分析（Softmax 内核）: one extra
// global load costs a third of the effective bandwidth).  RMSNorm reuses the same
// layout, load/store and reduction helpers (section 总结).
//
// Template parameters: E element type (F32 / BF16), P fp32 values per lane per
// row, R lanes per row, G workgroups per row, VEC 128-bit path or per-element
// path.  Two kernel kinds per op (see configs.hpp): block kernels (G = 1, one
// workgroup per few rows) and stream kernels (persistent, one row per workgroup
// at a time, the next row's loads issued before the current row is reduced;
// with G > 1 the G consecutive blocks of a row group meet in the workspace, each
// holding an interleaved share of the row: row_io.hpp, lane_of).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

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

// The row of lane group `sub` of this block (block kernels).  Rows past M are
// clamped (R >= 64) or lie past the end of the block's buffer (R < 64); either
// way they are only read, never written.
template <int R>
__device__ __forceinline__ RowView block_row_view(const char *base, int64_t M, int sub,
                                                  uint32_t row_bytes) {
    constexpr int RPB = rows_per_block_for(R);
    const int64_t first = (int64_t)blockIdx.x * RPB;
    if constexpr (R >= 64) {
        int64_t row = first + sub;
        if (row >= M) row = M - 1;
        return {make_buf(base + row * row_bytes, row_bytes), 0u, row_bytes};
    } else {
        const int64_t left = M - first;
        const uint32_t nrows = (uint32_t)(left < RPB ? left : RPB);
        return {make_buf(base + first * row_bytes, nrows * row_bytes), (uint32_t)sub * row_bytes,
                (uint32_t)(sub + 1) * row_bytes};
    }
}

// Row `row` of a stream kernel; past the last row the buffer is empty, so its
// loads return 0 without touching memory.
__device__ __forceinline__ RowView stream_row_view(const char *base, int64_t row, int64_t M,
                                                   uint32_t row_bytes) {
    const bool ok = row < M;
    return {make_buf(base + (ok ? row : 0) * row_bytes, ok ? row_bytes : 0u), 0u, row_bytes};
}

// Row loop of the stream kernels with D register buffers.  Rows group,
// group + groups, ... < M are processed in order; buffer k % D holds the k-th of
// them.  Before row k is finished, the loads of row k + D - 1 are issued, so
// D - 1 rows are in flight while one is reduced and written.  Loads past the
// last row read an empty buffer (no memory traffic).  `row` is the same for the
// whole workgroup, so every branch here is uniform.
template <int K, int D, class Step>
__device__ __forceinline__ bool stream_steps(Step &step) {
    if constexpr (K == D) {
        return true;
    } else {
        if (!step(std::integral_constant<int, K>{})) return false;
        return stream_steps<K + 1, D>(step);
    }
}

template <int D, int P, class Load, class Finish>
__device__ __forceinline__ void stream_rows(int64_t row, int64_t M, int groups, float (&buf)[D][P],
                                            Load load, Finish finish) {
    static_assert(D >= 2, "at least one row in flight");
#pragma unroll
    for (int k = 0; k < D - 1; ++k) load(buf[k], row + (int64_t)k * groups);
    auto step = [&](auto K) -> bool {
        constexpr int k = decltype(K)::value;
        if (row >= M) return false;
        load(buf[(k + D - 1) % D], row + (int64_t)(D - 1) * groups);
        finish(buf[k], row);
        row += groups;
        return true;
    };
    while (stream_steps<0, D>(step)) {
    }
}

// Everything a row body needs besides the row buffers.
struct RowCtx {
    int N;
    int l;          // lane within the row's lane group
    int member;     // workgroup index within the row (0 when G == 1)
    int it;         // row iteration of this workgroup (stream kernels)
    bool full;      // this lane group's part of the row has no padding
    float *red_a;   // LDS slots of this row, first reduction
    float *red_b;   // LDS slots of this row, second reduction
    float *bcast;   // LDS: merged split-row partials [0..1], "a wait timed out" flag [2]
    GroupRef g;
    int spin_limit;
    Lane ln = {0, 0};  // where this lane's chunks lie in the row (lane_of)

    // Slots for a row body with a single reduction.  A slot array may be written
    // again only after a later barrier (waves_combine), so a persistent kernel
    // alternates its two arrays from row to row: the barrier of row k + 1's
    // reduction separates the last read of row k's slots from row k + 2's writes.
    __device__ __forceinline__ float *one_reduction_slots() const {
        return (it & 1) ? red_b : red_a;
    }
};

// ---------------------------------------------------------------- softmax

// Merges of the split-row partials (grid_exchange.hpp): two pairs, or the pairs of
// W lanes by a butterfly; kEmpty* is the pair of a lane with no member.
struct MergeMaxSum {
    static constexpr float kEmptyA = -__builtin_inff(), kEmptyB = 0.0f;
    __device__ __forceinline__ void operator()(float &m, float &s, float mj, float sj) const {
        MaxSum r = merge(MaxSum{m, s}, MaxSum{mj, sj});
        m = r.m;
        s = r.s;
    }
    template <int W>
    __device__ __forceinline__ static void lanes(float &m, float &s) {
        MaxSum r = lanes_reduce<W>(MaxSum{m, s}, OpMerge{});
        m = r.m;
        s = r.s;
    }
};

// What a softmax kernel writes for a row, given e_j = exp(x_j - mu) in registers
// and the factor `scale` that turns e_j into the softmax p_j.  An output policy
// `Out` (a kernel argument) hands out one Epi per row:
//   capture<E, C, R, G, STREAM>(v, ctx)  sees the lane's raw values before the exp;
//   apply<E, C, R, STREAM>(v, scale, mu, M, S, ctx, valid)  turns e = exp(x - mu)
//                                   into the values to store and writes any
//                                   per-row outputs (M, S: the row's max and sum
//                                   of exp(x - M));
//   fixup<E, R, STREAM>(yv, valid)  runs after the lane's stores of the row.
// A stream kernel keeps kExtra more registers per row buffer for the row's own
// inputs: stash(extra, r) fills them when the row's loads are issued (so they
// arrive with the row), and epi(extra, r) builds the Epi when the row is
// finished.  Plain softmax stores p_j and has no per-row inputs.
struct SoftmaxOut {
    static constexpr int kCfg = kCfgSoftmax;  // configuration menu predicates
    static constexpr int kExtra = 0;
    struct Epi {
        template <class E, int C, int R, int G, bool STREAM>
        __device__ __forceinline__ void capture(const float *, const RowCtx &) {}
        template <class E, int C, int R, bool STREAM>
        __device__ __forceinline__ void apply(float *v, float scale, float, float, float,
                                              const RowCtx &, bool) {
#pragma unroll
            for (int j = 0; j < C * E::VPC; ++j) v[j] *= scale;
        }
        template <class E, int R, bool STREAM>
        __device__ __forceinline__ void fixup(RowView, bool) {}
    };
    __device__ __forceinline__ Epi row(int64_t) const { return {}; }
    __device__ __forceinline__ void stash(float *, int64_t) const {}
    __device__ __forceinline__ Epi epi(const float *, int64_t) const { return {}; }
};

// Passes 1 and 2 on a lane's loaded part v of the row: the row max m (over this
// workgroup's part), e = exp(x - m) in place and its sum s.
template <class E, int P, int R, int G, bool STREAM, class Epi>
__device__ __forceinline__ MaxSum softmax_local(float *v, RowCtx &c, Epi &epi) {
    constexpr int C = P / E::VPC;
    epi.template capture<E, C, R, G, STREAM>(v, c);
    if (!c.full) mask_part<E, C, R, STREAM>(c.ln, c.N, -INFINITY, v);

    // pass 1: row max
    float m = tree_reduce<P>(v, OpMax{});
    m = row_reduce<R>(m, c.red_a, c.l, OpMax{});

    // pass 2: e = exp(x - m) kept in place (padding: exp(-inf) = 0), and its sum
    const float mu = safe_max(m);
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] = exp_shift(v[j], mu);
    float s = tree_reduce<P>(v, OpSum{});
    s = row_reduce<R>(s, c.red_b, c.l, OpSum{});
    return {m, s};
}

// Pass 3: normalise with the row's (M, S) (for a split row, merged over its G
// workgroups; `loc` is this workgroup's own pair), then the store.  STREAM: called
// from a persistent kernel's row loop (row buffers that end with the row, masks
// kept inside the loop; see store_part and mask_part).
template <class E, int P, int R, int G, bool VEC, bool STREAM, class Epi>
__device__ __forceinline__ void softmax_apply(float *v, RowView yv, bool valid, RowCtx &c,
                                              Epi &epi, MaxSum loc, float Mrow, float Srow) {
    constexpr int C = P / E::VPC;
    float scale;
    if constexpr (G == 1)
        scale = __builtin_amdgcn_rcpf(Srow);
    else
        scale = exp_shift(loc.m, safe_max(Mrow)) * __builtin_amdgcn_rcpf(Srow);
    epi.template apply<E, C, R, STREAM>(v, scale, safe_max(loc.m), Mrow, Srow, c, valid);
    store_part<E, C, R, VEC, STREAM>(yv, c.ln, c.N, valid, c.full, v);
    epi.template fixup<E, R, STREAM>(yv, valid);
}

// Passes 1-3 on a lane's loaded part v of the row, then the store.
template <class E, int P, int R, int G, bool VEC, bool STREAM, class Epi>
__device__ __forceinline__ void softmax_finish(float *v, RowView yv, bool valid, RowCtx &c,
                                               Epi &epi) {
    const MaxSum loc = softmax_local<E, P, R, G, STREAM>(v, c, epi);
    if constexpr (G == 1) {
        softmax_apply<E, P, R, G, VEC, STREAM>(v, yv, valid, c, epi, loc, loc.m, loc.s);
    } else {
        exchange_pairs<G>(c.g, c.member, c.it, loc.m, loc.s, c.spin_limit, c.bcast,
                          MergeMaxSum{});
        softmax_apply<E, P, R, G, VEC, STREAM>(v, yv, valid, c, epi, loc, c.bcast[0], c.bcast[1]);
    }
}

template <class E, int P, int R, bool VEC, class Out = SoftmaxOut>
__global__ void __launch_bounds__(block_threads_for(R))
    softmax_block_kernel(const char *x, char *y, int64_t M, int N, Out out) {
    constexpr int C = P / E::VPC;
    constexpr int RPB = rows_per_block_for(R);
    constexpr int W = R > 64 ? R / 64 : 1;
    __shared__ float red_max[RPB * W];
    __shared__ float red_sum[RPB * W];
    const int sub = lane_group<R>();
    const uint32_t row_bytes = (uint32_t)N * E::BYTES;
    RowCtx c{N, (int)(threadIdx.x % R), 0, 0, part_full<Out::kCfg, E, C, R, 1>(0, N),
             red_max + sub * W, red_sum + sub * W, nullptr, GroupRef{}, 0};
    c.ln = lane_of<Out::kCfg, E, C, R, 1>(0, c.l);
    const int64_t row = (int64_t)blockIdx.x * RPB + sub;
    const bool valid = row < M;
    float v[P];
    load_part<E, C, R, VEC>(block_row_view<R>(x, M, sub, row_bytes), c.ln, v);
    auto epi = out.row(valid ? row : M - 1);
    softmax_finish<E, P, R, 1, VEC, false>(v, block_row_view<R>(y, M, sub, row_bytes), valid, c,
                                           epi);
}

template <class E, int P, int R, int G, bool VEC, class Out = SoftmaxOut,
          int D = stream_depth(kCfgSoftmax, P, R)>
__global__ void __launch_bounds__(R)
    __attribute__((amdgpu_waves_per_eu(stream_waves(Out::kCfg, E::BYTES, VEC, P, R, G))))
    softmax_stream_kernel(const char *x, char *y, int64_t M, int N, uint8_t *ws, int groups,
                          int spin_limit, Out out) {
    static_assert(R >= 64, "one row per workgroup");
    constexpr int C = P / E::VPC;
    constexpr int W = R / 64;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    __shared__ float bcast[3];
    RowCtx c{N, (int)threadIdx.x, 0, 0, true, red_max, red_sum, bcast, GroupRef{}, spin_limit};
    int group = blockIdx.x;
    if constexpr (G > 1) {
        member_of<G>(&group, &c.member);
        c.g = group_ref<G>(ws, group);
        if (threadIdx.x == 0) bcast[2] = 0.0f;  // read only after later barriers
    }
    c.ln = lane_of<Out::kCfg, E, C, R, G>(c.member, (int)threadIdx.x);
    c.full = part_full<Out::kCfg, E, C, R, G>(c.member, N);
    const uint32_t rb = (uint32_t)N * E::BYTES;

    // Per-row inputs of the output policy (if any) sit after a row's values in its
    // buffer and are loaded with it.
    constexpr int X = Out::kExtra;
    if constexpr (kDeferredExchange && defer_split(Out::kCfg, E::BYTES, VEC, P, R, G)) {
        // Split rows, deferred exchange: three buffers.  Row k is reduced and its
        // partial published before the workgroup waits for row k - 1's peers and
        // writes row k - 1; the loads of row k + 1 are in flight meanwhile.  The
        // exchange's latency is then hidden behind a whole row's reduction.
        float buf[3][P + X];
        typename Out::Epi epis[3];
        MaxSum pend = {0.0f, 0.0f};  // this workgroup's (max, sum) of the row waiting
        int64_t row = group;
        // A row in flight is held as its raw 16-byte chunks (bf16: half the
        // registers) and widened when it becomes the current row.
        auto load = [&](float *v, int64_t r) {
            if constexpr (VEC)
                load_part_raw<E, C, R>(stream_row_view(x, r, M, rb), c.ln, v);
            else
                load_part<E, C, R, VEC>(stream_row_view(x, r, M, rb), c.ln, v);
            if (r < M) out.stash(v + P, r);
        };
        load(buf[0], row);
        load(buf[1], row + groups);
        auto step = [&](auto Kc) -> bool {
            constexpr int K = decltype(Kc)::value, KP = (K + 2) % 3;
            const bool more = row < M;
            MaxSum cur = {0.0f, 0.0f};
            if (more) {
                if constexpr (VEC) widen_part<E, C>(buf[K]);
                epis[K] = out.epi(buf[K] + P, row);
                cur = softmax_local<E, P, R, G, true>(buf[K], c, epis[K]);
                publish_pair<G>(c.g, c.member, c.it, cur.m, cur.s);
            } else {
                // no reduction (and its barriers) in this step: every wave has read
                // the previous row's merged pair before wave 0 writes the next one
                __syncthreads();
            }
            if (c.it > 0) {  // complete the previous row
                wait_pairs<G>(c.g, c.it - 1, c.spin_limit, c.bcast, MergeMaxSum{});
                softmax_apply<E, P, R, G, VEC, true>(buf[KP], stream_row_view(y, row - groups, M, rb),
                                               true, c, epis[KP], pend, c.bcast[0], c.bcast[1]);
            }
            pend = cur;
            if (!more) return false;
            load(buf[KP], row + 2 * (int64_t)groups);
            ++c.it;
            row += groups;
            return true;
        };
        while (stream_steps<0, 3>(step)) {
        }
    } else {
        // D register buffers: the loads of the next D - 1 rows are in flight while
        // the current row is reduced, exchanged and written.
        float buf[D][P + X];
        stream_rows<D>(
            (int64_t)group, M, groups, buf,
            [&](float *v, int64_t r) {
                load_part<E, C, R, VEC>(stream_row_view(x, r, M, rb), c.ln, v);
                if (r < M) out.stash(v + P, r);
            },
            [&](float *v, int64_t r) {
                auto epi = out.epi(v + P, r);
                softmax_finish<E, P, R, G, VEC, true>(v, stream_row_view(y, r, M, rb), true, c,
                                                      epi);
                ++c.it;
            });
    }
    if constexpr (G > 1) {
        if (c.it > 0) depart_group<G>(c.g);
    }
}

// ---------------------------------------------------------------- RMSNorm

struct MergeSum {
    static constexpr float kEmptyA = 0.0f, kEmptyB = 0.0f;
    __device__ __forceinline__ void operator()(float &q, float &unused, float qj, float) const {
        q = q + qj;
        unused = 0.0f;
    }
    template <int W>
    __device__ __forceinline__ static void lanes(float &q, float &unused) {
        q = lanes_reduce<W>(q, OpSum{});
        unused = 0.0f;
    }
};

// Weight source of the block kernels: the lane's part of w, already in registers.
template <int P>
struct WeightRegs {
    const float *w;
    __device__ __forceinline__ void apply(float *v, int) const {
#pragma unroll
        for (int j = 0; j < P; ++j) v[j] *= w[j];
    }
};

// Weight source of the stream kernels: the workgroup's slice of w, decoded to
// fp32 in LDS once per launch.  Lane l keeps its values j = 4q..4q+3 at
// slot[q * R + l], so the 16-byte LDS reads of a wave are contiguous.
template <int P, int R>
struct WeightLds {
    const float4 *slot;
    __device__ __forceinline__ void apply(float *v, int l) const {
#pragma unroll
        for (int q = 0; q < P / 4; ++q) {
            const float4 w4 = slot[q * R + l];
            v[4 * q] *= w4.x;
            v[4 * q + 1] *= w4.y;
            v[4 * q + 2] *= w4.z;
            v[4 * q + 3] *= w4.w;
        }
    }
};

// No weight (already applied).
struct WeightNone {
    __device__ __forceinline__ void apply(float *, int) const {}
};

// Sum of squares of this workgroup's part of the row.
template <class E, int P, int R, bool STREAM>
__device__ __forceinline__ float rmsnorm_local(float *v, RowCtx &c) {
    constexpr int C = P / E::VPC;
    if (!c.full) mask_part<E, C, R, STREAM>(c.ln, c.N, 0.0f, v);
    const float q = tree_sum_squares<P>(v);
    return row_reduce<R>(q, c.one_reduction_slots(), c.l, OpSum{});
}

// y = (x * w) * r with r = rsqrt(Q / N + eps) for the row's sum of squares Q, then
// the store.
template <class E, int P, int R, bool VEC, bool STREAM, class Weight>
__device__ __forceinline__ void rmsnorm_apply(float *v, const Weight &w, float Q, RowView yv,
                                              float *rstd_out, float eps, bool valid,
                                              const RowCtx &c) {
    constexpr int C = P / E::VPC;
    const float r = __builtin_amdgcn_rsqf(Q / (float)c.N + eps);
    w.apply(v, c.l);
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] *= r;
    store_part<E, C, R, VEC, STREAM>(yv, c.ln, c.N, valid, c.full, v);
    if (rstd_out && valid && c.l == 0 && c.member == 0) *rstd_out = r;
}

template <class E, int P, int R, int G, bool VEC, bool STREAM, class Weight>
__device__ __forceinline__ void rmsnorm_finish(float *v, const Weight &w, RowView yv,
                                               float *rstd_out, float eps, bool valid, RowCtx &c) {
    float q = rmsnorm_local<E, P, R, STREAM>(v, c);
    if constexpr (G > 1) {
        exchange_pairs<G>(c.g, c.member, c.it, q, 0.0f, c.spin_limit, c.bcast, MergeSum{});
        q = c.bcast[0];
    }
    rmsnorm_apply<E, P, R, VEC, STREAM>(v, w, q, yv, rstd_out, eps, valid, c);
}

template <class E, int P, int R, bool VEC>
__global__ void __launch_bounds__(block_threads_for(R))
    rmsnorm_block_kernel(const char *x, const char *w, char *y, float *rstd, int64_t M, int N,
                         float eps) {
    constexpr int C = P / E::VPC;
    constexpr int RPB = rows_per_block_for(R);
    constexpr int W = R > 64 ? R / 64 : 1;
    __shared__ float red[RPB * W];
    const int sub = lane_group<R>();
    const uint32_t row_bytes = (uint32_t)N * E::BYTES;
    RowCtx c{N, (int)(threadIdx.x % R), 0, 0, part_full<kCfgRmsnorm, E, C, R, 1>(0, N),
             red + sub * W, nullptr, nullptr, GroupRef{}, 0};
    const int64_t row = (int64_t)blockIdx.x * RPB + sub;
    const bool valid = row < M;
    float v[P];
    c.ln = lane_of<kCfgRmsnorm, E, C, R, 1>(0, c.l);
    load_part<E, C, R, VEC>(block_row_view<R>(x, M, sub, row_bytes), c.ln, v);
    float wv[P];
    load_part<E, C, R, VEC, kReuseLoad>(RowView{make_buf(w, row_bytes), 0u, row_bytes}, c.ln, wv);
    rmsnorm_finish<E, P, R, 1, VEC, false>(v, WeightRegs<P>{wv}, block_row_view<R>(y, M, sub, row_bytes),
                                    rstd ? rstd + row : nullptr, eps, valid, c);
}

template <class E, int P, int R, int G, bool VEC, int D = stream_depth(kCfgRmsnorm, P, R)>
__global__ void __launch_bounds__(R)
    __attribute__((amdgpu_waves_per_eu(stream_waves(kCfgRmsnorm, E::BYTES, VEC, P, R, G))))
    rmsnorm_stream_kernel(const char *x, const char *w, char *y, float *rstd, int64_t M, int N,
                          float eps, uint8_t *ws, int groups, int spin_limit) {
    static_assert(R >= 64, "one row per workgroup");
    constexpr int C = P / E::VPC;
    constexpr int W = R / 64;
    __shared__ float red[2][W];
    __shared__ float bcast[3];
    __shared__ float4 wslot[(P / 4) * R];
    RowCtx c{N, (int)threadIdx.x, 0, 0, true, red[0], red[1], bcast, GroupRef{}, spin_limit};
    int group = blockIdx.x;
    if constexpr (G > 1) {
        member_of<G>(&group, &c.member);
        c.g = group_ref<G>(ws, group);
        if (threadIdx.x == 0) bcast[2] = 0.0f;  // read only after later barriers
    }
    c.ln = lane_of<kCfgRmsnorm, E, C, R, G>(c.member, (int)threadIdx.x);
    c.full = part_full<kCfgRmsnorm, E, C, R, G>(c.member, N);
    const uint32_t rb = (uint32_t)N * E::BYTES;

    // This workgroup's slice of w, once; each lane later reads back only the
    // slots it wrote, so no barrier is needed.
    {
        float t[P];
        load_part<E, C, R, VEC, kReuseLoad>(RowView{make_buf(w, rb), 0u, rb}, c.ln, t);
#pragma unroll
        for (int q = 0; q < P / 4; ++q)
            wslot[q * R + c.l] = make_float4(t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]);
    }
    const WeightLds<P, R> wsrc{wslot};

    if constexpr (kDeferredExchange && defer_split(kCfgRmsnorm, E::BYTES, VEC, P, R, G)) {
        // Split rows, deferred exchange (see the softmax stream kernel).
        float buf[3][P];
        int64_t row = group;
        auto load = [&](float *v, int64_t r) {
            if constexpr (VEC)
                load_part_raw<E, C, R>(stream_row_view(x, r, M, rb), c.ln, v);
            else
                load_part<E, C, R, VEC>(stream_row_view(x, r, M, rb), c.ln, v);
        };
        load(buf[0], row);
        load(buf[1], row + groups);
        auto step = [&](auto Kc) -> bool {
            constexpr int K = decltype(Kc)::value, KP = (K + 2) % 3;
            const bool more = row < M;
            if (more) {
                if constexpr (VEC) widen_part<E, C>(buf[K]);
                const float q = rmsnorm_local<E, P, R, true>(buf[K], c);
                publish_pair<G>(c.g, c.member, c.it, q, 0.0f);
                // x * w now rather than at the store: the store step then reads no
                // weight from LDS while three rows are live, which with 64 fp32
                // values per lane would not fit the registers; (x * w) * r as before
                wsrc.apply(buf[K], c.l);
            } else {
                __syncthreads();  // as in the softmax kernel: the merged sum is read
            }
            if (c.it > 0) {  // complete the previous row
                wait_pairs<G>(c.g, c.it - 1, c.spin_limit, c.bcast, MergeSum{});
                const int64_t rp = row - groups;
                rmsnorm_apply<E, P, R, VEC, true>(buf[KP], WeightNone{}, c.bcast[0],
                                            stream_row_view(y, rp, M, rb),
                                            rstd ? rstd + rp : nullptr, eps, true, c);
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
        float buf[D][P];
        stream_rows<D>(
            (int64_t)group, M, groups, buf,
            [&](float *v, int64_t r) {
                load_part<E, C, R, VEC>(stream_row_view(x, r, M, rb), c.ln, v);
            },
            [&](float *v, int64_t r) {
                rmsnorm_finish<E, P, R, G, VEC, true>(v, wsrc, stream_row_view(y, r, M, rb),
                                                rstd ? rstd + r : nullptr, eps, true, c);
                ++c.it;
            });
    }
    if constexpr (G > 1) {
        if (c.it > 0) depart_group<G>(c.g);
    }
}

}  // namespace rr
