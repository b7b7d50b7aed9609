// reduce.hpp -- the reduction ladder: registers -> wave64 lanes -> LDS -> global workspace.
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%), section 硬件感知的归约策略,
// reduces from the top of the memory hierarchy down and hands only reduced values to
// the next level: (1) each thread over its own registers, (2) a butterfly across the
// 32 lanes of a warp so that every lane ends with the result, (3) one slot per warp in
// a shared-memory buffer, a barrier, then every warp reads all slots, (4) across a
// cluster of blocks through distributed shared memory with an arrival barrier.
// The gfx950 ladder:
//   (1) tree_reduce      over a lane's P registers (a balanced tree: short dependency
//                        chains and a rounding error that grows with log2(P), not P);
//   (2) lanes_reduce<W>  butterfly over W <= 64 lanes of a wave64: DPP quad_perm for
//                        distances 1 and 2, DPP row_half_mirror and row_mirror inside a
//                        16-lane row, then the gfx950 permlane16/permlane32 swaps
//                        across rows; every lane ends with the same bits;
//   (3) waves_combine<W> one LDS slot per wave, a barrier, every lane reads the slots in
//                        wave order (so every wave gets the same bits);
//   (4) the grid exchange (grid_exchange.hpp): workgroups that share a row publish a
//       partial in a global workspace and wait for their peers.  This GPU has no
//       cluster / distributed-shared-memory level.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rr {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpSum {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// Balanced pairwise reduction of v[0..N).
template <int N, class Op>
__device__ __forceinline__ float tree_reduce(const float *v, Op op) {
    if constexpr (N == 1) {
        return v[0];
    } else {
        constexpr int H = N / 2;
        float a = tree_reduce<H>(v, op);
        float b = tree_reduce<N - H>(v + H, op);
        return op(a, b);
    }
}

// Balanced pairwise sum of v[i]^2 (squares formed at the leaves).
template <int N>
__device__ __forceinline__ float tree_sum_squares(const float *v) {
    if constexpr (N == 1) {
        return v[0] * v[0];
    } else {
        constexpr int H = N / 2;
        return tree_sum_squares<H>(v) + tree_sum_squares<N - H>(v + H);
    }
}

// Balanced pairwise sum of a[i] * b[i] (products formed at the leaves).
template <int N>
__device__ __forceinline__ float tree_dot(const float *a, const float *b) {
    if constexpr (N == 1) {
        return a[0] * b[0];
    } else {
        constexpr int H = N / 2;
        return tree_dot<H>(a, b) + tree_dot<N - H>(a + H, b + H);
    }
}

// ---- cross-lane moves -------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    // row_mask = bank_mask = 0xf: every lane is written; bound_ctrl: lanes whose
    // source is out of range read 0 (no such lane for the patterns used here).
    return __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xF, 0xF, true);
}

constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]: partner at distance 1
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]: partner at distance 2
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i inside each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i inside each 16 lanes

// op(x_lane, x_partner) for the 16-lane-row swap (rows 0<->1, 2<->3) and the
// half-wave swap (lanes 0..31 <-> 32..63).  The swap instructions return both
// halves of the exchange; combining them in a fixed operand order gives every
// lane of a pair the same bits.
template <class Op>
__device__ __forceinline__ float swap16_combine(float v, Op op) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <class Op>
__device__ __forceinline__ float swap32_combine(float v, Op op) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---- (2) butterfly over W lanes (W a power of two, 1..64) -------------------
//
// After the quad stages all 4 lanes of a quad hold the same value, so the mirror
// patterns (which are not xor patterns) still pair every lane with a lane of the
// other half of its 8- or 16-lane group.
template <int W, class Op>
__device__ __forceinline__ float lanes_reduce(float v, Op op) {
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W must be a power of two <= 64");
    if constexpr (W >= 2) v = op(v, dpp<kDppQuadSwap1>(v));
    if constexpr (W >= 4) v = op(v, dpp<kDppQuadSwap2>(v));
    if constexpr (W >= 8) v = op(v, dpp<kDppRowHalfMirror>(v));
    if constexpr (W >= 16) v = op(v, dpp<kDppRowMirror>(v));
    if constexpr (W >= 32) v = swap16_combine(v, op);
    if constexpr (W >= 64) v = swap32_combine(v, op);
    return v;
}

// ---- running (max, sum of exp) pairs ----------------------------------------
//
// (m, s) stands for s * exp(m) restricted to the values seen so far; merging two
// pairs rescales both sums to the larger max (the online-softmax rescaling).  An
// empty pair is (-inf, 0).  merge(a, b) and merge(b, a) give the same bits.
struct MaxSum {
    float m, s;
};

__device__ __forceinline__ float exp_shift(float v, float mu) {
    return __builtin_amdgcn_exp2f((v - mu) * kLog2e);
}

// The max to subtract: -inf (nothing seen) is replaced by 0 so that empty
// entries give exp(-inf) = 0 instead of NaN.
__device__ __forceinline__ float safe_max(float m) { return m == -INFINITY ? 0.0f : m; }

__device__ __forceinline__ MaxSum merge(MaxSum a, MaxSum b) {
    float M = fmaxf(a.m, b.m);
    float mu = safe_max(M);
    return {M, a.s * exp_shift(a.m, mu) + b.s * exp_shift(b.m, mu)};
}

struct OpMerge {
    __device__ __forceinline__ MaxSum operator()(MaxSum a, MaxSum b) const { return merge(a, b); }
};

template <int CTRL>
__device__ __forceinline__ MaxSum dpp(MaxSum v) {
    return {dpp<CTRL>(v.m), dpp<CTRL>(v.s)};
}

__device__ __forceinline__ MaxSum swap16_combine(MaxSum v, OpMerge op) {
    auto rm = __builtin_amdgcn_permlane16_swap(__float_as_uint(v.m), __float_as_uint(v.m), false,
                                               false);
    auto rs = __builtin_amdgcn_permlane16_swap(__float_as_uint(v.s), __float_as_uint(v.s), false,
                                               false);
    return op(MaxSum{__uint_as_float(rm[0]), __uint_as_float(rs[0])},
              MaxSum{__uint_as_float(rm[1]), __uint_as_float(rs[1])});
}
__device__ __forceinline__ MaxSum swap32_combine(MaxSum v, OpMerge op) {
    auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(v.m), __float_as_uint(v.m), false,
                                               false);
    auto rs = __builtin_amdgcn_permlane32_swap(__float_as_uint(v.s), __float_as_uint(v.s), false,
                                               false);
    return op(MaxSum{__uint_as_float(rm[0]), __uint_as_float(rs[0])},
              MaxSum{__uint_as_float(rm[1]), __uint_as_float(rs[1])});
}

template <int W>
__device__ __forceinline__ MaxSum lanes_reduce(MaxSum v, OpMerge op) {
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W must be a power of two <= 64");
    if constexpr (W >= 2) v = op(v, dpp<kDppQuadSwap1>(v));
    if constexpr (W >= 4) v = op(v, dpp<kDppQuadSwap2>(v));
    if constexpr (W >= 8) v = op(v, dpp<kDppRowHalfMirror>(v));
    if constexpr (W >= 16) v = op(v, dpp<kDppRowMirror>(v));
    if constexpr (W >= 32) v = swap16_combine(v, op);
    if constexpr (W >= 64) v = swap32_combine(v, op);
    return v;
}

// ---- (3) across the W waves that share a row, through LDS --------------------
//
// `slots` points at this row's W entries.  Every thread of the workgroup must call
// this (it holds a barrier).  A slot array may be written again only after another
// barrier has passed.
template <int W, class T, class Op>
__device__ __forceinline__ T waves_combine(T v, T *slots, int wave_in_row, int lane, Op op) {
    if (lane == 0) slots[wave_in_row] = v;
    __syncthreads();
    T r = slots[0];
#pragma unroll
    for (int w = 1; w < W; ++w) r = op(r, slots[w]);
    return r;
}

// Full row reduction for a lane group of R lanes (R <= 64: inside one wave,
// R > 64: R / 64 waves).  `slots` is unused when R <= 64.
template <int R, class T, class Op>
__device__ __forceinline__ T row_reduce(T v, T *slots, int l, Op op) {
    if constexpr (R <= 64) {
        return lanes_reduce<R>(v, op);
    } else {
        v = lanes_reduce<64>(v, op);
        return waves_combine<R / 64>(v, slots, l >> 6, l & 63, op);
    }
}

}  // namespace rr
