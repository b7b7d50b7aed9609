// xent_grad.hpp -- cross-entropy forward fused with its gradient: the output
// policy of the softmax kernels that turns a row's softmax into
//     dx_j = (p_j - [j == label]) * dloss,   lse = M + ln S,   loss = lse - x_label.
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%), section 让内存密集型内核达到"光速",
// names the cross-entropy loss among its memory-bound kernels and presents them as
// building blocks of training as well as inference.  Fusing the gradient into the
// forward keeps the row on chip: the logits are read from HBM once and the gradient
// written once (the forward alone reads the row once; a separate backward would read
// it again).  The gradient is the textbook derivative of the per-row loss, scaled by
// the row's upstream gradient dloss.  A label outside [0, N) makes the loss and the
// whole row of the gradient NaN.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "reduce.hpp"
#include "row_kernels.hpp"
#include "vec_io.hpp"

namespace rr {

struct XentGradOut {
    static constexpr int kCfg = kCfgXentGrad;  // configuration menu predicates
    const int32_t *labels;
    const float *dloss;
    float *loss;
    float *lse;  // may be null
    int64_t M;

    struct Epi {
        int label;
        float g;
        float *loss;
        float *lse;
        float x_label;
        bool has;  // this lane holds the label's column

        // The lane whose chunk holds the label keeps its raw value (no extra read).
        // Only that chunk is examined (a branch at most one lane of the row takes),
        // and inside it the element is picked by masks, not by a computed register
        // index: "pick one of these registers" turned into an address would move
        // the whole row out of registers.
        template <class E, int C, int R>
        __device__ __forceinline__ void capture(const float *v, Lane ln, int N) {
            constexpr int VPC = E::VPC;
            uint32_t bits = 0;
            bool found = false;
#pragma unroll
            for (int i = 0; i < C; ++i) {
                const int d = label - ln.chunk(i) * VPC;
                if ((unsigned)d < (unsigned)VPC && label < N) {
#pragma unroll
                    for (int e = 0; e < VPC; ++e)
                        bits |= __float_as_uint(v[i * VPC + e]) & (0u - (uint32_t)(d == e));
                    found = true;
                }
            }
            x_label = __uint_as_float(bits);
            has = found;
        }

        template <class E, int C, int R>
        __device__ __forceinline__ void apply(float *v, float scale, float Mrow, float Srow,
                                              const RowCtx &c, bool valid) {
            constexpr int VPC = E::VPC;
            const bool ok = label >= 0 && label < c.N;
            const float ge = ok ? g : __builtin_nanf("");
            const float sg = scale * ge;
#pragma unroll
            for (int j = 0; j < C * VPC; ++j) v[j] *= sg;
            if (has) {
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    const int d = label - (c.ln.chunk(i)) * VPC;
                    if ((unsigned)d < (unsigned)VPC) {
#pragma unroll
                        for (int e = 0; e < VPC; ++e) v[i * VPC + e] -= (d == e) ? ge : 0.0f;
                    }
                }
            }
            if (valid) {
                const float row_lse = Mrow + __builtin_amdgcn_logf(Srow) * kLn2;
                if (c.l == 0 && c.member == 0) {
                    if (lse) *lse = row_lse;
                    if (!ok) *loss = __builtin_nanf("");
                }
                if (ok && has) *loss = row_lse - x_label;
            }
        }
    };

    // Block kernels: plain loads (rows may differ between the lanes of a wave).
    __device__ __forceinline__ Epi row(int64_t r) const {
        return Epi{labels[r], dloss[r], loss + r, lse ? lse + r : nullptr, 0.0f, false};
    }

    // Stream kernels (one row per workgroup): the label and dloss are loaded with
    // vector-memory loads issued right after the row's own loads, so they complete
    // with it and no reduction barrier waits for them on its own.
    static constexpr int kExtra = 2;
    __device__ __forceinline__ void stash(float *extra, int64_t r) const {
        const Buf bl = make_buf(labels, (uint32_t)(M * 4));
        const Buf bg = make_buf(dloss, (uint32_t)(M * 4));
        const int off = (int)((uint32_t)r * 4u);
        extra[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bl.rsrc, off, 0, 0));
        extra[1] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bg.rsrc, off, 0, 0));
    }
    __device__ __forceinline__ Epi epi(const float *extra, int64_t r) const {
        return Epi{(int)__float_as_uint(extra[0]), extra[1], loss + r, lse ? lse + r : nullptr,
                   0.0f, false};
    }
};

}  // namespace rr
