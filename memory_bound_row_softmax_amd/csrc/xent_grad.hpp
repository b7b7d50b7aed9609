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

    // Where the label's element gets its "- dloss": in the registers, before the
    // row's stores (the owner's wave alone subtracts, all elements of the chunk
    // selected by masks), or by the owner lane rewriting that one element after
    // them.  The second keeps the row's registers out of a branch that changes
    // them, which cost 44 VGPRs in the 64-value bf16 stream kernels (three
    // workgroups per CU instead of two).  Offset-averaged GB/s on MI355X, 16384
    // rows, registers -> rewrite:
    //   bf16 64 x 256 lanes, 2 / 4 / 8 workgroups (N = 32768 / 65536 / 131072):
    //       5590 -> 5850, 5700 -> 6090, 5565 -> 6005
    //   bf16 32 x 512, 2 workgroups (N = 32768):   5520 -> 5740
    //   bf16 32 x 1024, 1 workgroup (N = 32768):   5700 -> 5550
    //   fp32 64 x 256, 8 workgroups (8192 x 131072): 6270 -> 6205
    //   bf16 block 32 x 256 (N = 8192):             6390 -> 6240
    template <class E, int R, bool STREAM>
    static constexpr bool rewrite_label() {
        return E::BYTES == 2 && STREAM && R <= 512;
    }

    struct Epi {
        int label;
        float g;
        float *loss;
        float *lse;
        bool has;         // this lane holds the label's column
        float x_label;
        float fix;        // the rewritten element

        // The lane whose part of the row holds the label's column keeps x[label]
        // from its registers (no extra read), picked by masks and not by a
        // computed register index: "pick one of these registers" turned into an
        // address would move the whole row out of registers.  With the rewrite the
        // owner is found from the label by inverting the lane layout and only its
        // wave scans; otherwise every lane tests each of its chunks (the code these
        // kernels were tuned with).
        template <class E, int C, int R, int G, bool STREAM>
        __device__ __forceinline__ void capture(const float *v, const RowCtx &c) {
            constexpr int VPC = E::VPC;
            uint32_t bits = 0;
            if constexpr (rewrite_label<E, R, STREAM>()) {
                has = false;
                int i = 0;
                if (label >= 0 && label < c.N) {
                    int member, l;
                    chunk_owner<kCfg, E, C, R, G>(label / VPC, member, l, i);
                    has = member == c.member && l == c.l && i < C;
                }
                if (has) {
                    const int d = label % VPC;
#pragma unroll
                    for (int k = 0; k < C; ++k) {
                        if (k == i) {
#pragma unroll
                            for (int e = 0; e < VPC; ++e)
                                bits |= __float_as_uint(v[k * VPC + e]) & (0u - (uint32_t)(d == e));
                        }
                    }
                }
            } else {
                bool found = false;
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    const int d = label - c.ln.chunk(i) * VPC;
                    if ((unsigned)d < (unsigned)VPC && label < c.N) {
#pragma unroll
                        for (int e = 0; e < VPC; ++e)
                            bits |= __float_as_uint(v[i * VPC + e]) & (0u - (uint32_t)(d == e));
                        found = true;
                    }
                }
                has = found;
            }
            x_label = __uint_as_float(bits);
        }

        template <class E, int C, int R, bool STREAM>
        __device__ __forceinline__ void apply(float *v, float scale, float mu, float Mrow,
                                              float Srow, const RowCtx &c, bool valid) {
            constexpr int VPC = E::VPC;
            const bool ok = label >= 0 && label < c.N;
            const float ge = ok ? g : __builtin_nanf("");
            const float sg = scale * ge;
#pragma unroll
            for (int j = 0; j < C * VPC; ++j) v[j] *= sg;
            if constexpr (rewrite_label<E, R, STREAM>()) {
                // e_label exactly as the row's e_j were computed
                if (has) fix = exp_shift(x_label, mu) * sg - ge;
            } else if (has) {
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    const int d = label - c.ln.chunk(i) * VPC;
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
                if (has) *loss = row_lse - x_label;
            }
        }

        // The same lane's second store to one address reaches memory after its first.
        template <class E, int R, bool STREAM>
        __device__ __forceinline__ void fixup(RowView yv, bool valid) {
            if constexpr (rewrite_label<E, R, STREAM>()) {
                if (has && valid) buf_store_elem<E>(yv.buf, yv.base + (uint32_t)label * E::BYTES, fix);
            }
        }
    };

    // Block kernels: plain loads (rows may differ between the lanes of a wave).
    __device__ __forceinline__ Epi row(int64_t r) const {
        return Epi{labels[r], dloss[r], loss + r, lse ? lse + r : nullptr};
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
        return Epi{(int)__float_as_uint(extra[0]), extra[1], loss + r, lse ? lse + r : nullptr};
    }
};

}  // namespace rr
