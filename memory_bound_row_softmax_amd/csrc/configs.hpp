// configs.hpp -- the menu of compiled kernel configurations.
//
// Shared by the planner (which may only pick what exists) and by the kernel
// files (which instantiate exactly this list).  No HIP here.
//
// Row-resident kernels (softmax, RMSNorm) come in two kinds, both named by
// (P, R, G):
//   P  fp32 values each lane keeps in registers per row (P / 4 chunks of 16
//      bytes for fp32 input, P / 8 for bf16),
//   R  lanes that share one row inside a workgroup (16..64: a slice of one
//      wave, 128..1024: several waves joined through LDS),
//   G  workgroups per row.
// One row holds at most P * R * G elements.
//
//  * block kernels (G = 1): one workgroup per rows_per_block_for(R) rows, as
//    many workgroups as that takes; the hardware overlaps the workgroups
//    resident on a CU.  For rows up to a few thousand elements.
//  * stream kernels (G >= 1): a persistent grid, one row per workgroup at a
//    time; each workgroup (or row group of G workgroups, which meet in a small
//    global workspace) loads its next row while it reduces and writes the
//    current one (two register buffers).  For long rows, where only one or two
//    workgroups fit on a CU and nothing else would hide the load latency.
//
// Cross-entropy kernels are named by (P, R): each of the R lanes of a row
// loads P values per step and keeps a running (max, sum).
#pragma once

#define RR_BLOCK_CONFIGS(X)                                                                 \
    X(8, 16) X(8, 32) X(8, 64) X(8, 128) X(8, 256) X(8, 512) X(8, 1024)                     \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) X(16, 256) X(16, 512) X(16, 1024)              \
    X(32, 16) X(32, 32) X(32, 64) X(32, 128) X(32, 256) X(32, 512) X(32, 1024)              \
    X(64, 16) X(64, 32) X(64, 64) X(64, 128) X(64, 256) X(64, 512) X(64, 1024)

#define RR_STREAM_CONFIGS(X)                                                                \
    X(16, 1024, 1) X(16, 1024, 2) X(16, 1024, 4) X(16, 1024, 8) X(16, 1024, 16)             \
    X(32, 512, 1) X(32, 512, 2) X(32, 512, 4) X(32, 512, 8) X(32, 512, 16)                  \
    X(32, 512, 32) X(32, 512, 64)                                                           \
    X(32, 1024, 1) X(32, 1024, 2) X(32, 1024, 4) X(32, 1024, 8) X(32, 1024, 16)             \
    X(64, 256, 1) X(64, 256, 2) X(64, 256, 4) X(64, 256, 8) X(64, 256, 16)                  \
    X(64, 512, 1) X(64, 512, 2) X(64, 512, 4) X(64, 512, 8) X(64, 512, 16)                  \
    X(64, 512, 32) X(64, 512, 64) X(64, 512, 128) X(64, 512, 256)                           \
    X(64, 512, 3) X(64, 512, 5) X(64, 512, 6)                                           \
    X(64, 256, 3) X(64, 256, 5) X(64, 256, 6) X(64, 256, 7) X(64, 256, 9) X(64, 256, 10)   \
    X(64, 256, 11) X(64, 256, 12) X(64, 256, 13) X(64, 256, 14) X(64, 256, 15)

// Packed bf16 RMSNorm stream kernels (128-bit path only, see packed_bf16.hpp),
// named by (R, G): each lane keeps kPackedP = 128 bf16 values as 64 VGPRs of raw
// chunks.  A plan names them with P = kPackedP.  256 lanes on 8 workgroups (two per
// CU) serve rows of 131073 to 262144 elements: offset-averaged GB/s against 512
// lanes on 4, 16384 x 262144 6034 -> 6402 (and 5769-6439 -> 6383-6430 over the
// offsets), 8192 and 32768 rows +1.5 and +2.4 %, 200000 elements +1.3 %, 160000 and
// 180000 within 1 %; at 16384 to 65536 elements 128 or 256 lanes lost 5-14 % to the
// unpacked kernels, and at 524288 and 1048576 256 lanes lost 5-6 % to 512.
// 512 lanes on 256 workgroups (one on every CU) hold rows of up to 16M elements.
constexpr int kPackedP = 128;
#define RR_PACKED_CONFIGS(X) \
    X(512, 1) X(512, 2) X(512, 4) X(512, 8) X(512, 16) X(512, 32) X(512, 64) X(512, 128) \
    X(512, 256) X(256, 8)

// The packed kernels defer the exchange (three buffers, 254 VGPRs) from 16
// workgroups per row.  Offset-averaged GB/s, bf16 RMSNorm, waiting at once ->
// deferred: 1048576 elements on 16 6041 -> 6075-6135, 2097152 on 32 5748 -> 6259-6295,
// 4194304 on 64 5307 -> 6099-6116, 8388608 on 128 5245 -> 6078-6127, 3000000 on 64
// 4754 -> 5410-5428; on 8 it lost 4 % (524288 elements 6555 -> 6288; 262144 on 8 of
// 256 lanes 6443 -> 6193).
constexpr int kPackedDeferMinG = 16;

// RMSNorm backward (persistent, see rmsnorm_bwd.hpp), named by (P, R, G): a lane
// keeps x, dy (two rows in flight), its w slice and its dw partials, about 6P + 45
// VGPRs, so P <= 32 on up to 512 lanes and P = 8 on 1024 lanes.
#define RR_RMSBWD_CONFIGS(X)                                                                \
    X(8, 16, 1) X(8, 32, 1) X(8, 64, 1) X(8, 128, 1) X(8, 256, 1) X(8, 512, 1) X(8, 1024, 1)  \
    X(16, 16, 1) X(16, 32, 1) X(16, 64, 1) X(16, 128, 1) X(16, 256, 1) X(16, 512, 1)          \
    X(32, 16, 1) X(32, 32, 1) X(32, 64, 1) X(32, 128, 1) X(32, 256, 1) X(32, 512, 1)          \
    X(16, 512, 2) X(16, 512, 4) X(16, 512, 8) X(16, 512, 16) X(16, 512, 32)                   \
    X(32, 512, 2) X(32, 512, 4) X(32, 512, 8) X(32, 512, 16)

#define RR_XENT_CONFIGS(X)                                                                  \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) X(16, 256) X(16, 512) X(16, 1024)              \
    X(32, 16) X(32, 32) X(32, 64) X(32, 128) X(32, 256) X(32, 512) X(32, 1024)

namespace rr {

// Op codes shared by the planner and the kernels.
constexpr int kCfgSoftmax = 0;
constexpr int kCfgRmsnorm = 1;
constexpr int kCfgXentGrad = 2;  // softmax kernels with the cross-entropy gradient epilogue
constexpr int kCfgSoftmaxBwd = 3;
constexpr int kCfgRmsnormBwd = 4;  // register budgets only (stream_waves)

// Which block configurations are compiled for (op, element bytes, vectorised
// path).  Excluded are those that would need more than the 128 VGPRs a lane of a
// 1024-thread workgroup can have, or whose per-element path holds more than 32
// values per lane; none of the compiled kernels uses scratch memory (the build
// checks this).  Register needs, measured on the gfx950 compiler:
//   softmax, 128-bit path:         about P + 40
//   RMSNorm:                       about 2P + 40 (row and weight both in registers)
//   per-element path:              grows with the per-element offsets, so P <= 32
//                                  (P <= 16 for RMSNorm with 1024 lanes)
//   softmax backward:              about 2P + 30 (y and dy both in registers)
constexpr bool block_config_enabled(int op, int elem_bytes, bool vec, int P, int R) {
    (void)elem_bytes;
    if (op == kCfgSoftmaxBwd) return (vec ? P : 2 * P) * (R == 1024 ? 2 : 1) <= 64;
    if (!vec && P > 32) return false;
    if (!vec && op == kCfgRmsnorm && R == 1024 && P > 16) return false;
    if (op == kCfgRmsnorm && R == 1024 && P == 64) return false;
    return true;
}

// Split rows take at most 128 workgroups per row (one wave polls the exchange slots,
// two per lane).
// Stream kernels hold two rows' worth of values per lane (about 2P + 40 VGPRs;
// RMSNorm about 3P + 30, its weight slice coming back from LDS); the weight slice
// of a workgroup lives in LDS as fp32 (4 * P * R bytes, at most 128 KiB).  The
// per-element path keeps P <= 16 (one exception below).  RMSNorm fp32 with 32
// values on 1024 lanes would need scratch when the row is split.
// The cross-entropy gradient epilogue keeps the label, dloss and the label's logit
// per row: fp32 with 32 values on 1024 lanes no longer fits in 128 VGPRs.
constexpr bool stream_config_enabled(int op, int elem_bytes, bool vec, int P, int R, int G) {
    // The per-element path keeps P <= 16, except unaligned bf16 softmax, RMSNorm and
    // cross-entropy gradient rows split over 2 to 8 workgroups: 32 values on 512
    // lanes (the planner uses them up to 81920 elements; the gradient at 8192 x
    // 50257 ran at 2363 GB/s on a 64 x 1024 block kernel, 3536 on 32 x 512 x 4).
    if (!vec && P > 16)
        return elem_bytes == 2 && P == 32 && R == 512 && G >= 2 && G <= 8 &&
               (op == kCfgSoftmax || op == kCfgRmsnorm || op == kCfgXentGrad);
    // 128 workgroups per row (4194304 elements on chip): softmax and RMSNorm forward
    if (G > 64 && op != kCfgSoftmax && op != kCfgRmsnorm) return false;
    // Workgroups per row that are not a power of two: bf16 softmax and cross-entropy
    // gradient rows, and fp32 softmax rows, on 64 values x 512 lanes, and bf16
    // cross-entropy gradient rows on 64 values x 256 lanes, take exactly as many as
    // the row needs (the planner), so that most registers hold an element.
    if ((G & (G - 1)) != 0) {
        if (R == 256) return vec && P == 64 && elem_bytes == 2 && op == kCfgXentGrad;
        return vec && P == 64 && R == 512 &&
               ((elem_bytes == 2 && (op == kCfgSoftmax || op == kCfgXentGrad)) ||
                (elem_bytes == 4 && op == kCfgSoftmax));
    }
    if (op == kCfgXentGrad && elem_bytes == 4 && P == 32 && R == 1024) return false;
    // softmax backward keeps two rows (y, dy) per buffer: about 4P + 40 VGPRs
    if (op == kCfgSoftmaxBwd) return vec ? (R == 1024 ? P <= 16 : P <= 32) : P <= 16;
    if (op == kCfgRmsnorm && elem_bytes == 4 && P == 32 && R == 1024 && G > 1) return false;
    return true;
}

// Register buffers of a stream kernel (rows held at once: one being reduced,
// the others' loads in flight).  A workgroup of 1024 lanes leaves each lane 128
// VGPRs, enough for a third buffer only when P <= 16; RMSNorm, which also
// reads its weight back from LDS, fits a third buffer only when P <= 32.
#ifndef RR_STREAM_DEPTH
#define RR_STREAM_DEPTH 2
#endif
constexpr int stream_depth(int op, int P, int R) {
    const bool fits = (R < 1024 || P <= 16) && (op != 1 || P <= 32);
    return (RR_STREAM_DEPTH > 2 && fits) ? RR_STREAM_DEPTH : 2;
}

// Two-pass long rows (past the split-row capacity): tiles of kLongP * kLongR elements
// (kLongPElem on the per-element path), G workgroups per row (long_row_groups
// below), rows up to kLongMaxN elements (byte offsets stay 32-bit).
constexpr int kLongP = 32;
constexpr int kLongPElem = 16;
constexpr int kLongR = 512;
constexpr int kLongG = 16;
// As many workgroups per row (16, 32 or 64) as keep a workgroup's share of the row
// (of y and dy for the softmax backward) at about 512 KiB or less.  On MI355X the
// two-read softmax ran fastest that way (fp32 rows of 3M and 4M elements on 32, of
// 8M on 64, bf16 rows of 2M and 4M on 16).  RMSNorm measured within 3 % for 16, 32
// and 64 at 4M and 8M elements, and 64 won on longer rows (offset-averaged GB/s, 16
// -> 64: bf16 32M elements 3450 -> 3767, 64M 3185 -> 3558; fp32 16M 3486 -> 4116,
// 9M 4090 -> 4252).
constexpr int long_row_groups(long long row_bytes) {
    int g = kLongG;
    while (g < 64 && row_bytes > (long long)g * (512 << 10)) g *= 2;
    return g;
}
constexpr long long kLongMaxN = 1ll << 28;

// RMSNorm backward: the per-element path keeps P <= 16 for fp32; bf16 (whose
// per-element loads take no branch) has 32 values per lane as well.
constexpr bool rmsbwd_config_enabled(bool vec, int P, int elem_bytes) {
    return vec || P <= 16 || (elem_bytes == 2 && P <= 32);
}

// RMSNorm backward partial rows: at most kBwdMaxWorkgroups / G row groups, each
// writing one fp32 partial row of dw; one column reduction pass adds them.
constexpr int kBwdMaxWorkgroups = 1024;

// Split rows with the deferred exchange: a row's partial is published, the next
// row reduced, and only then the wait for the peers' partials of the first row
// (three row buffers instead of two; a row in flight is kept as raw chunks, half
// the registers for bf16).  Used where it measured faster on MI355X: rows split
// over 8 or more workgroups, softmax with 64 values on 512 lanes (+5-9 % at
// 262144 elements), 16 values on 1024 lanes (+10-20 %) and the softmax backward
// with 32 values on 512 lanes (+11-24 % at 131072 and 262144 elements), and
// RMSNorm with 32 values on 512 lanes (fp32 at 262144 elements: 16 workgroups
// per row deferred beat 8 with 64 values by 5 %; at 1048576 elements 64 deferred
// beat 32 with 64 values by 15-22 %).  With 2 workgroups per
// row the exchange is cheap and the deferral only delays the stores (bf16 softmax
// at 65536 elements: -14 %); elsewhere the third buffer does not fit the
// registers or costs a workgroup per CU (-2 to -20 % for 32 values on 512 lanes,
// 64 on 256).
#ifndef RR_SPLIT_DEFER
#define RR_SPLIT_DEFER 1
#endif
constexpr bool kDeferredExchange = RR_SPLIT_DEFER != 0;

#ifndef RR_DEFER_MIN_G
#define RR_DEFER_MIN_G 8
#endif
constexpr bool defer_split(int op, int elem_bytes, bool vec, int P, int R, int G) {
    if (G < RR_DEFER_MIN_G) return false;
    if (op == kCfgSoftmaxBwd) return vec && P == 32 && R == 512;
    if (op == kCfgRmsnorm && P == 32 && R == 512) return true;
    // fp32 RMSNorm with 64 values (offset-averaged GB/s, waiting at once -> deferred):
    // 524288 elements on 16 6006 -> 6348, 1048576 on 32 5785 -> 6483, 2097152 on 64
    // 5250 -> 6253, 4194304 on 128 5187 -> 6341, 8388608 on 256 4684 -> 6224; on 8
    // it lost 1-3 % (200000 6144 -> 6013, 262144 6615 -> 6472)
    if (op == kCfgRmsnorm && P == 64 && R == 512) return G >= 16;
    // bf16 softmax on 8 and 16: two non-deferred workgroups per CU beat one deferred
    // (stream_waves; offset-averaged GB/s: 262144 elements on 8 6246 against 5849,
    // 524288 on 16 5746 against 5577, 400000 on 16 5299 against 4594; on 32 they
    // lost, 5443 against 5715 at 1048576)
    if (P == 64 && R == 512 && elem_bytes == 2 && (G == 8 || G == 16) && op == kCfgSoftmax)
        return false;
    if (P == 64 && R == 512) return op == kCfgSoftmax;
    if (P == 16 && R == 1024) return vec || op != kCfgXentGrad;
    return false;
}

// Granule, in 16-byte chunks, in which the chunks of a row split over G workgroups
// are dealt to them (row_io.hpp, lane_of); one workgroup holds S = C * R chunks of a
// row (C per lane).  Chosen by measurement on MI355X: softmax forward over 16384
// rows, GB/s averaged over six byte offsets between input and output (the spread
// over offsets reaches 10 %), against one contiguous part per workgroup:
//   G = 2:  512 chunks (8 KiB) +1 %
//   G = 4:  4 KiB +5 % (bf16, S = 4096); fp32 softmax (S = 8192) 8 KiB +1 % (4 KiB: -2 %)
//   G = 8:  4 KiB +2 to +6 %
//   G = 16: a contiguous part per workgroup for S = 8192 (fp32, 64 x 512: 4 KiB -7 %);
//           4 KiB for S = 4096 (softmax backward 32 x 512: +12 % bf16, +1 % fp32;
//           cross-entropy gradient 64 x 256: +5 %)
//   G = 5, 32, 64: a contiguous part per workgroup was best (4 KiB: -4 to -8 %)
// RMSNorm, the softmax backward and the cross-entropy gradient at G = 4 measured best
// with 4 KiB (+5 to +13 %).
constexpr int split_granule(int op, int C, int R, int G) {
    const int S = C * R;
#ifdef RR_SPLIT_GRANULE
    int K = RR_SPLIT_GRANULE == 0 ? S : RR_SPLIT_GRANULE;  // tuning builds; 0: contiguous
#else
    int K = S;
    if (G == 2) K = 512;
    if (G == 4) K = (op == kCfgSoftmax && S >= 8192) ? 512 : 256;
    if (G == 8) K = 256;
    if (G == 16 && S <= 4096) K = 256;
#endif
    if (K >= S) return S;
    if (K > R && C % (K / R) != 0) return S;
    return K;
}

// Waves per SIMD a persistent kernel is compiled for, as a register budget: with 4,
// a lane has at most 128 VGPRs and a CU holds two 512-lane workgroups, twice the
// bytes in flight of one.  Listed are the 512-lane kernels that fit that budget
// without spilling; 1 leaves the budget to the compiler.  bf16 softmax at G = 2..5
// measured +3 to +7 % (16384 rows of 65536 to 151936 elements), at G = 8 and 16
// (without the deferred exchange, which does not fit) +3 to +23 % (defer_split).
// The bf16 cross-entropy gradient on 64 values x 256 lanes (G >= 3) fits it too:
// four workgroups per CU instead of three, +2 to +11 % at 8 and 16 workgroups
// (16384 rows of 131072 to 262144 elements; 151936 on 16: 3990 -> 4415 GB/s).
constexpr int stream_waves(int op, int elem_bytes, bool vec, int P, int R, int G) {
    if (op == kCfgXentGrad && elem_bytes == 2 && vec && P == 64 && R == 256 && G >= 3) return 4;
    if (R != 512 || elem_bytes != 2) return 1;
    if (op == kCfgSoftmax && vec && P == 64 && G >= 2 && G <= 16) return 4;
    if (op == kCfgRmsnorm && !vec && P == 32 && (G == 2 || G == 4)) return 4;
    if (op == kCfgSoftmaxBwd && vec && P == 32 && G == 2) return 4;
    if (op == kCfgRmsnormBwd && !vec && P == 16 && G == 1) return 4;
    return 1;
}

// Threads per workgroup and rows per workgroup for a lane-group width R (block
// kernels; a stream kernel's workgroup is its R lanes).
constexpr int block_threads_for(int R) { return R < 256 ? 256 : R; }
constexpr int rows_per_block_for(int R) { return block_threads_for(R) / R; }

// Split-row workspace layout (bytes):
//   [0, 256)                 header: word 0 is the error word (non-zero: a wait timed
//                            out), the rest unused
//   256 + g * group_stride   record of row group g:
//       +0                   departure counter (uint32)
//       +64                  slots[kSlotSets][G][2] of uint64: (epoch << 32) | float bits
constexpr int kWsHeader = 256;
constexpr int kMaxGroups = 1024;
// Row groups at most, per G: kMaxGroups, and for G = 256 half of it, so that no split
// plan's workspace passes 256 + 1024 * group_stride_for(128) bytes (a grid of rows
// on 256 workgroups each has only a few row groups on a 256-CU device).
constexpr int max_groups_for(int G) { return G <= 128 ? kMaxGroups : kMaxGroups * 128 / G; }
constexpr int kSlotSets = 4;
constexpr int group_stride_for(int G) { return 64 + kSlotSets * G * 16; }

}  // namespace rr
