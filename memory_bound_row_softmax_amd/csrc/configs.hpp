// configs.hpp -- the menu of compiled kernel configurations.
//
// Shared by the planner (which may only pick what exists) and by the kernel
// files (which instantiate exactly this list).  No HIP here.
//
// Row-resident kernels (softmax, RMSNorm) are named by (P, R, G):
//   P  fp32 values each lane keeps in registers (P / 4 chunks of 16 bytes for
//      fp32 input, P / 8 for bf16),
//   R  lanes that share one row inside a workgroup (16..64: a slice of one
//      wave, 128..1024: several waves joined through LDS),
//   G  workgroups per row (1, or 2..16 on the grid path, where partial
//      results meet in a small global workspace).
// One row holds at most P * R * G elements.
//
// Streaming kernels (cross-entropy) are named by (P, R): each of the R lanes
// of a row loads P values per step and keeps a running (max, sum).
#pragma once

#define RR_ROW_CONFIGS(X)                                                                   \
    X(16, 16, 1) X(16, 32, 1) X(16, 64, 1) X(16, 128, 1) X(16, 256, 1) X(16, 512, 1)         \
    X(16, 1024, 1)                                                                           \
    X(32, 16, 1) X(32, 32, 1) X(32, 64, 1) X(32, 128, 1) X(32, 256, 1) X(32, 512, 1)         \
    X(32, 1024, 1)                                                                           \
    X(64, 16, 1) X(64, 32, 1) X(64, 64, 1) X(64, 128, 1) X(64, 256, 1) X(64, 512, 1)         \
    X(64, 1024, 1)                                                                           \
    X(32, 256, 2) X(32, 256, 4) X(32, 256, 8) X(32, 256, 16)                                 \
    X(32, 512, 2) X(32, 512, 4) X(32, 512, 8) X(32, 512, 16)                                 \
    X(32, 1024, 2) X(32, 1024, 4) X(32, 1024, 8) X(32, 1024, 16)                             \
    X(64, 256, 2) X(64, 256, 4) X(64, 256, 8) X(64, 256, 16)                                 \
    X(64, 512, 2) X(64, 512, 4) X(64, 512, 8) X(64, 512, 16)                                 \
    X(64, 1024, 2) X(64, 1024, 4) X(64, 1024, 8) X(64, 1024, 16)

#define RR_XENT_CONFIGS(X)                                                                  \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) X(16, 256) X(16, 512) X(16, 1024)              \
    X(32, 16) X(32, 32) X(32, 64) X(32, 128) X(32, 256) X(32, 512) X(32, 1024)

namespace rr {

// Op codes shared by the planner and the kernels.
constexpr int kCfgSoftmax = 0;
constexpr int kCfgRmsnorm = 1;

// Which row configurations are compiled for (op, element bytes, vectorised path).
// Excluded are those that would need more than the 128 VGPRs a lane of a
// 1024-thread workgroup can have, or whose per-element path holds more than 32
// values per lane; none of the compiled kernels uses scratch memory (the build
// checks this).  Register needs, measured on the gfx950 compiler:
//   softmax, 128-bit path:         about P + 40
//   RMSNorm:                       about 2P + 40 (row and weight both in registers)
//   per-element path:              grows with the per-element offsets, so P <= 32
//                                  (P <= 16 for RMSNorm with 1024 lanes)
constexpr bool row_config_enabled(int op, int elem_bytes, bool vec, int P, int R, int G) {
    (void)elem_bytes;
    (void)G;
    if (!vec && P > 32) return false;
    if (!vec && op == kCfgRmsnorm && R == 1024 && P > 16) return false;
    if (op == kCfgRmsnorm && R == 1024 && P == 64) return false;
    return true;
}

// Threads per workgroup and rows per workgroup for a lane-group width R.
constexpr int block_threads_for(int R) { return R < 256 ? 256 : R; }
constexpr int rows_per_block_for(int R) { return block_threads_for(R) / R; }

// Grid-path workspace layout (bytes):
//   [0, 256)                 header; word 0 is the error word (non-zero: a wait timed out)
//   256 + g * group_stride   record of row group g:
//       +0                   departure counter (uint32)
//       +64                  slots[2 parities][G][2] of uint64: (epoch << 32) | float bits
constexpr int kWsHeader = 256;
constexpr int kMaxGroups = 1024;
constexpr int group_stride_for(int G) { return 64 + 2 * G * 16; }

}  // namespace rr
