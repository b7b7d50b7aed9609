// plan.hpp -- host planner: picks the kernel configuration for (op, dtype, M, N).
// No HIP here, so it is testable on any machine.
#pragma once

#include <cstddef>
#include <cstdint>

namespace rr {

// kPathRow: block kernel; kPathSplit: stream kernel with G > 1 (split rows);
// kPathXent: cross-entropy; kPathStream: stream kernel with G = 1; kPathLong: rows
// past the on-chip capacity, read twice (softmax and RMSNorm forward).
enum PathKind { kPathRow = 0, kPathSplit = 1, kPathXent = 2, kPathStream = 3, kPathLong = 4 };
// kOpXentGrad (cross-entropy forward fused with its gradient) runs the softmax
// kernels with another epilogue and takes the softmax plan.
// kOpSoftmaxBwd: softmax backward from the forward output (two input rows).
// kOpRmsnormBwd: RMSNorm backward (dx per row, dw down the columns).
enum OpKind {
    kOpSoftmax = 0,
    kOpRmsnorm = 1,
    kOpXent = 2,
    kOpXentGrad = 3,
    kOpSoftmaxBwd = 4,
    kOpRmsnormBwd = 5
};
enum DtypeKind { kF32 = 0, kBf16 = 1 };
enum PlanResult { kPlanOk = 0, kPlanUnsupported = 1, kPlanInvalid = 2 };

struct Plan {
    int path = kPathRow;
    // RMSNorm backward: byte offset in the workspace of the dw partial rows, and
    // their count at most.
    size_t part_off = 0;
    int max_parts = 0;
    bool stream = false;  // persistent, double-buffered stream kernel
    bool vec = true;
    int P = 0, R = 0, G = 1;
    int block = 0, rows_per_block = 0;
    int64_t max_n = 0;
    size_t ws_bytes = 0;
};

// Whether a configuration is compiled (and usable) for (op, dtype, vec).
bool block_config_ok(int op, int dtype, bool vec, int P, int R);
bool stream_config_ok(int op, int dtype, bool vec, int P, int R, int G);
bool xent_config_exists(int P, int R);
bool rmsbwd_config_ok(int dtype, bool vec, int P, int R, int G);

// Chooses the plan.  `vec` says whether the 128-bit path is usable for these
// pointers.  Test-only overrides come from the environment: RR_FORCE_KIND
// ("block", "stream" or "long"), RR_FORCE_P, RR_FORCE_R and RR_FORCE_G (row ops), or
// RR_FORCE_P and RR_FORCE_R (cross-entropy); a forced configuration that is not
// compiled, or too small for N, is unsupported.
PlanResult make_plan(int op, int dtype, int64_t M, int64_t N, bool vec, Plan *out);

// Workspace bytes of the grid path for G workgroups per row and M rows.
size_t grid_ws_bytes(int G, int64_t M);

}  // namespace rr
