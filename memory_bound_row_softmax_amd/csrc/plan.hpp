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

// Test-only overrides, set through rr_set_test_overrides() and nowhere else (all
// zero unless a test sets them): the kernel kind, P, R and G of the plan, the row
// groups of a persistent grid and the bound of each split-row wait.
enum ForcedKind { kForceNone = 0, kForceBlock = 1, kForceStream = 2, kForceLong = 3 };
struct TestOverrides {
    int kind = kForceNone;
    int P = 0, R = 0, G = 0;  // 0: not forced
    int groups = 0;           // 0: as many row groups as fit on the device
    int spin = 0;             // 0: the default bound; -1: every wait gives up at once
};
void set_test_overrides(const TestOverrides &o);
TestOverrides test_overrides();

// Chooses the plan.  `vec` says whether the 128-bit path is usable for these
// pointers.  Under test overrides (kind, P, R, G for the row ops; P, R for
// cross-entropy) a forced configuration that is not compiled, or too small for N,
// is unsupported.
PlanResult make_plan(int op, int dtype, int64_t M, int64_t N, bool vec, Plan *out);

// Workspace bytes of the grid path for G workgroups per row and M rows.
size_t grid_ws_bytes(int G, int64_t M);

}  // namespace rr
