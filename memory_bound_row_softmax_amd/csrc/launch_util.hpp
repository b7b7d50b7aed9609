// launch_util.hpp -- shared host helpers for the per-op launch files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "configs.hpp"
#include "launch.hpp"

namespace rr {

// Row groups of a persistent launch with G workgroups per row: as many as fit on
// the device at once (so the whole grid normally runs at once), at most
// max_groups_for(G) and at most M.  Split rows need G workgroups of the kernel to fit at once (their
// members wait for each other; see grid_exchange.hpp).
template <class K>
hipError_t resident_groups(K kernel, int block, int G, int64_t M, const LaunchArgs &a,
                           int *groups) {
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0);
    if (e != hipSuccess) return e;
    int64_t g = (int64_t)per_cu * a.num_cus / G;
    // test override (rr_set_test_overrides): a grid larger than fits at once (split
    // rows must still drain when one XCD holds G workgroups)
    if (a.forced_groups > 0) g = a.forced_groups;
    if (g > max_groups_for(G)) g = max_groups_for(G);
    if (g > M) g = M;
    if (g < 1) return hipErrorCooperativeLaunchTooLarge;
    *groups = (int)g;
    return hipSuccess;
}

inline hipError_t blocks_for_rows(int64_t M, int rows_per_block, unsigned *blocks) {
    const int64_t b = (M + rows_per_block - 1) / rows_per_block;
    if (b < 1 || b > 0x7FFFFFFF) return hipErrorInvalidValue;
    *blocks = (unsigned)b;
    return hipSuccess;
}

}  // namespace rr
