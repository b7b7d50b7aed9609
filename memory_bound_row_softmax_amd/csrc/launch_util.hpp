// launch_util.hpp -- shared host helpers for the per-op launch files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "configs.hpp"
#include "launch.hpp"

namespace rr {

// Row groups of a cooperative (every block resident) launch with G blocks per row:
// as many as fit on the device at once, at most kMaxGroups and at most M, and a
// multiple of 8 when there are at least 8 (so each XCD gets whole groups).
template <class K>
hipError_t cooperative_groups(K kernel, int block, int G, int64_t M, const LaunchArgs &a,
                              int *groups) {
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0);
    if (e != hipSuccess) return e;
    int64_t g = (int64_t)per_cu * a.num_cus / G;
    if (g > kMaxGroups) g = kMaxGroups;
    if (g > M) g = M;
    if (g >= 8) g -= g % 8;
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
