// plan.cpp -- host planner (no HIP).
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%) chooses, before launch, how
// threads map onto the reduction dimension (section 硬件感知的加载与存储策略, the
// thread-value layout) and whether a row is reduced inside one block or across a
// cluster of blocks, depending on the size of the reduction dimension (section
// 硬件感知的归约策略, the last paragraph).  It also notes that the tuning is per
// operator and per shape (section 总结).  This file is that choice for gfx950:
//   * a row of up to P * R elements lives in the registers of R lanes
//     (R <= 64: part of one wave; R > 64: R / 64 waves joined through LDS);
//   * longer rows are split over G workgroups that exchange partial results
//     through global memory (the cluster / distributed-shared-memory level of
//     the pages has no counterpart on this GPU);
//   * cross-entropy writes no per-element output, so it streams its row with a
//     running (max, sum) instead of holding it.
#include "plan.hpp"

#include <cstdlib>

#include "configs.hpp"

namespace rr {

bool row_config_exists(int P, int R, int G) {
#define RR_X(p, r, g) \
    if (P == p && R == r && G == g) return true;
    RR_ROW_CONFIGS(RR_X)
#undef RR_X
    return false;
}

bool xent_config_exists(int P, int R) {
#define RR_X(p, r) \
    if (P == p && R == r) return true;
    RR_XENT_CONFIGS(RR_X)
#undef RR_X
    return false;
}

size_t grid_ws_bytes(int G, int64_t M) {
    int64_t groups = M < kMaxGroups ? M : kMaxGroups;
    if (groups < 1) groups = 1;
    return (size_t)kWsHeader + (size_t)groups * (size_t)group_stride_for(G);
}

static int64_t next_pow2(int64_t v) {
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

static int env_int(const char *name) {
    const char *s = std::getenv(name);
    if (!s || !*s) return 0;
    return std::atoi(s);
}

static void fill_geometry(Plan *p) {
    p->block = block_threads_for(p->R);
    p->rows_per_block = rows_per_block_for(p->R);
}

// Default row-resident choice: the fewest workgroups per row, then the preferred
// number of values per lane (more values per lane = more 128-bit loads in flight
// per lane; small rows prefer fewer so that one row still spans many lanes),
// then the narrowest lane group that holds the row.
static bool default_row(int op, int dtype, bool vec, int64_t N, int *P, int *R, int *G) {
    static const int kPrefSmall[3] = {16, 32, 64};
    static const int kPrefMid[3] = {32, 64, 16};
    static const int kPrefLarge[3] = {64, 32, 16};
    const int *pref = N <= 1024 ? kPrefSmall : (N <= 2048 ? kPrefMid : kPrefLarge);
    const int cfg_op = op == kOpSoftmax ? kCfgSoftmax : kCfgRmsnorm;
    const int ebytes = dtype == kBf16 ? 2 : 4;
    for (int g = 1; g <= 16; g *= 2) {
        for (int k = 0; k < 3; ++k) {
            const int p = pref[k];
            int64_t r = next_pow2((N + (int64_t)p * g - 1) / ((int64_t)p * g));
            if (r < 16) r = 16;
            if (g > 1 && r < 256) r = 256;
            if (r > 1024) continue;
            if (!row_config_exists(p, (int)r, g) ||
                !row_config_enabled(cfg_op, ebytes, vec, p, (int)r, g))
                continue;
            *P = p;
            *R = (int)r;
            *G = g;
            return true;
        }
    }
    return false;
}

static void default_xent(int64_t N, int *P, int *R) {
    *P = N <= 512 ? 16 : 32;
    int64_t r = next_pow2((N + *P - 1) / *P);
    if (r < 16) r = 16;
    if (r > 256) r = 256;
    *R = (int)r;
}

PlanResult make_plan(int op, int dtype, int64_t M, int64_t N, bool vec, Plan *out) {
    if (!out) return kPlanInvalid;
    if ((op != kOpSoftmax && op != kOpRmsnorm && op != kOpXent) ||
        (dtype != kF32 && dtype != kBf16) || M < 0 || (M > 0 && N < 1))
        return kPlanInvalid;
    if (N < 1) N = 1;  // M == 0: any plan will do, nothing is launched
    Plan p;
    p.vec = vec;
    const int fP = env_int("RR_FORCE_P"), fR = env_int("RR_FORCE_R"), fG = env_int("RR_FORCE_G");

    if (op == kOpXent) {
        if (N > INT32_MAX) return kPlanInvalid;
        int P, R;
        default_xent(N, &P, &R);
        if (fP) P = fP;
        if (fR) R = fR;
        if (!xent_config_exists(P, R)) return kPlanUnsupported;
        p.path = kPathStream;
        p.P = P;
        p.R = R;
        p.G = 1;
        p.max_n = INT32_MAX;
        p.ws_bytes = 0;
        fill_geometry(&p);
        *out = p;
        return kPlanOk;
    }

    int P = 0, R = 0, G = 1;
    if (fP || fR || fG) {
        P = fP ? fP : 64;
        R = fR ? fR : 1024;
        G = fG ? fG : 1;
    } else if (!default_row(op, dtype, vec, N, &P, &R, &G)) {
        return kPlanUnsupported;
    }
    const int cfg_op = op == kOpSoftmax ? kCfgSoftmax : kCfgRmsnorm;
    if (!row_config_exists(P, R, G) ||
        !row_config_enabled(cfg_op, dtype == kBf16 ? 2 : 4, vec, P, R, G))
        return kPlanUnsupported;
    p.P = P;
    p.R = R;
    p.G = G;
    p.max_n = (int64_t)P * R * G;
    if (N > p.max_n) return kPlanUnsupported;
    p.path = G > 1 ? kPathGrid : kPathRow;
    p.ws_bytes = G > 1 ? grid_ws_bytes(G, M) : 0;
    fill_geometry(&p);
    *out = p;
    return kPlanOk;
}

}  // namespace rr
