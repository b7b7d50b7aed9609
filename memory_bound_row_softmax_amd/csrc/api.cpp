// api.cpp -- the C ABI of librr: argument validation, planning, launch.
//
// Declarations and the meaning of every argument are in include/rr.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "launch.hpp"
#include "plan.hpp"
#include "rr.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];

int device_cus(int dev, hipError_t *err) {
    *err = hipSuccess;
    if (dev >= 0 && dev < kMaxDevices) {
        int c = g_num_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int c = 0;
    *err = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (*err != hipSuccess) return 0;
    if (dev >= 0 && dev < kMaxDevices) g_num_cus[dev].store(c, std::memory_order_relaxed);
    return c;
}

// Polls of each split-row wait before it gives up (about a second on MI355X).
constexpr int kSpinLimit = 1 << 20;

rr_status hip_status(hipError_t e) {
    if (e == hipSuccess) return RR_OK;
    g_last_hip_error = (int)e;
    if (e == hipErrorCooperativeLaunchTooLarge) return RR_ERR_UNSUPPORTED;
    return RR_ERR_HIP;
}

size_t elem_size(rr_dtype dt) { return dt == RR_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + n) and [b, b + n) share a byte but do not start at the same address.
bool partial_overlap(const void *a, const void *b, size_t n) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    if (pa == pb) return false;
    return pa < pb + n && pb < pa + n;
}

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

// Common checks of the matrix arguments.  Returns RR_OK and the matrix size in bytes.
rr_status check_matrix(int64_t M, int64_t N, rr_dtype dt, size_t *bytes) {
    if (dt != RR_F32 && dt != RR_BF16) return RR_ERR_INVALID_ARGUMENT;
    if (M < 0) return RR_ERR_INVALID_ARGUMENT;
    if (M == 0) {
        *bytes = 0;
        return RR_OK;
    }
    if (N < 1) return RR_ERR_INVALID_ARGUMENT;
    const size_t s = elem_size(dt);
    if ((uint64_t)M > (uint64_t)INT64_MAX / (uint64_t)N / s) return RR_ERR_INVALID_ARGUMENT;
    *bytes = (size_t)M * (size_t)N * s;
    return RR_OK;
}

rr_status plan_status(rr::PlanResult r) {
    switch (r) {
    case rr::kPlanOk: return RR_OK;
    case rr::kPlanUnsupported: return RR_ERR_UNSUPPORTED;
    default: return RR_ERR_INVALID_ARGUMENT;
    }
}

// A buffer of the call, for the workspace overlap check (p may be NULL).
struct Region {
    const void *p;
    size_t n;
};

// The part of the workspace the plan uses must exist, be aligned and share no byte
// with any operand of the call.
rr_status check_workspace(const rr::Plan &p, void *ws, size_t ws_bytes,
                          std::initializer_list<Region> operands) {
    if (p.ws_bytes == 0) return RR_OK;
    if (!ws || ws_bytes < p.ws_bytes || !aligned16(ws)) return RR_ERR_WORKSPACE;
    for (const Region &r : operands)
        if (r.p && overlap(ws, p.ws_bytes, r.p, r.n)) return RR_ERR_WORKSPACE;
    return RR_OK;
}

rr_status launch_args(hipStream_t stream, rr::LaunchArgs *a) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    const int cus = device_cus(dev, &e);
    if (e != hipSuccess) return hip_status(e);
    const rr::TestOverrides ov = rr::test_overrides();
    *a = rr::LaunchArgs{stream, cus, ov.spin != 0 ? (ov.spin < 0 ? 0 : ov.spin) : kSpinLimit,
                        ov.groups > 0 ? ov.groups : 0};
    return RR_OK;
}

static_assert(RR_STATIC_SCRATCH_BYTES == rr::kStaticScratchBytes,
              "the header states the size of the library-held workspace");

// rr_softmax_fwd, with the caller's workspace or (static_ws) the library's own.
rr_status softmax_fwd(const void *x, void *y, int64_t M, int64_t N, rr_dtype dt, void *ws,
                      size_t ws_bytes, bool static_ws, hipStream_t stream) {
    size_t bytes = 0;
    rr_status st = check_matrix(M, N, dt, &bytes);
    if (st != RR_OK || M == 0) return st;
    if (!x || !y || partial_overlap(x, y, bytes)) return RR_ERR_INVALID_ARGUMENT;
    const bool vec = aligned16(x) && aligned16(y) && ((size_t)N * elem_size(dt)) % 16 == 0;
    rr::Plan p;
    st = plan_status(rr::make_plan(rr::kOpSoftmax, dt, M, N, vec, &p));
    if (st != RR_OK) return st;
    if (static_ws) {
        if (p.ws_bytes > rr::kStaticScratchBytes) return RR_ERR_WORKSPACE;
        ws = nullptr;
        ws_bytes = 0;
        if (p.ws_bytes > 0) {
            int dev = 0;
            hipError_t e = hipGetDevice(&dev);
            if (e == hipSuccess) e = rr::static_scratch(dev, &ws);
            if (e != hipSuccess) return hip_status(e);
            ws_bytes = rr::kStaticScratchBytes;
        }
    }
    if ((st = check_workspace(p, ws, ws_bytes, {{x, bytes}, {y, bytes}})) != RR_OK) return st;
    rr::LaunchArgs a;
    if ((st = launch_args(stream, &a)) != RR_OK) return st;
    if (p.path == rr::kPathLong)
        return hip_status(rr::launch_long_row(p, rr::kOpSoftmax, dt, x, nullptr, y, nullptr, M, N,
                                              0.0f, ws, a));
    return hip_status(rr::launch_softmax(p, dt, x, y, M, N, ws, a));
}

}  // namespace

extern "C" {

rr_status rr_softmax_fwd(const void *x, void *y, int64_t M, int64_t N, rr_dtype dt, void *ws,
                         size_t ws_bytes, hipStream_t stream) {
    return softmax_fwd(x, y, M, N, dt, ws, ws_bytes, false, stream);
}

rr_status rr_softmax_fwd_static(const void *x, void *y, int64_t M, int64_t N, rr_dtype dt,
                                hipStream_t stream) {
    return softmax_fwd(x, y, M, N, dt, nullptr, 0, true, stream);
}

rr_status rr_rmsnorm_fwd(const void *x, const void *w, void *y, float *rstd, int64_t M,
                         int64_t N, rr_dtype dt, float eps, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
    size_t bytes = 0;
    rr_status st = check_matrix(M, N, dt, &bytes);
    if (st != RR_OK) return st;
    if (!(eps >= 0.0f) || eps == INFINITY) return RR_ERR_INVALID_ARGUMENT;
    if (M == 0) return RR_OK;
    if (!x || !w || !y || partial_overlap(x, y, bytes)) return RR_ERR_INVALID_ARGUMENT;
    const bool vec = aligned16(x) && aligned16(y) && aligned16(w) &&
                     ((size_t)N * elem_size(dt)) % 16 == 0;
    rr::Plan p;
    st = plan_status(rr::make_plan(rr::kOpRmsnorm, dt, M, N, vec, &p));
    if (st != RR_OK) return st;
    const size_t row_vec = (size_t)M * 4u;
    if ((st = check_workspace(p, ws, ws_bytes,
                              {{x, bytes}, {y, bytes}, {w, (size_t)N * elem_size(dt)},
                               {rstd, row_vec}})) != RR_OK)
        return st;
    rr::LaunchArgs a;
    if ((st = launch_args(stream, &a)) != RR_OK) return st;
    if (p.path == rr::kPathLong)
        return hip_status(rr::launch_long_row(p, rr::kOpRmsnorm, dt, x, w, y, rstd, M, N, eps, ws,
                                              a));
    return hip_status(rr::launch_rmsnorm(p, dt, x, w, y, rstd, M, N, eps, ws, a));
}

rr_status rr_cross_entropy_fwd(const void *logits, const int32_t *labels, float *loss,
                               float *lse, int64_t M, int64_t N, rr_dtype dt, void *ws,
                               size_t ws_bytes, hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    size_t bytes = 0;
    rr_status st = check_matrix(M, N, dt, &bytes);
    if (st != RR_OK || M == 0) return st;
    if (!logits || !labels || !loss || N > INT32_MAX) return RR_ERR_INVALID_ARGUMENT;
    const bool vec = aligned16(logits) && ((size_t)N * elem_size(dt)) % 16 == 0;
    rr::Plan p;
    st = plan_status(rr::make_plan(rr::kOpXent, dt, M, N, vec, &p));
    if (st != RR_OK) return st;
    rr::LaunchArgs a;
    if ((st = launch_args(stream, &a)) != RR_OK) return st;
    return hip_status(rr::launch_xent(p, dt, logits, labels, loss, lse, M, N, a));
}

rr_status rr_cross_entropy_fwd_bwd(const void *logits, const int32_t *labels, const float *dloss,
                                   float *loss, float *lse, void *dlogits, int64_t M, int64_t N,
                                   rr_dtype dt, void *ws, size_t ws_bytes, hipStream_t stream) {
    size_t bytes = 0;
    rr_status st = check_matrix(M, N, dt, &bytes);
    if (st != RR_OK || M == 0) return st;
    if (!logits || !labels || !dloss || !loss || !dlogits || N > INT32_MAX || M >= (1ll << 30) ||
        partial_overlap(logits, dlogits, bytes))
        return RR_ERR_INVALID_ARGUMENT;
    const bool vec = aligned16(logits) && aligned16(dlogits) && ((size_t)N * elem_size(dt)) % 16 == 0;
    rr::Plan p;
    st = plan_status(rr::make_plan(rr::kOpXentGrad, dt, M, N, vec, &p));
    if (st != RR_OK) return st;
    const size_t row_vec = (size_t)M * 4u;
    if ((st = check_workspace(p, ws, ws_bytes,
                              {{logits, bytes}, {dlogits, bytes}, {labels, row_vec},
                               {dloss, row_vec}, {loss, row_vec}, {lse, row_vec}})) != RR_OK)
        return st;
    rr::LaunchArgs a;
    if ((st = launch_args(stream, &a)) != RR_OK) return st;
    if (p.path == rr::kPathLong)
        return hip_status(rr::launch_long_row(p, rr::kOpXentGrad, dt, logits, nullptr, dlogits, lse,
                                              M, N, 0.0f, ws, a, {labels, dloss, loss}));
    return hip_status(rr::launch_xent_grad(p, dt, logits, labels, dloss, loss, lse, dlogits, M, N,
                                           ws, a));
}

rr_status rr_softmax_bwd(const void *y, const void *dy, void *dx, int64_t M, int64_t N,
                         rr_dtype dt, void *ws, size_t ws_bytes, hipStream_t stream) {
    size_t bytes = 0;
    rr_status st = check_matrix(M, N, dt, &bytes);
    if (st != RR_OK || M == 0) return st;
    if (!y || !dy || !dx || partial_overlap(y, dx, bytes) || partial_overlap(dy, dx, bytes))
        return RR_ERR_INVALID_ARGUMENT;
    const bool vec = aligned16(y) && aligned16(dy) && aligned16(dx) &&
                     ((size_t)N * elem_size(dt)) % 16 == 0;
    rr::Plan p;
    st = plan_status(rr::make_plan(rr::kOpSoftmaxBwd, dt, M, N, vec, &p));
    if (st != RR_OK) return st;
    if ((st = check_workspace(p, ws, ws_bytes, {{y, bytes}, {dy, bytes}, {dx, bytes}})) != RR_OK)
        return st;
    rr::LaunchArgs a;
    if ((st = launch_args(stream, &a)) != RR_OK) return st;
    if (p.path == rr::kPathLong)
        return hip_status(rr::launch_long_row(p, rr::kOpSoftmaxBwd, dt, y, dy, dx, nullptr, M, N,
                                              0.0f, ws, a));
    return hip_status(rr::launch_softmax_bwd(p, dt, y, dy, dx, M, N, ws, a));
}

rr_status rr_rmsnorm_bwd(const void *x, const void *w, const void *dy, const float *rstd,
                         void *dx, float *dw, int64_t M, int64_t N, rr_dtype dt, void *ws,
                         size_t ws_bytes, hipStream_t stream) {
    size_t bytes = 0;
    rr_status st = check_matrix(M, N, dt, &bytes);
    if (st != RR_OK) return st;
    if (N < 1 || N > INT32_MAX || !dw) return RR_ERR_INVALID_ARGUMENT;
    const size_t dw_bytes = (size_t)N * 4u;
    if (M > 0) {
        if (!x || !w || !dy || !rstd || !dx || partial_overlap(x, dx, bytes) ||
            partial_overlap(dy, dx, bytes) || overlap(dw, dw_bytes, dx, bytes) ||
            overlap(dw, dw_bytes, x, bytes) || overlap(dw, dw_bytes, dy, bytes))
            return RR_ERR_INVALID_ARGUMENT;
    }
    const bool vec = M > 0 && aligned16(x) && aligned16(dy) && aligned16(dx) && aligned16(w) &&
                     ((size_t)N * elem_size(dt)) % 16 == 0;
    rr::Plan p;
    st = plan_status(rr::make_plan(rr::kOpRmsnormBwd, dt, M, N, vec, &p));
    if (st != RR_OK) return st;
    if (M > 0 && (st = check_workspace(p, ws, ws_bytes,
                                       {{x, bytes}, {dy, bytes}, {dx, bytes},
                                        {w, (size_t)N * elem_size(dt)}, {rstd, (size_t)M * 4u},
                                        {dw, dw_bytes}})) != RR_OK)
        return st;
    rr::LaunchArgs a;
    if ((st = launch_args(stream, &a)) != RR_OK) return st;
    return hip_status(rr::launch_rmsnorm_bwd(p, dt, x, w, dy, rstd, dx, dw, M, N, ws, a));
}

size_t rr_workspace_bytes(rr_op op, int64_t M, int64_t N, rr_dtype dt, int device) {
    (void)device;
    if (M <= 0) return 0;
    // The pointers are not known here, so cover both the 128-bit and the
    // per-element plan (the latter holds fewer values per lane).
    size_t need = 0;
    for (int vec = 0; vec < 2; ++vec) {
        rr::Plan p;
        if (rr::make_plan(op, dt, M, N, vec != 0, &p) == rr::kPlanOk && p.ws_bytes > need)
            need = p.ws_bytes;
    }
    return need;
}

rr_status rr_workspace_check(void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!ws || ws_bytes < sizeof(uint32_t)) return RR_ERR_WORKSPACE;
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e);
    uint32_t word = 0;
    e = hipMemcpy(&word, ws, sizeof word, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e);
    if (word == 0) return RR_OK;
    const uint32_t zero = 0;
    e = hipMemcpy(ws, &zero, sizeof zero, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_status(e);
    return RR_ERR_GRID_TIMEOUT;
}

rr_status rr_plan_query(rr_op op, int64_t M, int64_t N, rr_dtype dt, int vectorized,
                        rr_plan_info *out) {
    if (!out) return RR_ERR_INVALID_ARGUMENT;
    rr::Plan p;
    rr_status st = plan_status(rr::make_plan(op, dt, M, N, vectorized != 0, &p));
    if (st != RR_OK) return st;
    out->path = p.path;
    out->vectorized = p.vec ? 1 : 0;
    out->vals_per_lane = p.P;
    out->lanes_per_row = p.R;
    out->groups_per_row = p.G;
    out->block_threads = p.block;
    out->rows_per_block = p.rows_per_block;
    out->max_n = p.max_n;
    out->ws_bytes = p.ws_bytes;
    return RR_OK;
}

rr_status rr_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    if (!src || !dst || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst) ||
        partial_overlap(src, dst, bytes) || src == dst)
        return RR_ERR_INVALID_ARGUMENT;
    if (bytes == 0) return RR_OK;
    rr::LaunchArgs a;
    rr_status st = launch_args(stream, &a);
    if (st != RR_OK) return st;
    return hip_status(rr::launch_copy(src, dst, bytes, a));
}

rr_status rr_set_test_overrides(const rr_test_overrides *o) {
    rr::TestOverrides t;
    if (o) {
        if (o->kind < 0 || o->kind > 3 || o->vals_per_lane < 0 || o->lanes_per_row < 0 ||
            o->groups_per_row < 0 || o->resident_groups < 0 || o->spin_limit < -1)
            return RR_ERR_INVALID_ARGUMENT;
        t.kind = o->kind;
        t.P = o->vals_per_lane;
        t.R = o->lanes_per_row;
        t.G = o->groups_per_row;
        t.groups = o->resident_groups;
        t.spin = o->spin_limit;
    }
    rr::set_test_overrides(t);
    return RR_OK;
}

size_t rr_stream_read_sink_bytes(size_t bytes) { return rr::stream_read_sink_bytes(bytes); }

rr_status rr_stream_read(const void *src, size_t bytes, void *sink, size_t sink_bytes,
                         hipStream_t stream) {
    if (!src || !sink || bytes % 16 != 0 || !aligned16(src) ||
        (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return RR_ERR_INVALID_ARGUMENT;
    if (bytes == 0) return RR_OK;
    const size_t need = rr::stream_read_sink_bytes(bytes);
    if (sink_bytes < need || overlap(src, bytes, sink, need)) return RR_ERR_INVALID_ARGUMENT;
    rr::LaunchArgs a;
    rr_status st = launch_args(stream, &a);
    if (st != RR_OK) return st;
    return hip_status(rr::launch_read(src, bytes, static_cast<uint32_t *>(sink), a));
}

rr_status rr_stream_fill(void *dst, size_t bytes, uint32_t value, hipStream_t stream) {
    if (!dst || bytes % 16 != 0 || !aligned16(dst)) return RR_ERR_INVALID_ARGUMENT;
    if (bytes == 0) return RR_OK;
    rr::LaunchArgs a;
    rr_status st = launch_args(stream, &a);
    if (st != RR_OK) return st;
    return hip_status(rr::launch_fill(dst, bytes, value, a));
}

const char *rr_status_string(rr_status status) {
    switch (status) {
    case RR_OK: return "RR_OK";
    case RR_ERR_INVALID_ARGUMENT: return "RR_ERR_INVALID_ARGUMENT: invalid argument";
    case RR_ERR_UNSUPPORTED: return "RR_ERR_UNSUPPORTED: shape or grid not supported";
    case RR_ERR_WORKSPACE:
        return "RR_ERR_WORKSPACE: workspace missing, too small, misaligned or overlapping an "
               "operand";
    case RR_ERR_HIP: return "RR_ERR_HIP: a HIP call failed (see rr_last_hip_error)";
    case RR_ERR_GRID_TIMEOUT: return "RR_ERR_GRID_TIMEOUT: a split row timed out waiting for peers";
    }
    return "unknown rr_status";
}

int rr_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
