/*
 * rr.h -- C ABI of librr: memory-bound row reductions on AMD Instinct MI355X
 * (gfx950).  Softmax, RMSNorm and cross-entropy forward over a row-major
 * M x N matrix, each reading every input element from HBM once and (softmax,
 * RMSNorm) writing every output element once.
 *
 * Source pages.  [QuACK] is the QbitAI article "无需CUDA代码，给H100加速33%-50%",
 * a summary of the QuACK tutorial on speed-of-light memory-bound kernels.
 * Its section 让内存密集型内核达到"光速" names the three operators (RMSNorm,
 * softmax, cross-entropy loss) over a (batch x reduction dimension) input;
 * its section 内存吞吐量 gives the shapes (batch 8k-32k, reduction dimension
 * 256-262k, fp32 and bf16).  The pages print no formula; the definitions
 * stated at each function below are the textbook ones.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers, owned by the caller.  The library keeps
 *    no per-call state and allocates nothing.
 *  - Matrices are contiguous and row-major: element (i, j) is at i * N + j.
 *    x, y and w have the element type `dt`; cross-entropy outputs are fp32.
 *  - Calls are stream-ordered and asynchronous: RR_OK means the work was
 *    enqueued on `stream`.  Faults during execution surface at the caller's
 *    next synchronisation.  No call aborts or throws.
 *  - M == 0 is a no-op returning RR_OK.
 *  - 16-byte aligned pointers with (N * element size) % 16 == 0 take the
 *    vectorised path (128-bit loads and stores); anything else takes a
 *    per-element path that gives the same results more slowly (it still moves
 *    whole 16-byte chunks at element-aligned addresses, and only each row's last
 *    partial chunk element by element).
 *  - `ws` is a workspace that only rows split over several workgroups need:
 *    when rr_workspace_bytes(...) returns 0 it may be NULL.  Otherwise it
 *    must hold at least that many bytes, be 16-byte aligned, be zero-filled
 *    once when allocated, and must not be shared by launches that may run at
 *    the same time.  Its first word is the error word rr_workspace_check()
 *    reads.  Every launch that completes normally leaves it zero-filled again,
 *    except for the dw partial rows of rr_rmsnorm_bwd (scratch that each call
 *    rewrites).
 *  - The workgroups that share a row wait for each other.  The G workgroups of
 *    a row group are G consecutive block ids, and the grid is sized so that all
 *    of it fits on an idle device at once.  When it does not all run at once
 *    (other work holding the device), the launch still completes if each XCD can
 *    hold ceil(G / 8) of them (block b runs on XCD b mod 8, and each XCD starts
 *    its blocks in id order).  Each wait is bounded (about a second).  A workgroup whose wait gives up
 *    writes NaN in place of its share of that row (and of every later row whose wait
 *    also fails) and sets the workspace's error word, which rr_workspace_check()
 *    reports: a launch never ends with wrong values that are not NaN.
 */
#ifndef RR_H
#define RR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RR_OK = 0,
    RR_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, M < 0, N < 1 with M > 0, bad dtype,
                                    eps < 0 or not finite, partial overlap of x and y, N too
                                    large for an int32 label (cross-entropy) */
    RR_ERR_UNSUPPORTED = 2,      /* N above the largest row the on-chip plan can hold, or the
                                    workgroups that share a row do not fit on the device at
                                    once */
    RR_ERR_WORKSPACE = 3,        /* ws is NULL, smaller than rr_workspace_bytes(), not
                                    16-byte aligned, or shares a byte with an operand */
    RR_ERR_HIP = 4,              /* a HIP call failed; see rr_last_hip_error() */
    RR_ERR_GRID_TIMEOUT = 5      /* reported by rr_workspace_check(): a split row waited for
                                    its peer workgroups longer than the spin limit */
} rr_status;

typedef enum { RR_F32 = 0, RR_BF16 = 1 } rr_dtype;

typedef enum {
    RR_OP_SOFTMAX = 0,
    RR_OP_RMSNORM = 1,
    RR_OP_XENT = 2,
    RR_OP_XENT_GRAD = 3,   /* rr_cross_entropy_fwd_bwd */
    RR_OP_SOFTMAX_BWD = 4, /* rr_softmax_bwd */
    RR_OP_RMSNORM_BWD = 5  /* rr_rmsnorm_bwd */
} rr_op;

/*
 * Softmax forward, per row i:  m = max_j x_ij,  y_ij = exp(x_ij - m) / sum_k exp(x_ik - m).
 * [QuACK] section NCU 性能分析（Softmax 内核） (row max, exponential sum, final values)
 * and the closing paragraph of 内存吞吐量 (the conventional three-pass softmax over
 * on-chip data).  Arithmetic in fp32; y has the input type (bf16: round to nearest
 * even).  y == x (exact aliasing) is allowed; any other overlap is rejected.
 */
rr_status rr_softmax_fwd(const void *x, void *y, int64_t M, int64_t N, rr_dtype dt, void *ws,
                         size_t ws_bytes, hipStream_t stream);

/*
 * rr_softmax_fwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): rows split over several workgroups use a buffer the library holds on
 * each GPU, a device array of RR_STATIC_SCRATCH_BYTES (8 MiB + 256 KiB, enough for
 * every softmax plan) kept until the process ends.  The call allocates nothing; its
 * first call on a device looks the array's address up with hipGetSymbolAddress (not
 * an allocation).  Same arguments, results, plans and kernels as rr_softmax_fwd (the
 * same bits).  Calls on one GPU share the array: calls that may overlap on one GPU
 * (other streams, other threads) race and must not be made.  A wait that gives up is
 * seen as NaN rows (there is no workspace to check).  Returns RR_ERR_WORKSPACE if a
 * plan would need more than the array holds (no softmax plan does), RR_ERR_HIP if the
 * address lookup fails; otherwise as rr_softmax_fwd.
 */
#define RR_STATIC_SCRATCH_BYTES (8388608u + 262144u)
rr_status rr_softmax_fwd_static(const void *x, void *y, int64_t M, int64_t N, rr_dtype dt,
                                hipStream_t stream);

/*
 * RMSNorm forward, per row i:  r_i = 1 / sqrt(sum_j x_ij^2 / N + eps),  y_ij = x_ij * r_i * w_j.
 * [QuACK] section 让内存密集型内核达到"光速" (RMSNorm among the three kernels) and
 * 总结 (RMSNorm's layout, loads/stores and reduction helpers reused for softmax).
 * eps sits inside the root; there is no bias and no mean subtraction.  w has N
 * elements of type dt.  rstd (may be NULL) receives r_i as fp32.  Arithmetic in
 * fp32; y has the input type.  y == x is allowed.
 */
rr_status rr_rmsnorm_fwd(const void *x, const void *w, void *y, float *rstd, int64_t M,
                         int64_t N, rr_dtype dt, float eps, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * Cross-entropy forward, per row i:  lse_i = log sum_j exp(x_ij),  loss_i = lse_i - x_i[label_i].
 * [QuACK] section 让内存密集型内核达到"光速" (the cross-entropy loss kernel).  One loss
 * per row, no reduction over rows, no label smoothing and no ignored index.  A label
 * outside [0, N) gives loss_i = NaN (lse_i is still written) and is never used as an
 * address.  labels: int32[M]; loss: fp32[M]; lse: fp32[M] or NULL.  N must fit int32.
 */
rr_status rr_cross_entropy_fwd(const void *logits, const int32_t *labels, float *loss,
                               float *lse, int64_t M, int64_t N, rr_dtype dt, void *ws,
                               size_t ws_bytes, hipStream_t stream);

/*
 * Cross-entropy forward fused with its gradient with respect to the logits, per row i
 * (p_i = softmax of row i, g_i = dloss_i, the upstream gradient of loss_i):
 *     lse_i = log sum_j exp(x_ij),   loss_i = lse_i - x_i[label_i],
 *     dlogits_ij = (p_ij - [j == label_i]) * g_i.
 * [QuACK] section 让内存密集型内核达到"光速" (the cross-entropy loss kernel, and these
 * kernels as building blocks of training); the gradient is the textbook derivative of
 * the per-row loss.  The row is read from HBM once and the gradient written once.
 * labels: int32[M]; dloss: fp32[M] (e.g. 1/M everywhere for a mean over rows);
 * loss: fp32[M]; lse: fp32[M] or NULL; dlogits: M x N of type dt (bf16: round to
 * nearest even).  dlogits == logits (exact aliasing) is allowed; any other overlap is
 * rejected.  A label outside [0, N) gives loss_i = NaN and a NaN row of dlogits (lse_i
 * is still written); it is never used as an address.  Plans and workspace are queried
 * with RR_OP_XENT_GRAD.  Rows past the on-chip plans (more than 2097152 elements, or
 * 262144 when logits or dlogits is not 16-byte aligned), up to 2^28 elements, take a
 * two-read kernel: the row's max and sum over a first read, dlogits from a second.
 * N must fit int32 and M be below 2^30.
 */
rr_status rr_cross_entropy_fwd_bwd(const void *logits, const int32_t *labels, const float *dloss,
                                   float *loss, float *lse, void *dlogits, int64_t M, int64_t N,
                                   rr_dtype dt, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Softmax backward from the forward output y and the upstream gradient dy, per row i:
 *     c_i = sum_k y_ik * dy_ik,   dx_ij = y_ij * (dy_ij - c_i).
 * [QuACK] sections NCU 性能分析（Softmax 内核） and 内存吞吐量 (the softmax) and
 * 让内存密集型内核达到"光速" (these kernels as building blocks of training); the formula
 * is the textbook derivative of the softmax.  y, dy and dx are M x N of type dt; y and
 * dy are each read once and dx written once.  dx may be y or dy itself (exact aliasing);
 * any other overlap among the three is rejected.  Arithmetic in fp32.  Rows of more than
 * 32768 elements are split over workgroups and need a workspace (RR_OP_SOFTMAX_BWD).
 * Rows past the on-chip plans (more than 1048576 elements, or 262144 when y, dy or dx
 * is not 16-byte aligned), up to 2^28 elements, take a two-read kernel: c_i is summed
 * over a first read of y and dy, and dx is written from a second read.
 */
rr_status rr_softmax_bwd(const void *y, const void *dy, void *dx, int64_t M, int64_t N,
                         rr_dtype dt, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * RMSNorm backward from x, w, the upstream gradient dy and the forward's rstd r
 * (per row i, as written by rr_rmsnorm_fwd):
 *     c_i = sum_k dy_ik w_k x_ik,   dx_ij = r_i (w_j dy_ij - x_ij r_i^2 c_i / N),
 *     dw_j = sum_i dy_ij x_ij r_i.
 * [QuACK] section 让内存密集型内核达到"光速" (RMSNorm among the memory-bound kernels,
 * which serve training as well as inference); the formulas are the textbook
 * derivative of the forward above (eps enters only through r).  x, dy, dx: M x N of
 * type dt; w: N of type dt; rstd: fp32[M]; dw: fp32[N] (always written, zeros when
 * M == 0).  x and dy are read once and dx written once; dw is reduced over the rows
 * through fp32 partial rows in the workspace (one per workgroup), added in a fixed
 * order, so repeated calls give the same bits.  dx may be x or dy itself (exact
 * aliasing); any other overlap among x, dy, dx and dw is rejected.  The workspace
 * (RR_OP_RMSNORM_BWD) is always needed when M > 0; only its first part (the header
 * and, for split rows, the exchange area) must start zero-filled, as for the other
 * calls.  N up to 262144.
 */
rr_status rr_rmsnorm_bwd(const void *x, const void *w, const void *dy, const float *rstd,
                         void *dx, float *dw, int64_t M, int64_t N, rr_dtype dt, void *ws,
                         size_t ws_bytes, hipStream_t stream);

/*
 * Bytes of workspace a call with these arguments needs (0 when it needs none),
 * whatever the alignment of the pointers it will get.  The value depends only on
 * (op, M, N, dt); `device` is accepted for callers that size per device and is
 * otherwise unused (pass -1).
 */
size_t rr_workspace_bytes(rr_op op, int64_t M, int64_t N, rr_dtype dt, int device);

/*
 * Reads (and clears) the error word of a workspace after the work on `stream`
 * has finished (this call synchronises the stream).  Returns RR_OK, or
 * RR_ERR_GRID_TIMEOUT if some split row gave up waiting for its peers, in which
 * case that launch's outputs are not valid.
 */
rr_status rr_workspace_check(void *ws, size_t ws_bytes, hipStream_t stream);

/* Plan chosen for a call, for inspection and tests.  Needs no GPU. */
typedef struct {
    int path;           /* 0: block kernel, one row per lane group or workgroup,
                           1: persistent stream kernel with each row split over
                              `groups_per_row` workgroups (split rows, workspace),
                           2: cross-entropy forward (streaming online max and sum),
                           3: persistent stream kernel, one workgroup per row,
                           4: two-read long-row kernel (softmax and RMSNorm forward,
                              softmax backward, cross-entropy gradient), `groups_per_row`
                              workgroups per row (workspace) */
    int vectorized;     /* 1: 128-bit path, 0: per-element path */
    int vals_per_lane;  /* values each lane holds (row paths: fp32 values, or 128 bf16 values
                           kept packed by the bf16 RMSNorm) or loads per step (streaming) */
    int lanes_per_row;  /* lanes that share one row inside a workgroup */
    int groups_per_row; /* workgroups per row (1 except on path 1) */
    int block_threads;  /* threads per workgroup */
    int rows_per_block; /* rows one workgroup processes at once */
    int64_t max_n;      /* largest N this configuration holds (row paths) */
    size_t ws_bytes;    /* workspace bytes the call needs */
} rr_plan_info;

rr_status rr_plan_query(rr_op op, int64_t M, int64_t N, rr_dtype dt, int vectorized,
                        rr_plan_info *out);

/*
 * Streaming ceilings, measured in the same run as the kernels they are compared with
 * ([QuACK] sections NCU 性能分析（Softmax 内核） and 内存吞吐量 report each kernel's DRAM
 * throughput as a share of what the memory delivers).  Not operators of the pages;
 * measurement aids.  Each moves every byte once, 16 bytes per lane per access, with
 * the row kernels' non-temporal cache policies, and assigns the blocks of every
 * 128 KiB region to the eight XCDs so that each XCD's accesses share address bits
 * 12..14 (the mapping measured fastest for one read plus one write per byte).
 * `bytes` is a multiple of 16 and the data pointers are 16-byte aligned; otherwise
 * RR_ERR_INVALID_ARGUMENT.  Stream-ordered like the operators.
 *
 * rr_stream_copy: copies src to dst (no overlap; one read and one write per byte).
 * rr_stream_read: reads src and writes one 32-bit XOR checksum per 16 KiB to `sink`
 *   (4-byte aligned, at least rr_stream_read_sink_bytes(bytes) bytes, no overlap
 *   with src), so the reads cannot be dropped.
 * rr_stream_fill: writes the 32-bit `value` over dst (one write per byte).
 */
rr_status rr_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);
size_t rr_stream_read_sink_bytes(size_t bytes);
rr_status rr_stream_read(const void *src, size_t bytes, void *sink, size_t sink_bytes,
                         hipStream_t stream);
rr_status rr_stream_fill(void *dst, size_t bytes, uint32_t value, hipStream_t stream);

/*
 * Test-only: forces plan and launch choices for every later call in the process, so
 * that tests reach each kernel path at sizes the oracle checks in seconds (a split row
 * at N = 3000, a grid several times larger than the device holds, a wait that gives
 * up).  Not for production use: a forced plan may be slow or unsupported, and a forced
 * spin limit makes split rows time out (their rows are then NaN and
 * rr_workspace_check() reports RR_ERR_GRID_TIMEOUT).  Nothing else in the library
 * reads these values, and no environment variable changes any plan.  NULL (or all
 * fields zero) restores the defaults.  Returns RR_ERR_INVALID_ARGUMENT for a negative
 * field (other than spin_limit = -1) or an unknown kind.  Process-wide; not meant to be
 * changed while calls run on other threads.
 */
typedef struct {
    int kind;            /* 0: the planner's choice, 1: block kernel, 2: stream kernel,
                            3: the two-read long-row kernel (softmax and RMSNorm forward,
                               softmax backward, cross-entropy gradient) */
    int vals_per_lane;   /* P of the plan (0: the planner's choice) */
    int lanes_per_row;   /* R of the plan (0: the planner's choice) */
    int groups_per_row;  /* G of the plan (0: the planner's choice) */
    int resident_groups; /* row groups of a persistent grid (0: as many as fit at once) */
    int spin_limit;      /* polls per split-row wait (0: the default of 2^20, about a
                            second); -1: every wait gives up at once */
} rr_test_overrides;

rr_status rr_set_test_overrides(const rr_test_overrides *overrides);

const char *rr_status_string(rr_status status);

/* hipError_t of the most recent RR_ERR_HIP in the calling thread (0 if none). */
int rr_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RR_H */
