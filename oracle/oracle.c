/*
 * oracle.c -- plain, slow, single-threaded CPU reference for the three
 * memory-bound row reductions: softmax, RMSNorm and cross-entropy forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this file's library.  The GPU library never includes,
 * links or calls it, and it shares no code with the GPU library.
 *
 * Source pages.  [QuACK] is the QbitAI article "无需CUDA代码，给H100加速33%-50%"
 * (a summary of the QuACK tutorial on speed-of-light memory-bound kernels).
 * It names the three operators (section 让内存密集型内核达到"光速": RMSNorm,
 * softmax and the cross-entropy loss, the three kernels used as examples) and
 * describes softmax as a row max followed by an exponential sum and a final
 * pass (sections NCU 性能分析（Softmax 内核） and 内存吞吐量, last paragraphs:
 * the conventional three-pass softmax).  It prints no formula for any of
 * them, so each function below is the textbook definition, written out once,
 * in the order the definition states it:
 *
 *   softmax:        m = max_j x_j,  e_j = exp(x_j - m),  S = sum_j e_j,
 *                   y_j = e_j / S
 *   RMSNorm:        Q = sum_j x_j^2,  r = 1 / sqrt(Q / N + eps),
 *                   y_j = x_j * r * w_j      (eps inside the root, weight
 *                   multiplied, no bias, no mean subtraction)
 *   cross-entropy:  lse = m + log(sum_j exp(x_j - m)),  loss = lse - x_label
 *                   (per row, no reduction over rows; a label outside
 *                   [0, N) gives loss = NaN)
 *
 * The same pages present these kernels as building blocks of training as well
 * as inference (section 让内存密集型内核达到"光速").  The backward passes are
 * again textbook calculus on the definitions above, written out directly:
 *
 *   cross-entropy gradient (fused with the forward): with p_j = e_j / S the
 *                   softmax of the row and g the row's upstream gradient
 *                   dloss, dx_j = (p_j - [j == label]) * g; a label outside
 *                   [0, N) makes the whole row of dx NaN, like its loss
 *   softmax backward, from the forward output y and the upstream gradient dy:
 *                   c = sum_k y_k * dy_k,  dx_j = y_j * (dy_j - c)
 *   RMSNorm backward, from x, w, dy and the forward's fp32 rstd r:
 *                   c = sum_k dy_k * w_k * x_k,
 *                   dx_j = r * w_j * dy_j - r^3 * x_j * c / N,
 *                   dw_j = sum_i dy_ij * x_ij * r_i   (over all rows)
 *
 * Arithmetic: every input decodes exactly to double (fp32 by conversion,
 * bf16 as its 16 bits placed in the top half of an fp32); all sums run
 * left to right in double; exp, log and sqrt are the C library's double
 * functions.  Results are returned in double, unrounded.
 *
 * Pins (what checks this file against something other than itself) live in
 * tests/test_oracle_pins.py: closed forms, invariants, an arbitrary-precision
 * brute force on tiny rows, a float64 library cross-check and planted
 * mistakes that the pins must catch.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Input element type codes of this file (independent of any other header). */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

static double load_elem(const void *base, int dtype, int64_t i) {
    if (dtype == ORACLE_F32) return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int bad_args(int dtype, int64_t M, int64_t N) {
    return (dtype != ORACLE_F32 && dtype != ORACLE_BF16) || M < 0 || (M > 0 && N < 1);
}

/* softmax over each row of the M x N row-major matrix x; y is M x N double. */
int oracle_softmax(const void *x, int dtype, int64_t M, int64_t N, double *y) {
    if (bad_args(dtype, M, N)) return -1;
    for (int64_t i = 0; i < M; ++i) {
        int64_t row = i * N;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            double v = load_elem(x, dtype, row + j);
            if (v > m || isnan(v)) m = v;
        }
        double S = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double e = exp(load_elem(x, dtype, row + j) - m);
            y[row + j] = e;
            S += e;
        }
        for (int64_t j = 0; j < N; ++j) y[row + j] = y[row + j] / S;
    }
    return 0;
}

/* RMSNorm of each row with weight w[N]; eps is the fp32 value the caller
 * uses, widened to double.  rstd (may be NULL) receives r per row. */
int oracle_rmsnorm(const void *x, const void *w, int dtype, int64_t M, int64_t N, float eps,
                   double *y, double *rstd) {
    if (bad_args(dtype, M, N) || !(eps >= 0.0f)) return -1;
    double e = (double)eps;
    for (int64_t i = 0; i < M; ++i) {
        int64_t row = i * N;
        double Q = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double v = load_elem(x, dtype, row + j);
            Q += v * v;
        }
        double r = 1.0 / sqrt(Q / (double)N + e);
        if (rstd) rstd[i] = r;
        for (int64_t j = 0; j < N; ++j)
            y[row + j] = load_elem(x, dtype, row + j) * r * load_elem(w, dtype, j);
    }
    return 0;
}

/* Cross-entropy forward per row: lse = logsumexp(x_i), loss = lse - x_i[label_i]. */
int oracle_cross_entropy(const void *x, const int32_t *labels, int dtype, int64_t M, int64_t N,
                         double *loss, double *lse) {
    if (bad_args(dtype, M, N)) return -1;
    for (int64_t i = 0; i < M; ++i) {
        int64_t row = i * N;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            double v = load_elem(x, dtype, row + j);
            if (v > m || isnan(v)) m = v;
        }
        double S = 0.0;
        for (int64_t j = 0; j < N; ++j) S += exp(load_elem(x, dtype, row + j) - m);
        double l = m + log(S);
        if (lse) lse[i] = l;
        int32_t t = labels[i];
        loss[i] = (t >= 0 && (int64_t)t < N) ? l - load_elem(x, dtype, row + t) : NAN;
    }
    return 0;
}

/* Cross-entropy forward and its gradient with respect to the logits, per row:
 * loss and lse as oracle_cross_entropy, dx_j = (p_j - [j == label]) * dloss_i
 * with p the row's softmax.  dloss is fp32 per row (the upstream gradient of
 * each row's loss).  A label outside [0, N) gives loss = NaN and a NaN row of
 * dx.  dx is M x N double. */
int oracle_cross_entropy_grad(const void *x, const int32_t *labels, const float *dloss, int dtype,
                              int64_t M, int64_t N, double *loss, double *lse, double *dx) {
    if (bad_args(dtype, M, N)) return -1;
    for (int64_t i = 0; i < M; ++i) {
        int64_t row = i * N;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            double v = load_elem(x, dtype, row + j);
            if (v > m || isnan(v)) m = v;
        }
        double S = 0.0;
        for (int64_t j = 0; j < N; ++j) S += exp(load_elem(x, dtype, row + j) - m);
        double l = m + log(S);
        if (lse) lse[i] = l;
        int32_t t = labels[i];
        int ok = t >= 0 && (int64_t)t < N;
        loss[i] = ok ? l - load_elem(x, dtype, row + t) : NAN;
        double g = (double)dloss[i];
        for (int64_t j = 0; j < N; ++j) {
            double p = exp(load_elem(x, dtype, row + j) - m) / S;
            double onehot = (j == (int64_t)t) ? 1.0 : 0.0;
            dx[row + j] = ok ? (p - onehot) * g : NAN;
        }
    }
    return 0;
}

/* Softmax backward per row from the forward output y and the upstream
 * gradient dy (both of the input dtype): c = sum_k y_k dy_k,
 * dx_j = y_j * (dy_j - c).  dx is M x N double. */
int oracle_softmax_backward(const void *y, const void *dy, int dtype, int64_t M, int64_t N,
                            double *dx) {
    if (bad_args(dtype, M, N)) return -1;
    for (int64_t i = 0; i < M; ++i) {
        int64_t row = i * N;
        double c = 0.0;
        for (int64_t k = 0; k < N; ++k)
            c += load_elem(y, dtype, row + k) * load_elem(dy, dtype, row + k);
        for (int64_t j = 0; j < N; ++j)
            dx[row + j] = load_elem(y, dtype, row + j) * (load_elem(dy, dtype, row + j) - c);
    }
    return 0;
}

/* RMSNorm backward from x, w, the upstream gradient dy (all of the input
 * dtype) and the forward's per-row rstd (fp32): per row c = sum_k dy_k w_k x_k,
 * dx_j = r w_j dy_j - r^3 x_j c / N; over all rows dw_j = sum_i dy_ij x_ij r_i.
 * dx is M x N double, dw is N double. */
int oracle_rmsnorm_backward(const void *x, const void *w, const void *dy, const float *rstd,
                            int dtype, int64_t M, int64_t N, double *dx, double *dw) {
    if (bad_args(dtype, M, N)) return -1;
    for (int64_t j = 0; j < N; ++j) dw[j] = 0.0;
    for (int64_t i = 0; i < M; ++i) {
        int64_t row = i * N;
        double r = (double)rstd[i];
        double c = 0.0;
        for (int64_t k = 0; k < N; ++k)
            c += load_elem(dy, dtype, row + k) * load_elem(w, dtype, k) * load_elem(x, dtype, row + k);
        for (int64_t j = 0; j < N; ++j) {
            double xj = load_elem(x, dtype, row + j);
            double gj = load_elem(dy, dtype, row + j);
            dx[row + j] = r * load_elem(w, dtype, j) * gj - r * r * r * xj * c / (double)N;
            dw[j] += gj * xj * r;
        }
    }
    return 0;
}
