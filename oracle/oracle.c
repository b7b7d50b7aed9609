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
