/*
 * CPU oracle for row softmax and the attention forward pass, fp16 in, fp16
 * out.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg load this library. The product path never
 * calls it and shares no code with it.
 *
 * What it computes follows "TileLang simplifica la creación de kernels GPU de
 * alto rendimiento", section "Softmax y FlashAttention sin materializar
 * matrices innecesarias":
 *
 *  * Row softmax: for each row, the maximum, the exponentials of the values
 *    minus it, their sum, and each exponential divided by the sum:
 *
 *        y[i][j] = exp(x[i][j] - max_k x[i][k]) / sum_k exp(x[i][k] - max_k x[i][k])
 *
 *  * Attention forward (the FlashAttention kernel's result; the page's blocked
 *    algorithm with running maxima, normalisation sums and rescaling reaches
 *    exactly this, up to rounding): for each batch b and head h, with
 *    Q[b][h] (Sq x D), K[b][h] and V[b][h] (Skv x D),
 *
 *        s[i][j] = scale * sum_d Q[i][d] K[j][d]
 *        p[i][j] = exp(s[i][j] - m_i) / l_i,  m_i = max_j s[i][j], l_i = sum_j exp(s[i][j] - m_i)
 *        O[i][d] = sum_j p[i][j] V[j][d]
 *
 *    with the maximum and the sums over the keys a query may see: all of
 *    them (non-causal), or, in the causal case, keys j <= i -- a position
 *    uses no information from later ones (the page's causal / non-causal
 *    distinction; "later" is counted from the first key, the convention of
 *    the PyTorch scaled-dot-product attention the page validates against).
 *    Also returned: the log-sum-exp lse_i = m_i + ln l_i.
 *
 * Everything is computed in double on the decoded fp16 inputs (exact decode,
 * the same hand-written binary16 definition as the GEMM oracle) and rounded
 * once to fp16, to nearest with ties to even. Sums run in index order.
 *
 * Plain C11, built with gcc -O2 (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

double oracle_f16_to_f64(uint16_t h);
uint16_t oracle_f64_to_f16_rne(double x);

/*
 * Row softmax of X[rows][cols] (fp16 bit patterns) into Y (fp16, rounded
 * once). yd, if not NULL, receives the double results. Returns 0, or -1 on a
 * bad argument or allocation failure.
 */
int oracle_softmax_rows_f16(int64_t rows, int64_t cols, const uint16_t* X, uint16_t* Y, double* yd)
{
    if (rows < 0 || cols < 0) return -1;
    if (rows == 0 || cols == 0) return 0;
    int err = 0;
#pragma omp parallel
    {
        double* e = (double*)malloc((size_t)cols * sizeof(double));
        if (!e) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = 0; i < rows; ++i) {
                const uint16_t* x = X + i * cols;
                double m = -INFINITY;
                for (int64_t j = 0; j < cols; ++j) {
                    const double v = oracle_f16_to_f64(x[j]);
                    if (v > m) m = v;
                }
                double l = 0.0;
                for (int64_t j = 0; j < cols; ++j) {
                    e[j] = exp(oracle_f16_to_f64(x[j]) - m);
                    l += e[j];
                }
                for (int64_t j = 0; j < cols; ++j) {
                    const double y = e[j] / l;
                    Y[i * cols + j] = oracle_f64_to_f16_rne(y);
                    if (yd) yd[i * cols + j] = y;
                }
            }
        }
        free(e);
    }
    return err ? -1 : 0;
}

/*
 * One query row: O[i][0..D) of batch-head bh, from the decoded scores. out:
 * fp16 row; od: double row (or NULL); lse: the log-sum-exp; pv: sum_j p_j
 * |V[j][d]| per d (or NULL), the scale of the rounding error a blocked
 * computation can make in O[i][d].
 */
static int attention_row(int64_t Sq, int64_t Skv, int64_t D, const uint16_t* Q, const uint16_t* K,
                         const uint16_t* V, double scale, int causal, int64_t i, uint16_t* out, double* od,
                         double* lse, double* pv)
{
    (void)Sq;
    const int64_t nkeys = causal ? (i + 1 < Skv ? i + 1 : Skv) : Skv;
    double* s = (double*)malloc((size_t)(nkeys > 0 ? nkeys : 1) * sizeof(double));
    double* o = (double*)calloc((size_t)(D > 0 ? D : 1), sizeof(double));
    double* a = (double*)calloc((size_t)(D > 0 ? D : 1), sizeof(double));
    if (!s || !o || !a) {
        free(s);
        free(o);
        free(a);
        return -1;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += oracle_f16_to_f64(Q[i * D + d]) * oracle_f16_to_f64(K[j * D + d]);
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t j = 0; j < nkeys; ++j) {
        const double p = s[j] / l;
        for (int64_t d = 0; d < D; ++d) {
            const double v = oracle_f16_to_f64(V[j * D + d]);
            o[d] += p * v;
            a[d] += p * fabs(v);
        }
    }
    for (int64_t d = 0; d < D; ++d) {
        out[d] = oracle_f64_to_f16_rne(nkeys > 0 ? o[d] : 0.0);
        if (od) od[d] = nkeys > 0 ? o[d] : 0.0;
        if (pv) pv[d] = a[d];
    }
    if (lse) *lse = nkeys > 0 ? m + log(l) : -INFINITY;
    free(s);
    free(o);
    free(a);
    return 0;
}

/*
 * Selected query rows of the attention forward pass. Q: [B*H][Sq][D],
 * K and V: [B*H][Skv][D], contiguous fp16. Row t is query qi[t] of batch-head
 * bh[t] (bh = b*H + h). Outputs per row t: out[t*D .. +D) (fp16), and, if not
 * NULL, od (double, same indexing), lse[t], pv[t*D .. +D).
 */
int oracle_attention_rows_f16(int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const uint16_t* Q,
                              const uint16_t* K, const uint16_t* V, double scale, int causal, int64_t nrows,
                              const int64_t* bh, const int64_t* qi, uint16_t* out, double* od, double* lse,
                              double* pv)
{
    if (BH < 0 || Sq < 0 || Skv < 0 || D < 0 || nrows < 0 || (causal != 0 && causal != 1)) return -1;
    for (int64_t t = 0; t < nrows; ++t)
        if (bh[t] < 0 || bh[t] >= BH || qi[t] < 0 || qi[t] >= Sq) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < nrows; ++t) {
        const int64_t g = bh[t];
        const int rc = attention_row(Sq, Skv, D, Q + g * Sq * D, K + g * Skv * D, V + g * Skv * D, scale, causal,
                                     qi[t], out + t * D, od ? od + t * D : NULL, lse ? lse + t : NULL,
                                     pv ? pv + t * D : NULL);
        if (rc) {
#pragma omp atomic write
            err = 1;
        }
    }
    return err ? -1 : 0;
}
