/*
 * CPU oracle for C = ReLU(A @ B), fp16 A[M,K], B[K,N], fp16 C[M,N].
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg load this library. The product path never
 * calls it and shares no code with it.
 *
 * What it computes follows the TileLang GEMM example ("Writing
 * high-performance kernels in TileLang", section "Escribamos un GEMM"): the
 * kernel there takes fp16 A (M x K) and B (K x N), accumulates the tile
 * products in a wider accumulator, applies max(x, 0) to the accumulator and
 * only then writes the result into an fp16 C (M x N); the example checks the
 * result against relu(a @ b). That result has a plain definition, so the
 * oracle is that definition written out:
 *
 *   1. decode every fp16 bit pattern to a double (IEEE binary16 definition);
 *   2. pre[i][j] = sum over k = 0, 1, ..., K-1 (in that order) of
 *      a[i][k] * b[k][j] in double precision -- each product of two fp16
 *      values is exact in double (11 + 11 significant bits);
 *   3. y = pre > 0 ? pre : +0 (the ReLU);
 *   4. encode y to fp16 with round to nearest, ties to even.
 *
 * The second operation is the fused epilogue of "TileLang simplifica la
 * creación de kernels GPU de alto rendimiento" (section "Fusionar operaciones
 * para reducir viajes a memoria"): the bias is added to the accumulator and
 * GELU applied before the single write of C. The page names GELU without a
 * formula; the oracle uses its definition, GELU(x) = x * Phi(x) with Phi the
 * standard normal distribution function, Phi(x) = erfc(-x / sqrt 2) / 2.
 * The page does not give the bias's type or shape either; the reading here
 * is one fp16 value per column of C (bias[j] added to every row), decoded
 * exactly like A and B:
 *
 *   pre[i][j] = sum over k (ascending) of a[i][k] * b[k][j]  +  bias[j]
 *   C[i][j]   = fp16_rne( GELU(pre[i][j]) )
 *
 * Transposed operands. The tile-level product of the same TileLang example
 * takes transpose_A / transpose_B flags (the notes under the program in
 * section "Escribamos un GEMM"): C = epilogue(op(A) @ op(B)), where op(A) is
 * either A as stored (M x K, leading dimension K) or the transpose of a
 * stored K x M matrix (leading dimension M), and op(B) is either B as stored
 * (K x N, leading dimension N) or the transpose of a stored N x K matrix
 * (leading dimension K). Only where the elements are read changes:
 *
 *   op(A)[i][k] = op_a ? A[k*M + i] : A[i*K + k]
 *   op(B)[k][j] = op_b ? B[j*K + k] : B[k*N + j]
 *
 * Readings where the pages are silent: the final rounding is IEEE
 * round-to-nearest-even (what an ordinary fp32 -> fp16 conversion does);
 * overflow past the largest finite fp16 becomes +inf; fp16 subnormals are
 * honoured on input and output; the sum over an empty K is 0.
 *
 * Each output element's summation order is fixed (k ascending), so results do
 * not depend on how many threads run the row loop.
 *
 * Plain C11, no fp16 compiler types, built with gcc -O2 (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- IEEE binary16 decode: sign, 5-bit exponent (bias 15), 10-bit fraction ---- */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;             /* inf / NaN */
    } else {
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a non-negative double q to the nearest integer, ties to even. */
static double round_half_even(double q)
{
    const double fl = floor(q);
    const double r = q - fl;                       /* exact for q < 2^52 */
    if (r > 0.5) return fl + 1.0;
    if (r < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* ---- IEEE binary16 encode, round to nearest, ties to even ---- */
uint16_t oracle_f64_to_f16_rne(double x)
{
    if (isnan(x)) return 0x7e00;
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const double a = fabs(x);
    /* 65504 is the largest finite value, its spacing is 32; half of it past
       65504 is 65520, which ties to the even neighbour 65536 = overflow. */
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; n == 1024 is the smallest normal */
        const double n = round_half_even(ldexp(a, 24));
        return sign | (uint16_t)n;
    }
    int E;
    (void)frexp(a, &E);                            /* a = f * 2^E, f in [0.5, 1) */
    int ex = E - 1;                                /* a in [2^ex, 2^(ex+1)) */
    double n = round_half_even(ldexp(a, 10 - ex)); /* in [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; ex += 1; }
    if (ex + 15 >= 31) return sign | 0x7c00;
    return sign | (uint16_t)(((ex + 15) << 10) | ((int)n - 1024));
}

void oracle_decode_f16(const uint16_t* h, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

void oracle_encode_f16(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16_rne(x[i]);
}

static uint16_t relu_to_f16(double pre)
{
    return oracle_f64_to_f16_rne(pre > 0.0 ? pre : 0.0);
}

/* GELU by its definition: x * Phi(x), with the standard normal distribution
   function written Phi(x) = erfc(-x / sqrt 2) / 2 -- the same function as
   (1 + erf(x / sqrt 2)) / 2, without the cancellation of that form for
   negative x. */
double oracle_gelu(double x)
{
    return x * (0.5 * erfc(-x / sqrt(2.0)));
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Element (i, k) of op(A), and element (k, j) of op(B), as stored. */
static uint16_t a_elem(const uint16_t* A, int op_a, int64_t M, int64_t K, int64_t i, int64_t k)
{
    return op_a ? A[k * M + i] : A[i * K + k];
}

static uint16_t b_elem(const uint16_t* B, int op_b, int64_t K, int64_t N, int64_t k, int64_t j)
{
    return op_b ? B[j * K + k] : B[k * N + j];
}

/* The epilogue: ReLU (bias == NULL) or bias + GELU. */
static uint16_t finish(double acc, const uint16_t* bias, int64_t j, double* pre_out)
{
    if (!bias) {
        if (pre_out) *pre_out = acc;
        return relu_to_f16(acc);
    }
    const double pre = acc + oracle_f16_to_f64(bias[j]);
    if (pre_out) *pre_out = pre;
    return oracle_f64_to_f16_rne(oracle_gelu(pre));
}

/*
 * Rows [row0, row1) of C. C points at row 0 of the full C (leading
 * dimension N). pre, if not NULL, receives the double pre-activation values
 * (same indexing as C); absdot, if not NULL, receives sum_k |a||b|.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
static int rows_impl(int64_t M, int64_t N, int64_t K, const uint16_t* A, int op_a, const uint16_t* B,
                     int op_b, const uint16_t* bias, uint16_t* C, double* pre, double* absdot,
                     int64_t row0, int64_t row1)
{
    if (M < 0 || N < 0 || K < 0 || row0 < 0 || row1 > M || row0 > row1) return -1;
    if (N == 0 || row0 == row1) return 0;
    /* op(B) decoded once, row k of op(B) at bd + k*N */
    double* bd = NULL;
    if (K > 0) {
        bd = (double*)malloc((size_t)K * (size_t)N * sizeof(double));
        if (!bd) return -1;
        for (int64_t k = 0; k < K; ++k)
            for (int64_t j = 0; j < N; ++j) bd[k * N + j] = oracle_f16_to_f64(b_elem(B, op_b, K, N, k, j));
    }
    int err = 0;
#pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)N * sizeof(double));
        double* sab = absdot ? (double*)malloc((size_t)N * sizeof(double)) : NULL;
        if (!acc || (absdot && !sab)) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = row0; i < row1; ++i) {
                for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
                if (sab) for (int64_t j = 0; j < N; ++j) sab[j] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double a = oracle_f16_to_f64(a_elem(A, op_a, M, K, i, k));
                    const double* brow = bd + k * N;
                    for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
                    if (sab) {
                        const double aa = fabs(a);
                        for (int64_t j = 0; j < N; ++j) sab[j] += aa * fabs(brow[j]);
                    }
                }
                for (int64_t j = 0; j < N; ++j) {
                    C[i * N + j] = finish(acc[j], bias, j, pre ? &pre[i * N + j] : NULL);
                    if (sab) absdot[i * N + j] = sab[j];
                }
            }
        }
        free(acc);
        free(sab);
    }
    free(bd);
    return err ? -1 : 0;
}

/*
 * Selected elements (ii[t], jj[t]), each summed in the same k-ascending order
 * as the full routine, so it gives the same values there.
 */
static int points_impl(int64_t M, int64_t N, int64_t K, const uint16_t* A, int op_a, const uint16_t* B,
                       int op_b, const uint16_t* bias, int64_t npts, const int64_t* ii, const int64_t* jj,
                       uint16_t* out, double* pre, double* absdot)
{
    if (M < 0 || N < 0 || K < 0 || npts < 0) return -1;
    for (int64_t t = 0; t < npts; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < npts; ++t) {
        const int64_t i = ii[t], j = jj[t];
        double acc = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = oracle_f16_to_f64(a_elem(A, op_a, M, K, i, k));
            const double b = oracle_f16_to_f64(b_elem(B, op_b, K, N, k, j));
            acc += a * b;
            s += fabs(a) * fabs(b);
        }
        out[t] = finish(acc, bias, j, pre ? &pre[t] : NULL);
        if (absdot) absdot[t] = s;
    }
    return 0;
}

/* Rows [row0, row1) of C = ReLU(A @ B). */
int oracle_gemm_relu_f16_rows(int64_t M, int64_t N, int64_t K,
                              const uint16_t* A, const uint16_t* B, uint16_t* C,
                              double* pre, double* absdot,
                              int64_t row0, int64_t row1)
{
    return rows_impl(M, N, K, A, 0, B, 0, NULL, C, pre, absdot, row0, row1);
}

/* The whole of C = ReLU(A @ B). */
int oracle_gemm_relu_f16(int64_t M, int64_t N, int64_t K,
                         const uint16_t* A, const uint16_t* B, uint16_t* C,
                         double* pre, double* absdot)
{
    return rows_impl(M, N, K, A, 0, B, 0, NULL, C, pre, absdot, 0, M);
}

/* Selected elements of C = ReLU(A @ B). */
int oracle_gemm_relu_f16_points(int64_t M, int64_t N, int64_t K,
                                const uint16_t* A, const uint16_t* B,
                                int64_t npts, const int64_t* ii, const int64_t* jj,
                                uint16_t* out, double* pre, double* absdot)
{
    return points_impl(M, N, K, A, 0, B, 0, NULL, npts, ii, jj, out, pre, absdot);
}

/* Rows [row0, row1) of C = GELU(A @ B + bias), bias: N fp16 values (one per column). */
int oracle_gemm_bias_gelu_f16_rows(int64_t M, int64_t N, int64_t K,
                                   const uint16_t* A, const uint16_t* B, const uint16_t* bias,
                                   uint16_t* C, double* pre, double* absdot,
                                   int64_t row0, int64_t row1)
{
    if (!bias && N > 0) return -1;
    return rows_impl(M, N, K, A, 0, B, 0, bias, C, pre, absdot, row0, row1);
}

/* Selected elements of C = GELU(A @ B + bias). */
int oracle_gemm_bias_gelu_f16_points(int64_t M, int64_t N, int64_t K,
                                     const uint16_t* A, const uint16_t* B, const uint16_t* bias,
                                     int64_t npts, const int64_t* ii, const int64_t* jj,
                                     uint16_t* out, double* pre, double* absdot)
{
    if (!bias && N > 0) return -1;
    return points_impl(M, N, K, A, 0, B, 0, bias, npts, ii, jj, out, pre, absdot);
}

/*
 * Rows [row0, row1) of C = epilogue(op(A) @ op(B)) with op_a, op_b in {0, 1}
 * (0: as stored, 1: transposed, see above); bias NULL gives the ReLU epilogue,
 * otherwise bias + GELU.
 */
int oracle_gemm_f16_rows_t(int64_t M, int64_t N, int64_t K, const uint16_t* A, int op_a,
                           const uint16_t* B, int op_b, const uint16_t* bias, uint16_t* C,
                           double* pre, double* absdot, int64_t row0, int64_t row1)
{
    if ((op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1)) return -1;
    return rows_impl(M, N, K, A, op_a, B, op_b, bias, C, pre, absdot, row0, row1);
}

/* Selected elements of C = epilogue(op(A) @ op(B)). */
int oracle_gemm_f16_points_t(int64_t M, int64_t N, int64_t K, const uint16_t* A, int op_a,
                             const uint16_t* B, int op_b, const uint16_t* bias, int64_t npts,
                             const int64_t* ii, const int64_t* jj, uint16_t* out, double* pre,
                             double* absdot)
{
    if ((op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1)) return -1;
    return points_impl(M, N, K, A, op_a, B, op_b, bias, npts, ii, jj, out, pre, absdot);
}
