/*
 * CPU oracle for the fused-epilogue GEMM  D = act(alpha * op(A) * op(B) + beta * C + bias).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or call this file;
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares
 * no code, header, table or constant with the HIP library.
 *
 * Sources (pages as data; cited by page title and section):
 *  - "CUTLASS: Fast Linear Algebra in CUDA C++", section "Efficient Matrix Multiplication on
 *    GPUs": the GEMM definition C = alpha*A*B + beta*C and three loop nests that compute it
 *    (the naive i-j-k nest, the nest with k outermost, and the nest tiled over M and N with k
 *    inside the tile loops).  All three add the K products of one output element in ascending
 *    k order, so in IEEE arithmetic without contraction they give the same bits.
 *  - same page, section "Fusing Element-wise Operations: An Example with SGEMM": the epilogue
 *    scales the product by alpha, adds a bias term and beta times the C element, then clamps
 *    with max(threshold, .); the threshold is 0 here.
 *  - "Flexible Performant GEMM Kernels on GPUs", section 5.3 (fusion): the bias is a vector
 *    added to every row of the product, i.e. bias[j] for output column j.
 *  - "Flexible Performant GEMM Kernels on GPUs", section 2.3 (Tensor Cores): fp16 inputs with
 *    fp32 accumulation; here the oracle accumulates exactly in fp64 (int64 for int8), which is
 *    the unrounded value every correct kernel approximates.
 *
 * Storage reading (the pages call the layouts N and T without fixing the storage order): every
 * matrix is row-major; op = N uses the array as stored, op = T means the stored array is the
 * transpose.  opA(A)[i][k] = A[i*lda + k] (N) or A[k*lda + i] (T); opB(B)[k][j] = B[k*ldb + j]
 * (N) or B[j*ldb + k] (T).
 *
 * Built with -O2 -ffp-contract=off and no fast-math so that every product and sum is one IEEE
 * double operation in the stated order.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes of this oracle (its own numbering) */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_I8 = 3, OR_I32 = 4, OR_F64 = 5 };

/* ---- exact decoders -------------------------------------------------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * normal: (-1)^s * 2^(e-15) * (1 + f/1024); subnormal (e=0): (-1)^s * 2^-14 * f/1024;
 * e=31: infinity (f=0) or NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                /* 2^-14 * f / 2^10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);    /* 2^(e-15) * (1024+f) / 2^10 */
    return s ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32: widen by appending 16 zero bits. */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double oracle_elem_f64(int dt, const void *p, int64_t idx)
{
    switch (dt) {
    case OR_F32: return (double)((const float *)p)[idx];
    case OR_F16: return oracle_f16_to_f64(((const uint16_t *)p)[idx]);
    case OR_BF16: return oracle_bf16_to_f64(((const uint16_t *)p)[idx]);
    case OR_I8: return (double)((const int8_t *)p)[idx];
    case OR_I32: return (double)((const int32_t *)p)[idx];
    case OR_F64: return ((const double *)p)[idx];
    }
    return NAN;
}

int64_t oracle_elem_i64(int dt, const void *p, int64_t idx)
{
    switch (dt) {
    case OR_I8: return ((const int8_t *)p)[idx];
    case OR_I32: return ((const int32_t *)p)[idx];
    }
    return 0;
}

int oracle_decode_f64(int dt, const void *src, int64_t n, double *dst)
{
    if (dt < OR_F32 || dt > OR_F64) return -1;
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_elem_f64(dt, src, i);
    return 0;
}

int oracle_decode_i64(int dt, const void *src, int64_t n, int64_t *dst)
{
    if (dt != OR_I8 && dt != OR_I32) return -1;
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_elem_i64(dt, src, i);
    return 0;
}

/* ---- rounding of the exact result to the output type (round to nearest, ties to even) ---- */

/* Round a double to the nearest binary16 value, ties to even, overflow to +-inf.
 * Works on the real value: in the binade [2^ue, 2^(ue+1)) binary16 values are spaced by
 * q = 2^(ue-10) (the subnormal range shares the spacing 2^-24 of the lowest binade), so the
 * nearest one is q * rint(|x| / q); rint rounds to nearest, ties to even (the C default mode),
 * and the division by a power of two is exact.  The result is re-encoded from that integer. */
uint16_t oracle_f64_to_f16(double x)
{
    if (isnan(x)) return 0x7e00;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return s;
    if (a >= 65520.0) return s | 0x7c00;  /* 65504 + half its spacing of 32, tie goes to even = inf */
    int e;
    frexp(a, &e);                         /* a = m * 2^e with m in [0.5, 1) */
    int ue = e - 1;
    if (ue < -14) ue = -14;
    double m = rint(a / ldexp(1.0, ue - 10)); /* integer in [0, 2048] */
    if (m == 2048.0) { ue += 1; m = 1024.0; }
    if (m < 1024.0) return s | (uint16_t)m;   /* subnormal: only when ue == -14 */
    return s | (uint16_t)((ue + 15) << 10) | (uint16_t)(m - 1024.0);
}

/* Round a double to the nearest bfloat16 value (8 exponent bits, bias 127, 7 fraction bits),
 * ties to even, by the same construction with spacing 2^(ue-7). */
uint16_t oracle_f64_to_bf16(double x)
{
    if (isnan(x)) return 0x7fc0;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return s;
    if (isinf(a)) return s | 0x7f80;
    int e;
    frexp(a, &e);
    int ue = e - 1;
    if (ue < -126) ue = -126;
    double m = rint(a / ldexp(1.0, ue - 7)); /* integer in [0, 256] */
    if (m == 256.0) { ue += 1; m = 128.0; }
    if (ue > 127) return s | 0x7f80;
    if (m < 128.0) return s | (uint16_t)m;
    return s | (uint16_t)((ue + 127) << 7) | (uint16_t)(m - 128.0);
}

float oracle_f64_to_f32(double x) { return (float)x; /* IEEE conversion, RNE */ }

int oracle_round_to(int dt, const double *src, int64_t n, void *dst)
{
    for (int64_t i = 0; i < n; ++i) {
        switch (dt) {
        case OR_F32: ((float *)dst)[i] = oracle_f64_to_f32(src[i]); break;
        case OR_F16: ((uint16_t *)dst)[i] = oracle_f64_to_f16(src[i]); break;
        case OR_BF16: ((uint16_t *)dst)[i] = oracle_f64_to_bf16(src[i]); break;
        default: return -1;
        }
    }
    return 0;
}

/* ---- gather: dense op(X) from the stored array ------------------------------------------- */

/* out[r*cols + c] = op(X)[r][c]; op = 0 (N): X[r*ldx + c]; op = 1 (T): X[c*ldx + r]. */
void oracle_gather_f64(int op, int64_t rows, int64_t cols, const double *X, int64_t ldx, double *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = op ? X[c * ldx + r] : X[r * ldx + c];
}

void oracle_gather_i64(int op, int64_t rows, int64_t cols, const int64_t *X, int64_t ldx, int64_t *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = op ? X[c * ldx + r] : X[r * ldx + c];
}

/* ---- the product acc = op(A) * op(B) on dense M x K and K x N operands --------------------
 * order 0: naive nest (i, j, k);  order 1: k outermost (k, i, j);  order 2: tiled nest over
 * Mtile x Ntile output tiles with k inside the tile loops, rows split over threads.
 * Rows [r0, r1) only; acc is M x N dense and only those rows are written. */

#define OR_MTILE 32
#define OR_NTILE 256

static void mm_ijk_f64(int64_t r0, int64_t r1, int64_t N, int64_t K, const double *A, const double *B, double *acc)
{
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += A[i * K + k] * B[k * N + j];
            acc[i * N + j] = s;
        }
}

static void mm_kij_f64(int64_t r0, int64_t r1, int64_t N, int64_t K, const double *A, const double *B, double *acc)
{
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < N; ++j) acc[i * N + j] = 0.0;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t i = r0; i < r1; ++i) {
            double a = A[i * K + k];
            for (int64_t j = 0; j < N; ++j) acc[i * N + j] += a * B[k * N + j];
        }
}

static void mm_tiled_f64(int64_t r0, int64_t r1, int64_t N, int64_t K, const double *A, const double *B, double *acc)
{
    for (int64_t m = r0; m < r1; m += OR_MTILE)
        for (int64_t n = 0; n < N; n += OR_NTILE) {
            int64_t me = m + OR_MTILE < r1 ? m + OR_MTILE : r1;
            int64_t ne = n + OR_NTILE < N ? n + OR_NTILE : N;
            for (int64_t i = m; i < me; ++i)
                for (int64_t j = n; j < ne; ++j) acc[i * N + j] = 0.0;
            for (int64_t k = 0; k < K; ++k)
                for (int64_t i = m; i < me; ++i) {
                    double a = A[i * K + k];
                    for (int64_t j = n; j < ne; ++j) acc[i * N + j] += a * B[k * N + j];
                }
        }
}

static void mm_ijk_i64(int64_t r0, int64_t r1, int64_t N, int64_t K, const int64_t *A, const int64_t *B, int64_t *acc)
{
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < N; ++j) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += A[i * K + k] * B[k * N + j];
            acc[i * N + j] = s;
        }
}

static void mm_kij_i64(int64_t r0, int64_t r1, int64_t N, int64_t K, const int64_t *A, const int64_t *B, int64_t *acc)
{
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < N; ++j) acc[i * N + j] = 0;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t i = r0; i < r1; ++i) {
            int64_t a = A[i * K + k];
            for (int64_t j = 0; j < N; ++j) acc[i * N + j] += a * B[k * N + j];
        }
}

static void mm_tiled_i64(int64_t r0, int64_t r1, int64_t N, int64_t K, const int64_t *A, const int64_t *B, int64_t *acc)
{
    for (int64_t m = r0; m < r1; m += OR_MTILE)
        for (int64_t n = 0; n < N; n += OR_NTILE) {
            int64_t me = m + OR_MTILE < r1 ? m + OR_MTILE : r1;
            int64_t ne = n + OR_NTILE < N ? n + OR_NTILE : N;
            for (int64_t i = m; i < me; ++i)
                for (int64_t j = n; j < ne; ++j) acc[i * N + j] = 0;
            for (int64_t k = 0; k < K; ++k)
                for (int64_t i = m; i < me; ++i) {
                    int64_t a = A[i * K + k];
                    for (int64_t j = n; j < ne; ++j) acc[i * N + j] += a * B[k * N + j];
                }
        }
}

typedef struct {
    int order, is_int;
    int64_t r0, r1, N, K;
    const void *A, *B;
    void *acc;
} mm_job;

static void *mm_worker(void *arg)
{
    mm_job *j = (mm_job *)arg;
    if (j->is_int) {
        const int64_t *A = j->A, *B = j->B;
        int64_t *acc = j->acc;
        if (j->order == 0) mm_ijk_i64(j->r0, j->r1, j->N, j->K, A, B, acc);
        else if (j->order == 1) mm_kij_i64(j->r0, j->r1, j->N, j->K, A, B, acc);
        else mm_tiled_i64(j->r0, j->r1, j->N, j->K, A, B, acc);
    } else {
        const double *A = j->A, *B = j->B;
        double *acc = j->acc;
        if (j->order == 0) mm_ijk_f64(j->r0, j->r1, j->N, j->K, A, B, acc);
        else if (j->order == 1) mm_kij_f64(j->r0, j->r1, j->N, j->K, A, B, acc);
        else mm_tiled_f64(j->r0, j->r1, j->N, j->K, A, B, acc);
    }
    return NULL;
}

/* Rows [r0, r1) are split into nthreads contiguous blocks (multiples of OR_MTILE), one thread
 * each; threads only split the work, every element is still summed by one thread in k order. */
static int mm_run(int order, int is_int, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                  void *acc, int64_t r0, int64_t r1, int nthreads)
{
    if (order < 0 || order > 2 || M < 0 || N < 0 || K < 0 || r0 < 0 || r1 > M || r0 > r1) return -1;
    if (nthreads < 1) nthreads = 1;
    int64_t rows = r1 - r0;
    int64_t per = (rows + nthreads - 1) / nthreads;
    per = (per + OR_MTILE - 1) / OR_MTILE * OR_MTILE;
    if (per == 0) per = OR_MTILE;
    mm_job jobs[256];
    pthread_t th[256];
    int nj = 0;
    for (int64_t s = r0; s < r1 && nj < 256; s += per, ++nj) {
        jobs[nj] = (mm_job){order, is_int, s, s + per < r1 ? s + per : r1, N, K, A, B, acc};
    }
    if (nj == 1) {
        mm_worker(&jobs[0]);
        return 0;
    }
    for (int t = 0; t < nj; ++t)
        if (pthread_create(&th[t], NULL, mm_worker, &jobs[t]) != 0) {
            mm_worker(&jobs[t]);
            th[t] = 0;
        }
    for (int t = 0; t < nj; ++t)
        if (th[t]) pthread_join(th[t], NULL);
    return 0;
}

int oracle_matmul_f64(int order, int64_t M, int64_t N, int64_t K, const double *Aop, const double *Bop,
                      double *acc, int64_t r0, int64_t r1, int nthreads)
{
    return mm_run(order, 0, M, N, K, Aop, Bop, acc, r0, r1, nthreads);
}

int oracle_matmul_i64(int order, int64_t M, int64_t N, int64_t K, const int64_t *Aop, const int64_t *Bop,
                      int64_t *acc, int64_t r0, int64_t r1, int nthreads)
{
    return mm_run(order, 1, M, N, K, Aop, Bop, acc, r0, r1, nthreads);
}

/* ---- the fused epilogue on the exact product ----------------------------------------------
 * out[i][j] = act(alpha*acc[i][j] + beta*C[i][j] + bias[j]); the beta term is present only when
 * beta != 0 (C is not read otherwise), the bias term only when bias != NULL, act = max(., 0)
 * when relu != 0.  acc, C and out are rows x N dense. */
void oracle_epilogue_f64(int64_t rows, int64_t N, const double *acc, double alpha, const double *C,
                         double beta, const double *bias, int relu, double *out)
{
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double t = alpha * acc[i * N + j];
            if (beta != 0.0) t += beta * C[i * N + j];
            if (bias) t += bias[j];
            if (relu && !(t > 0.0)) t = 0.0;
            out[i * N + j] = t;
        }
}

/* Integer epilogue (int8 inputs): alpha must be 1 and beta 0 or 1; the sums are exact. */
int oracle_epilogue_i64(int64_t rows, int64_t N, const int64_t *acc, int64_t alpha, const int64_t *C,
                        int64_t beta, const int64_t *bias, int relu, int64_t *out)
{
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < N; ++j) {
            int64_t t = alpha * acc[i * N + j];
            if (beta != 0) t += beta * C[i * N + j];
            if (bias) t += bias[j];
            if (relu && t < 0) t = 0;
            out[i * N + j] = t;
        }
    return 0;
}

/* ---- single output elements straight from the stored (raw) operands ----------------------
 * For outputs too large to recompute whole: for each point p, ref = act(alpha*sum_k
 * opA(A)[i][k]*opB(B)[k][j] + beta*C[i*ldc+j] + bias[j]) with the same ascending-k order,
 * decoding every element on access.  C and bias are raw too (types cd_dt and bias_dt). */
int oracle_points_f64(int64_t npts, const int64_t *ii, const int64_t *jj, int64_t K, int opa, int opb,
                      int ab_dt, const void *A, int64_t lda, const void *B, int64_t ldb, int cd_dt,
                      const void *C, int64_t ldc, int bias_dt, const void *bias, double alpha,
                      double beta, int relu, double *out)
{
    for (int64_t p = 0; p < npts; ++p) {
        int64_t i = ii[p], j = jj[p];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = oracle_elem_f64(ab_dt, A, opa ? k * lda + i : i * lda + k);
            double b = oracle_elem_f64(ab_dt, B, opb ? j * ldb + k : k * ldb + j);
            s += a * b;
        }
        double t = alpha * s;
        if (beta != 0.0) t += beta * oracle_elem_f64(cd_dt, C, i * ldc + j);
        if (bias) t += oracle_elem_f64(bias_dt, bias, j);
        if (relu && !(t > 0.0)) t = 0.0;
        out[p] = t;
    }
    return 0;
}

int oracle_points_i64(int64_t npts, const int64_t *ii, const int64_t *jj, int64_t K, int opa, int opb,
                      int ab_dt, const void *A, int64_t lda, const void *B, int64_t ldb, int cd_dt,
                      const void *C, int64_t ldc, int bias_dt, const void *bias, int64_t alpha,
                      int64_t beta, int relu, int64_t *out)
{
    for (int64_t p = 0; p < npts; ++p) {
        int64_t i = ii[p], j = jj[p];
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t a = oracle_elem_i64(ab_dt, A, opa ? k * lda + i : i * lda + k);
            int64_t b = oracle_elem_i64(ab_dt, B, opb ? j * ldb + k : k * ldb + j);
            s += a * b;
        }
        int64_t t = alpha * s;
        if (beta != 0) t += beta * oracle_elem_i64(cd_dt, C, i * ldc + j);
        if (bias) t += oracle_elem_i64(bias_dt, bias, j);
        if (relu && t < 0) t = 0;
        out[p] = t;
    }
    return 0;
}
