/*
 * oracle.c -- plain, slow CPU reference for the tiled GEMM  C = A * B.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The HIP library
 * never links it, includes it or calls it, and this file includes nothing
 * from the HIP library.
 *
 * What is computed.  "Hiding Memory Latency in CUDA: Asynchronous Loads and
 * Software Pipelines" (introduction) defines the work of a tiled GEMM as
 * the product of A and B, walked tile by tile along K; "Pipeline GPU Kernel"
 * (Schritt 5) states that pipelining only reorders the loads and leaves the
 * arithmetic unchanged.  The result of every pipelined variant is therefore
 * the plain definition
 *
 *        C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 *
 * over the already-rounded input values.  This file writes exactly that
 * definition out: the inputs are decoded exactly to double (float inputs)
 * or widened to int32 (int8 inputs), and each output is one dot product
 * accumulated in k order, in double (floats) or int32 (int8).  There is no
 * blocking, no reordering of the sum and no fused arithmetic beyond that.
 * OpenMP only splits the independent output rows between threads.
 *
 * Layouts (element (r,c) of a matrix):
 *   A  row-major M x K             A[i*lda + k]
 *   B  row-major K x N  (b_col=0)  B[k*ldb + j]
 *   B  col-major K x N  (b_col=1)  B[j*ldb + k]
 *   C  row-major M x N             C[i*ldc + j]
 * K = 0 gives C = 0 (the empty sum).  M = 0 or N = 0 writes nothing.
 *
 * dtype codes: 0 = binary16, 1 = bfloat16, 3 = binary32 (float inputs,
 * double output); int8 has its own entry points with int32 output.
 *
 * Return codes: 0 ok, -1 invalid argument, -2 int8 K too large for an
 * exact int32 sum (|a*b| <= 2^14, so K <= 131071 keeps every partial sum
 * inside int32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F16 0
#define ORACLE_BF16 1
#define ORACLE_F32 3
#define ORACLE_I8_MAX_K 131071

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Decoded from the format definition, exactly, into double. */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^(1-15-10) */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE 754 binary32 word. */
double oracle_bf16_to_f64(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

double oracle_f32_to_f64(uint32_t bits)
{
    float x;
    memcpy(&x, &bits, sizeof x);
    return (double)x;
}

static double decode(int dtype, const void* base, int64_t idx)
{
    switch (dtype) {
    case ORACLE_F16: return oracle_f16_to_f64(((const uint16_t*)base)[idx]);
    case ORACLE_BF16: return oracle_bf16_to_f64(((const uint16_t*)base)[idx]);
    default: return oracle_f32_to_f64(((const uint32_t*)base)[idx]);
    }
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

static int check_dims(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                      int b_col, int64_t ldc)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0; /* nothing is read or written */
    if (lda < (K > 0 ? K : 1)) return -1;
    if (b_col ? ldb < (K > 0 ? K : 1) : ldb < (N > 0 ? N : 1)) return -1;
    if (ldc < (N > 0 ? N : 1)) return -1;
    return 0;
}

/* Full product, float inputs, double output. */
int oracle_gemm_float(int dtype, int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda, const void* B, int64_t ldb,
                      int b_col, double* C, int64_t ldc, int nthreads)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_F32) return -1;
    if (check_dims(M, N, K, lda, ldb, b_col, ldc)) return -1;
    if (M == 0 || N == 0) return 0;

    /* Decode once: a[i][k] row-major, bt[j][k] so every dot product reads
     * two contiguous rows.  This is a change of layout only. */
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * (K ? K : 1)));
    double* bt = (double*)malloc(sizeof(double) * (size_t)(N * (K ? K : 1)));
    if (!a || !bt) { free(a); free(bt); return -1; }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) a[i * K + k] = decode(dtype, A, i * lda + k);
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            bt[j * K + k] = decode(dtype, B, b_col ? j * ldb + k : k * ldb + j);

    const int nt = set_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double* ai = a + i * K;
        for (int64_t j = 0; j < N; ++j) {
            const double* bj = bt + j * K;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += ai[k] * bj[k];
            C[i * ldc + j] = s;
        }
    }
    free(a);
    free(bt);
    return 0;
}

/* Selected outputs only: out[e] = C[rows[e]][cols[e]], each computed from
 * the raw inputs as one k-ordered double dot product. */
int oracle_gemm_float_entries(int dtype, int64_t K, const void* A, int64_t lda,
                              const void* B, int64_t ldb, int b_col, int64_t n_entries,
                              const int64_t* rows, const int64_t* cols, double* out,
                              int nthreads)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_F32) return -1;
    if (K < 0 || n_entries < 0) return -1;
    const int nt = set_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t e = 0; e < n_entries; ++e) {
        const int64_t i = rows[e], j = cols[e];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += decode(dtype, A, i * lda + k) *
                 decode(dtype, B, b_col ? j * ldb + k : k * ldb + j);
        out[e] = s;
    }
    return 0;
}

/* Full product, int8 inputs, int32 accumulation and output. */
int oracle_gemm_int8(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                     const int8_t* B, int64_t ldb, int b_col, int32_t* C, int64_t ldc,
                     int nthreads)
{
    if (check_dims(M, N, K, lda, ldb, b_col, ldc)) return -1;
    if (K > ORACLE_I8_MAX_K) return -2;
    if (M == 0 || N == 0) return 0;

    int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * (K ? K : 1)));
    int32_t* bt = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N * (K ? K : 1)));
    if (!a || !bt) { free(a); free(bt); return -1; }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) a[i * K + k] = A[i * lda + k];
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k) bt[j * K + k] = b_col ? B[j * ldb + k] : B[k * ldb + j];

    const int nt = set_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const int32_t* ai = a + i * K;
        for (int64_t j = 0; j < N; ++j) {
            const int32_t* bj = bt + j * K;
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += ai[k] * bj[k];
            C[i * ldc + j] = s;
        }
    }
    free(a);
    free(bt);
    return 0;
}

int oracle_gemm_int8_entries(int64_t K, const int8_t* A, int64_t lda, const int8_t* B,
                             int64_t ldb, int b_col, int64_t n_entries, const int64_t* rows,
                             const int64_t* cols, int32_t* out, int nthreads)
{
    if (K < 0 || n_entries < 0) return -1;
    if (K > ORACLE_I8_MAX_K) return -2;
    const int nt = set_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t e = 0; e < n_entries; ++e) {
        const int64_t i = rows[e], j = cols[e];
        int32_t s = 0;
        for (int64_t k = 0; k < K; ++k)
            s += (int32_t)A[i * lda + k] * (int32_t)(b_col ? B[j * ldb + k] : B[k * ldb + j]);
        out[e] = s;
    }
    return 0;
}

/* Exact decode of n stored values (dtype as above) into double. */
int oracle_decode_array(int dtype, const void* src, int64_t n, double* dst)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_F32) return -1;
    for (int64_t e = 0; e < n; ++e) dst[e] = decode(dtype, src, e);
    return 0;
}

int oracle_max_threads(void)
{
    return set_threads(0);
}

/*
 * The streaming pipeline of "Hiding Memory Latency in CUDA: Asynchronous
 * Loads and Software Pipelines" (section 8, the minimal example): every
 * element of a float vector is scaled by two,
 *
 *        y[i] = 2 * x[i]      (0 <= i < n),
 *
 * in float, as the page computes it.  Here each value is decoded exactly to
 * double, doubled there and rounded once back to float; doubling is exact in
 * both formats (overflow to infinity and NaN included), so this is the plain
 * definition.  x and y are raw binary32 bit patterns.  n = 0 writes nothing.
 */
int oracle_scale_by_two(int64_t n, const uint32_t* x, uint32_t* y)
{
    if (n < 0 || (n > 0 && (!x || !y))) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const double v = 2.0 * oracle_f32_to_f64(x[i]);
        const float f = (float)v;
        memcpy(&y[i], &f, sizeof f);
    }
    return 0;
}

/*
 * The attention-style consumer, the pages' high-ratio example.  "Kernel-
 * Engpass analysieren" counts the work of flash attention as
 * 4 * batch * heads * seq_len^2 * head_dim FLOP (Schritt 1: the two products
 * of every query row with every key row, then every probability with every
 * value row) and uses it as the kernel with many matrix instructions per tile
 * load (Schritt 4 and the pitfalls).  Flash attention computes softmax
 * attention; written out plainly for each of BH independent (batch, head)
 * slices:
 *
 *        S[i][j] = scale * sum_{d<D} Q[i][d] * K[j][d]
 *        m_i     = max_j S[i][j]
 *        P[i][j] = exp(S[i][j] - m_i) / sum_{j'} exp(S[i][j'] - m_i)
 *        O[i][d] = sum_{j<Sk} P[i][j] * V[j][d]
 *
 * No mask (the pages name none).  Subtracting the row maximum leaves P
 * unchanged and keeps exp finite.  Inputs are decoded exactly to double;
 * every sum is taken in index order, in double.
 *
 * Layouts (contiguous): Q [BH][Sq][D], K and V [BH][Sk][D], O [BH][Sq][D]
 * (double).  dtype 0 = binary16, 1 = bfloat16.  Sk = 0 is refused (a
 * softmax over no keys is undefined); BH = 0 or Sq = 0 writes nothing.
 * Return codes: 0 ok, -1 invalid argument or no memory.
 */
static int attention_row(int dtype, int64_t Sk, int64_t D, const void* Q, int64_t q_off, const void* K,
                         const void* V, int64_t kv_off, double scale, double* s, double* o)
{
    for (int64_t j = 0; j < Sk; ++j) {
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += decode(dtype, Q, q_off + d) * decode(dtype, K, kv_off + j * D + d);
        s[j] = scale * acc;
    }
    double m = s[0];
    for (int64_t j = 1; j < Sk; ++j)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    for (int64_t j = 0; j < Sk; ++j) s[j] = s[j] / z; /* P[i][j] */
    for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < Sk; ++j) acc += s[j] * decode(dtype, V, kv_off + j * D + d);
        o[d] = acc;
    }
    return 0;
}

int oracle_attention(int dtype, int64_t BH, int64_t Sq, int64_t Sk, int64_t D, const void* Q,
                     const void* K, const void* V, double scale, double* O, int nthreads)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (BH < 0 || Sq < 0 || Sk <= 0 || D <= 0) return -1;
    if (BH == 0 || Sq == 0) return 0;
    int bad = 0;
    const int nt = set_threads(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)Sk);
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static) collapse(2)
        for (int64_t b = 0; b < BH; ++b)
            for (int64_t i = 0; i < Sq; ++i)
                if (s) attention_row(dtype, Sk, D, Q, (b * Sq + i) * D, K, V, b * Sk * D, scale, s,
                                     O + (b * Sq + i) * D);
        free(s);
    }
    return bad ? -1 : 0;
}

/* Selected query rows only: out[e][0..D) = O[slices[e]][rows[e]][0..D). */
int oracle_attention_rows(int dtype, int64_t BH, int64_t Sq, int64_t Sk, int64_t D, const void* Q,
                          const void* K, const void* V, double scale, int64_t n_rows, const int64_t* slices,
                          const int64_t* rows, double* out, int nthreads)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (BH < 0 || Sq < 0 || Sk <= 0 || D <= 0 || n_rows < 0) return -1;
    for (int64_t e = 0; e < n_rows; ++e)
        if (slices[e] < 0 || slices[e] >= BH || rows[e] < 0 || rows[e] >= Sq) return -1;
    int bad = 0;
    const int nt = set_threads(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)Sk);
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (int64_t e = 0; e < n_rows; ++e)
            if (s) attention_row(dtype, Sk, D, Q, (slices[e] * Sq + rows[e]) * D, K, V, slices[e] * Sk * D, scale,
                                 s, out + e * D);
        free(s);
    }
    return bad ? -1 : 0;
}
