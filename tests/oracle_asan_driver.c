/*
 * Drives every entry point of oracle/oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_oracle_asan.py).  Operand
 * buffers are allocated to exactly the bytes the layout contract says are
 * read: A ends at element (M-1)*lda + K, row-major B at (K-1)*ldb + N,
 * column-major B at (N-1)*ldb + K, C at (M-1)*ldc + N.  Any read or write past
 * them, any use of freed memory, any leak and any signed overflow stops the
 * run with a report.  The checks of values are light (the pins of the test
 * suite check the arithmetic); the point is memory safety on every path:
 * padded pitches, both B layouts, K = 0, empty outputs, the sampled-entry
 * entry points, the int8 K limit, the decoders and the streaming example.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm_float(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                      int64_t ldb, int b_col, double* C, int64_t ldc, int nthreads);
int oracle_gemm_float_entries(int dtype, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                              int b_col, int64_t n_entries, const int64_t* rows, const int64_t* cols, double* out,
                              int nthreads);
int oracle_gemm_int8(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                     int b_col, int32_t* C, int64_t ldc, int nthreads);
int oracle_gemm_int8_entries(int64_t K, const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, int b_col,
                             int64_t n_entries, const int64_t* rows, const int64_t* cols, int32_t* out, int nthreads);
int oracle_decode_array(int dtype, const void* src, int64_t n, double* dst);
int oracle_scale_by_two(int64_t n, const uint32_t* x, uint32_t* y);

static int failures;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static int64_t extent(int64_t rows, int64_t pitch, int64_t used) { return rows > 0 ? (rows - 1) * pitch + used : 0; }

/* Small integer-valued inputs in every element format: 1 in binary16 and
 * bfloat16 patterns, 1.0f in binary32; products and sums stay exact. */
static void fill_ones(int dtype, void* p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == 0) ((uint16_t*)p)[i] = 0x3C00;
        else if (dtype == 1) ((uint16_t*)p)[i] = 0x3F80;
        else ((uint32_t*)p)[i] = 0x3F800000u;
    }
}

static void float_case(int dtype, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int b_col, int64_t ldc)
{
    const int elt = dtype == 3 ? 4 : 2;
    const int64_t na = extent(M, lda, K), nb = b_col ? extent(N, ldb, K) : extent(K, ldb, N);
    void* A = malloc((size_t)(na ? na : 1) * elt);
    void* B = malloc((size_t)(nb ? nb : 1) * elt);
    const int64_t nc = extent(M, ldc, N);
    double* C = (double*)malloc(sizeof(double) * (size_t)(nc ? nc : 1));
    fill_ones(dtype, A, na);
    fill_ones(dtype, B, nb);
    CHECK(oracle_gemm_float(dtype, M, N, K, A, lda, B, ldb, b_col, C, ldc, 4) == 0);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) CHECK(C[i * ldc + j] == (double)K);
    if (M > 0 && N > 0) {
        int64_t rows[3] = {0, M - 1, M / 2}, cols[3] = {N - 1, 0, N / 2};
        double out[3];
        CHECK(oracle_gemm_float_entries(dtype, K, A, lda, B, ldb, b_col, 3, rows, cols, out, 2) == 0);
        for (int e = 0; e < 3; ++e) CHECK(out[e] == (double)K);
    }
    free(A);
    free(B);
    free(C);
}

static void int8_case(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int b_col, int64_t ldc, int8_t v)
{
    const int64_t na = extent(M, lda, K), nb = b_col ? extent(N, ldb, K) : extent(K, ldb, N);
    int8_t* A = (int8_t*)malloc((size_t)(na ? na : 1));
    int8_t* B = (int8_t*)malloc((size_t)(nb ? nb : 1));
    const int64_t nc = extent(M, ldc, N);
    int32_t* C = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nc ? nc : 1));
    memset(A, v, (size_t)na);
    memset(B, v, (size_t)nb);
    CHECK(oracle_gemm_int8(M, N, K, A, lda, B, ldb, b_col, C, ldc, 4) == 0);
    const int64_t want = (int64_t)v * v * K;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) CHECK(C[i * ldc + j] == want);
    if (M > 0 && N > 0) {
        int64_t rows[2] = {M - 1, 0}, cols[2] = {0, N - 1};
        int32_t out[2];
        CHECK(oracle_gemm_int8_entries(K, A, lda, B, ldb, b_col, 2, rows, cols, out, 2) == 0);
        CHECK(out[0] == want && out[1] == want);
    }
    free(A);
    free(B);
    free(C);
}

int main(void)
{
    for (int dtype = 0; dtype <= 3; ++dtype) {
        if (dtype == 2) continue; /* int8 has its own entry points */
        for (int b_col = 0; b_col <= 1; ++b_col) {
            float_case(dtype, 5, 7, 9, 12, b_col ? 11 : 10, b_col, 9);
            float_case(dtype, 1, 1, 1, 1, 1, b_col, 1);
            float_case(dtype, 3, 4, 0, 1, b_col ? 1 : 4, b_col, 4); /* K = 0: C = 0 */
            float_case(dtype, 33, 17, 65, 70, b_col ? 66 : 17, b_col, 20);
        }
        float_case(dtype, 0, 5, 3, 3, 5, 0, 5); /* empty outputs */
        float_case(dtype, 5, 0, 3, 3, 1, 0, 1);
    }
    for (int b_col = 0; b_col <= 1; ++b_col) {
        int8_case(5, 7, 9, 12, b_col ? 11 : 10, b_col, 9, -128);
        int8_case(3, 4, 0, 1, b_col ? 1 : 4, b_col, 4, 1);
        int8_case(1, 1, 131071, 131071, b_col ? 131071 : 1, b_col, 1, -128); /* the exact-int32 limit */
    }
    {
        int8_t a = 1, b = 1;
        int32_t c = 0;
        CHECK(oracle_gemm_int8(1, 1, 131072, &a, 131072, &b, 131072, 1, &c, 1, 1) == -2); /* refused unread */
    }
    /* refused arguments touch nothing */
    CHECK(oracle_gemm_float(0, -1, 1, 1, NULL, 1, NULL, 1, 0, NULL, 1, 1) == -1);
    CHECK(oracle_gemm_float(0, 2, 2, 3, NULL, 2, NULL, 2, 0, NULL, 2, 1) == -1); /* lda < K */
    CHECK(oracle_gemm_float(2, 1, 1, 1, NULL, 1, NULL, 1, 0, NULL, 1, 1) == -1); /* int8 code here */
    CHECK(oracle_gemm_int8(2, 2, 2, NULL, 2, NULL, 1, 0, NULL, 2, 1) == -1);     /* ldb < N */
    {
        const uint16_t h[4] = {0x3C00, 0x0001, 0x7C00, 0xFC00};
        double d[4];
        CHECK(oracle_decode_array(0, h, 4, d) == 0 && d[0] == 1.0 && d[1] > 0 && d[2] > 1e300 && d[3] < -1e300);
        CHECK(oracle_decode_array(2, h, 4, d) == -1);
    }
    {
        uint32_t x[13], y[13];
        for (int i = 0; i < 13; ++i) x[i] = 0x3F800000u + (uint32_t)i;
        CHECK(oracle_scale_by_two(13, x, y) == 0 && y[0] == 0x40000000u);
        CHECK(oracle_scale_by_two(0, NULL, NULL) == 0);
        CHECK(oracle_scale_by_two(-1, x, y) == -1);
    }
    if (failures) return 1;
    printf("oracle ok under the sanitizers\n");
    return 0;
}
