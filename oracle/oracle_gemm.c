/*
 * Plain CPU reference for the dense matrix product C = A·B.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU path, and nothing on the GPU path
 * may call it.
 *
 * What it computes follows the problem statement of the lesson
 * "Matrix multiplication: reuse the inputs" (triton-cuda-lab, section
 * "The three dimensions have different jobs"): A is [M,K], B is [K,N],
 * C is [M,N], all row-major, and C[row,col] is the sum over the inner index
 * of A[row,inner]·B[inner,col].  The same chapter asks for the three-loop
 * CPU version first; this is that version, in fp64, with the loops ordered
 * row / inner / column so the innermost loop runs along contiguous rows of
 * B and C.  No blocking, no reordering of the sum beyond k = 0, 1, ..., K-1,
 * no BLAS.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * The row loop is split across OpenMP threads; every output element is
 * still summed by one thread in the order k = 0 .. K-1, so the result does
 * not depend on the thread count.
 *
 * The rounding helpers implement IEEE-754 round-to-nearest-even from fp64
 * to binary16 and to bfloat16 (8-bit significand, fp32's exponent range),
 * straight from the definition: scale by a power of two so the target
 * quantum becomes 1, round to the nearest integer with ties to even, scale
 * back, overflow to infinity, NaN stays a quiet NaN.  The pages only say the
 * fp32 accumulator is converted to the output type (lesson "Matrix
 * multiplication", section "Connect to the real implementation"; chapter
 * "Fast matrix multiplication", the Triton kernel's final cast); reading:
 * round-to-nearest-even, the IEEE default.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <time.h>
#include <omp.h>

/* C[i,j] = sum_{k=0}^{K-1} A[i,k]*B[k,j] for the full M x N output. */
void oracle_gemm_f64(const double* A, const double* B, double* C,
                     int64_t M, int64_t N, int64_t K, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* c = C + i * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = A[i * K + k];
            const double* b = B + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
        }
    }
}

/* Same product restricted to rows [row0, row0 + nrows) of C; C points at the
 * first of those rows.  Used to compute a bounded block of a large product. */
void oracle_gemm_rows_f64(const double* A, const double* B, double* C,
                          int64_t row0, int64_t nrows, int64_t N, int64_t K,
                          int nthreads)
{
    oracle_gemm_f64(A + row0 * K, B, C, nrows, N, K, nthreads);
}

/* One dot product per requested (row, col) pair: out[t] = C[rows[t], cols[t]]. */
void oracle_gemm_points_f64(const double* A, const double* B,
                            const int64_t* rows, const int64_t* cols, int64_t npts,
                            int64_t N, int64_t K, double* out, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t t = 0; t < npts; ++t) {
        const double* a = A + rows[t] * K;
        const int64_t col = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += a[k] * B[k * N + col];
        out[t] = s;
    }
}

/* Wall-clock seconds of one full product (compute only), for the baseline. */
double oracle_time_gemm_rows_f64(const double* A, const double* B, double* C,
                                 int64_t row0, int64_t nrows, int64_t N, int64_t K,
                                 int nthreads)
{
    struct timespec t0, t1;
    clock_gettime(CLOCK_MONOTONIC, &t0);
    oracle_gemm_rows_f64(A, B, C, row0, nrows, N, K, nthreads);
    clock_gettime(CLOCK_MONOTONIC, &t1);
    return (double)(t1.tv_sec - t0.tv_sec) + 1e-9 * (double)(t1.tv_nsec - t0.tv_nsec);
}

/* ---------------------------------------------------------------------------
 * Round-to-nearest-even from fp64 to a binary format with a p-bit significand
 * (hidden bit included), minimum normal exponent emin and maximum exponent
 * emax.  Returns the rounded value as a double (±inf on overflow).
 * ------------------------------------------------------------------------- */
static double rne_value(double x, int p, int emin, int emax)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    const double ax = fabs(x);
    int e2;
    (void)frexp(ax, &e2);          /* ax = m * 2^e2, 0.5 <= m < 1 */
    int e = e2 - 1;                /* ax in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;        /* subnormal range: fixed quantum */
    const int q = e - (p - 1);     /* quantum 2^q */
    const double y = ldexp(ax, -q);          /* exact: power-of-two scaling */
    const double r = nearbyint(y);           /* default mode: ties to even */
    double v = ldexp(r, q);
    const double maxfin = ldexp(ldexp(1.0, p) - 1.0, emax - (p - 1));
    if (v > maxfin) v = INFINITY;
    return x < 0 ? -v : v;
}

/* Encode a value already representable in the format as its bit pattern. */
static uint32_t encode_bits(double v, int p, int emin, int ebits, int sign_shift)
{
    const uint32_t sign = signbit(v) ? (1u << sign_shift) : 0u;
    const uint32_t mbits = (uint32_t)(p - 1);
    const uint32_t expmask = (1u << ebits) - 1u;
    if (isnan(v)) return sign | (expmask << mbits) | (1u << (mbits - 1));
    if (isinf(v)) return sign | (expmask << mbits);
    const double av = fabs(v);
    if (av == 0.0) return sign;
    int e2;
    (void)frexp(av, &e2);
    const int e = e2 - 1;
    const int bias = (1 << (ebits - 1)) - 1;
    if (e < emin) {                                   /* subnormal */
        const uint32_t mant = (uint32_t)ldexp(av, -(emin - (p - 1)));
        return sign | mant;
    }
    const uint32_t expfield = (uint32_t)(e + bias);
    const uint32_t mant = (uint32_t)(ldexp(av, -(e - (p - 1))) - ldexp(1.0, p - 1));
    return sign | (expfield << mbits) | mant;
}

/* fp64 -> IEEE binary16 bits, round to nearest even. */
void oracle_round_f16(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint16_t)encode_bits(rne_value(x[i], 11, -14, 15), 11, -14, 5, 15);
}

/* fp64 -> bfloat16 bits (8-bit significand, 8-bit exponent), nearest even. */
void oracle_round_bf16(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint16_t)encode_bits(rne_value(x[i], 8, -126, 127), 8, -126, 8, 15);
}

/* fp64 -> IEEE binary32 bits, round to nearest even. */
void oracle_round_f32(const double* x, uint32_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = encode_bits(rne_value(x[i], 24, -126, 127), 24, -126, 8, 31);
}
