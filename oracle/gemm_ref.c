/*
 * Oracle for the fused GEMM  C = act(A . B + bias)  -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this file's library.  It shares no code, header or constant with the HIP
 * path and is compiled separately with gcc.
 *
 * What it computes (page "Tile Selection: Cost Models Against Measurement",
 * opening section and "The structure of the search space": a matrix multiply
 * C = AB with C of shape M x N and reduction depth K, fused with a bias and an
 * activation; page "Tiling the hierarchy", fusion section: the activation is
 * applied on the GEMM output, the "nearly free" epilogue):
 *
 *     C[i][j] = act( sum_{k<K} A[i][k] * B[k][j] + bias[j] )
 *
 * with A [M x K] and B [K x N] row-major, bias [N] (or absent = 0).  Every
 * product and the running sum are in IEEE double; inputs stored as float32 or
 * bf16 widen to double exactly.  The loop order is the plain i-k-j nest.
 *
 * act: 0 = identity, 1 = ReLU max(0, x), 2 = GELU in its erf form
 * 0.5 x (1 + erf(x / sqrt 2)) (the pages only say "gelu"; the erf form is the
 * reading taken).
 *
 * Parity pins: closed forms (identity, one-hot and rank-1 operands), exactly
 * rounded brute force on tiny shapes and integer-exact inputs, in tests/.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* widen one stored element to double: in_bf16 = 0 -> float32, 1 -> bf16 bits */
static double widen(const void *base, int64_t idx, int in_bf16)
{
    if (in_bf16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[idx];
}

static double activation(double x, int act)
{
    if (act == 1)
        return x > 0.0 ? x : 0.0;
    if (act == 2)
        return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
    return x;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Full product into C (double, M x N).  Returns 0, or -1 on a bad argument.
 * Rows are distributed over OpenMP threads; each row is summed in the same
 * k order whatever the thread count.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                int in_bf16, const float *bias, int act, double *C)
{
    if (M < 0 || N < 0 || K < 0 || (act < 0 || act > 2))
        return -1;
    if ((M > 0 && K > 0 && !A) || (K > 0 && N > 0 && !B) || (M > 0 && N > 0 && !C))
        return -1;

    /* widen B once: a plain copy in double */
    double *Bd = NULL;
    if (K > 0 && N > 0) {
        Bd = (double *)malloc((size_t)K * (size_t)N * sizeof(double));
        if (!Bd)
            return -1;
        for (int64_t t = 0; t < K * N; ++t)
            Bd[t] = widen(B, t, in_bf16);
    }

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < M; ++i) {
        double *row = C + i * N;
        for (int64_t j = 0; j < N; ++j)
            row[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = widen(A, i * K + k, in_bf16);
            const double *brow = Bd + k * N;
            for (int64_t j = 0; j < N; ++j)
                row[j] += a * brow[j];
        }
        for (int64_t j = 0; j < N; ++j)
            row[j] = activation(row[j] + (bias ? (double)bias[j] : 0.0), act);
    }
    free(Bd);
    return 0;
}

/*
 * Selected entries only: out[t] = C[rows[t]][cols[t]], each summed over k in
 * increasing order (the same per-entry order as oracle_gemm).
 */
int oracle_gemm_entries(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                        int in_bf16, const float *bias, int act, int64_t n,
                        const int64_t *rows, const int64_t *cols, double *out)
{
    if (M < 0 || N < 0 || K < 0 || n < 0 || (act < 0 || act > 2))
        return -1;
    for (int64_t t = 0; t < n; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
            return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < n; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += widen(A, i * K + k, in_bf16) * widen(B, k * N + j, in_bf16);
        out[t] = activation(s + (bias ? (double)bias[j] : 0.0), act);
    }
    return 0;
}
