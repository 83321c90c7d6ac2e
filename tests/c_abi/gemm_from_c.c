/*
 * A C program (no C++, no Python) driving the library through include/tilegemm.h:
 * it tunes one shape, runs C = ReLU(A . B + bias) twice -- with the tuned
 * configuration looked up from the cache and with it passed explicitly -- and
 * writes C (float32, row-major) to a file for the test to compare with the
 * oracle.
 *
 *   gemm_from_c M N K seed out.f32
 *
 * Inputs are small integers from closed-form patterns (exact in bf16, and every
 * partial sum exact in fp32):
 *   A[i][k] = (7i + 3k + (k^2 mod 13) + (ik mod 7) + seed) mod 5 - 2,
 *   B[k][j] = (5k + 11j + (kj mod 7) + (k^2 mod 11) + 2 seed) mod 5 - 2,
 *   bias[j] = j mod 9 - 4.
 * Exit status 0 on success; on failure the library's message is printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tilegemm.h"

static uint16_t bf16_of_small_int(int v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);   /* exact: small integers need no rounding */
}

#define HIP_OK(x)                                                               \
    do {                                                                        \
        hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));             \
            return 1;                                                           \
        }                                                                       \
    } while (0)
#define TG_OK_(x)                                                               \
    do {                                                                        \
        int s_ = (x);                                                           \
        if (s_ != TG_OK) {                                                      \
            fprintf(stderr, "%s: status %d: %s\n", #x, s_, tg_last_error());    \
            return 1;                                                           \
        }                                                                       \
    } while (0)

int main(int argc, char** argv)
{
    if (argc != 6) {
        fprintf(stderr, "usage: %s M N K seed out.f32\n", argv[0]);
        return 2;
    }
    const int64_t M = atoll(argv[1]), N = atoll(argv[2]), K = atoll(argv[3]);
    const int seed = atoi(argv[4]);
    if (M <= 0 || N <= 0 || K <= 0 || M * K > (1 << 26) || K * N > (1 << 26) || M * N > (1 << 26)) {
        fprintf(stderr, "sizes out of this example's range\n");
        return 2;
    }
    uint16_t* hA = malloc((size_t)(M * K) * 2);
    uint16_t* hB = malloc((size_t)(K * N) * 2);
    float* hbias = malloc((size_t)N * 4);
    float* hC = malloc((size_t)(M * N) * 4);
    float* hC2 = malloc((size_t)(M * N) * 4);
    if (!hA || !hB || !hbias || !hC || !hC2)
        return 1;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            hA[i * K + k] = bf16_of_small_int((int)((7 * i + 3 * k + (k * k) % 13 + (i * k) % 7 + seed) % 5) - 2);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            hB[k * N + j] = bf16_of_small_int((int)((5 * k + 11 * j + (k * j) % 7 + (k * k) % 11 + 2 * seed) % 5) - 2);
    for (int64_t j = 0; j < N; ++j)
        hbias[j] = (float)(j % 9 - 4);

    void *dA, *dB, *dC;
    float* dbias;
    HIP_OK(hipMalloc(&dA, (size_t)(M * K) * 2));
    HIP_OK(hipMalloc(&dB, (size_t)(K * N) * 2));
    HIP_OK(hipMalloc((void**)&dbias, (size_t)N * 4));
    HIP_OK(hipMalloc(&dC, (size_t)(M * N) * 4));
    HIP_OK(hipMemcpy(dA, hA, (size_t)(M * K) * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dB, hB, (size_t)(K * N) * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dbias, hbias, (size_t)N * 4, hipMemcpyHostToDevice));

    TG_OK_(tg_set_stream(NULL));
    tg_cfg cfg;
    TG_OK_(gemm_autotune_ep(M, N, K, TG_BF16_F32OUT, TG_ACT_RELU, 1, &cfg));
    printf("tuned cfg: kind %d bm %d bn %d bk %d waves %dx%d stages %d split %d\n", cfg.kind, cfg.bm, cfg.bn, cfg.bk,
           cfg.wgm, cfg.wgn, cfg.stages, cfg.split_k);
    /* without a configuration: the cached choice */
    TG_OK_(gemm_bias_act(M, N, K, dA, dB, dbias, dC, TG_BF16_F32OUT, TG_ACT_RELU, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hC, dC, (size_t)(M * N) * 4, hipMemcpyDeviceToHost));
    /* with the configuration passed explicitly: the same kernel, the same bits */
    HIP_OK(hipMemset(dC, 0, (size_t)(M * N) * 4));
    TG_OK_(gemm_bias_act(M, N, K, dA, dB, dbias, dC, TG_BF16_F32OUT, TG_ACT_RELU, &cfg));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hC2, dC, (size_t)(M * N) * 4, hipMemcpyDeviceToHost));
    if (memcmp(hC, hC2, (size_t)(M * N) * 4) != 0) {
        fprintf(stderr, "cached and explicit configurations gave different results\n");
        return 1;
    }
    /* an infeasible request is refused with a message, and nothing runs */
    tg_cfg bad = cfg;
    bad.bm = 48;
    if (gemm_bias_act(M, N, K, dA, dB, dbias, dC, TG_BF16_F32OUT, TG_ACT_RELU, &bad) == TG_OK) {
        fprintf(stderr, "an infeasible configuration was accepted\n");
        return 1;
    }
    printf("refused as expected: %s\n", tg_last_error());

    FILE* f = fopen(argv[5], "wb");
    if (!f || fwrite(hC, 4, (size_t)(M * N), f) != (size_t)(M * N) || fclose(f) != 0) {
        fprintf(stderr, "cannot write %s\n", argv[5]);
        return 1;
    }
    hipFree(dA);
    hipFree(dB);
    hipFree(dbias);
    hipFree(dC);
    free(hA);
    free(hB);
    free(hbias);
    free(hC);
    free(hC2);
    printf("ok\n");
    return 0;
}
