/*
 * A plain C program that uses the library through include/sgemm_f32.h alone (no
 * C++, no Python): it reads A (M x K) and B (K x N) as raw float32 files, runs
 * sgemm_f32() and sgemm_f32_ex() (C = 2*A*B - C with both operands passed
 * transposed) on the GPU, and writes both results as raw float32 files.  It
 * also checks two argument errors.  Built by __graft_entry__.build() and
 * tests/test_c_abi.py; the results are compared with the oracle by the test.
 *
 * usage: consumer M N K a.bin b.bin c0.bin c.bin cex.bin
 */
#include <stdio.h>
#include <stdlib.h>

#include "sgemm_f32.h"

static float *read_all(const char *path, size_t n) {
    float *p = (float *)malloc(n * sizeof(float) + 1);
    FILE *f = fopen(path, "rb");
    if (!p || !f || fread(p, sizeof(float), n, f) != n) {
        fprintf(stderr, "cannot read %zu floats from %s\n", n, path);
        exit(2);
    }
    fclose(f);
    return p;
}

static void write_all(const char *path, const float *p, size_t n) {
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, sizeof(float), n, f) != n) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(2);
    }
    fclose(f);
}

#define CHECK(call)                                                                   \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

int main(int argc, char **argv) {
    if (argc != 9) {
        fprintf(stderr, "usage: %s M N K a.bin b.bin c0.bin c.bin cex.bin\n", argv[0]);
        return 2;
    }
    const int M = atoi(argv[1]), N = atoi(argv[2]), K = atoi(argv[3]);
    const size_t na = (size_t)M * K, nb = (size_t)K * N, nc = (size_t)M * N;
    float *A = read_all(argv[4], na), *B = read_all(argv[5], nb), *C0 = read_all(argv[6], nc);
    float *At = (float *)malloc(na * sizeof(float)), *Bt = (float *)malloc(nb * sizeof(float));
    float *C = (float *)malloc(nc * sizeof(float));
    for (int i = 0; i < M; ++i)
        for (int k = 0; k < K; ++k) At[(size_t)k * M + i] = A[(size_t)i * K + k];
    for (int k = 0; k < K; ++k)
        for (int j = 0; j < N; ++j) Bt[(size_t)j * K + k] = B[(size_t)k * N + j];

    float *dA, *dB, *dAt, *dBt, *dC;
    CHECK(hipMalloc((void **)&dA, na * sizeof(float)));
    CHECK(hipMalloc((void **)&dB, nb * sizeof(float)));
    CHECK(hipMalloc((void **)&dAt, na * sizeof(float)));
    CHECK(hipMalloc((void **)&dBt, nb * sizeof(float)));
    CHECK(hipMalloc((void **)&dC, nc * sizeof(float)));
    CHECK(hipMemcpy(dA, A, na * sizeof(float), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dB, B, nb * sizeof(float), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dAt, At, na * sizeof(float), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dBt, Bt, nb * sizeof(float), hipMemcpyHostToDevice));

    /* argument errors come back as hipErrorInvalidValue before any launch */
    if (sgemm_f32(-1, N, K, dA, K, dB, N, dC, N, 0) != hipErrorInvalidValue ||
        sgemm_f32(M, N, K, dA, K - 1, dB, N, dC, N, 0) != hipErrorInvalidValue) {
        fprintf(stderr, "invalid arguments were not rejected\n");
        return 1;
    }

    CHECK(sgemm_f32(M, N, K, dA, K, dB, N, dC, N, 0));
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(C, dC, nc * sizeof(float), hipMemcpyDeviceToHost));
    write_all(argv[7], C, nc);

    CHECK(hipMemcpy(dC, C0, nc * sizeof(float), hipMemcpyHostToDevice));
    CHECK(sgemm_f32_ex(SGEMM_F32_OP_T, SGEMM_F32_OP_T, M, N, K, 2.0f, dAt, M, dBt, K, -1.0f, dC,
                       N, 0));
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(C, dC, nc * sizeof(float), hipMemcpyDeviceToHost));
    write_all(argv[8], C, nc);

    printf("consumer ok: %d x %d x %d via %s\n", M, N, K,
           sgemm_f32_algo_name(sgemm_f32_select(M, N, K, dA, K, dB, N, dC, N)));
    hipFree(dA); hipFree(dB); hipFree(dAt); hipFree(dBt); hipFree(dC);
    free(A); free(B); free(C0); free(At); free(Bt); free(C);
    return 0;
}
