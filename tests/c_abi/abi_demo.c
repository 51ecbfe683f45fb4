/*
 * abi_demo.c -- calls libmi_sgemm through its C ABI from plain C, with device
 * memory from the HIP runtime and no Python or torch in the process.
 *
 * It runs the compute entry points on small integer-valued operands (so the
 * expected results are exact and are formed here with 64-bit integer sums),
 * checks a few argument errors, and prints "abi demo ok" on success; any
 * mismatch or error prints a line and gives exit status 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mi_sgemm.h"

#define HIP_OK(call)                                                            \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) {                                                 \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                           \
        }                                                                       \
    } while (0)

static int fail(const char *what, int status) {
    printf("%s: %s (status %d)\n", what, mi_status_string(status), status);
    return 1;
}

/* Values in {-3, ..., 3} from a fixed linear congruential sequence. */
static float small_int(uint32_t *s) {
    *s = *s * 1664525u + 1013904223u;
    return (float)((int)((*s >> 16) % 7u) - 3);
}

static int check(const char *what, const float *got, const int64_t *want, int m, int n) {
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < n; ++j)
            if (got[i * n + j] != (float)want[i * n + j]) {
                printf("%s: C[%d][%d] = %g, expected %lld\n", what, i, j, got[i * n + j],
                       (long long)want[i * n + j]);
                return 1;
            }
    return 0;
}

int main(void) {
    const int m = 67, n = 45, k = 129;
    float *hA = malloc(sizeof(float) * m * k), *hB = malloc(sizeof(float) * k * n);
    float *hAt = malloc(sizeof(float) * k * m), *hBt = malloc(sizeof(float) * n * k);
    float *hC = malloc(sizeof(float) * m * n);
    int64_t *want = malloc(sizeof(int64_t) * m * n);
    if (!hA || !hB || !hAt || !hBt || !hC || !want) return 1;
    uint32_t seed = 12345u;
    for (int i = 0; i < m * k; ++i) hA[i] = small_int(&seed);
    for (int i = 0; i < k * n; ++i) hB[i] = small_int(&seed);
    for (int i = 0; i < m; ++i)
        for (int t = 0; t < k; ++t) hAt[t * m + i] = hA[i * k + t];
    for (int t = 0; t < k; ++t)
        for (int j = 0; j < n; ++j) hBt[j * k + t] = hB[t * n + j];
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < n; ++j) {
            int64_t s = 0;
            for (int t = 0; t < k; ++t) s += (int64_t)hA[i * k + t] * (int64_t)hB[t * n + j];
            want[i * n + j] = s;
        }

    float *A, *B, *At, *Bt, *C, *x, *out;
    void *ws;
    HIP_OK(hipMalloc((void **)&A, sizeof(float) * m * k));
    HIP_OK(hipMalloc((void **)&B, sizeof(float) * k * n));
    HIP_OK(hipMalloc((void **)&At, sizeof(float) * k * m));
    HIP_OK(hipMalloc((void **)&Bt, sizeof(float) * n * k));
    HIP_OK(hipMalloc((void **)&C, sizeof(float) * m * n));
    HIP_OK(hipMemcpy(A, hA, sizeof(float) * m * k, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(B, hB, sizeof(float) * k * n, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(At, hAt, sizeof(float) * k * m, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(Bt, hBt, sizeof(float) * n * k, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    int st = mi_sgemm(m, n, k, 1.f, A, k, B, n, 0.f, C, n, stream);
    if (st) return fail("mi_sgemm", st);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(hC, C, sizeof(float) * m * n, hipMemcpyDeviceToHost));
    if (check("mi_sgemm", hC, want, m, n)) return 1;

    HIP_OK(hipMemset(C, 0, sizeof(float) * m * n));
    st = mi_sgemm_ex(MI_SGEMM_OP_T, MI_SGEMM_OP_T, m, n, k, 1.f, At, m, Bt, k, 0.f, C, n, stream);
    if (st) return fail("mi_sgemm_ex(T, T)", st);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(hC, C, sizeof(float) * m * n, hipMemcpyDeviceToHost));
    if (check("mi_sgemm_ex(T, T)", hC, want, m, n)) return 1;

    const size_t wsb = mi_sgemm_splitk_workspace_bytes(m, n, k, 4);
    HIP_OK(hipMalloc(&ws, wsb));
    HIP_OK(hipMemset(C, 0, sizeof(float) * m * n));
    st = mi_sgemm_splitk(m, n, k, 1.f, A, k, B, n, 0.f, C, n, 4, ws, wsb, stream);
    if (st) return fail("mi_sgemm_splitk", st);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(hC, C, sizeof(float) * m * n, hipMemcpyDeviceToHost));
    if (check("mi_sgemm_splitk", hC, want, m, n)) return 1;

    /* the allocation-free split-K entry: no workspace argument, the same
       result; a second call reuses the library's static scratch */
    for (int rep = 0; rep < 2; ++rep) {
        HIP_OK(hipMemset(C, 0, sizeof(float) * m * n));
        st = mi_sgemm_splitk_noalloc(MI_SGEMM_OP_N, MI_SGEMM_OP_N, m, n, k, 1.f, A, k, B, n,
                                     0.f, C, n, 3 + rep, stream);
        if (st) return fail("mi_sgemm_splitk_noalloc", st);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(hC, C, sizeof(float) * m * n, hipMemcpyDeviceToHost));
        if (check("mi_sgemm_splitk_noalloc", hC, want, m, n)) return 1;
    }
    if (mi_sgemm_splitk_noalloc(MI_SGEMM_OP_N, MI_SGEMM_OP_N, 2048, 2048, 4096, 1.f, A, 4096, B,
                                2048, 0.f, C, 2048, 8, stream) != MI_SGEMM_ERROR_SCRATCH_LIMIT)
        return fail("plan beyond the static scratch not rejected", -1);

    /* argument errors are reported before anything is enqueued */
    if (mi_sgemm(m, n, k, 1.f, A, k - 1, B, n, 0.f, C, n, stream) != MI_SGEMM_ERROR_INVALID_LD)
        return fail("short lda not rejected", -1);
    if (mi_sgemm_splitk(m, n, k, 1.f, A, k, B, n, 0.f, C, n, 4, ws, wsb - 1, stream) !=
        MI_SGEMM_ERROR_WORKSPACE)
        return fail("short workspace not rejected", -1);

    /* array sum of the integer-valued A: exact */
    const long long nx = (long long)m * k;
    const size_t rwb = mi_reduce_sum_workspace_bytes(nx);
    void *rws;
    HIP_OK(hipMalloc(&rws, rwb));
    HIP_OK(hipMalloc((void **)&out, sizeof(float)));
    x = A;
    st = mi_reduce_sum(nx, x, out, rws, rwb, stream);
    if (st) return fail("mi_reduce_sum", st);
    HIP_OK(hipStreamSynchronize(stream));
    float got;
    HIP_OK(hipMemcpy(&got, out, sizeof(float), hipMemcpyDeviceToHost));
    int64_t s = 0;
    for (long long i = 0; i < nx; ++i) s += (int64_t)hA[i];
    if (got != (float)s) {
        printf("mi_reduce_sum: %g, expected %lld\n", got, (long long)s);
        return 1;
    }

    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(A)); HIP_OK(hipFree(B)); HIP_OK(hipFree(At)); HIP_OK(hipFree(Bt));
    HIP_OK(hipFree(C)); HIP_OK(hipFree(ws)); HIP_OK(hipFree(rws)); HIP_OK(hipFree(out));
    free(hA); free(hB); free(hAt); free(hBt); free(hC); free(want);
    printf("abi demo ok\n");
    return 0;
}
