/* A plain C99 client of libaaren (test program): device memory from the HIP
 * runtime's C API, one aaren_scan call, and the inputs and output written to
 * a file as raw little-endian float32 (q [H][d], k and v [B][H][N][d], then
 * o [B][H][N][d]) for the test to compare with the CPU oracle.
 *
 * usage: c_client OUT_FILE
 * exit status 0 on success; any HIP or libaaren error is printed and ends
 * the program with status 1. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "aaren.h"

enum { B = 2, H = 3, N = 600, D = 64 };

static int hip_ok(hipError_t e, const char *what)
{
    if (e != hipSuccess) {
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return 0;
    }
    return 1;
}

/* uniform values in [-2, 2) from a 64-bit linear congruential sequence */
static float next_value(uint64_t *state)
{
    *state = *state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((double)(*state >> 40) / (double)(1ull << 24) * 4.0 - 2.0);
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUT_FILE\n", argv[0]);
        return 1;
    }
    const size_t nq = (size_t)H * D, nk = (size_t)B * H * N * D;
    float *q = malloc(nq * sizeof(float)), *k = malloc(nk * sizeof(float));
    float *v = malloc(nk * sizeof(float)), *o = malloc(nk * sizeof(float));
    if (!q || !k || !v || !o) {
        fprintf(stderr, "out of host memory\n");
        return 1;
    }
    uint64_t state = 12345;
    for (size_t i = 0; i < nq; ++i)
        q[i] = next_value(&state);
    for (size_t i = 0; i < nk; ++i)
        k[i] = next_value(&state);
    for (size_t i = 0; i < nk; ++i)
        v[i] = next_value(&state);

    void *dq = NULL, *dk = NULL, *dv = NULL, *dout = NULL, *ws = NULL;
    const size_t wsb = aaren_scan_workspace_size(B, H, N, D);
    if (wsb == 0) {
        fprintf(stderr, "workspace query rejected the shape\n");
        return 1;
    }
    if (!hip_ok(hipMalloc(&dq, nq * sizeof(float)), "hipMalloc q") ||
        !hip_ok(hipMalloc(&dk, nk * sizeof(float)), "hipMalloc k") ||
        !hip_ok(hipMalloc(&dv, nk * sizeof(float)), "hipMalloc v") ||
        !hip_ok(hipMalloc(&dout, nk * sizeof(float)), "hipMalloc o") ||
        !hip_ok(hipMalloc(&ws, wsb), "hipMalloc workspace") ||
        !hip_ok(hipMemset(ws, 0, wsb), "hipMemset workspace") ||
        !hip_ok(hipMemcpy(dq, q, nq * sizeof(float), hipMemcpyHostToDevice), "copy q") ||
        !hip_ok(hipMemcpy(dk, k, nk * sizeof(float), hipMemcpyHostToDevice), "copy k") ||
        !hip_ok(hipMemcpy(dv, v, nk * sizeof(float), hipMemcpyHostToDevice), "copy v"))
        return 1;

    const float scale = 0.125f; /* 1 / sqrt(64) */
    const aaren_status st = aaren_scan(dq, dk, dv, dout, B, H, N, D, scale, AAREN_F32,
                                       AAREN_F32, ws, wsb, NULL);
    if (st != AAREN_OK) {
        fprintf(stderr, "aaren_scan: %s (%s)\n", aaren_status_string(st), aaren_last_error());
        return 1;
    }
    if (!hip_ok(hipDeviceSynchronize(), "synchronize") ||
        !hip_ok(hipMemcpy(o, dout, nk * sizeof(float), hipMemcpyDeviceToHost), "copy o"))
        return 1;

    FILE *f = fopen(argv[1], "wb");
    if (!f || fwrite(q, sizeof(float), nq, f) != nq || fwrite(k, sizeof(float), nk, f) != nk ||
        fwrite(v, sizeof(float), nk, f) != nk || fwrite(o, sizeof(float), nk, f) != nk ||
        fclose(f) != 0) {
        fprintf(stderr, "cannot write %s\n", argv[1]);
        return 1;
    }
    hipFree(dq);
    hipFree(dk);
    hipFree(dv);
    hipFree(dout);
    hipFree(ws);
    free(q);
    free(k);
    free(v);
    free(o);
    printf("aaren_scan from C: %d x %d x %d x %d, version %d\n", B, H, N, D, aaren_version());
    return 0;
}
