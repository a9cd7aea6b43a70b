/*
 * fa_c_forward.c: a plain C99 caller of the library's C ABI (include/fa.h), with no Python, PyTorch or
 * C++ involved.  It reads one attention problem from a file, allocates device memory with the HIP
 * runtime, calls fa_fwd on the null stream, and writes O and lse back to a file, so that a test can
 * compare them with the float64 oracle and with the Python binding's result for the same inputs.
 *
 * Input file:  int32 B, H, N, d, causal, dtype; float32 scale; then q, k, v as raw [B,H,N,d] elements
 *              (2 bytes each for FA_F16 / FA_BF16, 4 for FA_F32).
 * Output file: o as raw [B,H,N,d] elements of the same type, then lse as float32 [B,H,N].
 * Exit status: 0 on success; 2 with the library's message when fa_fwd rejects the request; 1 on an
 * I/O or HIP runtime error.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "fa.h"

static int hip_ok(hipError_t e, const char* what) {
    if (e == hipSuccess) return 1;
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s INPUT OUTPUT\n", argv[0]);
        return 1;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) {
        perror(argv[1]);
        return 1;
    }
    int32_t hdr[6];
    float scale = 0.0f;
    if (fread(hdr, sizeof(int32_t), 6, in) != 6 || fread(&scale, sizeof(float), 1, in) != 1) {
        fprintf(stderr, "short header\n");
        fclose(in);
        return 1;
    }
    const int B = hdr[0], H = hdr[1], N = hdr[2], d = hdr[3], causal = hdr[4], dtype = hdr[5];
    const size_t eb = dtype == FA_F32 ? 4 : 2;
    if (B < 0 || H < 0 || N < 0 || d <= 0) {
        fprintf(stderr, "bad sizes\n");
        fclose(in);
        return 1;
    }
    const size_t n = (size_t)B * H * N * d, rows = (size_t)B * H * N;
    void* host[3] = {NULL, NULL, NULL};
    void* dev[3] = {NULL, NULL, NULL};
    void* h_o = malloc(n * eb + 16);
    float* h_lse = (float*)malloc(rows * sizeof(float) + 16);
    void* d_o = NULL;
    float* d_lse = NULL;
    int rc = 1;
    for (int t = 0; t < 3; ++t) {
        host[t] = malloc(n * eb + 16);
        if (!host[t] || fread(host[t], eb, n, in) != n) {
            fprintf(stderr, "short input tensor %d\n", t);
            goto done;
        }
    }
    for (int t = 0; t < 3; ++t) {
        if (!hip_ok(hipMalloc(&dev[t], n * eb + 16), "hipMalloc") ||
            !hip_ok(hipMemcpy(dev[t], host[t], n * eb, hipMemcpyHostToDevice), "hipMemcpy to device"))
            goto done;
    }
    if (!h_o || !h_lse || !hip_ok(hipMalloc(&d_o, n * eb + 16), "hipMalloc") ||
        !hip_ok(hipMalloc((void**)&d_lse, rows * sizeof(float) + 16), "hipMalloc"))
        goto done;
    {
        const int st = fa_fwd(dev[0], dev[1], dev[2], d_o, d_lse, B, H, N, d, causal, scale, dtype, NULL);
        if (st != FA_OK) {
            fprintf(stderr, "fa_fwd: %s: %s\n", fa_status_str(st), fa_last_error());
            rc = 2;
            goto done;
        }
    }
    if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize") ||
        !hip_ok(hipMemcpy(h_o, d_o, n * eb, hipMemcpyDeviceToHost), "hipMemcpy to host") ||
        !hip_ok(hipMemcpy(h_lse, d_lse, rows * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy to host"))
        goto done;
    {
        FILE* out = fopen(argv[2], "wb");
        if (!out) {
            perror(argv[2]);
            goto done;
        }
        const int ok = fwrite(h_o, eb, n, out) == n && fwrite(h_lse, sizeof(float), rows, out) == rows;
        if (fclose(out) != 0 || !ok) {
            fprintf(stderr, "write failed\n");
            goto done;
        }
    }
    rc = 0;
done:
    fclose(in);
    for (int t = 0; t < 3; ++t) {
        free(host[t]);
        if (dev[t]) hipFree(dev[t]);
    }
    if (d_o) hipFree(d_o);
    if (d_lse) hipFree(d_lse);
    free(h_o);
    free(h_lse);
    return rc;
}
