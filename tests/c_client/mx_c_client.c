/*
 * A plain C99 client of libmx: the small MXFP8 case end to end through the
 * C ABI of include/mx.h, with device memory and a stream from the HIP
 * runtime and no other runtime in between.
 *
 *   mx_c_client DIR M K N
 *
 * reads DIR/a.bin (bf16 A [M x K], row-major) and DIR/b.bin (bf16 B [K x N],
 * stored as written), quantizes A in row mode and B in transposed mode to
 * E4M3 (mx_quantize, mx_quantize_transpose), multiplies the two MX operands
 * (mx_gemm, fp32 C [M x N]) on one stream, and writes
 * DIR/{qa_codes,qa_scales,qb_codes,qb_scales,c}.bin.  Before any launch it
 * also checks that a bad argument comes back as MX_ERR_INVALID_ARG.  Exit
 * status 0 on success; otherwise the failing call is printed.
 *
 * Test infrastructure: tests/test_gpu_c_client.py writes the inputs and
 * checks the outputs against the oracle.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mx.h"

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)

#define MX_OK_(call)                                                                  \
    do {                                                                              \
        mx_status_t s_ = (call);                                                      \
        if (s_ != MX_OK) {                                                            \
            fprintf(stderr, "%s failed: %s\n", #call, mx_status_string(s_));          \
            exit(3);                                                                  \
        }                                                                             \
    } while (0)

static void *read_file(const char *dir, const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) { perror(path); exit(4); }
    void *p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read: %s\n", path); exit(4); }
    fclose(f);
    return p;
}

static void write_file(const char *dir, const char *name, const void *p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { perror(path); exit(4); }
    fclose(f);
}

/* device buffer of `bytes`, filled from host memory `src` when given */
static void *dev(size_t bytes, const void *src) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    if (src) HIP_OK(hipMemcpy(d, src, bytes, hipMemcpyHostToDevice));
    return d;
}

static void fetch(const char *dir, const char *name, const void *d, size_t bytes) {
    void *h = malloc(bytes);
    if (!h) exit(5);
    HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    write_file(dir, name, h, bytes);
    free(h);
}

int main(int argc, char **argv) {
    if (argc != 5) {
        fprintf(stderr, "usage: %s DIR M K N\n", argv[0]);
        return 1;
    }
    const char *dir = argv[1];
    const int64_t M = atoll(argv[2]), K = atoll(argv[3]), N = atoll(argv[4]);
    if (M <= 0 || K <= 0 || N <= 0 || K % 32 != 0) {
        fprintf(stderr, "bad sizes\n");
        return 1;
    }
    printf("libmx version %d\n", mx_version());

    /* argument errors are reported before anything touches the GPU */
    if (mx_gemm(NULL, NULL, MX_E4M3, NULL, NULL, MX_E4M3, 64, 64, 48, NULL, MX_OUT_F32, 64, NULL) !=
        MX_ERR_INVALID_ARG) {
        fprintf(stderr, "mx_gemm with K %% 32 != 0 was not rejected\n");
        return 6;
    }

    const size_t a_bytes = (size_t)(M * K * 2), b_bytes = (size_t)(K * N * 2);
    void *ha = read_file(dir, "a.bin", a_bytes), *hb = read_file(dir, "b.bin", b_bytes);
    void *da = dev(a_bytes, ha), *db = dev(b_bytes, hb);
    /* A [M x K] row mode; B [K x N] transposed mode -> the MX form of B^T, [N x K] */
    void *qa_c = dev((size_t)(M * K), NULL), *qa_s = dev((size_t)(M * K / 32), NULL);
    void *qb_c = dev((size_t)(N * K), NULL), *qb_s = dev((size_t)(N * K / 32), NULL);
    void *dc = dev((size_t)(M * N * 4), NULL);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    MX_OK_(mx_quantize(da, M, K, K, MX_E4M3, qa_c, qa_s, stream));
    MX_OK_(mx_quantize_transpose(db, K, N, N, MX_E4M3, qb_c, qb_s, stream));
    MX_OK_(mx_gemm(qa_c, qa_s, MX_E4M3, qb_c, qb_s, MX_E4M3, M, N, K, dc, MX_OUT_F32, N, stream));
    HIP_OK(hipStreamSynchronize(stream));

    fetch(dir, "qa_codes.bin", qa_c, (size_t)(M * K));
    fetch(dir, "qa_scales.bin", qa_s, (size_t)(M * K / 32));
    fetch(dir, "qb_codes.bin", qb_c, (size_t)(N * K));
    fetch(dir, "qb_scales.bin", qb_s, (size_t)(N * K / 32));
    fetch(dir, "c.bin", dc, (size_t)(M * N * 4));

    HIP_OK(hipStreamDestroy(stream));
    void *bufs[] = {da, db, qa_c, qa_s, qb_c, qb_s, dc};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; i++) HIP_OK(hipFree(bufs[i]));
    free(ha);
    free(hb);
    printf("ok\n");
    return 0;
}
