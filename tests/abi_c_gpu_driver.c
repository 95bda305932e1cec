/* A plain-C (C99) driver of the library on the GPU, with no Python and no
 * framework: device memory from the HIP runtime, every step through the
 * C ABI.
 *
 *   abi_c_gpu_driver IN OUT ROWS COLS
 *
 * IN holds ROWS x COLS bf16 bit patterns (uint16, row-major).  The driver
 * bootstraps the tensor scale (amax-only pass, refresh at step 0), quantizes
 * x row-wise and transposed with round to nearest (amax folded in again),
 * and runs fprop Y = X X^T from the row-wise operand.  OUT receives, in this
 * order: the tensor scale (fp32), the amax (fp32), row codes, row scales,
 * transposed codes, transposed scales (uint8) and Y (fp32, ROWS x ROWS). */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ue5m3fp4.h"

#define CHECK_HIP(x)                                                            \
    do {                                                                        \
        hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "%s: HIP error %d\n", #x, (int)e_);                 \
            return 2;                                                           \
        }                                                                       \
    } while (0)
#define CHECK_LIB(x)                                                            \
    do {                                                                        \
        int s_ = (x);                                                           \
        if (s_ != UE5M3FP4_OK) {                                                \
            fprintf(stderr, "%s: %s\n", #x, ue5m3fp4_status_string(s_));        \
            return 3;                                                           \
        }                                                                       \
    } while (0)

static int write_back(FILE* f, const void* dev, size_t bytes) {
    void* h = malloc(bytes ? bytes : 1);
    if (!h) return 4;
    if (hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
        free(h);
        return 2;
    }
    const size_t n = fwrite(h, 1, bytes, f);
    free(h);
    return n == bytes ? 0 : 5;
}

int main(int argc, char** argv) {
    if (argc != 5) {
        fprintf(stderr, "usage: %s IN OUT ROWS COLS\n", argv[0]);
        return 1;
    }
    const int64_t rows = atoll(argv[3]), cols = atoll(argv[4]);
    if (rows <= 0 || cols <= 0 || rows % 16 || cols % 16) return 1;
    const size_t n = (size_t)(rows * cols);
    uint16_t* hx = (uint16_t*)malloc(n * sizeof(uint16_t));
    FILE* in = fopen(argv[1], "rb");
    if (!hx || !in || fread(hx, sizeof(uint16_t), n, in) != n) return 1;
    fclose(in);

    uint16_t* x;
    uint8_t *rc, *rs, *cc, *cs;
    float *ts, *amax, *y;
    CHECK_HIP(hipMalloc((void**)&x, n * sizeof(uint16_t)));
    CHECK_HIP(hipMalloc((void**)&rc, n / 2));
    CHECK_HIP(hipMalloc((void**)&rs, n / 16));
    CHECK_HIP(hipMalloc((void**)&cc, n / 2));
    CHECK_HIP(hipMalloc((void**)&cs, n / 16));
    CHECK_HIP(hipMalloc((void**)&ts, sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&amax, sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&y, (size_t)(rows * rows) * sizeof(float)));
    const float one = 1.0f, zero = 0.0f;
    CHECK_HIP(hipMemcpy(x, hx, n * sizeof(uint16_t), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(ts, &one, sizeof(float), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(amax, &zero, sizeof(float), hipMemcpyHostToDevice));

    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    /* bootstrap: amax-only pass, then the refresh of step 0 */
    CHECK_LIB(ue5m3fp4_quantize_blockscale(x, rows, cols, cols, NULL, UE5M3FP4_RNE, 0, 0, NULL, NULL, NULL,
                                           NULL, amax, s));
    CHECK_LIB(ue5m3fp4_update_tensor_scale(amax, ts, 0, 1, 7168.0f, s));
    /* both orientations under the refreshed scale, amax folded in again */
    CHECK_LIB(ue5m3fp4_quantize_blockscale(x, rows, cols, cols, ts, UE5M3FP4_RNE, 0, 0, rc, rs, cc, cs, amax,
                                           s));
    /* fprop with W = X: Y[t][o] = sum_i X[t][i] X[o][i] */
    CHECK_LIB(ue5m3fp4_gemm_fprop(rc, rs, ts, rc, rs, ts, rows, cols, rows, y, s));
    CHECK_HIP(hipStreamSynchronize(s));

    FILE* out = fopen(argv[2], "wb");
    if (!out) return 1;
    int st = write_back(out, ts, sizeof(float));
    if (!st) st = write_back(out, amax, sizeof(float));
    if (!st) st = write_back(out, rc, n / 2);
    if (!st) st = write_back(out, rs, n / 16);
    if (!st) st = write_back(out, cc, n / 2);
    if (!st) st = write_back(out, cs, n / 16);
    if (!st) st = write_back(out, y, (size_t)(rows * rows) * sizeof(float));
    fclose(out);

    CHECK_HIP(hipStreamDestroy(s));
    hipFree(x);
    hipFree(rc);
    hipFree(rs);
    hipFree(cc);
    hipFree(cs);
    hipFree(ts);
    hipFree(amax);
    hipFree(y);
    free(hx);
    return st;
}
