/* The C ABI used from plain C (C99): the header compiles without C++, the
 * program links against libue5m3fp4.so, and calls whose arguments fail the
 * host-side checks return their status before any HIP call -- so this runs
 * without a GPU.  Prints one "name status" line per call. */
#include <stdint.h>
#include <stdio.h>

#include "ue5m3fp4.h"

int main(void) {
    uint8_t* none = NULL;
    float* fnone = NULL;
    static float ts_host[4];  /* a host address: never dereferenced, the checks fail first */
    int st;

    st = ue5m3fp4_quantize_blockscale(NULL, 32, 32, 32, ts_host, UE5M3FP4_RNE, 0, 0, none, none, none, none,
                                      fnone, NULL);
    printf("quantize_null_x %d\n", st);
    st = ue5m3fp4_quantize_blockscale(NULL, 32, 40, 40, ts_host, UE5M3FP4_RNE, 0, 0, none, none, none, none,
                                      fnone, NULL);
    printf("quantize_cols_not_16 %d\n", st);
    st = ue5m3fp4_quantize_blockscale(NULL, 32, 32, 32, ts_host, 7, 0, 0, none, none, none, none, fnone, NULL);
    printf("quantize_bad_rounding %d\n", st);
    st = ue5m3fp4_quantize_blockscale(NULL, (int64_t)1 << 31, 32, 32, ts_host, UE5M3FP4_SR, 0, 0, none, none,
                                      none, none, fnone, NULL);
    printf("quantize_rows_too_large %d\n", st);
    st = ue5m3fp4_quantize_blockscale(NULL, 0, 32, 32, ts_host, UE5M3FP4_RNE, 0, 0, none, none, none, none,
                                      fnone, NULL);
    printf("quantize_empty %d\n", st);
    st = ue5m3fp4_quantize_blockscale_2d(NULL, 32, 32, 32, ts_host, UE5M3FP4_RNE, 0, 0, none, none, none, none,
                                         fnone, NULL);
    printf("quantize_2d_no_output %d\n", st);
    st = ue5m3fp4_quantize_current_scaling(NULL, 32, 32, 32, 7168.0f, UE5M3FP4_RNE, 0, 0, none, none, none,
                                           none, fnone, fnone, NULL);
    printf("current_scaling_null %d\n", st);
    st = ue5m3fp4_dequantize(none, none, ts_host, 4, 24, fnone, NULL);
    printf("dequantize_cols_not_16 %d\n", st);
    st = ue5m3fp4_gemm_nt(none, none, ts_host, none, none, ts_host, 16, 16, 24, fnone, NULL);
    printf("gemm_nt_k_not_16 %d\n", st);
    st = ue5m3fp4_gemm_fprop(none, none, ts_host, none, none, ts_host, -1, 16, 16, fnone, NULL);
    printf("gemm_fprop_negative %d\n", st);
    st = ue5m3fp4_gemm_dgrad(none, none, ts_host, none, none, ts_host, 16, 16, 16, fnone, NULL);
    printf("gemm_dgrad_null %d\n", st);
    st = ue5m3fp4_gemm_wgrad(none, none, ts_host, none, none, ts_host, 0, 16, 16, fnone, NULL);
    printf("gemm_wgrad_null_out %d\n", st);
    st = ue5m3fp4_gemm_nt_bf16(none, none, ts_host, none, none, ts_host, 16, 16, 16, NULL, fnone, NULL);
    printf("gemm_bf16_null %d\n", st);
    st = ue5m3fp4_gemm_nt_bf16_quantized(none, none, ts_host, none, none, ts_host, 16, 16, 16, NULL, fnone,
                                         fnone, UE5M3FP4_RNE, 0, 0, none, none, none, none, NULL);
    printf("gemm_quantized_null_ts %d\n", st);
    st = ue5m3fp4_gemm_nt_mxfp4(none, none, ts_host, none, none, ts_host, 16, 16, 48, fnone, NULL);
    printf("gemm_mxfp4_k_not_32 %d\n", st);
    st = ue5m3fp4_update_tensor_scale(fnone, fnone, 0, 1, 7168.0f, NULL);
    printf("update_null %d\n", st);
    st = ue5m3fp4_update_tensor_scale(ts_host, ts_host + 1, 0, 0, 7168.0f, NULL);
    printf("update_period_0 %d\n", st);
    st = ue5m3fp4_update_tensor_scale(ts_host, ts_host + 1, 3, 2, 7168.0f, NULL);
    printf("update_not_this_step %d\n", st);
    st = ue5m3fp4_stream_reference(NULL, 40, none, none, none, none, NULL);
    printf("stream_reference_not_16 %d\n", st);
    printf("status_string %s\n", ue5m3fp4_status_string(UE5M3FP4_ESHAPE));
    return 0;
}
