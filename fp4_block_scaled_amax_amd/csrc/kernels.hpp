// Internal launch interface between the C ABI (api.hip) and the kernels.
// Callers have validated every argument; launchers only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ue5m3fp4 {

struct QuantizeArgs {
    const uint16_t* x;
    int64_t rows, cols, ld;
    const float* tensor_scale;
    bool stochastic;
    uint64_t seed;
    uint32_t offset;
    uint8_t* row_codes;
    uint8_t* row_scales;
    uint8_t* col_codes;
    uint8_t* col_scales;
    float* amax_inout;
    // current-tensor scaling (1-D quantizer only): tensor_scale becomes
    // fp32(*current_amax / fp32(6 max_safe)) when that amax is finite and > 0
    // (stored back to *tensor_scale); null for the periodic tensor scale
    const float* current_amax;
    float max_safe;
};

void launch_quantize_blockscale(const QuantizeArgs& a, hipStream_t stream);

// 16 x 16 tile scales (rows and cols multiples of 16, at least one output).
void launch_quantize_2d(const QuantizeArgs& a, hipStream_t stream);

void launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                       int64_t rows, int64_t cols, float* out, hipStream_t stream);

void launch_update_tensor_scale(float* amax_running, float* tensor_scale, float max_safe,
                                hipStream_t stream);

// Streaming reference of a quantize call's traffic (elems % 16 == 0; codes1
// and scales1 both null for one output).
void launch_stream_reference(const uint16_t* x, int64_t elems, uint8_t* codes0, uint8_t* scales0,
                             uint8_t* codes1, uint8_t* scales1, hipStream_t stream);

// *p = 0 (the running amax before a current-tensor-scaling amax pass).
void launch_zero_scalar(float* p, hipStream_t stream);

// Block-16 quantization of the GEMM's bf16 output in its epilogue, for the
// next linear: the stand-alone quantizer's outputs for the M x N output
// (row-wise along N, transposed along M), tensor scale *ts, nullable pairs.
struct OutputQuant {
    const float* ts;
    uint8_t* row_codes;
    uint8_t* row_scales;
    uint8_t* col_codes;
    uint8_t* col_scales;
    uint64_t seed;
    uint32_t offset;
    bool stochastic;
};

struct GemmArgs {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const float* a_ts;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const float* b_ts;
    int64_t M, N, K;
    float* c;             // fp32 output, or
    uint16_t* c_bf16;     // bf16 output (round to nearest even) ...
    float* amax;          // ... with max|C_bf16| folded into *amax (nullable)
    OutputQuant q;        // bf16 output only: its block-16 quantization (q.ts null: none)
};

void launch_gemm_nt(const GemmArgs& g, hipStream_t stream);

// Native MXFP4 comparison GEMM: a_scales / b_scales are E8M0 bytes, one per
// 32 elements along K ([rows][K/32]); fp32 output.
void launch_gemm_nt_mx(const GemmArgs& g, hipStream_t stream);

}  // namespace ue5m3fp4
