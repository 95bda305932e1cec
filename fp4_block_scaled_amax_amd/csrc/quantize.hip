// Block-16 E2M1/UE5M3 quantizer with fused transposed output, tensor-amax
// by-product, dequantizer and the periodic tensor-scale refresh (gfx950).
//
// Method: "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining"
// (arXiv 2609.02846), abstract: E2M1 payloads with UE5M3 scales per 16
// elements under a periodically refreshed fp32 tensor scale; stochastic
// rounding only for backward gradients.  "Stable FP4 Training via
// Transposition-Invariant Block Quantization" (related-papers summary): a
// 1-D-blocked tensor and its transpose get different scales, so the
// transposed GEMM operand is quantized again along its own axis -- here from
// the same bf16 registers, so the input is read from HBM once.
//
// Work decomposition.  One thread owns a 16-row x 8-column tile of x, loaded
// as 16 coalesced 16-byte row segments (a wave reads 2 rows x 512 bytes per
// instruction).  Along a row the thread holds half of a 16-element block; the
// partner lane (lane ^ 1) holds the other half, and one lane exchange gives
// the block amax.  Down a column the thread holds a whole 16-element block,
// so the transposed output needs no exchange at all.  A 256-thread workgroup
// covers 128 rows x 256 columns.
#include "formats.hpp"
#include "kernels.hpp"

namespace ue5m3fp4 {

namespace {

constexpr int kTileRows = 128;
constexpr int kTileCols = 256;
constexpr int kThreads = 256;

// |x| as an ordered integer: bf16 magnitude bits.  For non-negative floats
// the unsigned order of the bits is the numeric order, and a NaN (exponent
// all ones, mantissa != 0) sorts above +Inf, so an integer max propagates NaN.
__device__ __forceinline__ uint32_t max_abs_pair(uint32_t w) {
    const uint32_t lo = w & 0x7FFFu;
    const uint32_t hi = (w >> 16) & 0x7FFFu;
    return lo > hi ? lo : hi;
}

struct BlockScale {
    uint32_t code;  // UE5M3 byte
    float r;        // 1 / (ts * s_b); unused when special
    bool special;   // code 0x00 or 0xFF: payload magnitudes are 0
};

__device__ __forceinline__ BlockScale block_scale(uint32_t amax_bits16, float ts, float K) {
    BlockScale b;
    const float amax = __uint_as_float(amax_bits16 << 16);
    const float s_raw = amax / K;
    b.code = ue5m3_encode(s_raw);
    b.special = (b.code == 0u) || (b.code == kUe5m3Nan);
    const float d = ts * ue5m3_decode(b.special ? 0x78u : b.code);
    b.r = 1.0f / d;
    return b;
}

// Payload nibble of one bf16 element (in the low 16 bits of h).
template <bool SR>
__device__ __forceinline__ uint32_t element_code(uint32_t h16, const BlockScale& b, uint32_t u16) {
    const uint32_t sign = (h16 >> 12) & 8u;
    const float x = __uint_as_float(h16 << 16);
    const float a = fabsf(x * b.r);
    uint32_t idx = SR ? e2m1_sr_index(a, u16) : e2m1_rne_index(a);
    idx = b.special ? 0u : idx;
    return sign | idx;
}

template <bool ROW, bool COL, bool SR, bool AMAX>
__global__ __launch_bounds__(kThreads, 2) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ tensor_scale, uint64_t seed, uint32_t offset,
    uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
    uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales,
    float* __restrict__ amax_inout) {
    const int tx = threadIdx.x & 31;
    const int ty = threadIdx.x >> 5;
    const int64_t r0 = (int64_t)blockIdx.y * kTileRows + 16 * ty;
    const int64_t c0 = (int64_t)blockIdx.x * kTileCols + 8 * tx;
    const bool col_ok = c0 < cols;  // cols % 16 == 0: lane pairs agree

    // ---- load 16 rows x 8 bf16 (zeros outside the tensor)
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t r = r0 + i;
        if (col_ok && r < rows) {
            v[i] = *reinterpret_cast<const uint4*>(x + r * ld + c0);
        } else {
            v[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }

    float ts = 0.0f, K = 0.0f;
    if (ROW || COL) {
        ts = *tensor_scale;
        K = 6.0f * ts;
    }

    uint32_t tmax = 0u;  // max |x| of this thread, bf16 magnitude bits

    // ---- row-wise output: blocks along columns, half a block per lane
    if (ROW || AMAX) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t m = max_abs_pair(v[i].x);
            m = max(m, max_abs_pair(v[i].y));
            m = max(m, max_abs_pair(v[i].z));
            m = max(m, max_abs_pair(v[i].w));
            tmax = max(tmax, m);
            if (ROW) {
                const uint32_t other = __shfl_xor(m, 1);
                const int64_t r = r0 + i;
                const BlockScale b = block_scale(max(m, other), ts, K);
                U32x4 w;
                if (SR) {
                    const uint64_t e0 = (uint64_t)r * (uint64_t)cols + (uint64_t)c0;
                    w = sr_words(e0 >> 3, offset, 0u, seed);
                }
                const uint32_t words[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                uint32_t packed = 0u;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t h = (k & 1) ? (words[k >> 1] >> 16) : (words[k >> 1] & 0xFFFFu);
                    const uint32_t u = SR ? sr_u16(w, k) : 0u;
                    packed |= element_code<SR>(h, b, u) << (4 * k);
                }
                if (col_ok && r < rows) {
                    *reinterpret_cast<uint32_t*>(row_codes + r * (cols / 2) + c0 / 2) = packed;
                    if ((tx & 1) == 0) row_scales[r * (cols / 16) + c0 / 16] = (uint8_t)b.code;
                }
            }
        }
    }

    // ---- transposed output: blocks along rows, one whole block per column
    if (COL) {
        if (ROW || AMAX) {
            // Opaque to the optimizer: stops it from keeping the 128 unpacked
            // halves of the row pass alive for reuse here (that doubles the
            // live registers and spills).  No instruction is emitted.
#pragma unroll
            for (int i = 0; i < 16; ++i)
                asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t h[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t word = (j >> 1) == 0 ? v[i].x : (j >> 1) == 1 ? v[i].y
                                    : (j >> 1) == 2 ? v[i].z : v[i].w;
                h[i] = (j & 1) ? (word >> 16) : (word & 0xFFFFu);
            }
            uint32_t m = 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) m = max(m, h[i] & 0x7FFFu);
            const BlockScale b = block_scale(m, ts, K);
            const int64_t c = c0 + j;
            U32x4 w0, w1;
            if (SR) {
                const uint64_t e0 = (uint64_t)c * (uint64_t)rows + (uint64_t)r0;
                w0 = sr_words(e0 >> 3, offset, 1u, seed);
                w1 = sr_words((e0 >> 3) + 1u, offset, 1u, seed);
            }
            uint32_t lo = 0u, hi = 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t u = SR ? sr_u16(w0, i) : 0u;
                lo |= element_code<SR>(h[i], b, u) << (4 * i);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t u = SR ? sr_u16(w1, i) : 0u;
                hi |= element_code<SR>(h[8 + i], b, u) << (4 * i);
            }
            if (col_ok && r0 < rows) {
                *reinterpret_cast<uint2*>(col_codes + c * (rows / 2) + r0 / 2) = make_uint2(lo, hi);
                col_scales[c * (rows / 16) + r0 / 16] = (uint8_t)b.code;
            }
        }
    }

    // ---- tensor amax: wave reduction, one atomic per wave
    if (AMAX) {
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, s));
        if ((threadIdx.x & 63) == 0 && tmax != 0u) {
            atomicMax(reinterpret_cast<unsigned int*>(amax_inout), tmax << 16);
        }
    }
}

template <bool ROW, bool COL, bool SR, bool AMAX>
void launch_quantize(const QuantizeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.cols + kTileCols - 1) / kTileCols),
                    (unsigned)((a.rows + kTileRows - 1) / kTileRows));
    hipLaunchKernelGGL((quantize_kernel<ROW, COL, SR, AMAX>), grid, dim3(kThreads), 0, stream,
                       a.x, a.rows, a.cols, a.ld, a.tensor_scale, a.seed, a.offset, a.row_codes,
                       a.row_scales, a.col_codes, a.col_scales, a.amax_inout);
}

template <bool ROW, bool COL, bool SR>
void dispatch_amax(const QuantizeArgs& a, hipStream_t s) {
    if (a.amax_inout) launch_quantize<ROW, COL, SR, true>(a, s);
    else launch_quantize<ROW, COL, SR, false>(a, s);
}

template <bool ROW, bool COL>
void dispatch_sr(const QuantizeArgs& a, hipStream_t s) {
    if (a.stochastic) dispatch_amax<ROW, COL, true>(a, s);
    else dispatch_amax<ROW, COL, false>(a, s);
}

// ----------------------------------------------------------- dequantize --

__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ tensor_scale,
                                                         int64_t rows, int64_t cols,
                                                         float* __restrict__ out) {
    const int64_t groups = cols / 8;  // 8 elements (4 code bytes) per thread
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * groups) return;
    const int64_t r = t / groups;
    const int64_t g = t - r * groups;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + r * (cols / 2) + 4 * g);
    const uint32_t sc = scales[r * (cols / 16) + g / 2];
    const float ts = *tensor_scale;
    const float s = sc == kUe5m3Nan ? __uint_as_float(0x7FC00000u) : ue5m3_decode(sc);
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t n = (w >> (4 * k)) & 15u;
        const uint32_t idx = n & 7u;
        // E2M1 magnitude: idx 0/1 -> 0/0.5; otherwise 2^(e-1) * (1 + m/2)
        const uint32_t e = idx >> 1, m = idx & 1u;
        const uint32_t bits = e == 0u ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
        const float q = __uint_as_float(bits | ((n & 8u) << 28));
        const float qs = q * s;  // exact
        o[k] = qs * ts;
    }
    float4* dst = reinterpret_cast<float4*>(out + r * cols + 8 * g);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

// ------------------------------------------------------ tensor scale ----

__global__ void update_tensor_scale_kernel(float* __restrict__ amax_running,
                                           float* __restrict__ tensor_scale, float max_safe) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    const float amax = *amax_running;
    const uint32_t b = __float_as_uint(amax);
    const bool finite = (b & 0x7F800000u) != 0x7F800000u;
    if (finite && amax > 0.0f) {
        const float denom = 6.0f * max_safe;
        *tensor_scale = amax / denom;
    }
    *amax_running = 0.0f;
}

}  // namespace

void launch_quantize_blockscale(const QuantizeArgs& a, hipStream_t s) {
    const bool row = a.row_codes != nullptr;
    const bool col = a.col_codes != nullptr;
    if (row && col) dispatch_sr<true, true>(a, s);
    else if (row) dispatch_sr<true, false>(a, s);
    else if (col) dispatch_sr<false, true>(a, s);
    else launch_quantize<false, false, false, true>(a, s);  // amax-only pass
}

void launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts,
                       int64_t rows, int64_t cols, float* out, hipStream_t s) {
    const int64_t threads = rows * (cols / 8);
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(dequantize_kernel, dim3(blocks), dim3(256), 0, s, codes, scales, ts, rows,
                       cols, out);
}

void launch_update_tensor_scale(float* amax_running, float* tensor_scale, float max_safe,
                                hipStream_t s) {
    hipLaunchKernelGGL(update_tensor_scale_kernel, dim3(1), dim3(64), 0, s, amax_running,
                       tensor_scale, max_safe);
}

}  // namespace ue5m3fp4
