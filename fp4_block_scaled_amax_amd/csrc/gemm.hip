// Block-scaled "NT" GEMM on UE5M3/E2M1 operands for gfx950:
//   C[i][j] = tsA * tsB * sum_k A(i, k) * B(j, k),   fp32 accumulation,
// where both operands are stored as E2M1 codes with one UE5M3 scale per 16
// elements along K.  fprop, dgrad and wgrad are all this kernel with
// different operands ("Rethinking Shrinkage Bias in LLM FP4 Pretraining ...
// UFP4 Recipe", abstract: the three training GEMMs; "UE5M3 FP4 Block Scaling
// for Stable Language Model Pretraining", abstract: UE5M3 block-16 operands,
// software-emulated).
//
// Emulation.  gfx950's scaled FP4 MFMA takes power-of-two (E8M0) scales per
// 32 elements, which cannot carry a UE5M3 mantissa nor a 16-element block.
// A dequantized element q * s has at most 6 significant bits and lies in
// [2^-18, 688128], so it is exact in bf16; bf16 x bf16 products are exact in
// fp32.  The kernel therefore stages packed codes and scale bytes in LDS,
// dequantizes each MFMA fragment exactly to bf16 in registers and runs
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
//
// K order.  The sum over k may be taken in any order as long as A and B use
// the same one.  Lane (r, h) of a wave (r = lane % 32, h = lane / 32) owns
// elements [64h, 64h + 64) of a 128-element K-chunk of its row; MFMA step t
// (0..7) takes elements [64h + 8t, 64h + 8t + 8) from every lane, so one
// 4-byte LDS read per operand row feeds one MFMA and each step sees two
// different 16-blocks (one per half-wave), each dequantized with its own
// scale before the multiply.
#include "formats.hpp"
#include "kernels.hpp"

namespace ue5m3fp4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;             // workgroup tile rows (A)
constexpr int kBN = 128;             // workgroup tile cols (B)
constexpr int kBK = 128;             // K elements per chunk
constexpr int kCodeBytes = kBK / 2;  // 64 code bytes per row per chunk
constexpr int kScaleBytes = kBK / 16;
constexpr int kLdsStride = kCodeBytes + 16;  // padded row stride in LDS
constexpr int kThreads = 256;        // 4 waves, 2 x 2, each 64 x 64

// E2M1 nibble -> fp32 (exact): exponent field 0 is 0 / 0.5, otherwise
// 2^(e-1) * (1 + m/2); bit 3 is the sign.
__device__ __forceinline__ float e2m1_value(uint32_t n) {
    const uint32_t idx = n & 7u;
    const uint32_t e = idx >> 1, m = idx & 1u;
    const uint32_t bits = e == 0u ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
    return __uint_as_float(bits | ((n & 8u) << 28));
}

__device__ __forceinline__ float scale_value(uint32_t c) {
    return c == kUe5m3Nan ? __uint_as_float(0x7FC00000u) : ue5m3_decode(c);
}

// 8 codes (one dword, element k in nibble k) times one block scale -> 8 bf16.
// q * s is exact in fp32 and in bf16, so truncating to the top 16 bits is exact.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w, float s) {
    uint32_t p[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float lo = e2m1_value((w >> (8 * k)) & 15u) * s;
        const float hi = e2m1_value((w >> (8 * k + 4)) & 15u) * s;
        p[k] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    bf16x8_t out;
    __builtin_memcpy(&out, p, sizeof(p));
    return out;
}

__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, const float* __restrict__ b_ts, int64_t M, int64_t N,
    int64_t K, float* __restrict__ C) {
    __shared__ __align__(16) uint8_t sA[kBM * kLdsStride];
    __shared__ __align__(16) uint8_t sB[kBN * kLdsStride];
    __shared__ __align__(16) uint8_t sAs[kBM * kScaleBytes];
    __shared__ __align__(16) uint8_t sBs[kBN * kScaleBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 31, h = lane >> 5;
    const int64_t m0 = (int64_t)blockIdx.y * kBM;
    const int64_t n0 = (int64_t)blockIdx.x * kBN;
    const int64_t kbytes = K / 2, kblocks = K / 16;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    for (int64_t k0 = 0; k0 < K; k0 += kBK) {
        // ---- stage codes: 8-byte units = one 16-element block each
        for (int u = tid; u < kBM * (kCodeBytes / 8); u += kThreads) {
            const int row = u >> 3, part = u & 7;
            const int64_t gk = k0 + 16 * part;
            uint2 va = make_uint2(0u, 0u), vb = make_uint2(0u, 0u);
            if (gk < K) {
                if (m0 + row < M)
                    va = *reinterpret_cast<const uint2*>(a_codes + (m0 + row) * kbytes + gk / 2);
                if (n0 + row < N)
                    vb = *reinterpret_cast<const uint2*>(b_codes + (n0 + row) * kbytes + gk / 2);
            }
            *reinterpret_cast<uint2*>(sA + row * kLdsStride + part * 8) = va;
            *reinterpret_cast<uint2*>(sB + row * kLdsStride + part * 8) = vb;
        }
        // ---- stage scale bytes
        for (int u = tid; u < kBM * kScaleBytes; u += kThreads) {
            const int row = u >> 3, blk = u & 7;
            const int64_t gb = k0 / 16 + blk;
            uint8_t sa = 0, sb = 0;
            if (gb < kblocks) {
                if (m0 + row < M) sa = a_scales[(m0 + row) * kblocks + gb];
                if (n0 + row < N) sb = b_scales[(n0 + row) * kblocks + gb];
            }
            sAs[row * kScaleBytes + blk] = sa;
            sBs[row * kScaleBytes + blk] = sb;
        }
        __syncthreads();

#pragma unroll
        for (int t = 0; t < 8; ++t) {
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int arow = wm * 64 + g * 32 + r;
                const uint32_t wa =
                    *reinterpret_cast<const uint32_t*>(sA + arow * kLdsStride + 32 * h + 4 * t);
                af[g] = dequant8(wa, scale_value(sAs[arow * kScaleBytes + 4 * h + (t >> 1)]));
                const int brow = wn * 64 + g * 32 + r;
                const uint32_t wb =
                    *reinterpret_cast<const uint32_t*>(sB + brow * kLdsStride + 32 * h + 4 * t);
                bfr[g] = dequant8(wb, scale_value(sBs[brow * kScaleBytes + 4 * h + (t >> 1)]));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
        __syncthreads();
    }

    // ---- epilogue: C = (acc * tsA) * tsB.  Accumulator register e of lane
    // (r, h) holds row 8 * (e / 4) + 4 * h + e % 4, column r of a 32 x 32 tile.
    const float tsa = *a_ts, tsb = *b_ts;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + r;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (row < M && col < N) C[row * N + col] = (acc[i][j][e] * tsa) * tsb;
            }
        }
}

}  // namespace

void launch_gemm_nt(const GemmArgs& g, hipStream_t stream) {
    const dim3 grid((unsigned)((g.N + kBN - 1) / kBN), (unsigned)((g.M + kBM - 1) / kBM));
    hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(kThreads), 0, stream, g.a_codes, g.a_scales,
                       g.a_ts, g.b_codes, g.b_scales, g.b_ts, g.M, g.N, g.K, g.c);
}

}  // namespace ue5m3fp4
