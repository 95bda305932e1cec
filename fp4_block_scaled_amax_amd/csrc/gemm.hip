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
// 32 elements: it can carry neither the 3 mantissa bits of a UE5M3 scale nor
// a 16-element block.  Instead each element is dequantized exactly to fp16
// and fed to v_mfma_f32_32x32x16_f16 (fp32 accumulation; fp16 x fp16
// products are exact in fp32).  The fp16 value is q * s / 16: q * s has at
// most 6 significant bits and lies in [2^-18, 688128]; divided by 16 it lies
// in [2^-22, 43008], inside fp16's range and, below 2^-14, on fp16's
// subnormal grid (multiples of 2^-24) -- so every value is exact.  The
// epilogue multiplies by 256 * tsA * tsB.
//
// Dequantization of two elements costs two VALU operations:
//   v_cvt_scalef32_pk_f16_fp4  q * 2^E   (the instruction applies only the
//                                         exponent of its fp32 scale operand)
//   v_pk_mul_f16               * m       (m = 8 + f for a normal UE5M3 code
//                                         (e, f), f for a subnormal one)
// with E = max(e, 1) - 22, so q * 2^E * m = q * s / 16.  A 256-entry table in
// LDS holds (2^E as fp32, m as packed fp16) for every scale byte; 0xFF maps
// to m = NaN so a NaN block poisons its output as the format requires.
//
// Tiling.  256 x 256 workgroup tile, 4 waves of 128 x 128 (4 x 4 MFMA tiles,
// 256 fp32 accumulators per lane), K chunks of 128 elements double-buffered
// in LDS (codes: 64 bytes per row padded to 80, which makes the 16-byte
// fragment reads of 8 consecutive rows hit distinct banks; scales: 8 bytes
// per row).  Global loads for chunk c + 2 are issued while chunk c is
// computed, and stored to LDS during chunk c + 1.
//
// K order.  The sum over k may be taken in any order as long as A and B use
// the same one.  In half-chunk u (64 elements) lane (r, h) (r = lane % 32,
// h = lane / 32) owns elements [64h + 32u, 64h + 32u + 32) of its row -- one
// 16-byte LDS read -- and MFMA step t (0..3) takes its elements
// [.. + 8t, .. + 8t + 8) (one code dword).  So each MFMA sees two 16-blocks
// (one per half-wave), each dequantized with its own scale before the
// multiply.
//
// Tile order.  Consecutive workgroup ids are dispatched round-robin over
// the 8 XCDs, each with its own L2.  The id is remapped so that each XCD
// walks a contiguous range of tiles, grouped 4 tile-rows at a time, so the
// 32 workgroups in flight on one XCD share 4 A panels and 8 B panels in L2.
#include "formats.hpp"
#include "kernels.hpp"

namespace ue5m3fp4 {

namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kThreads = 256;
constexpr int kCodeBytes = kBK / 2;            // 64 code bytes per row per chunk
constexpr int kCodeStride = kCodeBytes + 16;   // padded LDS row stride
constexpr int kScaleBytes = kBK / 16;          // 8 scale bytes per row per chunk
constexpr int kCodesA = 0;
constexpr int kCodesB = kCodesA + kBM * kCodeStride;
constexpr int kScalesA = kCodesB + kBN * kCodeStride;
constexpr int kScalesB = kScalesA + kBM * kScaleBytes;
constexpr int kStage = kScalesB + kBN * kScaleBytes;  // 45056 bytes
constexpr int kLut = 2 * kStage;
constexpr int kSmem = kLut + 256 * 8;
constexpr int kGroupM = 4;  // tile rows per group in the tile order

struct ScalePair {
    float cvt;      // 2^E, consumed by the convert instruction (exponent only)
    f16x2_t mult;   // integer mantissa factor in both halves
};

// 8 E2M1 codes (one dword; element k in nibble k) -> 8 fp16 values q*s/16.
__device__ __forceinline__ f16x8_t dequant8(uint32_t w, const ScalePair& s) {
    const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.cvt, 0) * s.mult;
    const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.cvt, 1) * s.mult;
    const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.cvt, 2) * s.mult;
    const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.cvt, 3) * s.mult;
    f16x8_t out;
    out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
    out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
    return out;
}

__device__ __forceinline__ ScalePair lut_entry(const uint8_t* smem, uint32_t code) {
    const uint2 v = *reinterpret_cast<const uint2*>(smem + kLut + 8 * code);
    ScalePair s;
    s.cvt = __uint_as_float(v.x);
    __builtin_memcpy(&s.mult, &v.y, 4);
    return s;
}

// Workgroup id -> (tile row, tile col), XCD-aware and grouped.
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int& tm, int& tn) {
    const int n = tiles_m * tiles_n;
    int id = blockIdx.x;
    const int per_xcd = n / 8;
    if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;  // the tail keeps its id
    const int width = kGroupM * tiles_n;
    const int first_m = (id / width) * kGroupM;
    const int rows = min(tiles_m - first_m, kGroupM);
    tm = first_m + (id % width) % rows;
    tn = (id % width) / rows;
}

template <bool ALIGNED>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, const float* __restrict__ b_ts, int64_t M, int64_t N,
    int64_t K, float* __restrict__ C) {
    __shared__ __align__(16) uint8_t smem[kSmem];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 31, h = lane >> 5;

    // scale byte -> (2^E, m) table
    {
        const uint32_t c = (uint32_t)tid;
        const uint32_t e = c >> 3, f = c & 7u;
        const uint32_t eb = e > 0u ? e : 1u;
        const uint32_t cvt_bits = (eb + 105u) << 23;  // 2^(max(e,1) - 22)
        const _Float16 m = c == kUe5m3Nan ? (_Float16)__builtin_nanf("")
                                          : (_Float16)(float)(e > 0u ? 8u + f : f);
        uint16_t mb;
        __builtin_memcpy(&mb, &m, 2);
        *reinterpret_cast<uint2*>(smem + kLut + 8 * c) = make_uint2(cvt_bits, (uint32_t)mb * 0x10001u);
    }

    int tm, tn;
    tile_of((int)((M + kBM - 1) / kBM), (int)((N + kBN - 1) / kBN), tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t kbytes = K / 2, kblocks = K / 16;
    const int nchunks = (int)((K + kBK - 1) / kBK);

    // ---- global -> registers -> LDS staging
    // codes: 256 rows x 64 bytes per operand = 1024 16-byte units, 4 per thread
    // scales: 256 rows x 8 bytes per operand, one row per thread
    constexpr int kUnits = ALIGNED ? 4 : 8;  // 16-byte or 8-byte code units
    uint4 ra[ALIGNED ? 4 : 1], rb[ALIGNED ? 4 : 1];
    uint2 ra8[ALIGNED ? 1 : 8], rb8[ALIGNED ? 1 : 8];
    uint2 rsa, rsb;

    auto gload = [&](int chunk) {
        const int64_t k0 = (int64_t)chunk * kBK;
        if (ALIGNED) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int u = tid + kThreads * i;
                const int row = u >> 2, part = u & 3;
                const int64_t off = k0 / 2 + 16 * part;
                ra[i] = m0 + row < M ? *reinterpret_cast<const uint4*>(a_codes + (m0 + row) * kbytes + off)
                                     : make_uint4(0u, 0u, 0u, 0u);
                rb[i] = n0 + row < N ? *reinterpret_cast<const uint4*>(b_codes + (n0 + row) * kbytes + off)
                                     : make_uint4(0u, 0u, 0u, 0u);
            }
            rsa = m0 + tid < M ? *reinterpret_cast<const uint2*>(a_scales + (m0 + tid) * kblocks + k0 / 16)
                               : make_uint2(0u, 0u);
            rsb = n0 + tid < N ? *reinterpret_cast<const uint2*>(b_scales + (n0 + tid) * kblocks + k0 / 16)
                               : make_uint2(0u, 0u);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int u = tid + kThreads * i;
                const int row = u >> 3, part = u & 7;
                const int64_t gk = k0 + 16 * part;
                const bool kin = gk < K;
                ra8[i] = kin && m0 + row < M
                             ? *reinterpret_cast<const uint2*>(a_codes + (m0 + row) * kbytes + gk / 2)
                             : make_uint2(0u, 0u);
                rb8[i] = kin && n0 + row < N
                             ? *reinterpret_cast<const uint2*>(b_codes + (n0 + row) * kbytes + gk / 2)
                             : make_uint2(0u, 0u);
            }
            uint32_t sa[2] = {0u, 0u}, sb[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t blk = k0 / 16 + j;
                if (blk < kblocks) {
                    if (m0 + tid < M) sa[j >> 2] |= (uint32_t)a_scales[(m0 + tid) * kblocks + blk] << (8 * (j & 3));
                    if (n0 + tid < N) sb[j >> 2] |= (uint32_t)b_scales[(n0 + tid) * kblocks + blk] << (8 * (j & 3));
                }
            }
            rsa = make_uint2(sa[0], sa[1]);
            rsb = make_uint2(sb[0], sb[1]);
        }
    };

    auto lstore = [&](int stage) {
        uint8_t* base = smem + stage * kStage;
        if (ALIGNED) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int u = tid + kThreads * i;
                const int row = u >> 2, part = u & 3;
                *reinterpret_cast<uint4*>(base + kCodesA + row * kCodeStride + 16 * part) = ra[i];
                *reinterpret_cast<uint4*>(base + kCodesB + row * kCodeStride + 16 * part) = rb[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int u = tid + kThreads * i;
                const int row = u >> 3, part = u & 7;
                *reinterpret_cast<uint2*>(base + kCodesA + row * kCodeStride + 8 * part) = ra8[i];
                *reinterpret_cast<uint2*>(base + kCodesB + row * kCodeStride + 8 * part) = rb8[i];
            }
        }
        *reinterpret_cast<uint2*>(base + kScalesA + tid * kScaleBytes) = rsa;
        *reinterpret_cast<uint2*>(base + kScalesB + tid * kScaleBytes) = rsb;
    };
    (void)kUnits;

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (nchunks > 0) {
        gload(0);
        lstore(0);
        if (nchunks > 1) gload(1);
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const uint8_t* base = smem + (c & 1) * kStage;
#pragma unroll 1
        for (int u = 0; u < 2; ++u) {
            uint4 ca[4], cb[4];
            ScalePair sa[4][2], sb[4][2];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int arow = wm * 128 + g * 32 + r;
                const int brow = wn * 128 + g * 32 + r;
                ca[g] = *reinterpret_cast<const uint4*>(base + kCodesA + arow * kCodeStride + 32 * h + 16 * u);
                cb[g] = *reinterpret_cast<const uint4*>(base + kCodesB + brow * kCodeStride + 32 * h + 16 * u);
                const uint32_t s2a = *reinterpret_cast<const uint16_t*>(base + kScalesA + arow * kScaleBytes + 4 * h + 2 * u);
                const uint32_t s2b = *reinterpret_cast<const uint16_t*>(base + kScalesB + brow * kScaleBytes + 4 * h + 2 * u);
                sa[g][0] = lut_entry(smem, s2a & 0xFFu);
                sa[g][1] = lut_entry(smem, s2a >> 8);
                sb[g][0] = lut_entry(smem, s2b & 0xFFu);
                sb[g][1] = lut_entry(smem, s2b >> 8);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                f16x8_t fa[4], fb[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t wa = t == 0 ? ca[g].x : t == 1 ? ca[g].y : t == 2 ? ca[g].z : ca[g].w;
                    const uint32_t wb = t == 0 ? cb[g].x : t == 1 ? cb[g].y : t == 2 ? cb[g].z : cb[g].w;
                    fa[g] = dequant8(wa, sa[g][t >> 1]);
                    fb[g] = dequant8(wb, sb[g][t >> 1]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
        }
        if (c + 1 < nchunks) lstore((c + 1) & 1);
        if (c + 2 < nchunks) gload(c + 2);
        __syncthreads();
    }

    // ---- epilogue: C = (acc * 256 tsA) * tsB.  Accumulator register e of lane
    // (r, h) holds row 8 * (e / 4) + 4 * h + e % 4, column r of a 32 x 32 tile.
    const float sa256 = *a_ts * 256.0f, tsb = *b_ts;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 128 + j * 32 + r;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (row < M && col < N) C[row * N + col] = (acc[i][j][e] * sa256) * tsb;
            }
        }
}

}  // namespace

void launch_gemm_nt(const GemmArgs& g, hipStream_t stream) {
    const int64_t tiles = ((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
    const dim3 grid((unsigned)tiles);
    if (g.K % kBK == 0) {
        hipLaunchKernelGGL(gemm_nt_kernel<true>, grid, dim3(kThreads), 0, stream, g.a_codes,
                           g.a_scales, g.a_ts, g.b_codes, g.b_scales, g.b_ts, g.M, g.N, g.K, g.c);
    } else {
        hipLaunchKernelGGL(gemm_nt_kernel<false>, grid, dim3(kThreads), 0, stream, g.a_codes,
                           g.a_scales, g.a_ts, g.b_codes, g.b_scales, g.b_ts, g.M, g.N, g.K, g.c);
    }
}

}  // namespace ue5m3fp4
