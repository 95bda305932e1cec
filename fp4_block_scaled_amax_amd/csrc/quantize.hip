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
// Work decomposition.  A 256-thread workgroup owns a 128 x 256 tile; each
// thread a 16-row x 8-column piece, loaded as 16 coalesced 16-byte row
// segments (a wave reads 2 rows x 512 bytes per instruction).  Along a row
// the thread holds half of a 16-element block and the partner lane (lane ^ 1,
// one DPP swap) the other half; the pair splits the 16 row-block scale
// computations between them and swaps the results.  Down a column the thread
// holds a whole block.  Each row of the tile writes a complete 128-byte line
// of codes, each column 64 bytes.  One tile per workgroup: several resident
// workgroups per CU keep HBM busy while others compute.  Loads are unconditional (edge
// addresses are clamped into the tensor and the values zeroed at use), so
// the compiler issues all 16 back to back.
//
// Arithmetic per block: the block amax is an integer max over bf16
// magnitudes (packed 16-bit max; a NaN sorts above +Inf); s_raw = amax / (6 ts)
// and r = 1 / (ts * s_b) use the refined division / reciprocal of formats.hpp
// (equal to IEEE division in their guarded range); when s_raw falls in
// UE5M3's normal range the encode is one rounding add on the fp32 bits, and
// everything else (flushed, subnormal, saturated, NaN, out-of-range scales)
// takes the general path.  Round-to-nearest payloads come from
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0, which rounds an fp32 value to
// E2M1 exactly as the nearest-even definition does (checked on gfx950 for all
// 2^32 non-NaN inputs); a NaN never reaches it: blocks whose scale is NaN or
// whose reciprocal overflows take the software path.
#include "formats.hpp"
#include "kernels.hpp"

namespace ue5m3fp4 {

namespace {

constexpr int kTileRows = 128;
constexpr int kTileCols = 256;
constexpr int kThreads = 256;

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    u16x2_t x, y;
    __builtin_memcpy(&x, &a, 4);
    __builtin_memcpy(&y, &b, 4);
    const u16x2_t m = __builtin_elementwise_max(x, y);
    uint32_t out;
    __builtin_memcpy(&out, &m, 4);
    return out;
}

// value held by the partner lane (lane ^ 1)
__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

struct Ctx {
    float ts, K, yK;  // K = 6 ts, yK = RN(1 / K)
    bool fastK;       // K inside the range where the refined division is exact
};

struct BlockScale {
    uint32_t code;  // UE5M3 byte
    float r;        // 1 / (ts * s_b); 0 for a flushed block (payload = sign only);
                    // NaN for a NaN block; may be +Inf if ts * s_b underflows
};

// General path: any amax, any tensor scale.
__device__ __noinline__ BlockScale block_scale_general(float amax, Ctx c) {
    BlockScale b;
    b.code = ue5m3_encode(amax / c.K);
    if (b.code == 0u) b.r = 0.0f;
    else if (b.code == kUe5m3Nan) b.r = __uint_as_float(0x7FC00000u);
    else b.r = 1.0f / (c.ts * ue5m3_decode(b.code));
    return b;
}

__device__ __forceinline__ BlockScale block_scale(uint32_t amax_bits16, const Ctx& c) {
    const float amax = __uint_as_float(amax_bits16 << 16);
    // refined division amax / K (exact where guarded below)
    const float q = amax * c.yK;
    const float rr = __builtin_fmaf(-c.K, q, amax);
    const float s = __builtin_fmaf(rr, c.yK, q);
    // UE5M3 normal range: keep 3 mantissa bits, round the other 20 to nearest even
    const uint32_t sb = __float_as_uint(s);
    const uint32_t rounded = (sb + 0x7FFFFu + ((sb >> 20) & 1u)) >> 20;
    const uint32_t code = min(rounded - (112u << 3), kUe5m3MaxCode);  // rebias 127 -> 15
    const float sval = __uint_as_float((code + (112u << 3)) << 20);   // exact UE5M3 value
    const float d = c.ts * sval;
    const bool fast = c.fastK && amax >= 0x1p-100f && s >= 0x1p-14f && s <= 0x1p100f &&
                      d >= 0x1p-100f && d <= 0x1p100f;
    if (__builtin_expect(fast, 1)) {
        const float y = __builtin_amdgcn_rcpf(d);
        const float e = __builtin_fmaf(-d, y, 1.0f);
        BlockScale b;
        b.code = code;
        b.r = __builtin_fmaf(e, y, y);
        return b;
    }
    return block_scale_general(amax, c);
}

// Payload nibble of one element by the definition (software path): RNE or SR
// on |x * r|; a NaN block scale leaves only the sign bit.
template <bool SR>
__device__ __forceinline__ uint32_t element_code(float x, const BlockScale& b, uint32_t u16) {
    const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
    const float a = fabsf(x * b.r);
    const uint32_t idx = SR ? e2m1_sr_index(a, u16) : e2m1_rne_index(a);
    return sign | (b.code == kUe5m3Nan ? 0u : idx);
}

// 8 fp32 elements (already unpacked) -> 8 nibbles, element k in nibble k.
template <bool SR>
__device__ __forceinline__ uint32_t encode8(const float (&x)[8], const BlockScale& b,
                                           const U32x4& rnd) {
    if (!SR && __builtin_expect(b.r <= 3.4028235e38f, 1)) {
        uint32_t p = 0u;
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[0] * b.r, x[1] * b.r, 1.0f, 0);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[2] * b.r, x[3] * b.r, 1.0f, 1);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[4] * b.r, x[5] * b.r, 1.0f, 2);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[6] * b.r, x[7] * b.r, 1.0f, 3);
        return p;
    }
    uint32_t p = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) p |= element_code<SR>(x[k], b, SR ? sr_u16(rnd, k) : 0u) << (4 * k);
    return p;
}

__device__ __forceinline__ uint32_t comp(const uint4& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

template <bool ROW, bool COL, bool SR, bool AMAX>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ tensor_scale, uint64_t seed, uint32_t offset,
    uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
    uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales,
    float* __restrict__ amax_inout) {
    const int tx = threadIdx.x & 31;
    const int ty = threadIdx.x >> 5;
    const int64_t r0 = (int64_t)blockIdx.y * kTileRows + 16 * ty;
    const int64_t c0 = (int64_t)blockIdx.x * kTileCols + 8 * tx;
    const bool col_ok = c0 < cols;  // cols % 16 == 0: the two lanes of a pair agree

    // ---- 16 unconditional loads (clamped addresses), zeroed outside the tensor
    uint4 v[16];
    {
        const int64_t cc = col_ok ? c0 : cols - 8;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t r = r0 + i < rows ? r0 + i : rows - 1;
            v[i] = *reinterpret_cast<const uint4*>(x + r * ld + cc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (!(col_ok && r0 + i < rows)) v[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }

    Ctx ctx{0.0f, 0.0f, 0.0f, false};
    if (ROW || COL) {
        ctx.ts = *tensor_scale;
        ctx.K = 6.0f * ctx.ts;
        ctx.yK = 1.0f / ctx.K;
        ctx.fastK = ctx.K >= 0x1p-100f && ctx.K <= 0x1p100f;
    }

    // ---- amax of every row half-block and of every column pair
    uint32_t rmax[16];
    uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t m0 = v[i].x & 0x7FFF7FFFu, m1 = v[i].y & 0x7FFF7FFFu;
        const uint32_t m2 = v[i].z & 0x7FFF7FFFu, m3 = v[i].w & 0x7FFF7FFFu;
        if (COL) {
            cm[0] = pk_max_u16(cm[0], m0);
            cm[1] = pk_max_u16(cm[1], m1);
            cm[2] = pk_max_u16(cm[2], m2);
            cm[3] = pk_max_u16(cm[3], m3);
        }
        const uint32_t m = pk_max_u16(pk_max_u16(m0, m1), pk_max_u16(m2, m3));
        rmax[i] = max(m & 0xFFFFu, m >> 16);
    }

    uint32_t tmax = 0u;  // max |x| of this thread (bf16 magnitude bits)
    if (AMAX) {
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = max(tmax, rmax[i]);
    }

    // ---- row-wise output: blocks along columns
    if (ROW) {
        // The lane pair splits the row blocks: for rows 2k and 2k + 1, lane
        // parity p computes the scale of row 2k + p and swaps it with its partner.
        const uint32_t p = tx & 1;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t mine = p ? rmax[2 * k + 1] : rmax[2 * k];
            const uint32_t other = p ? rmax[2 * k] : rmax[2 * k + 1];
            // block amax of row 2k + p: my half of it and the partner's half
            const BlockScale own = block_scale(max(mine, swap_pair(other)), ctx);
            BlockScale par;
            par.code = swap_pair(own.code);
            par.r = __uint_as_float(swap_pair(__float_as_uint(own.r)));
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int i = 2 * k + q;
                const BlockScale& b = (q == (int)p) ? own : par;
                BlockScale bb;
                bb.code = q == 0 ? (p ? par.code : own.code) : (p ? own.code : par.code);
                bb.r = q == 0 ? (p ? par.r : own.r) : (p ? own.r : par.r);
                (void)b;
                const int64_t r = r0 + i;
                U32x4 rnd;
                if (SR) rnd = sr_words(((uint64_t)r * (uint64_t)cols + (uint64_t)c0) >> 3, offset, 0u, seed);
                float xs[8];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    xs[2 * m] = bf16_lo(comp(v[i], m));
                    xs[2 * m + 1] = bf16_hi(comp(v[i], m));
                }
                const uint32_t packed = encode8<SR>(xs, bb, rnd);
                if (col_ok && r < rows) {
                    *reinterpret_cast<uint32_t*>(row_codes + r * (cols / 2) + c0 / 2) = packed;
                    if (p == 0) row_scales[r * (cols / 16) + c0 / 16] = (uint8_t)bb.code;
                }
            }
        }
        if (COL) {
            // Opaque to the optimizer: stops it from keeping the unpacked
            // values of the row pass alive for reuse in the column pass (that
            // doubles the live registers).  No instruction is emitted.
#pragma unroll
            for (int i = 0; i < 16; ++i)
                asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
        }
    }

    // ---- transposed output: blocks along rows, one whole block per column
    if (COL) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t mj = (j & 1) ? (cm[j >> 1] >> 16) : (cm[j >> 1] & 0xFFFFu);
            const BlockScale b = block_scale(mj, ctx);
            const int64_t c = c0 + j;
            U32x4 rnd0, rnd1;
            if (SR) {
                const uint64_t n0 = ((uint64_t)c * (uint64_t)rows + (uint64_t)r0) >> 3;
                rnd0 = sr_words(n0, offset, 1u, seed);
                rnd1 = sr_words(n0 + 1u, offset, 1u, seed);
            }
            float lo[8], hi[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t wl = comp(v[i], j >> 1), wh = comp(v[8 + i], j >> 1);
                lo[i] = (j & 1) ? bf16_hi(wl) : bf16_lo(wl);
                hi[i] = (j & 1) ? bf16_hi(wh) : bf16_lo(wh);
            }
            const uint32_t plo = encode8<SR>(lo, b, rnd0);
            const uint32_t phi = encode8<SR>(hi, b, rnd1);
            if (col_ok && r0 < rows) {
                *reinterpret_cast<uint2*>(col_codes + c * (rows / 2) + r0 / 2) = make_uint2(plo, phi);
                col_scales[c * (rows / 16) + r0 / 16] = (uint8_t)b.code;
            }
        }
    }

    // ---- tensor amax: wave reduction; the atomic is issued only when the
    // wave's max exceeds the running value already there.  Atomics on one
    // address from every wave serialize across the XCDs and would cost more
    // than the whole quantization; a max only grows, so skipping when the
    // (possibly stale) value read is already >= ours is exact.
    if (AMAX) {
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, s));
        if ((threadIdx.x & 63) == 0 && tmax != 0u) {
            unsigned int* dst = reinterpret_cast<unsigned int*>(amax_inout);
            const unsigned int seen = __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((tmax << 16) > seen) atomicMax(dst, tmax << 16);
        }
    }
}

template <bool ROW, bool COL, bool SR, bool AMAX>
void launch_quantize(const QuantizeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.cols + kTileCols - 1) / kTileCols),
                    (unsigned)((a.rows + kTileRows - 1) / kTileRows));
    hipLaunchKernelGGL((quantize_kernel<ROW, COL, SR, AMAX>), grid, dim3(kThreads), 0, stream, a.x,
                       a.rows, a.cols, a.ld, a.tensor_scale, a.seed, a.offset, a.row_codes,
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
