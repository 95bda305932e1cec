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
// with E = max(e, 1) - 22, so q * 2^E * m = q * s / 16.  Both factors live in
// one "expanded scale" dword: its fp32 exponent field carries E, its low
// half carries m as fp16 (the multiply broadcasts the low half).  A 256-entry
// table maps each scale byte to its dword; 0xFF maps to m = NaN so a NaN
// block poisons its outputs as the format requires.
//
// Tiling.  256 x 256 workgroup tile, 4 waves of 128 x 128 (4 x 4 MFMA tiles,
// 256 fp32 accumulators per lane), K chunks of 128 elements double-buffered
// in LDS: codes 64 bytes per row padded to 72 (the 8-byte fragment reads of
// 32 consecutive rows then hit distinct banks), expanded scales as
// [block][row] dwords with each block's 256 rows padded by 32 bytes (the two
// half-waves read disjoint banks).  Scales are expanded once, while staging.
//
// Pipeline.  Lane (r, h) (r = lane % 32, h = lane / 32) owns K elements
// [64h + 16b, 64h + 16b + 16) of each chunk row in block-step b (0..3): one
// 16-block, one expanded scale, two MFMA steps of 8 elements.  A and B use
// the same K order, so the dot products are unchanged.  Per MFMA step the
// kernel issues 16 MFMAs on the current fragments while it dequantizes the
// next step's fragments (2 register sets); LDS reads run one block-step
// ahead (2 sets).  Staging of chunk c + 1 (LDS writes from registers) and
// the global loads of chunk c + 2 run inside chunk c's MFMA stream, and the
// one barrier per chunk sits before its last block-step, whose operands are
// already in registers: after it the waves read chunk c + 1's first block
// while their last MFMAs of chunk c issue.
//
// Tile order.  Consecutive workgroup ids are dispatched round-robin over
// the 8 XCDs, each with its own L2.  The id is remapped so that each XCD
// walks a contiguous range of tiles, grouped 4 tile-rows at a time, so the
// 32 workgroups in flight on one XCD share 4 A panels and 8 B panels in L2.
#include "formats.hpp"
#include "kernels.hpp"
#include "quant_block.hpp"

namespace ue5m3fp4 {

namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kThreads = 256;
constexpr int kCodeStride = kBK / 2 + 8;       // 64 code bytes per row, padded to 72
constexpr int kCodesA = 0;
constexpr int kCodesB = kCodesA + kBM * kCodeStride;
constexpr int kScaleBlockStride = kBM * 4 + 32;       // one block's 256 rows, padded
constexpr int kScalesA = kCodesB + kBN * kCodeStride;  // [8 blocks][256 rows] dwords
constexpr int kScalesB = kScalesA + 8 * kScaleBlockStride;
constexpr int kStage = kScalesB + 8 * kScaleBlockStride;  // 53760 bytes
constexpr int kLut = 2 * kStage;
constexpr int kSmem = kLut + 256 * 4;
constexpr int kGroupM = 4;  // tile rows per group in the tile order
// quantizing epilogue: the 256 x 256 bf16 output tile (512 bytes per row,
// 16-byte units XOR-swizzled by the row's 16-row block) and a reciprocal
// table, reusing the staging buffers
constexpr int kQTile = kBM * kBN * 2;
constexpr int kSmemQ = kQTile + 256 * 4;

// sched_group_barrier masks
constexpr int kSchedMfma = 0x008, kSchedValu = 0x002, kSchedDsRead = 0x100,
              kSchedDsWrite = 0x200, kSchedVmemRead = 0x020;

// Expanded scale of one UE5M3 byte c = (e, f): a dword whose fp32 exponent
// field is max(e, 1) + 105 (the convert applies 2^(max(e,1) - 22)) and whose
// low half is the fp16 mantissa factor m = 8 + f (normal) or f (subnormal),
// NaN for 0xFF.  q * 2^(max(e,1)-22) * m = q * s / 16 exactly.
__device__ __forceinline__ uint32_t expand_scale(uint32_t c) {
    const uint32_t e = c >> 3, f = c & 7u;
    const uint32_t eb = e > 0u ? e : 1u;
    const _Float16 m = c == kUe5m3Nan ? (_Float16)__builtin_nanf("") : (_Float16)(float)(e > 0u ? 8u + f : f);
    uint16_t mb;
    __builtin_memcpy(&mb, &m, 2);
    return ((eb + 105u) << 23) | (uint32_t)mb;
}

// 8 E2M1 codes (one dword; element k in nibble k) -> 8 fp16 values q*s/16.
__device__ __forceinline__ f16x8_t dequant8(uint32_t w, uint32_t S) {
    const float sc = __uint_as_float(S);
    const uint16_t mb = (uint16_t)S;
    _Float16 m;
    __builtin_memcpy(&m, &mb, 2);
    const f16x2_t mm = {m, m};
    const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0) * mm;
    const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1) * mm;
    const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2) * mm;
    const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3) * mm;
    f16x8_t out;
    out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
    out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
    return out;
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

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// One 16-byte unit (32 codes) of a row's K chunk starting at k0: part p
// covers elements [k0 + 32p, k0 + 32p + 32).  Unaligned K (a multiple of 16
// only): each 16-element half is clamped into the row; halves past K are
// zeroed through their scale.
template <bool ALIGNED>
__device__ __forceinline__ u32x4 load_unit(const uint8_t* row, int64_t K, int64_t k0, int part) {
    if (ALIGNED) return *reinterpret_cast<const u32x4*>(row + k0 / 2 + 16 * part);
    const int64_t ka = min(k0 + 32 * part, K - 16), kb = min(k0 + 32 * part + 16, K - 16);
    const u32x2 x = *reinterpret_cast<const u32x2*>(row + ka / 2);
    const u32x2 y = *reinterpret_cast<const u32x2*>(row + kb / 2);
    return u32x4{x.x, x.y, y.x, y.y};
}

// The 8 scale bytes of a row's K chunk (block index b0 = k0 / 16); bytes
// past the row's kblocks blocks are 0.
template <bool ALIGNED>
__device__ __forceinline__ u32x2 load_scales(const uint8_t* row, int64_t kblocks, int64_t b0) {
    if (ALIGNED) return *reinterpret_cast<const u32x2*>(row + b0);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t v = row[min(b0 + j, kblocks - 1)];
        w[j >> 2] |= (b0 + j < kblocks ? v : 0u) << (8 * (j & 3));
    }
    return u32x2{w[0], w[1]};
}

// One lane's operands for one block-step (16 elements of K per row): the
// code dwords of its 4 A rows and 4 B rows, and their expanded scales.
struct BlockStep {
    uint2 ca[4], cb[4];
    uint32_t sa[4], sb[4];
};

struct Frags {
    f16x8_t a[4], b[4];
};

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t to_bf16(float f) {
    const __bf16 b = (__bf16)f;
    uint16_t u;
    __builtin_memcpy(&u, &b, 2);
    return u;
}

// max of |bf16| bits over the workgroup folded into *amax (fp32 bits of a
// non-negative float order as integers; NaN above +Inf): wave and LDS
// reduction, one atomic per workgroup, skipped when the running value is
// already at least as large.
__device__ __forceinline__ void amax_commit(uint32_t m, float* amax) {
    __shared__ uint32_t wave_max[kThreads / 64];
    m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    m = max(m, (uint32_t)__shfl_xor((int)m, 16));
    m = max(m, (uint32_t)__shfl_xor((int)m, 8));
    m = max(m, (uint32_t)__shfl_xor((int)m, 4));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2));
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t w = 0u;
#pragma unroll
        for (int i = 0; i < kThreads / 64; ++i) w = max(w, wave_max[i]);
        if (w != 0u) {
            unsigned int* dst = reinterpret_cast<unsigned int*>(amax);
            const unsigned int seen = __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((w << 16) > seen) atomicMax(dst, w << 16);
        }
    }
}

// Byte offset of element (row, col) of the bf16 output tile in LDS.
__device__ __forceinline__ int qtile_offset(int row, int col) {
    return row * (kBN * 2) + ((((col >> 3) ^ (row >> 4)) & 31) << 4) + ((col & 7) << 1);
}

// Row-wise block-16 quantization of the bf16 output tile held in LDS
// (blocks along N): thread t takes 16-byte unit t % 32 of tile rows
// t / 32 + 8k, eight rows per batch.  The lane pair (t, t ^ 1) shares a
// block: lane parity p computes the block scales of the batch's rows 2m + p
// and the pair swaps them (DPP), as in the stand-alone quantizer.  The
// batch's LDS reads issue together, and the path check is once per batch.
// Output row m0 + row of the M x N output, stochastic bits from orientation
// 0 of that shape.  Each unit inside the output is also written to the bf16
// output C (a wave stores two whole 512-byte tile rows; N % 16 == 0 here) and
// its magnitudes are folded into tmax.
template <bool SR>
__device__ __forceinline__ void quantize_tile_rows(const uint8_t* tile, const Ctx& ctx, const float* rlut,
                                                   const OutputQuant& q, int64_t m0, int64_t n0,
                                                   int64_t M, int64_t N, uint16_t* __restrict__ Cb,
                                                   uint32_t& tmax) {
    const int t = threadIdx.x, u = t & 31;
    const uint32_t p = t & 1;
    const int64_t gc = n0 + 8 * u;
#pragma unroll 1
    for (int batch = 0; batch < kBM / 64; ++batch) {
        u32x4 w[8];
        uint32_t hmax[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int row = (t >> 5) + 8 * (8 * batch + k);
            w[k] = *reinterpret_cast<const u32x4*>(tile + qtile_offset(row, 8 * u));
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            hmax[k] = max_abs8(w[k]);
            const int64_t gr = m0 + (t >> 5) + 8 * (8 * batch + k);
            if (gr < M && gc < N) {
                *reinterpret_cast<u32x4*>(Cb + gr * N + gc) = w[k];
                tmax = max(tmax, hmax[k]);
            }
        }
        uint32_t code[8];
        float rr[8];
        bool ok = ctx.fastK;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t mine = p ? hmax[2 * m + 1] : hmax[2 * m];
            const uint32_t other = p ? hmax[2 * m] : hmax[2 * m + 1];
            const BlockScale own = block_scale(max(mine, swap_pair(other)), ctx, rlut, ok);
            const uint32_t pc = swap_pair(own.code);
            const float pr = __uint_as_float(swap_pair(__float_as_uint(own.r)));
            code[2 * m] = p ? pc : own.code;
            rr[2 * m] = p ? pr : own.r;
            code[2 * m + 1] = p ? own.code : pc;
            rr[2 * m + 1] = p ? own.r : pr;
        }
        // both lanes of the pair take the same path; the exchange runs in
        // every lane
        const uint32_t ok_bit = ok ? 1u : 0u;
        const bool pair_ok = (ok_bit & swap_pair(ok_bit)) != 0u;
        uint32_t packed[8];
        if (__builtin_expect(pair_ok, 1)) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float v[8];
                unpack8(w[k], v);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = v[e] * rr[k];
                U32x4 rnd;
                if (SR) {
                    const int64_t gr = m0 + (t >> 5) + 8 * (8 * batch + k);
                    rnd = sr_words(((uint64_t)gr * (uint64_t)N + (uint64_t)gc) >> 3, q.offset, 0u, q.seed);
                }
                packed[k] = encode8<SR>(v, rnd);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t blk = max(hmax[k], swap_pair(hmax[k]));  // both lanes active here
                const BlockScale b = block_scale_general(blk, ctx.ts, ctx.K);
                U32x4 rnd;
                if (SR) {
                    const int64_t gr = m0 + (t >> 5) + 8 * (8 * batch + k);
                    rnd = sr_words(((uint64_t)gr * (uint64_t)N + (uint64_t)gc) >> 3, q.offset, 0u, q.seed);
                }
                packed[k] = encode8_general<SR>(w[k], b.code, b.r, rnd);
                code[k] = b.code;
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t gr = m0 + (t >> 5) + 8 * (8 * batch + k);
            if (gr < M && gc < N) {
                *reinterpret_cast<uint32_t*>(q.row_codes + gr * (N / 2) + gc / 2) = packed[k];
                if (p == 0) q.row_scales[gr * (N / 16) + gc / 16] = (uint8_t)code[k];
            }
        }
    }
}

// The bf16 output tile held in LDS written to C (used when only the
// transposed quantization is requested, so N may be any size): thread t
// copies 16-byte unit t % 32 of tile rows t / 32 + 8k, element by element at
// a ragged right edge or when N % 8 != 0; the stored magnitudes are folded
// into tmax.
__device__ __forceinline__ void store_tile(const uint8_t* tile, int64_t m0, int64_t n0, int64_t M, int64_t N,
                                           uint16_t* __restrict__ Cb, uint32_t& tmax) {
    const int t = threadIdx.x, u = t & 31;
    const int64_t gc = n0 + 8 * u;
    const bool whole = N % 8 == 0 && gc + 8 <= N;
#pragma unroll 4
    for (int k = 0; k < kBM / 8; ++k) {
        const int row = (t >> 5) + 8 * k;
        const int64_t gr = m0 + row;
        if (gr >= M || gc >= N) continue;
        const u32x4 w = *reinterpret_cast<const u32x4*>(tile + qtile_offset(row, 8 * u));
        if (whole) {
            *reinterpret_cast<u32x4*>(Cb + gr * N + gc) = w;
            tmax = max(tmax, max_abs8(w));
        } else {
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (gc + e < N) {
                    const uint16_t b = (uint16_t)(ws[e >> 1] >> (16 * (e & 1)));
                    Cb[gr * N + gc + e] = b;
                    tmax = max(tmax, (uint32_t)(b & 0x7FFFu));
                }
            }
        }
    }
}

// Transposed block-16 quantization of the tile (blocks along M): in pass p
// wave w takes 16-byte unit J = w + 4p (8 columns); lane (rb, cp) =
// (lane % 16, lane / 16) reads the 4-byte column pair cp of J over tile rows
// 16 rb .. 16 rb + 15 (64 distinct banks) and quantizes its two columns.
template <bool SR>
__device__ __forceinline__ void quantize_tile_cols(const uint8_t* tile, const Ctx& ctx, const float* rlut,
                                                   const OutputQuant& q, int64_t m0, int64_t n0,
                                                   int64_t M, int64_t N) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int rb = lane & 15, cp = lane >> 4;
    const int64_t gr = m0 + 16 * rb;
#pragma unroll 2
    for (int p = 0; p < kBN / 32; ++p) {
        const int J = wv + 4 * p;
        const int c = 8 * J + 2 * cp;  // tile column of the pair's first column
        uint32_t cw[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            cw[i] = *reinterpret_cast<const uint32_t*>(tile + qtile_offset(16 * rb + i, c));
        uint32_t m2 = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) m2 = pk_max_u16(m2, cw[i] & 0x7FFF7FFFu);
        bool ok = ctx.fastK;
        BlockScale ba = block_scale(m2 & 0xFFFFu, ctx, rlut, ok);
        BlockScale bb = block_scale(m2 >> 16, ctx, rlut, ok);
        const int64_t gca = n0 + c, gcb = gca + 1;
        U32x4 rnd[4];
        if (SR) {
            const uint64_t na = ((uint64_t)gca * (uint64_t)M + (uint64_t)gr) >> 3;
            const uint64_t nb = ((uint64_t)gcb * (uint64_t)M + (uint64_t)gr) >> 3;
            rnd[0] = sr_words(na, q.offset, 1u, q.seed);
            rnd[1] = sr_words(na + 1u, q.offset, 1u, q.seed);
            rnd[2] = sr_words(nb, q.offset, 1u, q.seed);
            rnd[3] = sr_words(nb + 1u, q.offset, 1u, q.seed);
        }
        uint32_t pa[2], pb[2];
        if (__builtin_expect(ok, 1)) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float va[8], vb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    va[i] = bf16_lo(cw[8 * hh + i]) * ba.r;
                    vb[i] = bf16_hi(cw[8 * hh + i]) * bb.r;
                }
                pa[hh] = encode8<SR>(va, rnd[hh]);
                pb[hh] = encode8<SR>(vb, rnd[2 + hh]);
            }
        } else {
            ba = block_scale_general(m2 & 0xFFFFu, ctx.ts, ctx.K);
            bb = block_scale_general(m2 >> 16, ctx.ts, ctx.K);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                uint32_t la[4], lb[4];  // per-column words of 8 rows
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t w0 = cw[8 * hh + 2 * i], w1 = cw[8 * hh + 2 * i + 1];
                    la[i] = (w0 & 0xFFFFu) | (w1 << 16);
                    lb[i] = (w0 >> 16) | (w1 & 0xFFFF0000u);
                }
                pa[hh] = encode8_general<SR>(u32x4{la[0], la[1], la[2], la[3]}, ba.code, ba.r, rnd[hh]);
                pb[hh] = encode8_general<SR>(u32x4{lb[0], lb[1], lb[2], lb[3]}, bb.code, bb.r, rnd[2 + hh]);
            }
        }
        if (gr < M) {
            if (gca < N) {
                *reinterpret_cast<u32x2*>(q.col_codes + gca * (M / 2) + gr / 2) = u32x2{pa[0], pa[1]};
                q.col_scales[gca * (M / 16) + gr / 16] = (uint8_t)ba.code;
            }
            if (gcb < N) {
                *reinterpret_cast<u32x2*>(q.col_codes + gcb * (M / 2) + gr / 2) = u32x2{pb[0], pb[1]};
                q.col_scales[gcb * (M / 16) + gr / 16] = (uint8_t)bb.code;
            }
        }
    }
}

template <bool ALIGNED, bool BF16, bool QUANT>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, const float* __restrict__ b_ts, int64_t M, int64_t N,
    int64_t K, float* __restrict__ C, uint16_t* __restrict__ Cb, float* __restrict__ amax,
    OutputQuant q) {
    __shared__ __align__(16) uint8_t smem[QUANT ? kSmemQ : kSmem];
    uint32_t* lut = reinterpret_cast<uint32_t*>(smem + kLut);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 31, h = lane >> 5;

    lut[tid] = expand_scale((uint32_t)tid);

    int tm, tn;
    tile_of((int)((M + kBM - 1) / kBM), (int)((N + kBN - 1) / kBN), tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t kbytes = K / 2, kblocks = K / 16;
    const int nchunks = (int)((K + kBK - 1) / kBK);

    // ---- staging: global -> registers -> LDS.  Every load is unconditional
    // (rows clamped into the operand, K offsets into the row); rows outside
    // the operand and blocks past K get scale byte 0, whose factor m = 0 makes
    // them dequantize to exactly 0.  Thread tid stages 16-byte part tid % 4 of
    // rows srow + 64 i (i = 0..3) of each operand's 256 x 64 code bytes, and
    // the 8 scale bytes of row tid.  A wave stores 16 rows, 4 rows x 4 parts
    // per 16 lanes.  The LDS takes each 8-byte half of such a store 16 lanes
    // per cycle over 32 four-byte banks (measured: the bank-conflict count
    // follows this model exactly); at the 18-dword row stride rows o, o + 1,
    // o + 8 and o + 9 start 0, 18, 16 and 2 banks apart, so a 16-lane group
    // holding them writes each bank once, where 4 consecutive rows put two
    // dwords on half the banks.  A wave still loads 16 whole 64-byte row
    // chunks from global memory.  The staging registers are plain vector
    // values (no arrays), so they stay in VGPRs.
    u32x4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
    u32x2 rsa, rsb;
    u32x8 ea, eb;
    const bool a_valid = m0 + tid < M, b_valid = n0 + tid < N;
    const int64_t a_srow = a_valid ? m0 + tid : M - 1, b_srow = b_valid ? n0 + tid : N - 1;
    const int sq = (tid >> 2) & 15, spart = tid & 3;  // rows srow + 64 i, part spart
    const int srow = 16 * (tid >> 6) + 2 * (sq >> 2) + (sq & 1) + 8 * ((sq >> 1) & 1);
    const uint8_t* a_rows[4];
    const uint8_t* b_rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_rows[i] = a_codes + min(m0 + srow + 64 * i, M - 1) * kbytes;
        b_rows[i] = b_codes + min(n0 + srow + 64 * i, N - 1) * kbytes;
    }
    const uint8_t* a_srow_p = a_scales + a_srow * kblocks;
    const uint8_t* b_srow_p = b_scales + b_srow * kblocks;

    auto gload = [&](int chunk) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)chunk * kBK;
        ra0 = load_unit<ALIGNED>(a_rows[0], K, k0, spart);
        ra1 = load_unit<ALIGNED>(a_rows[1], K, k0, spart);
        ra2 = load_unit<ALIGNED>(a_rows[2], K, k0, spart);
        ra3 = load_unit<ALIGNED>(a_rows[3], K, k0, spart);
        rb0 = load_unit<ALIGNED>(b_rows[0], K, k0, spart);
        rb1 = load_unit<ALIGNED>(b_rows[1], K, k0, spart);
        rb2 = load_unit<ALIGNED>(b_rows[2], K, k0, spart);
        rb3 = load_unit<ALIGNED>(b_rows[3], K, k0, spart);
        rsa = load_scales<ALIGNED>(a_srow_p, kblocks, k0 / 16) & (a_valid ? ~0u : 0u);
        rsb = load_scales<ALIGNED>(b_srow_p, kblocks, k0 / 16) & (b_valid ? ~0u : 0u);
    };
    auto lstore_codes = [&](uint8_t* base) __attribute__((always_inline)) {
        // rows are 8-byte aligned (72-byte stride): two 8-byte stores per unit
        uint8_t* pa = base + kCodesA + srow * kCodeStride + 16 * spart;
        uint8_t* pb = base + kCodesB + srow * kCodeStride + 16 * spart;
        auto st = [](uint8_t* p, u32x4 v) __attribute__((always_inline)) {
            *reinterpret_cast<u32x2*>(p) = v.xy;
            *reinterpret_cast<u32x2*>(p + 8) = v.zw;
        };
        st(pa + 0 * 64 * kCodeStride, ra0);
        st(pa + 1 * 64 * kCodeStride, ra1);
        st(pa + 2 * 64 * kCodeStride, ra2);
        st(pa + 3 * 64 * kCodeStride, ra3);
        st(pb + 0 * 64 * kCodeStride, rb0);
        st(pb + 1 * 64 * kCodeStride, rb1);
        st(pb + 2 * 64 * kCodeStride, rb2);
        st(pb + 3 * 64 * kCodeStride, rb3);
    };
    auto lut_fetch = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t wa = j < 4 ? rsa.x : rsa.y, wb = j < 4 ? rsb.x : rsb.y;
            ea[j] = lut[(wa >> (8 * (j & 3))) & 0xFFu];
            eb[j] = lut[(wb >> (8 * (j & 3))) & 0xFFu];
        }
    };
    auto lstore_scales = [&](uint8_t* base) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            *reinterpret_cast<uint32_t*>(base + kScalesA + j * kScaleBlockStride + tid * 4) = ea[j];
            *reinterpret_cast<uint32_t*>(base + kScalesB + j * kScaleBlockStride + tid * 4) = eb[j];
        }
    };

    // ---- per-lane LDS read offsets.  Lane (r, h) covers K elements
    // [64h + 16b, 64h + 16b + 16) of every chunk row in block-step b (its
    // block 4h + b), 8 of them per MFMA step.
    const int a_code_off = kCodesA + (wm * 128 + r) * kCodeStride + 32 * h;
    const int b_code_off = kCodesB + (wn * 128 + r) * kCodeStride + 32 * h;
    const int a_sc_off = kScalesA + 4 * h * kScaleBlockStride + (wm * 128 + r) * 4;
    const int b_sc_off = kScalesB + 4 * h * kScaleBlockStride + (wn * 128 + r) * 4;

    auto read_bs = [&](BlockStep& bs, const uint8_t* base, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bs.ca[g] = *reinterpret_cast<const uint2*>(base + a_code_off + g * 32 * kCodeStride + 8 * b);
            bs.cb[g] = *reinterpret_cast<const uint2*>(base + b_code_off + g * 32 * kCodeStride + 8 * b);
            bs.sa[g] = *reinterpret_cast<const uint32_t*>(base + a_sc_off + b * kScaleBlockStride + g * 128);
            bs.sb[g] = *reinterpret_cast<const uint32_t*>(base + b_sc_off + b * kScaleBlockStride + g * 128);
        }
    };
    auto dequant = [&](Frags& f, const BlockStep& bs, int t1) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f.a[g] = dequant8(t1 ? bs.ca[g].y : bs.ca[g].x, bs.sa[g]);
            f.b[g] = dequant8(t1 ? bs.cb[g].y : bs.cb[g].x, bs.sb[g]);
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (nchunks > 0) {
        __syncthreads();  // table visible
        gload(0);
        lut_fetch();
        lstore_codes(smem);
        lstore_scales(smem);
        gload(min(1, nchunks - 1));
        __syncthreads();

        BlockStep bsr[2];
        Frags fr[2];
        read_bs(bsr[0], smem, 0);
        dequant(fr[0], bsr[0], 0);

        for (int c = 0; c < nchunks; ++c) {
            uint8_t* cur = smem + (c & 1) * kStage;
            uint8_t* nxt = smem + ((c + 1) & 1) * kStage;
#pragma unroll
            for (int J = 0; J < 8; ++J) {
                const Frags& f = fr[J & 1];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
                // LDS reads one block-step ahead; the next chunk's first
                // block-step only after the barrier
                if (J == 0 || J == 2 || J == 4) read_bs(bsr[((J >> 1) + 1) & 1], cur, (J >> 1) + 1);
                if (J == 6) read_bs(bsr[0], nxt, 0);
                // staging of chunk c + 1 into the other buffer, loads of c + 2
                if (J == 1) {
                    lstore_codes(nxt);
                    lut_fetch();
                    gload(min(c + 2, nchunks - 1));
                }
                if (J == 2) lstore_scales(nxt);
                // fragments of the next MFMA step
                dequant(fr[(J + 1) & 1], bsr[((J + 1) >> 1) & 1], (J + 1) & 1);
                // interleave: each MFMA followed by up to 5 VALU, 2 LDS and
                // 2 global-load instructions, so the dequantization of the
                // next step issues while the matrix core works
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedValu, 5, 0);
                    if (q < 10) __builtin_amdgcn_sched_group_barrier(kSchedDsRead | kSchedDsWrite, 2, 0);
                    if (q < 8) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 2, 0);
                }
                if (J == 5) __syncthreads();
            }
        }
    }

    // ---- epilogue: C = (acc * 256 tsA) * tsB, stored as fp32, or rounded to
    // bf16 with the tensor amax of the stored values folded into *amax.
    // Accumulator register e of lane (r, h) holds row 8 * (e / 4) + 4 * h +
    // e % 4, column r of a 32 x 32 tile.  With QUANT the bf16 values also go
    // to an LDS copy of the output tile, which is then quantized block-16
    // (row-wise and/or transposed) under the output's tensor scale.
    const float sa256 = *a_ts * 256.0f, tsb = *b_ts;
    const int64_t row0 = m0 + wm * 128 + 4 * h, col0 = n0 + wn * 128 + r;
    const int trow0 = wm * 128 + 4 * h, tcol0 = wn * 128 + r;  // within the tile
    uint32_t tmax = 0u;  // max |bf16| bits stored by this lane
    if (QUANT) {
        // The bf16 tile goes to LDS only (the staging buffers are free once
        // every wave is past its last MFMA); the passes below write it to C
        // from there, 16 bytes per lane, and quantize it.  Values outside
        // the output share no 16-block with stored ones (the quantized axes
        // are multiples of 16).
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<uint16_t*>(
                        smem + qtile_offset(trow0 + i * 32 + 8 * (e >> 2) + (e & 3), tcol0 + j * 32)) =
                        to_bf16((acc[i][j][e] * sa256) * tsb);
        float* rlut = reinterpret_cast<float*>(smem + kQTile);
        const Ctx ctx = make_ctx(*q.ts);
        rlut[tid] = q.stochastic ? rcp_entry<true>((uint32_t)tid, ctx.ts) : rcp_entry<false>((uint32_t)tid, ctx.ts);
        __syncthreads();  // tile and table visible
        if (q.row_codes) {
            if (q.stochastic) quantize_tile_rows<true>(smem, ctx, rlut, q, m0, n0, M, N, Cb, tmax);
            else quantize_tile_rows<false>(smem, ctx, rlut, q, m0, n0, M, N, Cb, tmax);
        } else {
            store_tile(smem, m0, n0, M, N, Cb, tmax);
        }
        if (q.col_codes) {
            if (q.stochastic) quantize_tile_cols<true>(smem, ctx, rlut, q, m0, n0, M, N);
            else quantize_tile_cols<false>(smem, ctx, rlut, q, m0, n0, M, N);
        }
    } else if (m0 + kBM <= M && n0 + kBN <= N) {
        // interior tile: one row pointer per accumulator row, the 4 column
        // tiles at immediate offsets
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t off = (row0 + i * 32 + 8 * (e >> 2) + (e & 3)) * N + col0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v = (acc[i][j][e] * sa256) * tsb;
                    if (BF16) {
                        const uint16_t b = to_bf16(v);
                        Cb[off + j * 32] = b;
                        tmax = max(tmax, (uint32_t)(b & 0x7FFFu));
                    } else {
                        C[off + j * 32] = v;
                    }
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t col = col0 + j * 32;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = row0 + i * 32 + 8 * (e >> 2) + (e & 3);
                    const float v = (acc[i][j][e] * sa256) * tsb;
                    if (row < M && col < N) {
                        if (BF16) {
                            const uint16_t b = to_bf16(v);
                            Cb[row * N + col] = b;
                            tmax = max(tmax, (uint32_t)(b & 0x7FFFu));
                        } else {
                            C[row * N + col] = v;
                        }
                    }
                }
            }
    }
    if (BF16 && amax != nullptr) amax_commit(tmax, amax);
}

}  // namespace

template <bool ALIGNED, bool BF16, bool QUANT>
void launch_gemm(const GemmArgs& g, hipStream_t stream) {
    const int64_t tiles = ((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
    hipLaunchKernelGGL((gemm_nt_kernel<ALIGNED, BF16, QUANT>), dim3((unsigned)tiles), dim3(kThreads), 0,
                       stream, g.a_codes, g.a_scales, g.a_ts, g.b_codes, g.b_scales, g.b_ts, g.M, g.N, g.K,
                       g.c, g.c_bf16, g.amax, g.q);
}

void launch_gemm_nt(const GemmArgs& g, hipStream_t stream) {
    const bool aligned = g.K % kBK == 0;
    if (g.c_bf16 && g.q.ts) {
        if (aligned) launch_gemm<true, true, true>(g, stream);
        else launch_gemm<false, true, true>(g, stream);
    } else if (g.c_bf16) {
        if (aligned) launch_gemm<true, true, false>(g, stream);
        else launch_gemm<false, true, false>(g, stream);
    } else {
        if (aligned) launch_gemm<true, false, false>(g, stream);
        else launch_gemm<false, false, false>(g, stream);
    }
}

}  // namespace ue5m3fp4
