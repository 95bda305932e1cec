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
// the same bf16 tile, so the input is read from HBM once.
//
// Work decomposition.  A 256-thread workgroup owns a TR x 256 tile (TR = 32
// or 64 rows).  Thread t loads 16-byte unit t % 32 (8 columns) of tile rows
// t / 32 + 8k: a wave reads 2 rows x 512 bytes per load, all loads issued
// back to back (edge addresses are clamped into the tensor; the duplicated
// values never reach an output).
//  - Row-wise pass, from registers: a 16-element row block spans a lane pair
//    (lane ^ 1, one DPP swap); the pair splits the block-scale computations
//    and swaps the results.  A wave writes 2 rows x 128 bytes of codes.
//  - Transposed pass, through LDS: the bf16 tile is written once to an
//    XOR-swizzled LDS buffer, and each lane reads one 4-byte column pair over
//    a 16-row block (conflict-free), quantizing two column blocks.
//  - Tile order: each XCD takes a contiguous range of an order that runs down
//    bands of 256 rows column by column, so tiles sharing 128-byte lines of
//    the transposed output meet in one L2.
//  - Cache policy: x is read once, so its loads are non-temporal (streamed
//    past the caches instead of displacing the partial lines of transposed
//    codes and scales that neighbouring tiles are still filling in L2), and so
//    are the row-wise code stores, whose wave stores cover whole lines.  The
//    partial-line outputs (transposed codes, all scale bytes) stay cached:
//    written non-temporally they reach HBM unmerged (measured 1.2-2x slower).
//
// Arithmetic per block and element: quant_block.hpp.
#include "formats.hpp"
#include "kernels.hpp"
#include "quant_block.hpp"

namespace ue5m3fp4 {

namespace {

// Tile shape: TR (32 or 64) rows x 256 columns per 256-thread workgroup.
// Row-only calls use 32-row tiles (more resident workgroups hide more load
// latency); calls with the transposed output use 64-row tiles (32-byte runs
// of transposed codes per column instead of 16).
template <int TR>
struct Shape {
    static constexpr int kTileRows = TR;
    static constexpr int kRowsPerThread = TR / 8;        // tile rows t / 32 + 8k
    static constexpr int kRowBlocks = TR / 16;           // 16-row blocks per column
    static constexpr int kPairsPerWave = 64 / kRowBlocks;  // column pairs per wave and pass
    static constexpr int kColPasses = 128 / (4 * kPairsPerWave);
    static constexpr int kBand = 256 / TR;               // tiles sharing a transposed line
    static_assert(TR == 32 || TR == 64, "tile height");
};
constexpr int kTileCols = 256;
constexpr int kThreads = 256;
constexpr int kLdsRowBytes = kTileCols * 2;  // one bf16 tile row

// LDS position of 16-byte unit u (8 columns) of tile row `row`: the unit
// index is XORed with the row's 16-row block times 16 / kRowBlocks, so the
// column pass (lanes over kRowBlocks row blocks x kPairsPerWave column pairs)
// reads 64 distinct banks.
template <int TR>
__device__ __forceinline__ int lds_offset(int row, int u) {
    constexpr int kRowBlocks = Shape<TR>::kRowBlocks;
    return row * kLdsRowBytes + ((u ^ (((row >> 4) & (kRowBlocks - 1)) * (16 / kRowBlocks))) << 4);
}

// Workgroup id -> tile origin.  Workgroups are dispatched round-robin over
// the 8 XCDs, each with its own L2.  Each XCD takes a contiguous range of a
// tile order that runs down bands of kBand tile rows (256 rows), column by
// column: the tiles of a band column share the 128-byte lines of the
// transposed output and the 8 neighbouring band columns share the lines of the
// row-wise scales, so their partial lines meet in one L2 while resident and
// reach HBM as whole lines.
template <int TR>
__device__ __forceinline__ void tile_of(uint32_t tiles_r, uint32_t tiles_c, int64_t& R0, int64_t& C0) {
    constexpr int kBand = Shape<TR>::kBand, kTileRows = TR;
    const uint32_t n = tiles_r * tiles_c;
    uint32_t j = blockIdx.x;
    const uint32_t per_xcd = n / 8;
    if (j < per_xcd * 8) j = (j % 8) * per_xcd + j / 8;  // the tail keeps its id
    const uint32_t band = j / (kBand * tiles_c);
    const uint32_t rem = j - band * kBand * tiles_c;
    const uint32_t h = min((uint32_t)kBand, tiles_r - kBand * band);  // rows in this band
    const uint32_t tc = rem / h, tr = kBand * band + (rem - tc * h);
    R0 = (int64_t)tr * kTileRows;
    C0 = (int64_t)tc * kTileCols;
}

// Tensor amax of a workgroup (bf16 magnitude bits of each thread's max)
// folded into *amax (fp32 bits; a non-negative float orders as its bits, and
// a NaN's bits above +Inf).  Wave reduction, then the workgroup's waves meet
// in LDS and one lane issues the atomic -- only when the workgroup's max
// exceeds the (possibly stale) running value: same-address atomics
// serialize across the XCDs, and a max only grows, so skipping is exact.
__device__ __forceinline__ void amax_commit(uint32_t tmax, float* amax) {
    __shared__ uint32_t wave_max[16];
    tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, 32));
    tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, 16));
    tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, 8));
    tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, 4));
    tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, 2));
    tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, 1));
    const int wv = threadIdx.x >> 6, waves = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) wave_max[wv] = tmax;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = 0u;
        for (int i = 0; i < waves; ++i) m = max(m, wave_max[i]);
        if (m != 0u) {
            unsigned int* dst = reinterpret_cast<unsigned int*>(amax);
            const unsigned int seen = __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((m << 16) > seen) atomicMax(dst, m << 16);
        }
    }
}

// Amax-only pass (the bootstrap before the first refresh, and the first step
// of current-tensor scaling): a grid-stride max over |x| with 16-byte loads,
// four in flight per thread, one atomic per workgroup.
__global__ __launch_bounds__(1024) void amax_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ld,
                                                    float* __restrict__ amax) {
    const int64_t units_row = cols / 8;  // 16-byte units per row (cols % 16 == 0)
    const int64_t units = rows * units_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t m = 0u;
    auto unit_max = [&](int64_t i) __attribute__((always_inline)) {
        const int64_t r = ld == cols ? 0 : i / units_row;
        const int64_t off = ld == cols ? i * 8 : r * ld + (i - r * units_row) * 8;
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off));
        const uint32_t p = pk_max_u16(pk_max_u16(w.x & 0x7FFF7FFFu, w.y & 0x7FFF7FFFu),
                                      pk_max_u16(w.z & 0x7FFF7FFFu, w.w & 0x7FFF7FFFu));
        return p;
    };
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t p2 = 0u;
    for (; i + 3 * stride < units; i += 4 * stride) {
        const uint32_t a = unit_max(i), b = unit_max(i + stride);
        const uint32_t c = unit_max(i + 2 * stride), d = unit_max(i + 3 * stride);
        p2 = pk_max_u16(p2, pk_max_u16(pk_max_u16(a, b), pk_max_u16(c, d)));
    }
    for (; i < units; i += stride) p2 = pk_max_u16(p2, unit_max(i));
    m = max(p2 & 0xFFFFu, p2 >> 16);
    amax_commit(m, amax);
}

// current_amax (nullable): current-tensor scaling -- the tensor scale is
// fp32(amax / fp32(6 max_safe)) of this tensor's amax (from the amax pass
// before), or *tensor_scale as passed when that amax is 0 or not finite, and
// workgroup 0 stores it to *tensor_scale.  Every workgroup computes the same
// value, and one that reads *tensor_scale after the store reads it only in
// the case where the store wrote back the value it found.
// W32 (stochastic rounding only): every call number of the launch is below
// 2^32 (fewer than 2^35 elements), so the counter's second word is 0 and
// sr_words32 applies.
template <int TR, bool ROW, bool COL, bool SR, bool AMAX, bool W32>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    float* tensor_scale, uint64_t seed, uint32_t offset,
    uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
    uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales,
    float* __restrict__ amax_inout, const float* __restrict__ current_amax, float max_safe) {
    using S = Shape<TR>;
    constexpr int kTileRows = S::kTileRows, kRowsPerThread = S::kRowsPerThread,
                  kRowBlocks = S::kRowBlocks, kPairsPerWave = S::kPairsPerWave,
                  kColPasses = S::kColPasses;
    __shared__ __align__(16) uint8_t tile[COL ? kTileRows * kLdsRowBytes : 16];
    __shared__ float rlut[(ROW || COL) ? 256 : 1];
    const int t = threadIdx.x;
    int64_t R0, C0;
    tile_of<TR>((uint32_t)((rows + kTileRows - 1) / kTileRows), (uint32_t)((cols + kTileCols - 1) / kTileCols),
            R0, C0);
    const bool interior = R0 + kTileRows <= rows && C0 + kTileCols <= cols;

    // ---- loads: thread t owns 16-byte unit u = t % 32 (8 columns) of tile
    // rows t / 32 + 8k, k < kRowsPerThread; a wave reads 2 rows x 512 bytes
    // per load.
    // Loads are unconditional: addresses outside the tensor are clamped to
    // its last row / last 8 columns.  The duplicated values never reach an
    // output (cols % 16 == 0, and rows % 16 == 0 when the transposed output
    // is written) and cannot raise the tensor amax.
    const int u = t & 31, rbase = t >> 5;
    const int64_t c0 = C0 + 8 * u;
    const bool col_ok = c0 < cols;
    u32x4 w[kRowsPerThread];
    if (interior) {
        // one base address, then a stride common to the launch
        const uint16_t* src = x + (R0 + rbase) * ld + c0;
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k)
            w[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(8 * k) * ld));
    } else {
        const uint16_t* src = x + (col_ok ? c0 : cols - 8);
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k) {
            const int64_t r = min(R0 + rbase + 8 * k, rows - 1);
            w[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + r * ld));
        }
    }

    // Random words of the row-wise output (stochastic rounding): they depend
    // on coordinates only -- call n of row R0 + rbase + 8k is n0 + k * cols.
    // Row-only calls draw them here, while the loads are in flight; with the
    // transposed output as well, the 32 registers they would hold meanwhile
    // cost a resident workgroup, so they are drawn where they are used.
    // With W32 the counter's second word is 0 (sr_words32).
    const uint64_t n0 = ((uint64_t)(R0 + rbase) * (uint64_t)cols + (uint64_t)c0) >> 3;
    auto row_words = [&](int k) {
        const uint64_t n = n0 + (uint64_t)k * (uint64_t)cols;
        if constexpr (W32) return sr_words32((uint32_t)n, offset, 0u, seed);
        else return sr_words(n, offset, 0u, seed);
    };
    constexpr bool kEarlyWords = SR && ROW && !COL;
    U32x4 early[kEarlyWords ? kRowsPerThread : 1];
    if constexpr (kEarlyWords) {
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k) early[k] = row_words(k);
    }

    Ctx ctx{0.0f, 0.0f, 0.0f, false, false};
    if (ROW || COL) {
        ctx.ts = *tensor_scale;
        if (current_amax != nullptr) {
            const float a = *current_amax;
            if ((__float_as_uint(a) & 0x7F800000u) != 0x7F800000u && a > 0.0f) ctx.ts = a / (6.0f * max_safe);
            if (blockIdx.x == 0 && t == 0) *tensor_scale = ctx.ts;
        }
        ctx.K = 6.0f * ctx.ts;
        ctx.yK = 1.0f / ctx.K;
        ctx.fastK = ctx.K >= 0x1p-100f && ctx.K <= 0x1p100f;
        ctx.tinyOK = ctx.K >= 1.0f;
        rlut[t] = rcp_entry<SR>((uint32_t)t, ctx.ts);
    }

    // ---- row half-block amax (bf16 magnitude bits; NaN sorts above Inf)
    uint32_t hmax[kRowsPerThread];
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
        const uint32_t m = pk_max_u16(pk_max_u16(w[k].x & 0x7FFF7FFFu, w[k].y & 0x7FFF7FFFu),
                                      pk_max_u16(w[k].z & 0x7FFF7FFFu, w[k].w & 0x7FFF7FFFu));
        hmax[k] = max(m & 0xFFFFu, m >> 16);
    }
    uint32_t tmax = 0u;
    if (AMAX) {
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k) tmax = max(tmax, hmax[k]);
    }

    if (COL) {
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k)
            *reinterpret_cast<u32x4*>(tile + lds_offset<TR>(rbase + 8 * k, u)) = w[k];
    }
    if (ROW || COL) __syncthreads();  // reciprocal table (and tile) visible

    // ---- row-wise output.  The lane pair (t, t ^ 1) shares each 16-block;
    // lane parity p computes the scales of rows k = 2m + p and the pair swaps
    // them.
    if (ROW) {
        const uint32_t p = t & 1;
        uint32_t code[kRowsPerThread];
        float rr[kRowsPerThread];
        bool ok = ctx.fastK;
#pragma unroll
        for (int m = 0; m < kRowsPerThread / 2; ++m) {
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
        // both lanes of the pair must take the same path; the exchange runs in
        // every lane (a short-circuit && would skip it where ok is false)
        const uint32_t ok_bit = ok ? 1u : 0u;
        const bool pair_ok = (ok_bit & swap_pair(ok_bit)) != 0u;
        uint32_t packed[kRowsPerThread];
        if (__builtin_expect(pair_ok, 1)) {
#pragma unroll
            for (int k = 0; k < kRowsPerThread; ++k) {
                float v[8];
                unpack8(w[k], v);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = v[e] * rr[k];
                U32x4 rnd;
                if constexpr (kEarlyWords) rnd = early[k];
                else if (SR) rnd = row_words(k);
                packed[k] = encode8<SR>(v, rnd);
            }
        } else {
#pragma unroll
            for (int k = 0; k < kRowsPerThread; ++k) {
                const uint32_t blk = max(hmax[k], swap_pair(hmax[k]));  // both lanes active here
                const BlockScale b = block_scale_general(blk, ctx.ts, ctx.K);
                U32x4 rnd;
                if constexpr (kEarlyWords) rnd = early[k];
                else if (SR) rnd = row_words(k);
                packed[k] = encode8_general<SR>(w[k], b.code, b.r, rnd);
                code[k] = b.code;
            }
        }
        uint8_t* pc = row_codes + (R0 + rbase) * (cols / 2) + c0 / 2;
        uint8_t* ps = row_scales + (R0 + rbase) * (cols / 16) + c0 / 16;
        const int64_t cstep = 8 * (cols / 2), sstep = 8 * (cols / 16);
        if (interior) {
            // both lanes of a pair store the block's scale byte (same value)
#pragma unroll
            for (int k = 0; k < kRowsPerThread; ++k) {
                __builtin_nontemporal_store(packed[k], reinterpret_cast<uint32_t*>(pc + k * cstep));
                ps[k * sstep] = (uint8_t)code[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < kRowsPerThread; ++k) {
                if (col_ok && R0 + rbase + 8 * k < rows) {
                    *reinterpret_cast<uint32_t*>(pc + k * cstep) = packed[k];
                    if (p == 0) ps[k * sstep] = (uint8_t)code[k];
                }
            }
        }
    }

    // ---- transposed output: lane (rb, cp) = (lane % kRowBlocks,
    // lane / kRowBlocks) of wave w quantizes columns 2j, 2j + 1
    // (j = kPairsPerWave (w + 4 pass) + cp) over tile rows 16 rb .. 16 rb + 15:
    // one 16-block per column.  The kRowBlocks lanes of a column write its
    // tile rows as kTileRows / 2 contiguous bytes.
    if (COL) {
        const int lane = t & 63, wv = t >> 6;
        const int rb = lane % kRowBlocks, cp = lane / kRowBlocks;
        const int64_t r0 = R0 + 16 * rb;
#pragma unroll 1
        for (int pass = 0; pass < kColPasses; ++pass) {
            const int j = kPairsPerWave * (wv + 4 * pass) + cp;  // column pair within the tile
            const int64_t ca = C0 + 2 * j;
            uint32_t cw[16];
            const uint8_t* src = tile + lds_offset<TR>(16 * rb, j >> 2) + 4 * (j & 3);
#pragma unroll
            for (int i = 0; i < 16; ++i) cw[i] = *reinterpret_cast<const uint32_t*>(src + i * kLdsRowBytes);
            uint32_t m2 = 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) m2 = pk_max_u16(m2, cw[i] & 0x7FFF7FFFu);
            bool ok = ctx.fastK;
            const BlockScale ba = block_scale(m2 & 0xFFFFu, ctx, rlut, ok);
            const BlockScale bb = block_scale(m2 >> 16, ctx, rlut, ok);
            uint32_t pa[2], pb[2];
            U32x4 rnd[4];
            if (SR) {
                const uint64_t na = ((uint64_t)ca * (uint64_t)rows + (uint64_t)r0) >> 3;
                const uint64_t nb = na + (uint64_t)(rows >> 3);
                if constexpr (W32) {
                    rnd[0] = sr_words32((uint32_t)na, offset, 1u, seed);
                    rnd[1] = sr_words32((uint32_t)na + 1u, offset, 1u, seed);
                    rnd[2] = sr_words32((uint32_t)nb, offset, 1u, seed);
                    rnd[3] = sr_words32((uint32_t)nb + 1u, offset, 1u, seed);
                } else {
                    rnd[0] = sr_words(na, offset, 1u, seed);
                    rnd[1] = sr_words(na + 1u, offset, 1u, seed);
                    rnd[2] = sr_words(nb, offset, 1u, seed);
                    rnd[3] = sr_words(nb + 1u, offset, 1u, seed);
                }
            }
            uint32_t code_a = ba.code, code_b = bb.code;
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
                const BlockScale ga = block_scale_general(m2 & 0xFFFFu, ctx.ts, ctx.K);
                const BlockScale gb = block_scale_general(m2 >> 16, ctx.ts, ctx.K);
                code_a = ga.code;
                code_b = gb.code;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    // words holding (column a, column b) of 8 rows -> per-column words
                    uint32_t la[4], lb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t w0 = cw[8 * hh + 2 * i], w1 = cw[8 * hh + 2 * i + 1];
                        la[i] = (w0 & 0xFFFFu) | (w1 << 16);
                        lb[i] = (w0 >> 16) | (w1 & 0xFFFF0000u);
                    }
                    pa[hh] = encode8_general<SR>(u32x4{la[0], la[1], la[2], la[3]}, ga.code, ga.r, rnd[hh]);
                    pb[hh] = encode8_general<SR>(u32x4{lb[0], lb[1], lb[2], lb[3]}, gb.code, gb.r, rnd[2 + hh]);
                }
            }
            if (interior || (ca < cols && r0 < rows)) {
                *reinterpret_cast<u32x2*>(col_codes + ca * (rows / 2) + r0 / 2) = u32x2{pa[0], pa[1]};
                *reinterpret_cast<u32x2*>(col_codes + (ca + 1) * (rows / 2) + r0 / 2) = u32x2{pb[0], pb[1]};
                col_scales[ca * (rows / 16) + r0 / 16] = (uint8_t)code_a;
                col_scales[(ca + 1) * (rows / 16) + r0 / 16] = (uint8_t)code_b;
            }
        }
    }

    // ---- tensor amax: one atomic per workgroup
    if (AMAX) amax_commit(tmax, amax_inout);
}

// Stochastic-rounding call numbers fit 32 bits: fewer than 2^35 elements.
bool words32(int64_t rows, int64_t cols) { return (uint64_t)rows * (uint64_t)cols < ((uint64_t)1 << 35); }

template <bool ROW, bool COL, bool SR, bool AMAX, bool W32>
void launch_quantize_w(const QuantizeArgs& a, hipStream_t stream) {
    constexpr int TR = COL ? 64 : 32;
    const int64_t tiles = ((a.cols + kTileCols - 1) / kTileCols) * ((a.rows + TR - 1) / TR);
    hipLaunchKernelGGL((quantize_kernel<TR, ROW, COL, SR, AMAX, W32>), dim3((unsigned)tiles), dim3(kThreads), 0,
                       stream, a.x, a.rows, a.cols, a.ld, const_cast<float*>(a.tensor_scale), a.seed, a.offset,
                       a.row_codes, a.row_scales, a.col_codes, a.col_scales, a.amax_inout, a.current_amax, a.max_safe);
}

template <bool ROW, bool COL, bool SR, bool AMAX>
void launch_quantize(const QuantizeArgs& a, hipStream_t stream) {
    if constexpr (SR) {
        if (words32(a.rows, a.cols)) return launch_quantize_w<ROW, COL, SR, AMAX, true>(a, stream);
    }
    launch_quantize_w<ROW, COL, SR, AMAX, false>(a, stream);
}

// Compute units of the current device (the runtime caches the attribute).
int cu_count() {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
        return c;
    return 256;
}

void launch_amax(const QuantizeArgs& a, hipStream_t s) {
    const int64_t units = a.rows * (a.cols / 8);
    const int64_t want = (units + 4 * 1024 - 1) / (4 * 1024);
    const int64_t grid = max((int64_t)1, min(want, (int64_t)cu_count() * 2));
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)grid), dim3(1024), 0, s, a.x, a.rows, a.cols, a.ld,
                       a.amax_inout);
}

// Streaming reference (measurement only, no quantization arithmetic): the
// byte traffic of a quantize call as contiguous streams -- per 16-element
// block, 32 bytes read, then 8 bytes of "codes" and 1 "scale" byte written
// per output (the codes are XORs of the input words).  Its time is what HBM
// gives for the quantizer's read/write mix without the quantizer's access
// pattern or arithmetic.
__global__ __launch_bounds__(256) void stream_reference_kernel(const u32x4* __restrict__ x, int64_t blocks,
                                                               u32x2* __restrict__ c0, uint8_t* __restrict__ s0,
                                                               u32x2* __restrict__ c1, uint8_t* __restrict__ s1) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < blocks; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(x + 2 * i), b = __builtin_nontemporal_load(x + 2 * i + 1);
        const uint32_t h = a.x ^ a.y ^ a.z ^ a.w, g = b.x ^ b.y ^ b.z ^ b.w;
        __builtin_nontemporal_store(u32x2{h, g}, c0 + i);
        s0[i] = (uint8_t)(h ^ g);
        if (c1 != nullptr) {
            __builtin_nontemporal_store(u32x2{g, h}, c1 + i);
            s1[i] = (uint8_t)((h ^ g) >> 8);
        }
    }
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

// ------------------------------------------------- 2-D (16 x 16) blocks --
//
// Transposition-invariant scaling ("Stable FP4 Training via Transposition-
// Invariant Block Quantization", related-papers summary): one UE5M3 scale per
// aligned 16 x 16 tile, each element rounded once, and the transposed operand
// made of the same codes.  A 256-thread workgroup owns a 64 x 256 tile; wave
// w holds tile rows 16w .. 16w + 15, lane (h, u) = (lane / 32, lane % 32)
// loading 16-byte unit u (8 columns) of rows 16w + h + 2k, k < 8 (a wave
// reads 2 rows x 512 bytes per load).  The 16 x 16 block b lives in lanes
// (h, 2b) and (h, 2b + 1): one DPP swap and one exchange across the wave
// halves give every one of its four lanes the tile amax.  Codes are computed
// row-wise only (stochastic rounding draws the row-wise counter stream); the
// transposed output is an 8 x 8 nibble transpose of the packed row codes
// through LDS, with no second rounding.

__device__ __forceinline__ void swap_bits(uint32_t& x, uint32_t& y, int s, uint32_t m) {
    const uint32_t d = ((x >> s) ^ y) & m;
    y ^= d;
    x ^= d << s;
}

// w[i] holds 8 codes of row i (column j in nibble j); afterwards w[j] holds
// the 8 codes of column j (row i in nibble i).  Three rounds of masked swaps:
// nibbles within bytes, bytes within halfwords, halfwords within words.
__device__ __forceinline__ void transpose_nibbles8(uint32_t (&w)[8]) {
#pragma unroll
    for (int a = 0; a < 4; ++a) swap_bits(w[2 * a], w[2 * a + 1], 4, 0x0F0F0F0Fu);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        swap_bits(w[4 * c], w[4 * c + 2], 8, 0x00FF00FFu);
        swap_bits(w[4 * c + 1], w[4 * c + 3], 8, 0x00FF00FFu);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) swap_bits(w[m], w[4 + m], 16, 0x0000FFFFu);
}

constexpr int k2dRows = 64;   // tile rows: 4 waves x 16
constexpr int k2dWords = 33;  // LDS words per tile row of packed codes (32 + 1: conflict-free columns)

template <bool ROW, bool COL, bool SR, bool AMAX, bool W32>
__global__ __launch_bounds__(kThreads) void quantize2d_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ tensor_scale, uint64_t seed, uint32_t offset,
    uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
    uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales,
    float* __restrict__ amax_inout) {
    __shared__ uint32_t packed_lds[COL ? k2dRows * k2dWords : 1];
    __shared__ uint8_t tcode[COL ? 4 * 16 : 1];
    __shared__ float rlut[256];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int u = lane & 31, h = lane >> 5;
    int64_t R0, C0;
    tile_of<k2dRows>((uint32_t)((rows + k2dRows - 1) / k2dRows), (uint32_t)((cols + kTileCols - 1) / kTileCols),
                     R0, C0);
    const bool interior = R0 + k2dRows <= rows && C0 + kTileCols <= cols;

    // ---- loads (edge addresses clamped into the tensor: rows and cols are
    // multiples of 16, so a clamped value only ever shares a 16 x 16 block
    // with other clamped values, and never reaches an output)
    const int64_t c0 = C0 + 8 * u;
    const bool col_ok = c0 < cols;
    const int64_t rb = R0 + 16 * wv + h;  // row of k = 0; row k is rb + 2k
    u32x4 w[8];
    if (interior) {
        const uint16_t* src = x + rb * ld + c0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            w[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(2 * k) * ld));
    } else {
        const uint16_t* src = x + (col_ok ? c0 : cols - 8);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t r = min(rb + 2 * k, rows - 1);
            w[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + r * ld));
        }
    }
    // stochastic rounding: call n of row rb + 2k is n0 + k * cols / 4; the
    // counter's second word is 0 when every call number is below 2^32 (W32)
    const uint64_t n0 = ((uint64_t)rb * (uint64_t)cols + (uint64_t)c0) >> 3;
    auto row_words = [&](int k) {
        const uint64_t n = n0 + (uint64_t)k * (uint64_t)(cols >> 2);
        if constexpr (W32) return sr_words32((uint32_t)n, offset, 0u, seed);
        else return sr_words(n, offset, 0u, seed);
    };

    Ctx ctx;
    ctx.ts = *tensor_scale;
    ctx.K = 6.0f * ctx.ts;
    ctx.yK = 1.0f / ctx.K;
    ctx.fastK = ctx.K >= 0x1p-100f && ctx.K <= 0x1p100f;
    ctx.tinyOK = ctx.K >= 1.0f;
    rlut[t] = rcp_entry<SR>((uint32_t)t, ctx.ts);

    // ---- tile amax (bf16 magnitude bits; NaN sorts above Inf)
    uint32_t m2 = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        m2 = pk_max_u16(m2, pk_max_u16(pk_max_u16(w[k].x & 0x7FFF7FFFu, w[k].y & 0x7FFF7FFFu),
                                       pk_max_u16(w[k].z & 0x7FFF7FFFu, w[k].w & 0x7FFF7FFFu)));
    const uint32_t tmax = max(m2 & 0xFFFFu, m2 >> 16);
    uint32_t amax16 = max(tmax, swap_pair(tmax));
    amax16 = max(amax16, (uint32_t)__shfl_xor((int)amax16, 32));
    __syncthreads();  // reciprocal table visible

    // ---- codes, once.  The four lanes of a block hold the same amax, so
    // they take the same path.
    bool ok = ctx.fastK;
    BlockScale b = block_scale(amax16, ctx, rlut, ok);
    uint32_t packed[8];
    if (__builtin_expect(ok, 1)) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float v[8];
            unpack8(w[k], v);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] * b.r;
            U32x4 rnd;
            if (SR) rnd = row_words(k);
            packed[k] = encode8<SR>(v, rnd);
        }
    } else {
        b = block_scale_general(amax16, ctx.ts, ctx.K);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            U32x4 rnd;
            if (SR) rnd = row_words(k);
            packed[k] = encode8_general<SR>(w[k], b.code, b.r, rnd);
        }
    }

    // ---- row-wise output: codes of rows rb + 2k; the block's scale byte is
    // repeated on its 16 rows (the even lane of the pair writes rows k < 4,
    // the odd lane rows k >= 4)
    if (ROW) {
        uint8_t* pc = row_codes + rb * (cols / 2) + c0 / 2;
        uint8_t* ps = row_scales + rb * (cols / 16) + c0 / 16;
        const int64_t cstep = 2 * (cols / 2), sstep = 2 * (cols / 16);
        const int k0 = 4 * (u & 1);
        if (interior) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                __builtin_nontemporal_store(packed[k], reinterpret_cast<uint32_t*>(pc + k * cstep));
#pragma unroll
            for (int k = 0; k < 4; ++k) ps[(k0 + k) * sstep] = (uint8_t)b.code;
        } else if (col_ok) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (rb + 2 * k < rows) {
                    *reinterpret_cast<uint32_t*>(pc + k * cstep) = packed[k];
                    if ((k >> 2) == (u & 1)) ps[k * sstep] = (uint8_t)b.code;
                }
            }
        }
    }

    // ---- transposed output: thread (q, v) = (t % 8, t / 8) transposes the
    // 8 x 8 code block of tile rows 8q .. 8q + 7 and columns 8v .. 8v + 7; the
    // 8 threads of a column group write its 64 tile rows as 32 contiguous
    // bytes.  Thread t writes the scale bytes of tile column t.
    if (COL) {
#pragma unroll
        for (int k = 0; k < 8; ++k) packed_lds[(16 * wv + h + 2 * k) * k2dWords + u] = packed[k];
        if (h == 0 && (u & 1) == 0) tcode[16 * wv + (u >> 1)] = (uint8_t)b.code;
        __syncthreads();
        const int q = t & 7, vcol = t >> 3;
        uint32_t cw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) cw[i] = packed_lds[(8 * q + i) * k2dWords + vcol];
        transpose_nibbles8(cw);
        const int64_t r8 = R0 + 8 * q, cb = C0 + 8 * vcol;
        uint8_t* dst = col_codes + cb * (rows / 2) + r8 / 2;
        if (interior || (r8 < rows && cb < cols)) {
#pragma unroll
            for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t*>(dst + j * (rows / 2)) = cw[j];
        }
        const int64_t c = C0 + t;
        if (c < cols) {
            const int blk = t >> 4;
            uint8_t* sd = col_scales + c * (rows / 16) + R0 / 16;
            if (R0 + k2dRows <= rows && (rows / 16) % 4 == 0) {
                *reinterpret_cast<uint32_t*>(sd) = (uint32_t)tcode[blk] | ((uint32_t)tcode[16 + blk] << 8) |
                                                   ((uint32_t)tcode[32 + blk] << 16) |
                                                   ((uint32_t)tcode[48 + blk] << 24);
            } else {
                for (int g = 0; g < 4 && R0 + 16 * g < rows; ++g) sd[g] = tcode[16 * g + blk];
            }
        }
    }

    if (AMAX) amax_commit(tmax, amax_inout);
}

template <bool ROW, bool COL, bool SR, bool AMAX, bool W32>
void launch_quantize2d_w(const QuantizeArgs& a, hipStream_t stream) {
    const int64_t tiles = ((a.cols + kTileCols - 1) / kTileCols) * ((a.rows + k2dRows - 1) / k2dRows);
    hipLaunchKernelGGL((quantize2d_kernel<ROW, COL, SR, AMAX, W32>), dim3((unsigned)tiles), dim3(kThreads), 0,
                       stream, a.x, a.rows, a.cols, a.ld, a.tensor_scale, a.seed, a.offset, a.row_codes,
                       a.row_scales, a.col_codes, a.col_scales, a.amax_inout);
}

template <bool ROW, bool COL, bool SR, bool AMAX>
void launch_quantize2d_t(const QuantizeArgs& a, hipStream_t stream) {
    if constexpr (SR) {
        if (words32(a.rows, a.cols)) return launch_quantize2d_w<ROW, COL, SR, AMAX, true>(a, stream);
    }
    launch_quantize2d_w<ROW, COL, SR, AMAX, false>(a, stream);
}

template <bool ROW, bool COL>
void dispatch_2d(const QuantizeArgs& a, hipStream_t s) {
    if (a.stochastic) {
        if (a.amax_inout) launch_quantize2d_t<ROW, COL, true, true>(a, s);
        else launch_quantize2d_t<ROW, COL, true, false>(a, s);
    } else {
        if (a.amax_inout) launch_quantize2d_t<ROW, COL, false, true>(a, s);
        else launch_quantize2d_t<ROW, COL, false, false>(a, s);
    }
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

__global__ void zero_scalar_kernel(float* __restrict__ p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0.0f;
}

}  // namespace

void launch_zero_scalar(float* p, hipStream_t s) {
    hipLaunchKernelGGL(zero_scalar_kernel, dim3(1), dim3(64), 0, s, p);
}

void launch_quantize_blockscale(const QuantizeArgs& a, hipStream_t s) {
    const bool row = a.row_codes != nullptr;
    const bool col = a.col_codes != nullptr;
    if (row && col) dispatch_sr<true, true>(a, s);
    else if (row) dispatch_sr<true, false>(a, s);
    else if (col) dispatch_sr<false, true>(a, s);
    else launch_amax(a, s);  // amax-only pass
}

void launch_quantize_2d(const QuantizeArgs& a, hipStream_t s) {
    const bool row = a.row_codes != nullptr;
    const bool col = a.col_codes != nullptr;
    if (row && col) dispatch_2d<true, true>(a, s);
    else if (row) dispatch_2d<true, false>(a, s);
    else dispatch_2d<false, true>(a, s);
}

void launch_stream_reference(const uint16_t* x, int64_t elems, uint8_t* codes0, uint8_t* scales0,
                             uint8_t* codes1, uint8_t* scales1, hipStream_t s) {
    const int64_t blocks = elems / 16;
    const int64_t grid = max((int64_t)1, min((blocks + 255) / 256, (int64_t)cu_count() * 32));
    hipLaunchKernelGGL(stream_reference_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       reinterpret_cast<const u32x4*>(x), blocks, reinterpret_cast<u32x2*>(codes0), scales0,
                       reinterpret_cast<u32x2*>(codes1), scales1);
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
