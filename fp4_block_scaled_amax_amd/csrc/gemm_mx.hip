// Native MXFP4 "NT" GEMM for gfx950, the comparison point that measures the
// cost of emulating UE5M3 block-16 scales:
//   C[i][j] = tsA * tsB * sum_k A(i, k) * B(j, k),   fp32 accumulation,
// with both operands E2M1 (element 2j in the low nibble) and one E8M0 scale
// (2^(c - 127), 0xFF = NaN) per 32 elements along K -- the OCP Microscaling
// format the hardware takes natively ("format-aware fusion" article: the
// MXFP4 route; "UE5M3 FP4 Block Scaling ...", abstract: UE5M3 itself has to
// be emulated).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands: lane (r, h) supplies
// 32 E2M1 codes (16 bytes) of row r covering K elements [32h, 32h + 32) of
// the instruction's 64, and the E8M0 scale of exactly that 32-element block;
// accumulator register e of lane (r, h) holds row 8(e/4) + 4h + e%4,
// column r (checked on gfx950 with random codes and per-lane scales).
//
// Tiling as the UE5M3 kernel: 256 x 256 workgroup tile, 4 waves of 128 x 128
// (4 x 4 MFMA tiles, 256 fp32 accumulators per lane).  K chunks of 256
// elements (4 MFMA steps) double-buffered in LDS: codes 128 bytes per row
// padded to 144 (the 16-byte fragment reads of 8 consecutive rows hit
// distinct banks), scales 8 bytes per row.  The fragments of the next MFMA
// step are read while the current step's 16 MFMAs issue; the staging of
// chunk c + 1 and the global loads of chunk c + 2 run inside chunk c; one
// barrier per chunk, before its last step.  XCD-aware tile order.
#include "kernels.hpp"

namespace ue5m3fp4 {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 256, kBK = 256;
constexpr int kThreads = 256;
constexpr int kCodeStride = kBK / 2 + 16;                // 128 code bytes per row, padded
constexpr int kCodesA = 0;
constexpr int kCodesB = kCodesA + kBM * kCodeStride;
constexpr int kScalesA = kCodesB + kBN * kCodeStride;     // 8 bytes per row
constexpr int kScalesB = kScalesA + kBM * 8;
constexpr int kStage = kScalesB + kBN * 8;                // 77824 bytes
constexpr int kSmem = 2 * kStage;
constexpr int kGroupM = 4;
constexpr int kFmtFp4 = 4;  // cbsz / blgp: E2M1 operands

constexpr int kSchedMfma = 0x008, kSchedValu = 0x002, kSchedDs = 0x100 | 0x200, kSchedVmemRead = 0x020;

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

// 16-byte unit (32 codes = one MX block) of a row's chunk; blocks past K are
// zero codes.  ALIGNED: K % 256 == 0.
template <bool ALIGNED>
__device__ __forceinline__ u32x4 load_unit(const uint8_t* row, int64_t K, int64_t k0, int part) {
    const int64_t k = k0 + 32 * part;
    if (ALIGNED) return *reinterpret_cast<const u32x4*>(row + k / 2);
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + min(k, K - 32) / 2);
    return k < K ? v : u32x4{0u, 0u, 0u, 0u};
}

// The 8 scale bytes of a row's chunk; blocks past K get 127 (1.0), so their
// zero codes contribute exactly 0.
template <bool ALIGNED>
__device__ __forceinline__ u32x2 load_scales(const uint8_t* row, int64_t kblocks, int64_t b0) {
    if (ALIGNED) return *reinterpret_cast<const u32x2*>(row + b0);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t v = row[min(b0 + j, kblocks - 1)];
        w[j >> 2] |= (b0 + j < kblocks ? v : 127u) << (8 * (j & 3));
    }
    return u32x2{w[0], w[1]};
}

struct Frag {
    u32x4 a[4], b[4];
};

template <bool ALIGNED>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_mx_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, const float* __restrict__ b_ts, int64_t M, int64_t N,
    int64_t K, float* __restrict__ C) {
    __shared__ __align__(16) uint8_t smem[kSmem];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 31, h = lane >> 5;

    int tm, tn;
    tile_of((int)((M + kBM - 1) / kBM), (int)((N + kBN - 1) / kBN), tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t kbytes = K / 2, kblocks = K / 32;
    const int nchunks = (int)((K + kBK - 1) / kBK);

    // ---- staging: thread tid stages 16-byte units tid + 256 i (i = 0..7) of
    // each operand's 256 x 128 code bytes (row unit / 8, part unit % 8) and the
    // 8 scale bytes of row tid.  Loads are unconditional (rows clamped).
    const int srow = tid >> 3, spart = tid & 7;  // unit tid + 256 i: row srow + 32 i
    const uint8_t* a_srow = a_scales + min(m0 + tid, M - 1) * kblocks;
    const uint8_t* b_srow = b_scales + min(n0 + tid, N - 1) * kblocks;
    u32x4 ra0, ra1, ra2, ra3, ra4, ra5, ra6, ra7, rb0, rb1, rb2, rb3, rb4, rb5, rb6, rb7;
    u32x2 rsa, rsb;

    // row i of this thread's units, clamped into the operand
    auto arow = [&](int i) __attribute__((always_inline)) {
        return a_codes + min(m0 + srow + 32 * i, M - 1) * kbytes;
    };
    auto brow = [&](int i) __attribute__((always_inline)) {
        return b_codes + min(n0 + srow + 32 * i, N - 1) * kbytes;
    };
    auto gload = [&](int chunk) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)chunk * kBK;
        ra0 = load_unit<ALIGNED>(arow(0), K, k0, spart); ra1 = load_unit<ALIGNED>(arow(1), K, k0, spart);
        ra2 = load_unit<ALIGNED>(arow(2), K, k0, spart); ra3 = load_unit<ALIGNED>(arow(3), K, k0, spart);
        ra4 = load_unit<ALIGNED>(arow(4), K, k0, spart); ra5 = load_unit<ALIGNED>(arow(5), K, k0, spart);
        ra6 = load_unit<ALIGNED>(arow(6), K, k0, spart); ra7 = load_unit<ALIGNED>(arow(7), K, k0, spart);
        rb0 = load_unit<ALIGNED>(brow(0), K, k0, spart); rb1 = load_unit<ALIGNED>(brow(1), K, k0, spart);
        rb2 = load_unit<ALIGNED>(brow(2), K, k0, spart); rb3 = load_unit<ALIGNED>(brow(3), K, k0, spart);
        rb4 = load_unit<ALIGNED>(brow(4), K, k0, spart); rb5 = load_unit<ALIGNED>(brow(5), K, k0, spart);
        rb6 = load_unit<ALIGNED>(brow(6), K, k0, spart); rb7 = load_unit<ALIGNED>(brow(7), K, k0, spart);
        rsa = load_scales<ALIGNED>(a_srow, kblocks, k0 / 32);
        rsb = load_scales<ALIGNED>(b_srow, kblocks, k0 / 32);
    };
    auto lstore = [&](uint8_t* base) __attribute__((always_inline)) {
        uint8_t* pa = base + kCodesA + srow * kCodeStride + 16 * spart;
        uint8_t* pb = base + kCodesB + srow * kCodeStride + 16 * spart;
        constexpr int step = 32 * kCodeStride;
        *reinterpret_cast<u32x4*>(pa + 0 * step) = ra0; *reinterpret_cast<u32x4*>(pa + 1 * step) = ra1;
        *reinterpret_cast<u32x4*>(pa + 2 * step) = ra2; *reinterpret_cast<u32x4*>(pa + 3 * step) = ra3;
        *reinterpret_cast<u32x4*>(pa + 4 * step) = ra4; *reinterpret_cast<u32x4*>(pa + 5 * step) = ra5;
        *reinterpret_cast<u32x4*>(pa + 6 * step) = ra6; *reinterpret_cast<u32x4*>(pa + 7 * step) = ra7;
        *reinterpret_cast<u32x4*>(pb + 0 * step) = rb0; *reinterpret_cast<u32x4*>(pb + 1 * step) = rb1;
        *reinterpret_cast<u32x4*>(pb + 2 * step) = rb2; *reinterpret_cast<u32x4*>(pb + 3 * step) = rb3;
        *reinterpret_cast<u32x4*>(pb + 4 * step) = rb4; *reinterpret_cast<u32x4*>(pb + 5 * step) = rb5;
        *reinterpret_cast<u32x4*>(pb + 6 * step) = rb6; *reinterpret_cast<u32x4*>(pb + 7 * step) = rb7;
        *reinterpret_cast<u32x2*>(base + kScalesA + tid * 8) = rsa;
        *reinterpret_cast<u32x2*>(base + kScalesB + tid * 8) = rsb;
    };

    // ---- per-lane LDS offsets.  MFMA step s (0..3) of a chunk covers K
    // elements [64 s, 64 s + 64); lane (r, h) reads its row's 16 bytes at
    // 32 s + 16 h and uses scale byte 2 s + h.
    const int a_off = kCodesA + (wm * 128 + r) * kCodeStride + 16 * h;
    const int b_off = kCodesB + (wn * 128 + r) * kCodeStride + 16 * h;
    const int as_off = kScalesA + (wm * 128 + r) * 8;
    const int bs_off = kScalesB + (wn * 128 + r) * 8;
    auto read_frag = [&](Frag& f, const uint8_t* base, int s) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f.a[g] = *reinterpret_cast<const u32x4*>(base + a_off + g * 32 * kCodeStride + 32 * s);
            f.b[g] = *reinterpret_cast<const u32x4*>(base + b_off + g * 32 * kCodeStride + 32 * s);
        }
    };
    auto read_scales = [&](u32x2 (&sa)[4], u32x2 (&sb)[4], const uint8_t* base) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            sa[g] = *reinterpret_cast<const u32x2*>(base + as_off + g * 32 * 8);
            sb[g] = *reinterpret_cast<const u32x2*>(base + bs_off + g * 32 * 8);
        }
    };
    auto scale_byte = [&](const u32x2& s2, int s) __attribute__((always_inline)) {
        const int b = 2 * s + h;  // 0..7
        return (int)(((b < 4 ? s2.x : s2.y) >> (8 * (b & 3))) & 0xFFu);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (nchunks > 0) {
        gload(0);
        lstore(smem);
        gload(min(1, nchunks - 1));
        __syncthreads();

        Frag fr[2];
        u32x2 sa[4], sb[4];
        read_frag(fr[0], smem, 0);
        read_scales(sa, sb, smem);

        for (int c = 0; c < nchunks; ++c) {
            uint8_t* cur = smem + (c & 1) * kStage;
            uint8_t* nxt = smem + ((c + 1) & 1) * kStage;
            u32x2 sa_n[4], sb_n[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                const Frag& f = fr[J & 1];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const i32x8_t av = {(int)f.a[i].x, (int)f.a[i].y, (int)f.a[i].z, (int)f.a[i].w, 0, 0, 0, 0};
                        const i32x8_t bv = {(int)f.b[j].x, (int)f.b[j].y, (int)f.b[j].z, (int)f.b[j].w, 0, 0, 0, 0};
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            av, bv, acc[i][j], kFmtFp4, kFmtFp4, 0, scale_byte(sa[i], J), 0,
                            scale_byte(sb[j], J));
                    }
                if (J < 3) read_frag(fr[(J + 1) & 1], cur, J + 1);
                if (J == 3) {
                    read_frag(fr[0], nxt, 0);
                    read_scales(sa_n, sb_n, nxt);
                }
                if (J == 0) {
                    lstore(nxt);
                    gload(min(c + 2, nchunks - 1));
                }
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    if (q < 12) __builtin_amdgcn_sched_group_barrier(kSchedDs, 1, 0);
                    if (q < 8) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedValu, 2, 0);
                }
                if (J == 2) __syncthreads();
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                sa[g] = sa_n[g];
                sb[g] = sb_n[g];
            }
        }
    }

    // ---- epilogue: C = (acc * tsA) * tsB
    const float tsa = *a_ts, tsb = *b_ts;
    const int64_t row0 = m0 + wm * 128 + 4 * h, col0 = n0 + wn * 128 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = col0 + j * 32;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = row0 + i * 32 + 8 * (e >> 2) + (e & 3);
                if (row < M && col < N) C[row * N + col] = (acc[i][j][e] * tsa) * tsb;
            }
        }
}

}  // namespace

void launch_gemm_nt_mx(const GemmArgs& g, hipStream_t stream) {
    const int64_t tiles = ((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
    if (g.K % kBK == 0)
        hipLaunchKernelGGL(gemm_nt_mx_kernel<true>, dim3((unsigned)tiles), dim3(kThreads), 0, stream,
                           g.a_codes, g.a_scales, g.a_ts, g.b_codes, g.b_scales, g.b_ts, g.M, g.N, g.K,
                           g.c);
    else
        hipLaunchKernelGGL(gemm_nt_mx_kernel<false>, dim3((unsigned)tiles), dim3(kThreads), 0, stream,
                           g.a_codes, g.a_scales, g.a_ts, g.b_codes, g.b_scales, g.b_ts, g.M, g.N, g.K,
                           g.c);
}

}  // namespace ue5m3fp4
