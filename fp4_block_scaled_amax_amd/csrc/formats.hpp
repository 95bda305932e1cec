// Device-side E2M1 / UE5M3 format arithmetic and the Philox4x32-10 generator.
//
// Method: "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining"
// (arXiv 2609.02846), abstract -- E2M1 payloads, unsigned E5M3 block scales,
// block 16, stochastic rounding on backward gradients.  Layouts and the
// exact arithmetic are stated in include/ue5m3fp4.h.
//
// Everything here is plain fp32 / integer code with one IEEE rounding per
// operation; the translation units are compiled with -ffp-contract=off so
// that no multiply-add is fused implicitly.  The only FMAs are the explicit
// correction steps of rcp_rn / div_rn, whose results equal IEEE division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ue5m3fp4 {

// ------------------------------------------------------------------ bf16 --

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ----------------------------------------------------------------- UE5M3 --
// Byte: bits 7..3 exponent e (bias 15), bits 2..0 mantissa f.  e == 0 is
// subnormal (f * 2^-17); 0xFF is NaN; 0xFE = 1.75 * 2^16 is the largest value.

constexpr uint32_t kUe5m3Nan = 0xFFu;
constexpr uint32_t kUe5m3MaxCode = 0xFEu;

// Round-to-nearest-even, saturating encode of an fp32 scale.  +-0 -> 0x00;
// NaN, +Inf and negative values -> 0xFF.
__device__ __forceinline__ uint32_t ue5m3_encode(float s) {
    if (s == 0.0f) return 0u;
    const uint32_t b = __float_as_uint(s);
    if (!(s > 0.0f) || b >= 0x7F800000u) return kUe5m3Nan;
    const int e = (int)(b >> 23) - 127;  // floor(log2 s) for normal fp32
    const uint32_t man = b & 0x7FFFFFu;
    uint32_t code;
    if (e >= -14) {
        // normal UE5M3: keep the top 3 mantissa bits, round the other 20
        code = ((uint32_t)(e + 15) << 3) | (man >> 20);
        const uint32_t rem = man & 0xFFFFFu;
        code += (rem > 0x80000u) || (rem == 0x80000u && (code & 1u));
        code = code < kUe5m3MaxCode ? code : kUe5m3MaxCode;
    } else {
        // subnormal UE5M3: m = round(s / 2^-17) = round(sig * 2^(e - 6))
        const int sh = 6 - e;  // >= 21
        if (sh > 31 || (b >> 23) == 0u) return 0u;  // s < 2^-25: rounds to 0
        const uint32_t sig = man | 0x800000u;
        code = sig >> sh;
        const uint32_t rem = sig & ((1u << sh) - 1u);
        const uint32_t half = 1u << (sh - 1);
        code += (rem > half) || (rem == half && (code & 1u));
    }
    return code;
}

// Value of a finite UE5M3 code (0x00..0xFE) as fp32 (exact).
__device__ __forceinline__ float ue5m3_decode(uint32_t c) {
    const uint32_t e = c >> 3, f = c & 7u;
    if (e == 0u) return (float)f * 0x1p-17f;
    return __uint_as_float(((e + 112u) << 23) | (f << 20));  // (1 + f/8) * 2^(e-15)
}

// ------------------------------------------------- correctly rounded ops --
// Round-to-nearest fp32 reciprocal and division built from v_rcp_f32 plus one
// FMA-based correction (Markstein's refinement).  Checked exhaustively on
// gfx950 against IEEE division: the reciprocal over every normal fp32 input,
// the division over every bf16 dividend mantissa against every divisor
// mantissa for quotients in the normal range.  Outside the guarded range the
// callers fall back to the IEEE division.

__device__ __forceinline__ float rcp_rn(float d) {
    if (!(d >= 0x1p-100f && d <= 0x1p100f)) return 1.0f / d;
    const float y = __builtin_amdgcn_rcpf(d);
    const float e = __builtin_fmaf(-d, y, 1.0f);
    return __builtin_fmaf(e, y, y);
}

// a / b rounded to nearest, given y = RN(1 / b) and fast_b = b in [2^-100, 2^100].
__device__ __forceinline__ float div_rn(float a, float b, float y, bool fast_b) {
    const float q = a * y;
    const float r = __builtin_fmaf(-b, q, a);
    const float q1 = __builtin_fmaf(r, y, q);
    if (fast_b && a >= 0x1p-100f && q1 >= 0x1p-100f && q1 <= 0x1p100f) return q1;
    return a / b;
}

// ------------------------------------------------------------------ E2M1 --
// Nibble: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.  Index
// 0..7 = magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.

// Round-to-nearest-even magnitude index of a = |v|.  Each comparison is a
// midpoint of the grid; at a midpoint the even index wins.  a >= 6 (and +Inf)
// gives 7; NaN fails every comparison and gives 0.
__device__ __forceinline__ uint32_t e2m1_rne_index(float a) {
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
           (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
           (uint32_t)(a > 5.0f);
}

// Stochastic-rounding magnitude index of a = |v| with 16 random bits u:
// with lo the grid value below a and step the gap to the next one, round up
// iff u < 65536 * (a - lo) / step.  Branch-free: within each stretch of the
// grid with one step (0..2 step 0.5, 2..4 step 1, 4..6 step 2) a is scaled by
// 1/step (a power of two, exact), so the integer part gives lo's index (plus
// 0, 2 or 4) and the fraction (exact by Sterbenz) is (a - lo) / step.  a >= 6
// gives 7; NaN gives 0.
__device__ __forceinline__ uint32_t e2m1_sr_index(float a, uint32_t u) {
    const bool r1 = a < 2.0f, r2 = a < 4.0f;
    const float scale = r1 ? 2.0f : (r2 ? 1.0f : 0.5f);
    const uint32_t add = r1 ? 0u : (r2 ? 2u : 4u);
    const float t = fminf(a, 7.0f) * scale;  // in [0, 4): exact
    const float fl = truncf(t);
    const float frac = t - fl;
    const uint32_t up = (float)u < frac * 65536.0f;
    const uint32_t idx = (uint32_t)fl + add + up;
    return a >= 6.0f ? 7u : (a == a ? idx : 0u);
}

// ---------------------------------------------------------------- Philox --
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): per round, words 0 and
// 2 are multiplied by 0xD2511F53 and 0xCD9E8D57 (64-bit products); the new
// words are (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is bumped by
// 0x9E3779B9 / 0xBB67AE85 between rounds.

struct U32x4 {
    uint32_t v[4];
};

__device__ __forceinline__ U32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input XOR in one v_bitop3_b32 (truth table 0x96)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    U32x4 out;
    out.v[0] = c0;
    out.v[1] = c1;
    out.v[2] = c2;
    out.v[3] = c3;
    return out;
}

// The eight 16-bit values of call n for output orientation o.
__device__ __forceinline__ U32x4 sr_words(uint64_t n, uint32_t offset, uint32_t o, uint64_t seed) {
    return philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), offset, o, (uint32_t)seed,
                         (uint32_t)(seed >> 32));
}

// The same for a call number below 2^32 (the counter's second word is 0):
// the first half of rounds 1 and 2 then depends only on the offset, the
// orientation and the key, which are the same for every lane of a launch,
// so that part is computed once per wave instead of per lane.
__device__ __forceinline__ U32x4 sr_words32(uint32_t n, uint32_t offset, uint32_t o, uint64_t seed) {
    return philox4x32_10(n, 0u, offset, o, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t sr_u16(const U32x4& w, int k) {
    return (w.v[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
}

}  // namespace ue5m3fp4
