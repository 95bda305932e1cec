// Block-16 quantization steps shared by the stand-alone quantizer and the
// GEMM epilogue that quantizes its own output: the block scale of a block
// amax, the element codes, and the small lane helpers they use.
//
// Method: "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining"
// (arXiv 2609.02846), abstract: E2M1 payloads, one UE5M3 scale per 16
// elements, fp32 tensor scale.  Per block: s_raw = amax / (6 ts) by the
// refined division of formats.hpp (equal to IEEE division wherever the code
// depends on it); the UE5M3 code from the bits of s_raw without branches
// (normal, subnormal, saturated); r = 1 / (ts * s_b) from a 256-entry table
// each workgroup builds with IEEE division (times 2^17 for stochastic
// rounding); round-to-nearest payloads from v_cvt_scalef32_pk_fp4_f32 with
// scale 1.0 (equal to the nearest-even definition for every non-NaN fp32
// input, checked on gfx950), stochastic ones from its SR sibling; blocks the
// fast path cannot take are redone by the definition.
#pragma once

#include "formats.hpp"

namespace ue5m3fp4 {
namespace {

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
    bool tinyOK;      // K >= 1: a block amax below 2^-100 gives scale code 0
};

struct BlockScale {
    uint32_t code;  // UE5M3 byte
    float r;        // RN(1 / (ts * s_b)); 0 for code 0 (payload = sign only)
};

// Block scale by the definition (any amax, any tensor scale): IEEE division,
// the integer encoder and decoder.  r is NaN for a NaN block.
__device__ __noinline__ BlockScale block_scale_general(uint32_t amax16, float ts, float K) {
    const float amax = __uint_as_float(amax16 << 16);
    BlockScale b;
    b.code = ue5m3_encode(amax / K);
    if (b.code == 0u) b.r = 0.0f;
    else if (b.code == kUe5m3Nan) b.r = __uint_as_float(0x7FC00000u);
    else b.r = 1.0f / (ts * ue5m3_decode(b.code));
    return b;
}

// Reciprocal table entry for scale code c: RN(1 / RN(ts * s_c)) by IEEE
// division, 0 for code 0; NaN marks codes the fast path must not use (the
// NaN code, and reciprocals that overflow or are NaN).  With stochastic
// rounding the entry is that reciprocal times 2^17 (an exact scaling, see
// encode8), and also NaN where the scaled value would overflow or where the
// reciprocal is at most 2^-17 (there an element could round to 0 in
// x * r but not in x * r * 2^17).
template <bool SR>
__device__ __forceinline__ float rcp_entry(uint32_t c, float ts) {
    if (c == 0u) return 0.0f;
    if (c == kUe5m3Nan) return __uint_as_float(0x7FC00000u);
    const float r = 1.0f / (ts * ue5m3_decode(c));
    if (!SR) return fabsf(r) <= 3.4028235e38f ? r : __uint_as_float(0x7FC00000u);
    return (r > 0x1p-17f && r <= 0x1p110f) ? r * 0x1p17f : __uint_as_float(0x7FC00000u);
}

// Fast block scale.  s = amax / K by the refined division (exact for
// amax >= 2^-100 and K in [2^-100, 2^100] wherever the code depends on it:
// quotients below 2^-100 give code 0 and above 2^100 saturate either way).
// Normal range (s >= 2^-14, or s overflowed to NaN): keep 3 mantissa bits of
// s, round the other 20 to nearest even, saturate at 0xFE.  Below 2^-14:
// code = rint(s * 2^17) (0..8; 8 is the smallest normal code).  r comes
// from the per-workgroup table.  `ok` is cleared for blocks the fast path
// cannot take (Inf/NaN amax, tiny amax with K < 1, NaN table entries).
__device__ __forceinline__ BlockScale block_scale(uint32_t amax16, const Ctx& c,
                                                  const float* __restrict__ rlut, bool& ok) {
    const float amax = __uint_as_float(amax16 << 16);
    const float q = amax * c.yK;
    const float rr = __builtin_fmaf(-c.K, q, amax);
    const float s = __builtin_fmaf(rr, c.yK, q);
    const uint32_t sb = __float_as_uint(s);
    const uint32_t rounded = min((sb + 0x7FFFFu + ((sb >> 20) & 1u)) >> 20, (112u << 3) + kUe5m3MaxCode);
    // clamped to [0, 8] so the conversion is defined for every s
    const uint32_t code_s = (uint32_t)fminf(fmaxf(__builtin_rintf(s * 0x1p17f), 0.0f), 8.0f);
    const uint32_t code_n = (rounded - (112u << 3)) & 0xFFu;
    const uint32_t sub = s < 0x1p-14f ? ~0u : 0u;
    BlockScale b;
    b.code = (code_s & sub) | (code_n & ~sub);
    b.r = rlut[b.code];
    ok = ok & (amax16 < 0x7F80u) & ((amax16 >= 0x0D80u) | c.tinyOK) & (b.r == b.r);
    return b;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// |a| rounded up to an integer, a's sign kept.
__device__ __forceinline__ float round_away(float a) {
    return __uint_as_float(__float_as_uint(__builtin_ceilf(fabsf(a))) | (__float_as_uint(a) & 0x80000000u));
}

// v_cvt_scalef32_sr_pk_fp4_f32 with scale 2^17 into byte J of p, the other
// three bytes kept.  The compiler's builtin for this instruction treats its
// destination as written whole (the bytes it does not select are left
// undefined), so for J > 0 the instruction is issued with the destination
// tied to p; J == 0 goes through the builtin and defines byte 0 only.
template <int J>
__device__ __forceinline__ void cvt_sr_byte(uint32_t& p, f32x2_t v, uint32_t seed) {
    if constexpr (J == 0)
        p = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, v, seed, 0x1p17f, 0);
    else if constexpr (J == 1)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(p) : "v"(v), "v"(seed), "s"(0x1p17f));
    else if constexpr (J == 2)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(p) : "v"(v), "v"(seed), "s"(0x1p17f));
    else
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(p) : "v"(v), "v"(seed), "s"(0x1p17f));
}

// Stochastic rounding of the element pair (a, b) = elements (2J, 2J + 1),
// random word w (u_a in its low half, u_b in its high half); a and b hold
// x * r * 2^17.  The instruction sees the pair as (b, a): its first slot
// rounds b under the seed, its second rounds a under the seed shifted left
// by one.  Byte J of pb receives b's code in its low nibble, byte J of pa
// receives a's code in its high nibble; the other nibble of each is the
// other slot's code under the wrong seed and is discarded.  See encode8.
template <int J>
__device__ __forceinline__ void sr_pair(uint32_t& pa, uint32_t& pb, float a, float b, uint32_t w) {
    const f32x2_t ba = f32x2_t{round_away(b), round_away(a)};
    cvt_sr_byte<J>(pb, ba, ~(w & 0xFFFF0000u));  // ~(u_b << 16), low half all ones
    cvt_sr_byte<J>(pa, ba, ~(w << 15));          // shifted: ~(u_a << 16) | 0xFFFE
}

// 8 fp32 values -> 8 E2M1 nibbles (element k in nibble k).
// RNE: v holds x * r.  v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds an
// fp32 value to E2M1 exactly as the nearest-even definition does, sign
// included (checked on gfx950 for all 2^32 non-NaN inputs).
// SR: v holds x * r * 2^17 (the table entries carry the 2^17).
template <bool SR>
__device__ __forceinline__ uint32_t encode8(const float (&v)[8], const U32x4& rnd) {
    if (!SR) {
        uint32_t p = 0u;
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0], v[1], 1.0f, 0);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2], v[3], 1.0f, 1);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4], v[5], 1.0f, 2);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6], v[7], 1.0f, 3);
        return p;
    }
    // Stochastic rounding on v_cvt_scalef32_sr_pk_fp4_f32, which divides its
    // input by the scale operand.  Measured on gfx950: its first element
    // rounds up iff F + seed >= 2^32, F being the fraction f of |v| between
    // its two E2M1 neighbours (sign copied, saturation at 6, +-Inf to +-6)
    // taken to 22 bits: F = floor(f * 2^22) * 2^10; its second element does
    // the same with seed << 1.  The definition, round up iff u < 65536 f,
    // depends on f only through ceil(65536 f), so |v| is first rounded up to
    // a multiple of 2^-17: f becomes ceil(65536 f) / 65536 in [0, 2) (and
    // keeps the same ceil(65536 f) in [2, 6) as well, where the grid step is
    // 1 or 2), F is then exact, and with a seed whose high 16 bits are
    // 65535 - u and whose next two bits are set, the instruction rounds up
    // iff ceil(65536 f) > u, i.e. iff u < 65536 f -- for every v, tiny ones
    // included (checked on gfx950 for both slots and both signs against the
    // integer form of the definition: every 2^-17 step of |v| up to 6.5 with
    // every third value of u, and every value of u below |v| = 0.52).  The
    // rounding up is
    // ceil(|x r 2^17|) with x's sign, and the scale operand 2^17 undoes the
    // 2^17.  Each element takes one instruction (the two slots read
    // overlapping seed bits, so one instruction cannot round two elements
    // with independent u); an instruction holds both elements of its pair
    // and keeps the code of the slot its seed serves.  pb collects the odd
    // elements' codes in low nibbles, pa the even elements' in high nibbles,
    // and one shift each and a bit-field merge put them in place.
    uint32_t pa, pb;
    sr_pair<0>(pa, pb, v[0], v[1], rnd.v[0]);
    sr_pair<1>(pa, pb, v[2], v[3], rnd.v[1]);
    sr_pair<2>(pa, pb, v[4], v[5], rnd.v[2]);
    sr_pair<3>(pa, pb, v[6], v[7], rnd.v[3]);
    return ((pa >> 4) & 0x0F0F0F0Fu) | ((pb << 4) & 0xF0F0F0F0u);
}

// Software element codes for blocks from block_scale_general: the same
// definition with the NaN-block rule (sign only) and any r.  The 8 bf16
// inputs arrive as 4 words (element 2i in the low half of word i).
template <bool SR>
__device__ __noinline__ uint32_t encode8_general(u32x4 w, uint32_t code, float r, U32x4 rnd) {
    uint32_t p = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t word = k < 2 ? w.x : k < 4 ? w.y : k < 6 ? w.z : w.w;
        const float x = (k & 1) ? bf16_hi(word) : bf16_lo(word);
        const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
        const float a = fabsf(x * r);
        const uint32_t idx = SR ? e2m1_sr_index(a, sr_u16(rnd, k)) : e2m1_rne_index(a);
        p |= (sign | (code == kUe5m3Nan ? 0u : idx)) << (4 * k);
    }
    return p;
}

__device__ __forceinline__ void unpack8(u32x4 w, float (&x)[8]) {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
    x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
    x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

// Per-call constants of the tensor scale ts (a device scalar read once).
__device__ __forceinline__ Ctx make_ctx(float ts) {
    Ctx c;
    c.ts = ts;
    c.K = 6.0f * ts;
    c.yK = 1.0f / c.K;
    c.fastK = c.K >= 0x1p-100f && c.K <= 0x1p100f;
    c.tinyOK = c.K >= 1.0f;
    return c;
}

// Largest bf16 magnitude bits among the 8 elements of a 16-byte unit (a NaN
// sorts above Inf).
__device__ __forceinline__ uint32_t max_abs8(u32x4 w) {
    const uint32_t m = pk_max_u16(pk_max_u16(w.x & 0x7FFF7FFFu, w.y & 0x7FFF7FFFu),
                                  pk_max_u16(w.z & 0x7FFF7FFFu, w.w & 0x7FFF7FFFu));
    return max(m & 0xFFFFu, m >> 16);
}

}  // namespace
}  // namespace ue5m3fp4
