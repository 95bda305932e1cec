/*
 * libue5m3fp4 -- UE5M3-FP4 block-16 quantization and the block-scaled
 * training GEMMs of a linear layer, for AMD Instinct MI355X (gfx950).
 *
 * The method: "UE5M3 FP4 Block Scaling for Stable Language Model
 * Pretraining" (arXiv 2609.02846), abstract.  Tensors are stored as E2M1
 * (4-bit float) payloads with one unsigned-E5M3 (UE5M3) scale per block of 16
 * elements and one fp32 tensor scale that is refreshed periodically rather
 * than recomputed before every quantization.  Backward gradients (dY) use
 * stochastic rounding, everything else round-to-nearest-even.  The three
 * GEMMs of a linear layer ("Rethinking Shrinkage Bias in LLM FP4 Pretraining
 * ... UFP4 Recipe", arXiv 2606.20381, abstract) consume these operands, each
 * quantized along its own contraction axis ("Stable FP4 Training via
 * Transposition-Invariant Block Quantization", related-papers summary: 1-D
 * blocks give a tensor and its transpose different scales).
 *
 * Formats (byte layouts of the library):
 *   E2M1 code (nibble): bit 3 sign, bits 2..1 exponent (bias 1), bit 0
 *     mantissa; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no Inf/NaN.
 *   UE5M3 scale (byte): bits 7..3 exponent e (bias 15), bits 2..0 mantissa f;
 *     e == 0: f * 2^-17; otherwise (1 + f/8) * 2^(e-15); 0xFF = NaN (no Inf);
 *     largest 0xFE = 114688.  Rounded to nearest even, saturating.
 *   A quantized R x C operand (blocks along C, C % 16 == 0):
 *     codes  [R][C/2]  uint8, element 2j in the low nibble of byte j;
 *     scales [R][C/16] uint8, row-major;
 *     value(i, j) = ts * ue5m3(scales[i][j/16]) * e2m1(code(i, j)).
 *
 * Quantization arithmetic (fp32, round-to-nearest-even, no fused ops):
 *   amax_b = max|x| over the block; K = 6 * ts; s_raw = amax_b / K;
 *   code_b = ue5m3(s_raw); if code_b is 0x00 or 0xFF every element of the
 *   block keeps only its sign bit; otherwise r = 1 / (ts * s_b) and the
 *   payload is round(x * r) on the E2M1 grid, saturating at +-6; the sign
 *   bit is always copied from x.
 * Stochastic rounding: Philox4x32-10 (Salmon et al., SC'11).  Output element
 *   (i, j) of an R_o x C_o output in orientation o (0 = row-wise, 1 =
 *   transposed) has e = i * C_o + j; call n = e >> 3 uses counter
 *   (n lo, n hi, offset, o) and key (seed lo, seed hi); element e takes the
 *   low (e even) or high (e odd) 16 bits u of output word (e & 7) >> 1 and
 *   rounds |v| up to the next grid value iff u < 65536 * frac, frac being
 *   the position of |v| between its two grid neighbours.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers (HBM) unless stated; the caller owns all
 *     memory.  No call allocates, frees, synchronizes, or keeps a pointer
 *     after it returns.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the null stream) and runs asynchronously; errors inside a kernel
 *     surface at the caller's next synchronization.
 *   - Arguments are validated on the host before any HIP call; a failed
 *     check returns a negative status and launches nothing.  Sizes of 0 are
 *     valid and launch nothing (except the GEMMs with K == 0, which write
 *     zeros).
 *   - Array base pointers must be 16-byte aligned; scalar pointers (tensor
 *     scales, amax) 4-byte aligned.
 *   - The library holds no global state and is safe to call from several
 *     host threads; calls on one stream execute in order.
 */
#ifndef UE5M3FP4_H
#define UE5M3FP4_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define UE5M3FP4_API __attribute__((visibility("default")))
#else
#define UE5M3FP4_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum ue5m3fp4_status {
    UE5M3FP4_OK = 0,
    UE5M3FP4_EINVAL = -1, /* NULL pointer, negative size, unknown mode, bad period */
    UE5M3FP4_ESHAPE = -2, /* a dimension violates the block-16 layout or sizes disagree */
    UE5M3FP4_EALIGN = -3, /* a pointer or leading dimension is misaligned */
    UE5M3FP4_EHIP = -4,   /* the HIP runtime reported an error at launch */
    UE5M3FP4_ERANGE = -5  /* a size exceeds the library's index range */
};

enum ue5m3fp4_rounding {
    UE5M3FP4_RNE = 0, /* round to nearest, ties to even: X and W */
    UE5M3FP4_SR = 1   /* stochastic rounding: backward gradients dY only */
};

/* Quantize a bf16 tensor x (rows x cols, row stride ld elements) under the
 * fp32 tensor scale *tensor_scale (device scalar).  Method: UE5M3 paper,
 * abstract (block-16 E2M1/UE5M3, periodic tensor scaling, SR on gradients).
 *
 *   row_codes/row_scales: x quantized along cols: [rows][cols/2], [rows][cols/16].
 *   col_codes/col_scales: x^T quantized along rows (the transposed operand of
 *       dgrad/wgrad), computed from the same bf16 read: [cols][rows/2],
 *       [cols][rows/16].
 *   Each pair is both NULL (not produced) or both non-NULL.  Both pairs NULL
 *   with amax_inout set is an amax-only pass (the bootstrap before the first
 *   tensor-scale refresh).
 *   amax_inout: nullable device fp32; receives max(*amax_inout, max|x|)
 *       (a NaN in x propagates).  This is the running amax that
 *       ue5m3fp4_update_tensor_scale consumes.
 *   rounding: UE5M3FP4_RNE or UE5M3FP4_SR; seed/offset select the SR stream
 *       (ignored for RNE).  The caller gives each quantize call of a step a
 *       distinct (seed, offset).
 * Requirements: cols % 16 == 0; rows % 16 == 0 when the transposed output is
 * requested; ld >= cols, ld % 8 == 0; rows, cols < 2^31; rows * ld < 2^40.
 * x and the outputs must not overlap. */
UE5M3FP4_API int ue5m3fp4_quantize_blockscale(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                 const float* tensor_scale, int rounding, uint64_t seed,
                                 uint32_t offset, uint8_t* row_codes, uint8_t* row_scales,
                                 uint8_t* col_codes, uint8_t* col_scales, float* amax_inout,
                                 void* stream);

/* Quantize x with one UE5M3 scale per aligned 16 x 16 tile instead of per
 * 16-element row block ("Stable FP4 Training via Transposition-Invariant
 * Block Quantization", summary in the UE5M3 paper's related-papers list:
 * 2-D blocks give a value the same scale in the forward operand and in the
 * transposed operand of the backward GEMMs).  Per tile: amax over its 256
 * elements, the block-scale and element steps of ue5m3fp4_quantize_blockscale
 * with that amax; each element is rounded once (SR bits: the row-wise stream
 * of ue5m3fp4_quantize_blockscale with the same seed/offset), so col_codes is
 * exactly the transpose of row_codes.
 *   row_codes/row_scales, col_codes/col_scales: the layouts of
 *       ue5m3fp4_quantize_blockscale, the tile's scale byte repeated on each
 *       of its 16 rows (row_scales[i][J] = tile (i/16, J)) and columns
 *       (col_scales[j][I] = tile (I, j/16)), so the GEMM entry points take
 *       either output unchanged.  At least one pair is required (EINVAL).
 *   amax_inout, rounding, seed, offset, tensor_scale: as
 *       ue5m3fp4_quantize_blockscale.
 * Requirements: rows % 16 == 0 and cols % 16 == 0 (ESHAPE); other rules as
 * ue5m3fp4_quantize_blockscale. */
UE5M3FP4_API int ue5m3fp4_quantize_blockscale_2d(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                    const float* tensor_scale, int rounding, uint64_t seed,
                                    uint32_t offset, uint8_t* row_codes, uint8_t* row_scales,
                                    uint8_t* col_codes, uint8_t* col_scales, float* amax_inout,
                                    void* stream);

/* Current-tensor scaling, the alternative to the periodic refresh: the
 * tensor scale comes from this tensor's own amax, which costs one more read
 * of x (UE5M3 paper, abstract: the UE5M3 range is what lets the recipe use
 * periodic instead of current tensor scaling; this call measures what that
 * saves).  Three steps on `stream`:
 *   1. *amax_out = max|x| (an amax pass; a NaN in x propagates);
 *   2. *tensor_scale = fp32(*amax_out / fp32(6 * max_safe)) when *amax_out
 *      is finite and > 0, else *tensor_scale is left as passed;
 *   3. the block quantization of ue5m3fp4_quantize_blockscale with that
 *      tensor scale (same outputs, layouts, rounding and random stream).
 * At least one output pair is required; tensor_scale and amax_out are device
 * fp32 scalars (tensor_scale is read only in the fallback of step 2).
 * max_safe > 0 and finite.  Other rules as ue5m3fp4_quantize_blockscale. */
UE5M3FP4_API int ue5m3fp4_quantize_current_scaling(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                      float max_safe, int rounding, uint64_t seed, uint32_t offset,
                                      uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                                      uint8_t* col_scales, float* tensor_scale, float* amax_out,
                                      void* stream);

/* Dequantize one block-scaled operand: the value that the UE5M3 paper's
 * two-level format stores ("UE5M3 FP4 Block Scaling for Stable Language
 * Model Pretraining", abstract: E2M1 payloads, one unsigned-E5M3 scale per
 * 16-element block, an fp32 tensor scale):
 *   out[i][j] = fp32(fp32(e2m1 * ue5m3) * ts) for a quantized rows x cols
 * operand (the product q * s_b is exact, so there is one rounding).
 *   codes [rows][cols/2], scales [rows][cols/16] (the quantizer's layouts),
 *   tensor_scale: device fp32 scalar; out: fp32 [rows][cols], row stride cols.
 * Blocks with scale 0xFF give NaN.  cols % 16 == 0 (UE5M3FP4_ESHAPE); NULL
 * pointers UE5M3FP4_EINVAL; misaligned pointers UE5M3FP4_EALIGN. */
UE5M3FP4_API int ue5m3fp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                        int64_t rows, int64_t cols, float* out, void* stream);

/* Generic block-scaled GEMM, both operands blocked along K:
 *   C[i][j] = (tsA * tsB) * sum_k A(i, k) * B(j, k),  fp32 accumulation,
 * A: codes [M][K/2], scales [M][K/16];  B: codes [N][K/2], scales [N][K/16];
 * C: fp32 [M][N] (row stride N).  K % 16 == 0.  M, N, K < 2^31. */
UE5M3FP4_API int ue5m3fp4_gemm_nt(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                     const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                     int64_t M, int64_t N, int64_t K, float* c, void* stream);

/* ue5m3fp4_gemm_nt with its output fused for the next linear layer:
 * C = (tsA * tsB) * sum_k A(i,k) B(j,k) computed as in ue5m3fp4_gemm_nt,
 * then rounded to bf16 (round to nearest even; NaN stays NaN) and stored as
 * bf16 [M][N] (row stride N); when amax_inout is non-NULL, max |C_bf16| over
 * the stored values is folded into *amax_inout (the running amax the next
 * quantization's tensor scale is refreshed from; a NaN propagates).
 * Format-aware fusion article (similar-articles list of the UFP4 page):
 * fusing the steps around the FP4 GEMM is where the throughput is.  c must
 * be 16-byte aligned, amax_inout 4-byte aligned.  Other rules as
 * ue5m3fp4_gemm_nt. */
UE5M3FP4_API int ue5m3fp4_gemm_nt_bf16(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                          const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                          int64_t M, int64_t N, int64_t K, uint16_t* c, float* amax_inout,
                          void* stream);

/* ue5m3fp4_gemm_nt_bf16 whose epilogue also quantizes the bf16 output for
 * the next linear layer ("format-aware fusion" article in the UFP4 page's
 * similar-articles list: scale computation and packing fused with the GEMM).
 * The quantized outputs are exactly those of ue5m3fp4_quantize_blockscale
 * applied to the bf16 C that this call writes (rows = M, cols = N, ld = N):
 *   c_row_codes/c_row_scales: [M][N/2], [M][N/16] (blocks along N; N % 16);
 *   c_col_codes/c_col_scales: [N][M/2], [N][M/16] (C^T, blocks along M;
 *       M % 16);
 *   c_tensor_scale: device fp32 scalar, the output's (periodic) tensor scale;
 *   rounding, seed, offset: as ue5m3fp4_quantize_blockscale (SR streams of
 *       the M x N output, orientation 0 row-wise and 1 transposed).
 * Each pair is both NULL or both non-NULL; at least one pair (EINVAL).
 * amax_inout (nullable) receives max(*amax_inout, max|C|) as in
 * ue5m3fp4_gemm_nt_bf16 -- the running amax of the next tensor-scale
 * refresh.  Other rules as ue5m3fp4_gemm_nt_bf16; c and the outputs must not
 * overlap. */
UE5M3FP4_API int ue5m3fp4_gemm_nt_bf16_quantized(const uint8_t* a_codes, const uint8_t* a_scales,
                                    const float* a_ts, const uint8_t* b_codes,
                                    const uint8_t* b_scales, const float* b_ts, int64_t M,
                                    int64_t N, int64_t K, uint16_t* c, float* amax_inout,
                                    const float* c_tensor_scale, int rounding, uint64_t seed,
                                    uint32_t offset, uint8_t* c_row_codes, uint8_t* c_row_scales,
                                    uint8_t* c_col_codes, uint8_t* c_col_scales, void* stream);

/* Native MXFP4 comparison GEMM: the block format gfx950's scaled FP4 MFMA
 * takes natively (OCP Microscaling: E2M1 elements, one E8M0 scale 2^(c-127)
 * per 32 elements, 0xFF = NaN), with the same tensor-scale epilogue as
 * ue5m3fp4_gemm_nt:  C = (tsA * tsB) * sum_k A(i,k) B(j,k), fp32 [M][N].
 * It measures what emulating UE5M3 block-16 costs (UE5M3 paper, abstract:
 * UE5M3 is software-emulated; format-aware fusion article: the MXFP4
 * route).  a_codes [M][K/2], b_codes [N][K/2] (element 2j in the low nibble);
 * a_scales [M][K/32], b_scales [N][K/32] E8M0 bytes.  K % 32 == 0
 * (UE5M3FP4_ESHAPE otherwise); alignment and sizes as ue5m3fp4_gemm_nt. */
UE5M3FP4_API int ue5m3fp4_gemm_nt_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                           const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                           int64_t M, int64_t N, int64_t K, float* c, void* stream);

/* fprop: Y = X W^T.  UFP4 paper, abstract (three training GEMMs).
 *   x: X [tokens][in] quantized row-wise (codes [tokens][in/2]);
 *   w: W [out][in] quantized row-wise (codes [out][in/2]);
 *   y: fp32 [tokens][out].  in % 16 == 0. */
UE5M3FP4_API int ue5m3fp4_gemm_fprop(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_ts,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_ts,
                        int64_t tokens, int64_t in_features, int64_t out_features, float* y,
                        void* stream);

/* dgrad: dX = dY W.  The second of the three training GEMMs of a linear
 * layer ("Rethinking Shrinkage Bias in LLM FP4 Pretraining ... UFP4
 * Recipe", abstract), run on block-scaled FP4 operands with stochastic
 * rounding on dY only ("UE5M3 FP4 Block Scaling ...", abstract: selective
 * stochastic rounding for backward gradients); W enters through its
 * transposed quantization, blocked along the contraction axis ("Stable FP4
 * Training via Transposition-Invariant Block Quantization", related-papers
 * summary: 1-D blocks give W and W^T different scales).
 *   dy: dY [tokens][out] quantized row-wise (codes [tokens][out/2]);
 *   wt: the transposed output of W's quantization, W^T [in][out] blocked
 *       along out (codes [in][out/2]);
 *   dx: fp32 [tokens][in].  out % 16 == 0. */
UE5M3FP4_API int ue5m3fp4_gemm_dgrad(const uint8_t* dy_codes, const uint8_t* dy_scales, const float* dy_ts,
                        const uint8_t* wt_codes, const uint8_t* wt_scales, const float* w_ts,
                        int64_t tokens, int64_t in_features, int64_t out_features, float* dx,
                        void* stream);

/* wgrad: dW = dY^T X.  The third training GEMM of a linear layer ("Rethinking
 * Shrinkage Bias in LLM FP4 Pretraining ... UFP4 Recipe", abstract): it
 * contracts over tokens, so both operands are the transposed quantizations
 * of dY and X, each blocked along tokens ("Stable FP4 Training via
 * Transposition-Invariant Block Quantization", related-papers summary).
 *   dyt: the transposed output of dY's quantization, dY^T [out][tokens]
 *        blocked along tokens (codes [out][tokens/2]);
 *   xt:  the transposed output of X's quantization, X^T [in][tokens]
 *        (codes [in][tokens/2]);
 *   dw: fp32 [out][in].  tokens % 16 == 0. */
UE5M3FP4_API int ue5m3fp4_gemm_wgrad(const uint8_t* dyt_codes, const uint8_t* dyt_scales, const float* dy_ts,
                        const uint8_t* xt_codes, const uint8_t* xt_scales, const float* x_ts,
                        int64_t tokens, int64_t in_features, int64_t out_features, float* dw,
                        void* stream);

/* Periodic tensor-scale refresh.  UE5M3 paper, abstract: the UE5M3 range
 * permits periodic (not current) tensor scaling.  If step % period == 0:
 * when *amax_running is finite and > 0,
 * *tensor_scale = fp32(*amax_running / fp32(6 * max_safe)); then
 * *amax_running = 0.  Otherwise nothing is launched.  period < 1 or
 * step < 0 is UE5M3FP4_EINVAL.  max_safe (> 0, finite;
 * 7168 = 114688 / 16 by default in the bindings) is the block scale the
 * tensor's largest block receives at refresh time.  Both pointers are device
 * fp32 scalars. */
UE5M3FP4_API int ue5m3fp4_update_tensor_scale(float* amax_running, float* tensor_scale, int64_t step,
                                 int64_t period, float max_safe, void* stream);

/* Measurement aid, not part of the method (it does no quantization): moves
 * the bytes of a quantize call as contiguous streams, so that its time is
 * the HBM rate available to the quantizer's read/write mix.  Reads x, elems
 * bf16 values (elems % 16 == 0, contiguous); per 16-value block writes 8
 * bytes to codes0 and 1 byte to scales0 (buffers of elems/2 and elems/16
 * bytes), and the same to codes1 / scales1 when both are non-NULL (one pair
 * NULL and the other not: UE5M3FP4_EINVAL).  Byte 0..7 of block i's codes
 * hold the XOR of words 0..3 and of words 4..7 of the block (little-endian
 * u32 pair; codes1 holds the pair swapped); scales0 byte i is the low byte of
 * their XOR, scales1 byte i the next byte.  x and codes 16-byte aligned
 * (UE5M3FP4_EALIGN), NULL x / codes0 / scales0 UE5M3FP4_EINVAL, elems < 0
 * UE5M3FP4_EINVAL, elems % 16 != 0 UE5M3FP4_ESHAPE, elems >= 2^40
 * UE5M3FP4_ERANGE. */
UE5M3FP4_API int ue5m3fp4_stream_reference(const uint16_t* x, int64_t elems, uint8_t* codes0, uint8_t* scales0,
                                           uint8_t* codes1, uint8_t* scales1, void* stream);

/* Static, NUL-terminated description of a status code. */
UE5M3FP4_API const char* ue5m3fp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* UE5M3FP4_H */
