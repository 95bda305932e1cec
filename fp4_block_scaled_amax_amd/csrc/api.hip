// C ABI of libue5m3fp4 (declared in include/ue5m3fp4.h): argument checks on
// the host, then one launch on the caller's stream.  No allocation, no
// synchronization, no retained state.
#include <cmath>

#include "../../include/ue5m3fp4.h"
#include "kernels.hpp"

namespace {

using namespace ue5m3fp4;

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// The runtime's last-error slot is per thread and also holds the errors of
// earlier, unrelated calls (a caller's failed query, a framework's lazy
// initialization).  It is cleared right before this library's launches, so
// that launch_status reports only their own failures.
void clear_stale_error() { (void)hipGetLastError(); }

int launch_status() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? UE5M3FP4_OK : UE5M3FP4_EHIP;
}

int check_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                   const float* tensor_scale, int rounding, const uint8_t* row_codes,
                   const uint8_t* row_scales, const uint8_t* col_codes, const uint8_t* col_scales,
                   const float* amax_inout) {
    if (rows < 0 || cols < 0 || ld < 0) return UE5M3FP4_EINVAL;
    if (rounding != UE5M3FP4_RNE && rounding != UE5M3FP4_SR) return UE5M3FP4_EINVAL;
    if (cols % 16 != 0) return UE5M3FP4_ESHAPE;
    if (rows >= kMaxDim || cols >= kMaxDim || ld >= kMaxElems) return UE5M3FP4_ERANGE;
    if (ld > 0 && rows > (kMaxElems - 1) / ld) return UE5M3FP4_ERANGE;  // rows * ld >= 2^40, unmultiplied
    if (rows == 0 || cols == 0) return UE5M3FP4_OK;  // empty tensor: nothing to do
    const bool row = row_codes || row_scales;
    const bool col = col_codes || col_scales;
    if (!x) return UE5M3FP4_EINVAL;
    if ((row_codes == nullptr) != (row_scales == nullptr)) return UE5M3FP4_EINVAL;
    if ((col_codes == nullptr) != (col_scales == nullptr)) return UE5M3FP4_EINVAL;
    if (!row && !col && !amax_inout) return UE5M3FP4_EINVAL;  // nothing requested
    if ((row || col) && !tensor_scale) return UE5M3FP4_EINVAL;
    if (col && rows % 16 != 0) return UE5M3FP4_ESHAPE;
    if (ld < cols) return UE5M3FP4_ESHAPE;
    if (ld % 8 != 0 || !aligned16(x)) return UE5M3FP4_EALIGN;
    if ((row && (!aligned16(row_codes) || !aligned16(row_scales))) ||
        (col && (!aligned16(col_codes) || !aligned16(col_scales))) ||
        (tensor_scale && !aligned4(tensor_scale)) || (amax_inout && !aligned4(amax_inout)))
        return UE5M3FP4_EALIGN;
    return UE5M3FP4_OK;
}

int check_gemm(const uint8_t* ac, const uint8_t* as, const float* at, const uint8_t* bc,
               const uint8_t* bs, const float* bt, int64_t M, int64_t N, int64_t K,
               const void* c) {
    if (M < 0 || N < 0 || K < 0) return UE5M3FP4_EINVAL;
    if (K % 16 != 0) return UE5M3FP4_ESHAPE;
    if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return UE5M3FP4_ERANGE;
    if (M * N >= kMaxElems || M * K >= kMaxElems || N * K >= kMaxElems) return UE5M3FP4_ERANGE;
    if (M == 0 || N == 0) return UE5M3FP4_OK;  // nothing is read or written
    if (!at || !bt || !c) return UE5M3FP4_EINVAL;
    if (K > 0 && (!ac || !as || !bc || !bs)) return UE5M3FP4_EINVAL;
    if (!aligned16(c) || !aligned4(at) || !aligned4(bt)) return UE5M3FP4_EALIGN;
    if (K > 0 && (!aligned16(ac) || !aligned16(as) || !aligned16(bc) || !aligned16(bs)))
        return UE5M3FP4_EALIGN;
    return UE5M3FP4_OK;
}

int run_gemm(const uint8_t* ac, const uint8_t* as, const float* at, const uint8_t* bc,
             const uint8_t* bs, const float* bt, int64_t M, int64_t N, int64_t K, float* c,
             void* stream) {
    const int st = check_gemm(ac, as, at, bc, bs, bt, M, N, K, c);
    if (st != UE5M3FP4_OK) return st;
    if (M == 0 || N == 0) return UE5M3FP4_OK;
    GemmArgs g{ac, as, at, bc, bs, bt, M, N, K, c, nullptr, nullptr};
    clear_stale_error();
    launch_gemm_nt(g, (hipStream_t)stream);
    return launch_status();
}

int run_gemm_bf16(const uint8_t* ac, const uint8_t* as, const float* at, const uint8_t* bc,
                  const uint8_t* bs, const float* bt, int64_t M, int64_t N, int64_t K, uint16_t* c,
                  float* amax, const OutputQuant& q, void* stream) {
    const int st = check_gemm(ac, as, at, bc, bs, bt, M, N, K, c);
    if (st != UE5M3FP4_OK) return st;
    if (amax && !aligned4(amax)) return UE5M3FP4_EALIGN;
    if (M == 0 || N == 0) return UE5M3FP4_OK;
    GemmArgs g{ac, as, at, bc, bs, bt, M, N, K, nullptr, c, amax, q};
    clear_stale_error();
    launch_gemm_nt(g, (hipStream_t)stream);
    return launch_status();
}

// Arguments of the quantizing epilogue, checked before the GEMM's own.
int check_output_quant(int64_t M, int64_t N, const float* ts, int rounding, const uint8_t* rc,
                       const uint8_t* rs, const uint8_t* cc, const uint8_t* cs) {
    if (!ts) return UE5M3FP4_EINVAL;
    if (rounding != UE5M3FP4_RNE && rounding != UE5M3FP4_SR) return UE5M3FP4_EINVAL;
    if ((rc == nullptr) != (rs == nullptr) || (cc == nullptr) != (cs == nullptr)) return UE5M3FP4_EINVAL;
    if (!rc && !cc) return UE5M3FP4_EINVAL;  // no quantized output requested
    if ((rc && N % 16 != 0) || (cc && M % 16 != 0)) return UE5M3FP4_ESHAPE;
    if (!aligned4(ts) || (rc && (!aligned16(rc) || !aligned16(rs))) ||
        (cc && (!aligned16(cc) || !aligned16(cs))))
        return UE5M3FP4_EALIGN;
    return UE5M3FP4_OK;
}

}  // namespace

extern "C" {

int ue5m3fp4_quantize_blockscale(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                 const float* tensor_scale, int rounding, uint64_t seed,
                                 uint32_t offset, uint8_t* row_codes, uint8_t* row_scales,
                                 uint8_t* col_codes, uint8_t* col_scales, float* amax_inout,
                                 void* stream) {
    const int st = check_quantize(x, rows, cols, ld, tensor_scale, rounding, row_codes, row_scales,
                                  col_codes, col_scales, amax_inout);
    if (st != UE5M3FP4_OK || rows == 0 || cols == 0) return st;
    QuantizeArgs a{x,         rows,      cols,      ld,        tensor_scale, rounding == UE5M3FP4_SR,
                   seed,      offset,    row_codes, row_scales, col_codes,   col_scales,
                   amax_inout};
    clear_stale_error();
    launch_quantize_blockscale(a, (hipStream_t)stream);
    return launch_status();
}

int ue5m3fp4_quantize_blockscale_2d(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                    const float* tensor_scale, int rounding, uint64_t seed,
                                    uint32_t offset, uint8_t* row_codes, uint8_t* row_scales,
                                    uint8_t* col_codes, uint8_t* col_scales, float* amax_inout,
                                    void* stream) {
    if (!row_codes && !row_scales && !col_codes && !col_scales) return UE5M3FP4_EINVAL;
    const int st = check_quantize(x, rows, cols, ld, tensor_scale, rounding, row_codes, row_scales,
                                  col_codes, col_scales, amax_inout);
    if (st != UE5M3FP4_OK) return st;
    if (rows % 16 != 0) return UE5M3FP4_ESHAPE;
    if (rows == 0 || cols == 0) return UE5M3FP4_OK;
    QuantizeArgs a{x,         rows,      cols,      ld,        tensor_scale, rounding == UE5M3FP4_SR,
                   seed,      offset,    row_codes, row_scales, col_codes,   col_scales,
                   amax_inout};
    clear_stale_error();
    launch_quantize_2d(a, (hipStream_t)stream);
    return launch_status();
}

int ue5m3fp4_quantize_current_scaling(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                      float max_safe, int rounding, uint64_t seed, uint32_t offset,
                                      uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                                      uint8_t* col_scales, float* tensor_scale, float* amax_out,
                                      void* stream) {
    if (!tensor_scale || !amax_out) return UE5M3FP4_EINVAL;
    if (!(max_safe > 0.0f) || !std::isfinite(max_safe)) return UE5M3FP4_EINVAL;
    if (!row_codes && !col_codes) return UE5M3FP4_EINVAL;  // no output requested
    const int st = check_quantize(x, rows, cols, ld, tensor_scale, rounding, row_codes, row_scales,
                                  col_codes, col_scales, amax_out);
    if (st != UE5M3FP4_OK || rows == 0 || cols == 0) return st;
    const hipStream_t s = (hipStream_t)stream;
    // 1. amax pass over x
    clear_stale_error();
    launch_zero_scalar(amax_out, s);
    QuantizeArgs pre{x, rows, cols, ld, nullptr, false, 0, 0, nullptr, nullptr, nullptr, nullptr, amax_out,
                     nullptr, 0.0f};
    launch_quantize_blockscale(pre, s);
    // 2. block quantization under this tensor's own scale, which the
    //    quantizer derives from the amax (and stores to *tensor_scale)
    QuantizeArgs q{x,         rows,      cols,      ld,        tensor_scale, rounding == UE5M3FP4_SR,
                   seed,      offset,    row_codes, row_scales, col_codes,   col_scales,
                   nullptr,   amax_out,  max_safe};
    launch_quantize_blockscale(q, s);
    return launch_status();
}

int ue5m3fp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                        int64_t rows, int64_t cols, float* out, void* stream) {
    if (rows < 0 || cols < 0) return UE5M3FP4_EINVAL;
    if (cols % 16 != 0) return UE5M3FP4_ESHAPE;
    if (rows >= kMaxDim || cols >= kMaxDim || rows * cols >= kMaxElems) return UE5M3FP4_ERANGE;
    if (rows == 0 || cols == 0) return UE5M3FP4_OK;
    if (!codes || !scales || !tensor_scale || !out) return UE5M3FP4_EINVAL;
    if (!aligned16(codes) || !aligned16(scales) || !aligned4(tensor_scale) || !aligned16(out))
        return UE5M3FP4_EALIGN;
    clear_stale_error();
    launch_dequantize(codes, scales, tensor_scale, rows, cols, out, (hipStream_t)stream);
    return launch_status();
}

int ue5m3fp4_stream_reference(const uint16_t* x, int64_t elems, uint8_t* codes0, uint8_t* scales0,
                              uint8_t* codes1, uint8_t* scales1, void* stream) {
    if (elems < 0) return UE5M3FP4_EINVAL;
    if (elems % 16 != 0) return UE5M3FP4_ESHAPE;
    if (elems >= kMaxElems) return UE5M3FP4_ERANGE;
    if (elems == 0) return UE5M3FP4_OK;
    if (!x || !codes0 || !scales0 || (codes1 == nullptr) != (scales1 == nullptr)) return UE5M3FP4_EINVAL;
    if (!aligned16(x) || !aligned16(codes0) || (codes1 && !aligned16(codes1))) return UE5M3FP4_EALIGN;
    clear_stale_error();
    launch_stream_reference(x, elems, codes0, scales0, codes1, scales1, (hipStream_t)stream);
    return launch_status();
}

int ue5m3fp4_gemm_nt(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                     const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                     int64_t M, int64_t N, int64_t K, float* c, void* stream) {
    return run_gemm(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, M, N, K, c, stream);
}

int ue5m3fp4_gemm_nt_bf16(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                          const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                          int64_t M, int64_t N, int64_t K, uint16_t* c, float* amax_inout,
                          void* stream) {
    return run_gemm_bf16(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, M, N, K, c, amax_inout,
                         OutputQuant{}, stream);
}

int ue5m3fp4_gemm_nt_bf16_quantized(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                                    const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                                    int64_t M, int64_t N, int64_t K, uint16_t* c, float* amax_inout,
                                    const float* c_tensor_scale, int rounding, uint64_t seed,
                                    uint32_t offset, uint8_t* c_row_codes, uint8_t* c_row_scales,
                                    uint8_t* c_col_codes, uint8_t* c_col_scales, void* stream) {
    if (M < 0 || N < 0 || K < 0) return UE5M3FP4_EINVAL;
    const int st = check_output_quant(M, N, c_tensor_scale, rounding, c_row_codes, c_row_scales,
                                      c_col_codes, c_col_scales);
    if (st != UE5M3FP4_OK) return st;
    const OutputQuant q{c_tensor_scale, c_row_codes, c_row_scales, c_col_codes, c_col_scales,
                        seed, offset, rounding == UE5M3FP4_SR};
    return run_gemm_bf16(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, M, N, K, c, amax_inout, q,
                         stream);
}

int ue5m3fp4_gemm_nt_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                           const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                           int64_t M, int64_t N, int64_t K, float* c, void* stream) {
    if (K >= 0 && K % 32 != 0) return UE5M3FP4_ESHAPE;
    const int st = check_gemm(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, M, N, K, c);
    if (st != UE5M3FP4_OK || M == 0 || N == 0) return st;
    GemmArgs g{a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, M, N, K, c, nullptr, nullptr};
    if (K == 0) {  // an empty sum: the UE5M3 kernel writes the zeros
        clear_stale_error();
        launch_gemm_nt(g, (hipStream_t)stream);
        return launch_status();
    }
    clear_stale_error();
    launch_gemm_nt_mx(g, (hipStream_t)stream);
    return launch_status();
}

int ue5m3fp4_gemm_fprop(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_ts,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_ts,
                        int64_t tokens, int64_t in_features, int64_t out_features, float* y,
                        void* stream) {
    // Y[t][o] = sum_i X[t][i] W[o][i]
    return run_gemm(x_codes, x_scales, x_ts, w_codes, w_scales, w_ts, tokens, out_features,
                    in_features, y, stream);
}

int ue5m3fp4_gemm_dgrad(const uint8_t* dy_codes, const uint8_t* dy_scales, const float* dy_ts,
                        const uint8_t* wt_codes, const uint8_t* wt_scales, const float* w_ts,
                        int64_t tokens, int64_t in_features, int64_t out_features, float* dx,
                        void* stream) {
    // dX[t][i] = sum_o dY[t][o] W^T[i][o]
    return run_gemm(dy_codes, dy_scales, dy_ts, wt_codes, wt_scales, w_ts, tokens, in_features,
                    out_features, dx, stream);
}

int ue5m3fp4_gemm_wgrad(const uint8_t* dyt_codes, const uint8_t* dyt_scales, const float* dy_ts,
                        const uint8_t* xt_codes, const uint8_t* xt_scales, const float* x_ts,
                        int64_t tokens, int64_t in_features, int64_t out_features, float* dw,
                        void* stream) {
    // dW[o][i] = sum_t dY^T[o][t] X^T[i][t]
    return run_gemm(dyt_codes, dyt_scales, dy_ts, xt_codes, xt_scales, x_ts, out_features,
                    in_features, tokens, dw, stream);
}

int ue5m3fp4_update_tensor_scale(float* amax_running, float* tensor_scale, int64_t step,
                                 int64_t period, float max_safe, void* stream) {
    if (!amax_running || !tensor_scale) return UE5M3FP4_EINVAL;
    if (period < 1 || step < 0) return UE5M3FP4_EINVAL;
    if (!(max_safe > 0.0f) || !std::isfinite(max_safe)) return UE5M3FP4_EINVAL;
    if (!aligned4(amax_running) || !aligned4(tensor_scale)) return UE5M3FP4_EALIGN;
    if (step % period != 0) return UE5M3FP4_OK;
    clear_stale_error();
    launch_update_tensor_scale(amax_running, tensor_scale, max_safe, (hipStream_t)stream);
    return launch_status();
}

const char* ue5m3fp4_status_string(int status) {
    switch (status) {
        case UE5M3FP4_OK: return "ok";
        case UE5M3FP4_EINVAL: return "invalid argument (NULL pointer, negative size, unknown mode)";
        case UE5M3FP4_ESHAPE: return "shape violates the block-16 layout or sizes disagree";
        case UE5M3FP4_EALIGN: return "misaligned pointer or leading dimension";
        case UE5M3FP4_EHIP: return "HIP runtime error at launch";
        case UE5M3FP4_ERANGE: return "size exceeds the library's index range";
        default: return "unknown status";
    }
}

}  // extern "C"
