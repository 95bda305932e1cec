"""Python binding of libue5m3fp4: UE5M3-FP4 block-16 quantization and the
block-scaled training GEMMs on MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of
libue5m3fp4.so (built in-tree by fp4_block_scaled_amax_amd/build.py).  The
functions take torch tensors for device memory and use torch's current HIP
stream unless one is given.  There is no fallback: if the library is missing
or a call fails, an exception is raised.

The method: "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining"
(arXiv 2609.02846), abstract.  The C ABI and all layouts are documented in
include/ue5m3fp4.h.
"""

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libue5m3fp4.so")

RNE = 0
SR = 1
MAX_SAFE_DEFAULT = 7168.0  # 114688 / 16: block scale of the largest block at refresh time

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64

_SIGNATURES = {
    "ue5m3fp4_quantize_blockscale": [_c_void_p, _i64, _i64, _i64, _c_void_p, ctypes.c_int,
                                     ctypes.c_uint64, ctypes.c_uint32, _c_void_p, _c_void_p,
                                     _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "ue5m3fp4_quantize_blockscale_2d": [_c_void_p, _i64, _i64, _i64, _c_void_p, ctypes.c_int,
                                        ctypes.c_uint64, ctypes.c_uint32, _c_void_p, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "ue5m3fp4_dequantize": [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p],
    "ue5m3fp4_gemm_nt": [_c_void_p] * 6 + [_i64, _i64, _i64, _c_void_p, _c_void_p],
    "ue5m3fp4_gemm_nt_bf16": [_c_void_p] * 6 + [_i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p],
    "ue5m3fp4_gemm_nt_bf16_quantized": [_c_void_p] * 6 + [_i64, _i64, _i64, _c_void_p, _c_void_p,
                                                          _c_void_p, ctypes.c_int, ctypes.c_uint64,
                                                          ctypes.c_uint32] + [_c_void_p] * 5,
    "ue5m3fp4_gemm_nt_mxfp4": [_c_void_p] * 6 + [_i64, _i64, _i64, _c_void_p, _c_void_p],
    "ue5m3fp4_gemm_fprop": [_c_void_p] * 6 + [_i64, _i64, _i64, _c_void_p, _c_void_p],
    "ue5m3fp4_gemm_dgrad": [_c_void_p] * 6 + [_i64, _i64, _i64, _c_void_p, _c_void_p],
    "ue5m3fp4_gemm_wgrad": [_c_void_p] * 6 + [_i64, _i64, _i64, _c_void_p, _c_void_p],
    "ue5m3fp4_update_tensor_scale": [_c_void_p, _c_void_p, _i64, _i64, ctypes.c_float,
                                     _c_void_p],
    "ue5m3fp4_quantize_current_scaling": [_c_void_p, _i64, _i64, _i64, ctypes.c_float, ctypes.c_int,
                                          ctypes.c_uint64, ctypes.c_uint32, _c_void_p, _c_void_p,
                                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "ue5m3fp4_stream_reference": [_c_void_p, _i64] + [_c_void_p] * 5,
}

_lib = None


class Ue5m3Fp4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def load_library(path=LIB_PATH):
    """Load libue5m3fp4.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m fp4_block_scaled_amax_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(path)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.ue5m3fp4_status_string.argtypes = [ctypes.c_int]
    lib.ue5m3fp4_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status):
    return load_library().ue5m3fp4_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise Ue5m3Fp4Error(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _require(t, dtypes, name, dims=None, contiguous=False):
    if t is None:
        raise ValueError(f"{name} is required")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_scalar(t, name):
    """A device fp32 scalar (tensor scale, amax): one element."""
    import torch

    _require(t, (torch.float32,), name)
    if t.numel() != 1:
        raise ValueError(f"{name} must hold exactly one fp32 value (has {t.numel()})")


def _check_pair(codes, scales, rows, cols, name):
    """Code and scale buffers of a rows x cols operand blocked along cols:
    contiguous uint8 [rows][cols/2] and [rows][cols/16] on the device."""
    import torch

    _require(codes, (torch.uint8,), f"{name} codes", 2, contiguous=True)
    _require(scales, (torch.uint8,), f"{name} scales", 2, contiguous=True)
    if tuple(codes.shape) != (rows, cols // 2) or tuple(scales.shape) != (rows, cols // 16):
        raise ValueError(f"{name}: codes {tuple(codes.shape)} / scales {tuple(scales.shape)} do not "
                         f"match a {rows} x {cols} operand ([{rows}][{cols // 2}], [{rows}][{cols // 16}])")
    if codes.device != scales.device:
        raise ValueError(f"{name}: codes and scales are on different devices")


def _check_operand(q, name):
    """A Quantized operand: contiguous device codes [R][C/2] and scales
    [R][C/16] (C % 16 == 0), and a one-element device fp32 tensor scale."""
    if not isinstance(q, Quantized):
        raise ValueError(f"{name} must be a Quantized operand")
    _require(q.codes, (__import__("torch").uint8,), f"{name} codes", 2)
    if q.codes.shape[1] % 8 != 0:
        raise ValueError(f"{name}: cols ({q.codes.shape[1] * 2}) must be a multiple of 16")
    _check_pair(q.codes, q.scales, q.codes.shape[0], q.codes.shape[1] * 2, name)
    _require_scalar(q.ts, f"{name} ts")
    if q.ts.device != q.codes.device:
        raise ValueError(f"{name}: ts is on another device than its codes")


def _same_device(name, *ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"{name}: tensors on different devices {sorted(map(str, devs))}")


@dataclass
class Quantized:
    """One block-scaled operand: codes [R][C/2] uint8, scales [R][C/16] uint8,
    ts = device fp32 tensor scale (1 element).  Blocks run along C."""

    codes: "object"
    scales: "object"
    ts: "object"

    @property
    def rows(self):
        return self.codes.shape[0]

    @property
    def cols(self):
        return self.codes.shape[1] * 2


def empty_quantized(rows, cols, ts, device=None):
    """Allocate the code and scale buffers of a rows x cols operand."""
    import torch

    device = device if device is not None else ts.device
    return Quantized(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                     torch.empty((rows, cols // 16), dtype=torch.uint8, device=device), ts)


def _quantize_operands(x, tensor_scale, row, col, amax):
    """Check and unpack the arguments shared by the quantizer entry points."""
    import torch

    _require(x, (torch.bfloat16, torch.int16, torch.uint16), "x", 2)
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along its columns")
    rows, cols = x.shape
    rc, rs, cc, cs = _output_pairs(row, col, rows, cols)
    if tensor_scale is not None:
        _require_scalar(tensor_scale, "tensor_scale")
    if amax is not None:
        _require_scalar(amax, "amax")
    _same_device("quantize", x, rc, rs, cc, cs, tensor_scale, amax)
    return rows, cols, rc, rs, cc, cs


def _output_pairs(row, col, rows, cols):
    """(codes, scales) of the row-wise output (rows x cols, blocked along
    cols) and of the transposed output (cols x rows, blocked along rows),
    each None or checked: contiguous device uint8 of the exact shapes."""
    rc = rs = cc = cs = None
    if row is not None:
        rc, rs = (row.codes, row.scales) if isinstance(row, Quantized) else row
        _check_pair(rc, rs, rows, cols, "row output")
    if col is not None:
        cc, cs = (col.codes, col.scales) if isinstance(col, Quantized) else col
        _check_pair(cc, cs, cols, rows, "col output")
    return rc, rs, cc, cs


def quantize_blockscale(x, tensor_scale, rounding=RNE, seed=0, offset=0, row=None, col=None,
                        amax=None, stream=None):
    """Quantize a bf16 (rows x cols) tensor.  row / col: Quantized outputs (or
    (codes, scales) pairs) for the row-wise and the transposed orientation, or
    None.  amax: device fp32 scalar that receives max(amax, max|x|)."""
    rows, cols, rc, rs, cc, cs = _quantize_operands(x, tensor_scale, row, col, amax)
    st = load_library().ue5m3fp4_quantize_blockscale(
        _ptr(x), rows, cols, x.stride(0), _ptr(tensor_scale), int(rounding), int(seed),
        int(offset), _ptr(rc), _ptr(rs), _ptr(cc), _ptr(cs), _ptr(amax), _stream(stream))
    _check(st, "ue5m3fp4_quantize_blockscale")


def quantize_blockscale_2d(x, tensor_scale, rounding=RNE, seed=0, offset=0, row=None, col=None,
                           amax=None, stream=None):
    """Quantize with one scale per 16 x 16 tile (transposition-invariant):
    the same arguments and output layouts as quantize_blockscale, the tile
    scale repeated over its rows / columns; col codes are the transpose of
    the row codes.  rows and cols must be multiples of 16."""
    rows, cols, rc, rs, cc, cs = _quantize_operands(x, tensor_scale, row, col, amax)
    st = load_library().ue5m3fp4_quantize_blockscale_2d(
        _ptr(x), rows, cols, x.stride(0), _ptr(tensor_scale), int(rounding), int(seed),
        int(offset), _ptr(rc), _ptr(rs), _ptr(cc), _ptr(cs), _ptr(amax), _stream(stream))
    _check(st, "ue5m3fp4_quantize_blockscale_2d")


def dequantize(q, out, stream=None):
    """out (fp32 [R][C]) = ts * s_b * e2m1 of the quantized operand q."""
    import torch

    _check_operand(q, "q")
    _require(out, (torch.float32,), "out", 2, contiguous=True)
    if tuple(out.shape) != (q.rows, q.cols):
        raise ValueError("out has the wrong shape")
    _same_device("dequantize", q.codes, out)
    st = load_library().ue5m3fp4_dequantize(_ptr(q.codes), _ptr(q.scales), _ptr(q.ts), q.rows,
                                            q.cols, _ptr(out), _stream(stream))
    _check(st, "ue5m3fp4_dequantize")
    return out


def stream_reference(x, row, col=None, stream=None):
    """Measurement aid (no quantization): the byte traffic of a quantize call
    on x (bf16 [R][C], contiguous) as contiguous streams into the code and
    scale buffers of `row` (and `col`), each a (codes, scales) pair or a
    Quantized of the matching shape.  Its time is the HBM rate the
    quantizer's read/write mix can reach."""
    import torch

    _require(x, (torch.bfloat16, torch.int16, torch.uint16), "x", 2, contiguous=True)
    rows, cols = x.shape
    if cols % 16 != 0:
        raise ValueError("x: cols must be a multiple of 16")
    pairs = []
    for name, out, r, c in (("row", row, rows, cols), ("col", col, cols, rows)):
        if out is None:
            pairs.append((None, None))
            continue
        codes, scales = (out.codes, out.scales) if isinstance(out, Quantized) else out
        _check_pair(codes, scales, r, c, name)
        _same_device("stream_reference", x, codes)
        pairs.append((codes, scales))
    if pairs[0][0] is None:
        raise ValueError("row is required")
    st = load_library().ue5m3fp4_stream_reference(_ptr(x), rows * cols, _ptr(pairs[0][0]), _ptr(pairs[0][1]),
                                                  _ptr(pairs[1][0]), _ptr(pairs[1][1]), _stream(stream))
    _check(st, "ue5m3fp4_stream_reference")


def _gemm_out(out, m, n, dtypes=None):
    import torch

    _require(out, dtypes or (torch.float32,), "out", 2)
    if tuple(out.shape) != (m, n) or not out.is_contiguous():
        raise ValueError(f"output must be a contiguous [{m}][{n}] tensor")


def _gemm_operands(a, b, out, na="A", nb="B"):
    """Both operands checked, blocked along the same K, on out's device."""
    _check_operand(a, na)
    _check_operand(b, nb)
    if a.cols != b.cols:
        raise ValueError(f"{na} and {nb} disagree on the contraction axis ({a.cols} vs {b.cols})")
    _same_device("gemm", a.codes, b.codes, out)


def gemm_nt(a, b, out, stream=None):
    """out[M][N] = tsA * tsB * A B^T with A (M x K) and B (N x K) blocked along K."""
    _gemm_operands(a, b, out)
    _gemm_out(out, a.rows, b.rows)
    st = load_library().ue5m3fp4_gemm_nt(_ptr(a.codes), _ptr(a.scales), _ptr(a.ts),
                                         _ptr(b.codes), _ptr(b.scales), _ptr(b.ts), a.rows,
                                         b.rows, a.cols, _ptr(out), _stream(stream))
    _check(st, "ue5m3fp4_gemm_nt")
    return out


def gemm_nt_bf16(a, b, out, amax=None, stream=None):
    """out[M][N] (bf16) = bf16(tsA * tsB * A B^T), round to nearest even;
    amax (device fp32 scalar or None) receives max(amax, max|out|)."""
    import torch

    _gemm_operands(a, b, out)
    _gemm_out(out, a.rows, b.rows, (torch.bfloat16, torch.int16, torch.uint16))
    if amax is not None:
        _require_scalar(amax, "amax")
        _same_device("gemm_nt_bf16", out, amax)
    st = load_library().ue5m3fp4_gemm_nt_bf16(_ptr(a.codes), _ptr(a.scales), _ptr(a.ts),
                                              _ptr(b.codes), _ptr(b.scales), _ptr(b.ts), a.rows,
                                              b.rows, a.cols, _ptr(out), _ptr(amax), _stream(stream))
    _check(st, "ue5m3fp4_gemm_nt_bf16")
    return out


def gemm_nt_bf16_quantized(a, b, out, out_ts, rounding=RNE, seed=0, offset=0, row=None, col=None,
                           amax=None, stream=None):
    """gemm_nt_bf16 whose epilogue also quantizes the bf16 output for the next
    linear: row / col (Quantized or (codes, scales), or None) receive exactly
    what quantize_blockscale(out, out_ts, rounding, seed, offset, ...) would
    write.  out_ts: the output's device fp32 tensor scale."""
    import torch

    _gemm_operands(a, b, out)
    M, N = a.rows, b.rows
    _gemm_out(out, M, N, (torch.bfloat16, torch.int16, torch.uint16))
    _require_scalar(out_ts, "out_ts")
    if amax is not None:
        _require_scalar(amax, "amax")
    rc, rs, cc, cs = _output_pairs(row, col, M, N)
    _same_device("gemm_nt_bf16_quantized", out, out_ts, amax, rc, rs, cc, cs)
    st = load_library().ue5m3fp4_gemm_nt_bf16_quantized(
        _ptr(a.codes), _ptr(a.scales), _ptr(a.ts), _ptr(b.codes), _ptr(b.scales), _ptr(b.ts), M, N,
        a.cols, _ptr(out), _ptr(amax), _ptr(out_ts), int(rounding), int(seed), int(offset), _ptr(rc),
        _ptr(rs), _ptr(cc), _ptr(cs), _stream(stream))
    _check(st, "ue5m3fp4_gemm_nt_bf16_quantized")
    return out


def gemm_nt_mxfp4(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, out, stream=None):
    """Native MXFP4 comparison GEMM: out[M][N] = tsA * tsB * A B^T with E2M1
    codes ([rows][K/2]) and E8M0 scales per 32 elements ([rows][K/32])."""
    import torch

    for t, n in ((a_codes, "a_codes"), (a_scales, "a_scales"), (b_codes, "b_codes"), (b_scales, "b_scales")):
        _require(t, (torch.uint8,), n, 2, contiguous=True)
    _require_scalar(a_ts, "a_ts")
    _require_scalar(b_ts, "b_ts")
    m, k = a_codes.shape[0], a_codes.shape[1] * 2
    n = b_codes.shape[0]
    if b_codes.shape[1] * 2 != k or tuple(a_scales.shape) != (m, k // 32) or tuple(b_scales.shape) != (n, k // 32):
        raise ValueError("MXFP4 operand shapes disagree")
    _gemm_out(out, m, n)
    _same_device("gemm_nt_mxfp4", a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, out)
    st = load_library().ue5m3fp4_gemm_nt_mxfp4(_ptr(a_codes), _ptr(a_scales), _ptr(a_ts), _ptr(b_codes),
                                               _ptr(b_scales), _ptr(b_ts), m, n, k, _ptr(out),
                                               _stream(stream))
    _check(st, "ue5m3fp4_gemm_nt_mxfp4")
    return out


def gemm_fprop(x_row, w_row, y, stream=None):
    """Y [tokens][out] = X W^T from X and W quantized row-wise."""
    _check_operand(x_row, "x_row")
    _check_operand(w_row, "w_row")
    tokens, in_f = x_row.rows, x_row.cols
    out_f = w_row.rows
    if w_row.cols != in_f:
        raise ValueError("X and W disagree on in_features")
    _gemm_out(y, tokens, out_f)
    st = load_library().ue5m3fp4_gemm_fprop(_ptr(x_row.codes), _ptr(x_row.scales), _ptr(x_row.ts),
                                            _ptr(w_row.codes), _ptr(w_row.scales), _ptr(w_row.ts),
                                            tokens, in_f, out_f, _ptr(y), _stream(stream))
    _check(st, "ue5m3fp4_gemm_fprop")
    return y


def gemm_dgrad(dy_row, w_col, dx, stream=None):
    """dX [tokens][in] = dY W from dY row-wise and W's transposed output."""
    _check_operand(dy_row, "dy_row")
    _check_operand(w_col, "w_col")
    tokens, out_f = dy_row.rows, dy_row.cols
    in_f = w_col.rows
    if w_col.cols != out_f:
        raise ValueError("dY and W^T disagree on out_features")
    _gemm_out(dx, tokens, in_f)
    st = load_library().ue5m3fp4_gemm_dgrad(_ptr(dy_row.codes), _ptr(dy_row.scales),
                                            _ptr(dy_row.ts), _ptr(w_col.codes),
                                            _ptr(w_col.scales), _ptr(w_col.ts), tokens, in_f,
                                            out_f, _ptr(dx), _stream(stream))
    _check(st, "ue5m3fp4_gemm_dgrad")
    return dx


def gemm_wgrad(dy_col, x_col, dw, stream=None):
    """dW [out][in] = dY^T X from the transposed outputs of dY and X."""
    _check_operand(dy_col, "dy_col")
    _check_operand(x_col, "x_col")
    out_f, tokens = dy_col.rows, dy_col.cols
    in_f = x_col.rows
    if x_col.cols != tokens:
        raise ValueError("dY^T and X^T disagree on tokens")
    _gemm_out(dw, out_f, in_f)
    st = load_library().ue5m3fp4_gemm_wgrad(_ptr(dy_col.codes), _ptr(dy_col.scales),
                                            _ptr(dy_col.ts), _ptr(x_col.codes),
                                            _ptr(x_col.scales), _ptr(x_col.ts), tokens, in_f,
                                            out_f, _ptr(dw), _stream(stream))
    _check(st, "ue5m3fp4_gemm_wgrad")
    return dw


def quantize_current_scaling(x, tensor_scale, amax, rounding=RNE, seed=0, offset=0, row=None,
                             col=None, max_safe=MAX_SAFE_DEFAULT, stream=None):
    """Current-tensor scaling: amax pass over x into `amax`, tensor_scale =
    amax / (6 max_safe) (left as passed when the amax is 0 or not finite),
    then the block quantization with it.  row / col as in
    quantize_blockscale (at least one)."""
    import torch

    _require(x, (torch.bfloat16, torch.int16, torch.uint16), "x", 2)
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along its columns")
    _require_scalar(tensor_scale, "tensor_scale")
    _require_scalar(amax, "amax")
    rows, cols = x.shape
    rc, rs, cc, cs = _output_pairs(row, col, rows, cols)
    _same_device("quantize_current_scaling", x, tensor_scale, amax, rc, rs, cc, cs)
    st = load_library().ue5m3fp4_quantize_current_scaling(
        _ptr(x), rows, cols, x.stride(0), float(max_safe), int(rounding), int(seed), int(offset),
        _ptr(rc), _ptr(rs), _ptr(cc), _ptr(cs), _ptr(tensor_scale), _ptr(amax), _stream(stream))
    _check(st, "ue5m3fp4_quantize_current_scaling")


def update_tensor_scale(amax_running, tensor_scale, step, period=1,
                        max_safe=MAX_SAFE_DEFAULT, stream=None):
    """Periodic refresh: at step % period == 0, ts = amax / (6 max_safe) if
    amax is finite and > 0, and amax is reset to 0 (both device scalars)."""
    _require_scalar(amax_running, "amax_running")
    _require_scalar(tensor_scale, "tensor_scale")
    _same_device("update_tensor_scale", amax_running, tensor_scale)
    st = load_library().ue5m3fp4_update_tensor_scale(_ptr(amax_running), _ptr(tensor_scale),
                                                     int(step), int(period), float(max_safe),
                                                     _stream(stream))
    _check(st, "ue5m3fp4_update_tensor_scale")
