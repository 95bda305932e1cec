"""CPU tests of the C ABI: the library loads, exports every function that
include/ue5m3fp4.h declares, and rejects bad arguments on the host before any
HIP call (so no GPU is needed: the pointers below are never dereferenced).
"""

import ctypes
import os
import re

import pytest

import fp4_block_scaled_amax_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ue5m3fp4.h")

OK, EINVAL, ESHAPE, EALIGN, EHIP, ERANGE = 0, -1, -2, -3, -4, -5
P = 0x10000  # a 16-byte aligned fake device address (never dereferenced)
M4 = 0x10004  # 4-byte but not 16-byte aligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        pytest.fail("libue5m3fp4.so is not built (python -m fp4_block_scaled_amax_amd.build)")
    return lib.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"UE5M3FP4_API\s+(?:const\s+)?\w+\**\s+\**(ue5m3fp4_\w+)\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 14, names
    for n in names:
        assert hasattr(L, n), n
    # and only those: internal C++ symbols stay hidden
    out = os.popen(f"nm -D --defined-only {lib.LIB_PATH}").read()
    exported = sorted(re.findall(r" T (\S+)", out))
    assert exported == names, exported


def test_status_strings(L):
    for s in (OK, EINVAL, ESHAPE, EALIGN, EHIP, ERANGE):
        assert len(lib.status_string(s)) >= 2
    assert lib.status_string(12345) == "unknown status"


def q(L, x=P, rows=32, cols=32, ld=32, ts=P, rnd=0, rc=P, rs=P, cc=P, cs=P, amax=None):
    return L.ue5m3fp4_quantize_blockscale(x, rows, cols, ld, ts, rnd, 0, 0, rc, rs, cc, cs, amax,
                                          None)


def test_quantize_argument_checks(L):
    assert q(L, rows=-1) == EINVAL
    assert q(L, rnd=2) == EINVAL
    assert q(L, x=None) == EINVAL
    assert q(L, rc=None) == EINVAL              # half of a pair
    assert q(L, cs=None) == EINVAL
    assert q(L, rc=None, rs=None, cc=None, cs=None) == EINVAL  # nothing requested
    assert q(L, ts=None) == EINVAL
    assert q(L, cols=40, ld=40) == ESHAPE       # cols % 16
    assert q(L, rows=40) == ESHAPE              # transposed output needs rows % 16
    assert q(L, ld=16) == ESHAPE                # ld < cols
    assert q(L, ld=36) == EALIGN                # ld % 8
    assert q(L, x=P + 8) == EALIGN
    assert q(L, rc=P + 4) == EALIGN
    assert q(L, ts=P + 2) == EALIGN
    assert q(L, rows=1 << 31) == ERANGE
    assert q(L, rows=1 << 20, ld=1 << 20) == ERANGE   # rows * ld = 2^40
    assert q(L, rows=(1 << 31) - 1, ld=1 << 39) == ERANGE  # a product past 2^63 must not wrap
    assert q(L, ld=1 << 62) == ERANGE
    # empty tensors are valid no-ops and touch nothing (even NULL pointers)
    assert q(L, rows=0, x=None, rc=None, rs=None, cc=None, cs=None) == OK
    assert q(L, cols=0, ld=0, x=None) == OK


def q2(L, x=P, rows=32, cols=32, ld=32, ts=P, rnd=0, rc=P, rs=P, cc=P, cs=P, amax=None):
    return L.ue5m3fp4_quantize_blockscale_2d(x, rows, cols, ld, ts, rnd, 0, 0, rc, rs, cc, cs, amax,
                                             None)


def test_quantize_2d_argument_checks(L):
    assert q2(L, rows=-1) == EINVAL
    assert q2(L, rnd=2) == EINVAL
    assert q2(L, x=None) == EINVAL
    assert q2(L, rc=None) == EINVAL             # half of a pair
    assert q2(L, rc=None, rs=None, cc=None, cs=None, amax=P) == EINVAL  # no output
    assert q2(L, ts=None) == EINVAL
    assert q2(L, cols=40, ld=40) == ESHAPE      # cols % 16
    assert q2(L, rows=40, cc=None, cs=None) == ESHAPE  # rows % 16, even row-only
    assert q2(L, ld=16) == ESHAPE
    assert q2(L, ld=36) == EALIGN
    assert q2(L, cc=P + 4) == EALIGN
    assert q2(L, amax=P + 2) == EALIGN
    assert q2(L, rows=1 << 31) == ERANGE
    assert q2(L, rows=0, x=None) == OK          # empty tensor: nothing launched


def qc(L, x=P, rows=32, cols=32, ld=32, ms=7168.0, rnd=0, rc=P, rs=P, cc=P, cs=P, ts=P, amax=P):
    return L.ue5m3fp4_quantize_current_scaling(x, rows, cols, ld, ms, rnd, 0, 0, rc, rs, cc, cs, ts,
                                               amax, None)


def test_current_scaling_argument_checks(L):
    assert qc(L, ts=None) == EINVAL
    assert qc(L, amax=None) == EINVAL
    assert qc(L, ms=0.0) == EINVAL
    assert qc(L, ms=float("inf")) == EINVAL
    assert qc(L, ms=float("nan")) == EINVAL
    assert qc(L, rc=None, rs=None, cc=None, cs=None) == EINVAL  # an amax pass alone is not this call
    assert qc(L, rnd=3) == EINVAL
    assert qc(L, cols=40, ld=40) == ESHAPE
    assert qc(L, rows=40) == ESHAPE
    assert qc(L, amax=P + 2) == EALIGN
    assert qc(L, x=P + 8) == EALIGN
    assert qc(L, rows=0, x=None) == OK  # empty tensor: nothing launched


def test_gemm_argument_checks(L):
    g = L.ue5m3fp4_gemm_nt
    assert g(P, P, P, P, P, P, -1, 4, 16, P, None) == EINVAL
    assert g(P, P, P, P, P, P, 4, 4, 24, P, None) == ESHAPE       # K % 16
    assert g(None, P, P, P, P, P, 4, 4, 16, P, None) == EINVAL
    assert g(P, P, None, P, P, P, 4, 4, 16, P, None) == EINVAL
    assert g(P, P, P, P, P, P, 4, 4, 16, None, None) == EINVAL
    assert g(P + 8, P, P, P, P, P, 4, 4, 16, P, None) == EALIGN
    assert g(P, P, M4, P, P, M4, 4, 4, 16, P + 4, None) == EALIGN  # output alignment
    assert g(P, P, P, P, P, P, 1 << 31, 4, 16, P, None) == ERANGE
    assert g(None, None, None, None, None, None, 0, 4, 16, None, None) == OK  # empty output
    # (tokens, in, out) with the contraction axis of each GEMM not a multiple of 16;
    # every call here must fail validation (the fake pointers are never launched on)
    for name, dims in (("ue5m3fp4_gemm_fprop", (16, 24, 16)),
                       ("ue5m3fp4_gemm_dgrad", (16, 16, 24)),
                       ("ue5m3fp4_gemm_wgrad", (24, 16, 16))):
        fn = getattr(L, name)
        assert fn(P, P, P, P, P, P, *dims, P, None) == ESHAPE
        assert fn(P, P, P, P, P, P, 0, 0, 0, None, None) == OK


def test_gemm_bf16_argument_checks(L):
    g = L.ue5m3fp4_gemm_nt_bf16
    assert g(P, P, P, P, P, P, 4, 4, 24, P, None, None) == ESHAPE       # K % 16
    assert g(P, P, P, P, P, P, 4, 4, 16, None, None, None) == EINVAL     # no output
    assert g(P, P, P, P, P, P, 4, 4, 16, P + 2, None, None) == EALIGN
    assert g(P, P, P, P, P, P, 4, 4, 16, P, P + 2, None) == EALIGN       # amax alignment
    assert g(P, P, P, P, P, P, 1 << 31, 4, 16, P, None, None) == ERANGE
    assert g(None, None, None, None, None, None, 4, 0, 16, None, None, None) == OK  # empty


def test_gemm_bf16_quantized_argument_checks(L):
    def g(M=32, N=32, K=32, c=P, ts=P, rnd=0, rc=P, rs=P, cc=P, cs=P, ac=P):
        return L.ue5m3fp4_gemm_nt_bf16_quantized(ac, P, P, P, P, P, M, N, K, c, None, ts, rnd, 0, 0,
                                                 rc, rs, cc, cs, None)
    assert g(M=-1) == EINVAL
    assert g(ts=None) == EINVAL
    assert g(rnd=2) == EINVAL
    assert g(rc=None) == EINVAL                       # half of a pair
    assert g(rc=None, rs=None, cc=None, cs=None) == EINVAL  # nothing to quantize
    assert g(N=40) == ESHAPE                          # row output needs N % 16
    assert g(M=40) == ESHAPE                          # transposed output needs M % 16
    assert g(K=24) == ESHAPE                          # K % 16
    assert g(rc=P + 4) == EALIGN
    assert g(ts=P + 2) == EALIGN
    assert g(c=None) == EINVAL
    assert g(ac=None) == EINVAL


def test_gemm_mxfp4_argument_checks(L):
    g = L.ue5m3fp4_gemm_nt_mxfp4
    assert g(P, P, P, P, P, P, 4, 4, 48, P, None) == ESHAPE       # K % 32
    assert g(P, P, P, P, P, P, -1, 4, 32, P, None) == EINVAL
    assert g(None, P, P, P, P, P, 4, 4, 32, P, None) == EINVAL
    assert g(P, P, P, P, P, P, 4, 4, 32, P + 4, None) == EALIGN
    assert g(P, P, P, P, P, P, 1 << 31, 4, 32, P, None) == ERANGE
    assert g(None, None, None, None, None, None, 0, 4, 32, None, None) == OK


def test_fprop_dgrad_wgrad_contract_the_right_axis(L):
    """fprop contracts over in_features, dgrad over out_features, wgrad over
    tokens: only that axis has to be a multiple of 16."""
    f, d, w = L.ue5m3fp4_gemm_fprop, L.ue5m3fp4_gemm_dgrad, L.ue5m3fp4_gemm_wgrad
    # (tokens, in, out) = (8, 24, 16): in % 16 != 0
    assert f(P, P, P, P, P, P, 0, 24, 16, None, None) == ESHAPE
    assert d(P, P, P, P, P, P, 0, 24, 16, None, None) == OK
    # (tokens, in, out) = (24, 16, 8): tokens % 16 != 0 only matters for wgrad
    assert w(P, P, P, P, P, P, 24, 0, 0, None, None) == ESHAPE


def test_dequantize_and_update_checks(L):
    dq = L.ue5m3fp4_dequantize
    assert dq(P, P, P, 4, 24, P, None) == ESHAPE
    assert dq(None, P, P, 4, 16, P, None) == EINVAL
    assert dq(P, P, P, 4, 16, P + 4, None) == EALIGN
    assert dq(None, None, None, 0, 16, None, None) == OK
    up = L.ue5m3fp4_update_tensor_scale
    assert up(None, P, 0, 1, ctypes.c_float(7168.0), None) == EINVAL
    assert up(P, P, 0, 0, ctypes.c_float(7168.0), None) == EINVAL    # period < 1
    assert up(P, P, -1, 1, ctypes.c_float(7168.0), None) == EINVAL
    assert up(P, P, 0, 1, ctypes.c_float(0.0), None) == EINVAL
    assert up(P, P, 0, 1, ctypes.c_float(float("inf")), None) == EINVAL
    assert up(P + 2, P, 0, 1, ctypes.c_float(7168.0), None) == EALIGN
    assert up(P, P, 3, 2, ctypes.c_float(7168.0), None) == OK        # not a refresh step


def test_binding_requires_built_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        lib._lib, saved = None, lib._lib
        try:
            lib.load_library(str(tmp_path / "nope.so"))
        finally:
            lib._lib = saved


def test_stream_reference_checks(L):
    sr = L.ue5m3fp4_stream_reference
    assert sr(P, 24, P, P, None, None, None) == ESHAPE
    assert sr(P, -16, P, P, None, None, None) == EINVAL
    assert sr(None, 16, P, P, None, None, None) == EINVAL
    assert sr(P, 16, P, None, None, None, None) == EINVAL
    assert sr(P, 16, P, P, P, None, None) == EINVAL       # one of the second pair
    assert sr(M4, 16, P, P, None, None, None) == EALIGN
    assert sr(P, 16, P, P, M4, P, None) == EALIGN
    assert sr(P, 1 << 40, P, P, None, None, None) == ERANGE
    assert sr(None, 0, None, None, None, None, None) == OK
