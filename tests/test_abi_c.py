"""The C ABI from plain C: tests/abi_c_check.c includes include/ue5m3fp4.h,
compiles as strict C99 with warnings as errors, links against the built
libue5m3fp4.so and runs calls whose arguments fail the host-side checks, so
each returns its status before any HIP call (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

import fp4_block_scaled_amax_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

EXPECTED = {
    "quantize_null_x": -1, "quantize_cols_not_16": -2, "quantize_bad_rounding": -1,
    "quantize_rows_too_large": -5, "quantize_empty": 0, "quantize_2d_no_output": -1,
    "current_scaling_null": -1, "dequantize_cols_not_16": -2, "gemm_nt_k_not_16": -2,
    "gemm_fprop_negative": -1, "gemm_dgrad_null": -1, "gemm_wgrad_null_out": -1, "gemm_bf16_null": -1,
    "gemm_quantized_null_ts": -1, "gemm_mxfp4_k_not_32": -2, "update_null": -1, "update_period_0": -1,
    "update_not_this_step": 0, "stream_reference_not_16": -2,
}


def test_header_is_c99_and_checks_run_without_gpu(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    so = lib.LIB_PATH
    if not os.path.exists(so):
        pytest.fail("libue5m3fp4.so is not built (python -m fp4_block_scaled_amax_amd.build)")
    exe = str(tmp_path / "abi_c_check")
    libdir = os.path.dirname(so)
    subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_c_check.c"), "-L", libdir, "-l:" + os.path.basename(so),
                    "-Wl,-rpath," + libdir, "-o", exe], check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=60).stdout.splitlines()
    got = dict(line.split(" ", 1) for line in out)
    assert got.pop("status_string") == lib.status_string(-2)  # ESHAPE
    assert {k: int(v) for k, v in got.items()} == EXPECTED
