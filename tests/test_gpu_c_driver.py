"""The library driven from plain C on the GPU, with no Python or framework
in the process (tests/abi_c_gpu_driver.c: HIP runtime allocations, then the
C ABI for the amax bootstrap, the tensor-scale refresh, the two-orientation
quantization and fprop).  Its outputs against the oracle: tensor scale and
amax exactly, codes and scales of both orientations bit for bit, Y = X X^T
within 1e-5 sum|a b|."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import quantize, tensor_scale
from workloads import random_bf16

from devhelpers import assert_gemm_close

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_driver_matches_oracle(cuda_device, tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    so = lib.LIB_PATH
    exe = str(tmp_path / "driver")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_c_gpu_driver.c"),
                    "-L", os.path.dirname(so), "-l:" + os.path.basename(so), "-L", os.path.join(ROCM, "lib"),
                    "-lamdhip64", "-Wl,-rpath," + os.path.dirname(so), "-Wl,-rpath," + os.path.join(ROCM, "lib"),
                    "-o", exe], check=True, capture_output=True, text=True)
    R, C = 528, 528
    bits = random_bf16((R, C), seed=528, kind="heavy")
    src, dst = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    bits.astype(np.uint16).tofile(src)
    r = subprocess.run([exe, src, dst, str(R), str(C)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(dst, dtype=np.uint8)
    parts, at = [], 0
    for size in (4, 4, R * C // 2, R * C // 16, R * C // 2, R * C // 16, 4 * R * R):
        parts.append(raw[at:at + size])
        at += size
    assert at == raw.size
    ts, amax = parts[0].view(np.float32)[0], parts[1].view(np.float32)[0]
    amax_ref = quantize.tensor_amax(bits)
    _, ts_ref = tensor_scale.update_tensor_scale(amax_ref, np.float32(1.0), 0, 1)
    assert ts == ts_ref and amax == amax_ref
    oc0, os0 = quantize.quantize_blockscale(bits, ts_ref, quantize.RNE, 0, 0, 0)
    oc1, os1 = quantize.quantize_blockscale(bits, ts_ref, quantize.RNE, 0, 0, 1)
    assert np.array_equal(parts[2].reshape(R, C // 2), oc0) and np.array_equal(parts[3].reshape(R, C // 16), os0)
    assert np.array_equal(parts[4].reshape(C, R // 2), oc1) and np.array_equal(parts[5].reshape(C, R // 16), os1)
    y = parts[6].view(np.float32).reshape(R, R)
    assert_gemm_close(y, oc0, os0, ts_ref, oc0, os0, ts_ref)
