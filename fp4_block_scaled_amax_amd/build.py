"""Build libue5m3fp4.so (gfx950) in-tree with hipcc.

Usage: python -m fp4_block_scaled_amax_amd.build   (or build() from Python)
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libue5m3fp4.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "gemm_mx.hip"]

HIP_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # one IEEE rounding per operation: no fused multiply-add anywhere
    "-ffp-contract=off",
    # no packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
]


# Per-source code-generation options.  The GEMMs' main loops are long
# straight-line blocks of MFMAs interleaved with dequantization (or operand
# moves), LDS and global-load instructions; LLVM's iterative ILP scheduling
# strategy orders them measurably better than the default on MI355X (about
# 6 % for the block-scaled GEMM, 11 % for the MXFP4 one at 8192 x 4096 x
# 16384).  The quantizer gains nothing from it.
SOURCE_FLAGS = {
    "gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "gemm_mx.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def _code_only(text):
    """C++ source text without comments and with runs of white space folded:
    what the compiler sees, so that editing a comment leaves the fingerprint
    alone.  String and character literals are kept whole."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_fingerprint(src):
    """SHA-256 of a source file's code, the code of the headers beside it
    (every source includes some of them) and the options it is compiled
    with: what a recorded measurement of its kernels refers to.  Comments
    and white space do not count."""
    import hashlib

    h = hashlib.sha256()
    for name in [src] + sorted(f for f in os.listdir(CSRC) if f.endswith(".hpp")):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    h.update(repr((HIP_FLAGS, SOURCE_FLAGS.get(src, []))).encode())
    return h.hexdigest()


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build")


def build(verbose=False):
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)  # the host pass ignores the GPU feature
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
