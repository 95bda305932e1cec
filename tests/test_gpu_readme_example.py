"""The README's usage example runs as written, and its three GEMM outputs
agree with fp64 products of the dequantized operands (the library's own
dequantize entry point) to within 1e-5 of sum |a b| per element."""

import os

import pytest

import fp4_block_scaled_amax_amd as lib

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def readme_example():
    text = open(os.path.join(ROOT, "README.md")).read()
    start = text.index("```python\n") + len("```python\n")
    return text[start:text.index("```", start)]


def dequant(q):
    import torch

    return lib.dequantize(q, torch.empty((q.rows, q.cols), dtype=torch.float32, device="cuda"))


def test_readme_example(cuda_device):
    import torch

    ns = {}
    exec(compile(readme_example(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    X, W, D = (ns["state"][k][3:] for k in ("x", "w", "dy"))
    for out, a, b in ((ns["y"], X[0], W[0]), (ns["dx"], D[0], W[1]), (ns["dw"], D[1], X[1])):
        da, db = dequant(a).double(), dequant(b).double()
        ref = da @ db.t()
        bound = 1e-5 * (da.abs() @ db.abs().t())
        assert bool(torch.isfinite(out).all())
        assert bool(((out.double() - ref).abs() <= bound).all())
        assert float(ref.abs().max()) > 0.0
