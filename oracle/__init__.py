"""CPU oracle for UE5M3-FP4 block-16 quantization and the block-scaled training GEMMs.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite (tests/), the smoke
check in __graft_entry__.py and the cpu_baseline leg of bench.py may import,
call or execute anything in this package.  The HIP library never calls it and
this package never imports the library: the two implementations share no code,
tables or constants.  Both only consume the same seeded inputs (workloads/).

The oracle is deliberately plain and slow: numpy, one step per line, in the
order the method takes them.

Sources (cited by title and section throughout):
  [UE5M3]  "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining"
           (arXiv 2609.02846), abstract.  E2M1 payloads paired with unsigned
           E5M3 block scales, block-16, periodic tensor scaling, stochastic
           rounding on backward gradients only, FP4 in the internal linears.
  [UFP4]   "Rethinking Shrinkage Bias in LLM FP4 Pretraining: Geometric
           Origin, Systemic Impact, and UFP4 Recipe" (arXiv 2606.20381),
           abstract.  Names the three training GEMMs of a linear layer and
           restricts stochastic rounding to dY.
  [TIBQ]   "Stable FP4 Training via Transposition-Invariant Block
           Quantization", summary in the UE5M3 paper's related-papers list.
           1-D blocks give the transposed operand different scales, so each
           GEMM operand is quantized along its own contraction axis.
  [Philox] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
           1, 2, 3", SC'11: the Philox4x32 counter-based generator.

Where the pages leave a step open, the module that implements it states the
reading it takes ("Reading:").

Pin status (see tests/test_oracle_*.py):
  formats.py      pinned: exhaustive brute force over every fp32 input,
                  numpy float16 decode of the 248 codes it can represent.
  philox.py       pinned against rocRAND's open-source Philox4x32-10 engine
                  (compiled from its headers at test time) and a pure-Python
                  scalar twin.
  quantize.py     pinned: hand-built worked blocks, closed-form special cases,
                  transpose invariant, exact stochastic-rounding probabilities
                  and unbiasedness (mean of 10^5 seeded draws within 1e-3).
  gemm.py         pinned: exact rational triple loop on tiny shapes, an exact
                  integer special case.
  tensor_scale.py pinned: closed-form state machine cases.
"""

from . import formats, philox, quantize, gemm, tensor_scale  # noqa: F401
