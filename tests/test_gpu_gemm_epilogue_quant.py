"""GPU parity of the GEMM whose epilogue quantizes its bf16 output for the
next linear layer ("format-aware fusion" article in the UFP4 page's
similar-articles list: scale computation and packing fused with the GEMM;
reading R19: the output is quantized as the stand-alone quantizer would
quantize the stored bf16(C)).

Oracle parity uses operands on which every fp32 partial sum of the GEMM is
exact (payload magnitudes 0, 0.5 and 1, scales in [1, 1.875], power-of-two
tensor scales): each product is then a multiple of 2^-8 below 3.6, so for
K <= 4112 every partial sum is a multiple of 2^-8 below 2^14 -- 22
significant bits -- and C is the exact sum whatever the accumulation order.
The oracle computes C (fp64, exact), rounds it to bf16 itself, and quantizes
that: the bf16 output, its amax and the fused codes and scales are compared
bit for bit with values the oracle alone produced.

Operands with the full E2M1 and UE5M3 ranges make the accumulation order
visible in the last bit, so there the fused outputs are checked for
consistency: the bf16 output equals the plain bf16-output GEMM's, lies in the
oracle's rounded tolerance band, and the fused codes and scales equal what the
stand-alone quantizer (itself oracle-pinned) writes for that stored output."""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import formats, quantize
from oracle import gemm as ogemm

from devhelpers import dev_scalar, host

pytestmark = pytest.mark.gpu

EXACT_CODES = np.array([0, 1, 2, 8, 9, 10], dtype=np.uint8)  # 0, 0.5, 1 and their negatives


def _device_operand(codes, scales, ts):
    import torch

    return lib.Quantized(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), dev_scalar(ts))


def _exact_operand(rng, rows, k, ts, zero_rows=()):
    """Codes from EXACT_CODES, scales 0x78..0x7F (1 .. 1.875); rows listed in
    zero_rows are all zero (their output rows give zero blocks)."""
    nib = rng.choice(EXACT_CODES, size=(rows, k))
    nib[list(zero_rows)] = 0
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(0x78, 0x80, size=(rows, k // 16), dtype=np.uint8)
    return _device_operand(codes, scales, ts), codes, scales


def _wide_operand(rng, rows, k, ts, lo=0x40, hi=0xB0):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, k // 16), dtype=np.uint8)
    return _device_operand(codes, scales, ts), codes, scales


def _oracle_output(ac, asc, tsa, bc, bsc, tsb):
    """bf16 bits of the exact GEMM output, rounded by the oracle."""
    ref, _ = ogemm.gemm_nt(ac, asc, tsa, bc, bsc, tsb)
    ref = ref + 0.0  # an exact zero is +0 (the accumulators start at +0)
    ref32 = ref.astype(np.float32)
    finite = np.isfinite(ref)
    assert np.array_equal(ref32[finite].astype(np.float64), ref[finite]), "operands do not give exact sums"
    return formats.f32_to_bf16_rne(ref32)


def _run(a, b, out_ts, rounding, seed, offset, row, col):
    import torch

    M, N = a.rows, b.rows
    ts = dev_scalar(out_ts)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    amax = dev_scalar(0.0)
    qr = lib.empty_quantized(M, N, ts) if row else None
    qc = lib.empty_quantized(N, M, ts) if col else None
    lib.gemm_nt_bf16_quantized(a, b, y, ts, rounding, seed, offset, row=qr, col=qc, amax=amax)
    return y, amax, qr, qc


def _bits(y):
    import torch

    return host(y.view(torch.int16)).view(np.uint16)


def _check_exact(a, b, ybits, out_ts, rounding, seed, offset, row=True, col=True):
    """GPU outputs against the oracle's: bf16 output, amax, codes, scales."""
    y, amax, qr, qc = _run(a, b, out_ts, rounding, seed, offset, row, col)
    got = _bits(y)
    assert np.array_equal(got, ybits), "bf16 output differs from the oracle's rounding of the exact sum"
    y32 = formats.bf16_to_f32(ybits)
    assert host(amax)[0] == np.float32(np.max(np.abs(y32)))
    ts = np.float32(out_ts)
    for q, o in ((qr, 0), (qc, 1)):
        if q is None:
            continue
        oc, os_ = quantize.quantize_blockscale(ybits, ts, rounding, seed, offset, o)
        bad = np.argwhere(host(q.scales) != os_)
        assert bad.size == 0, f"orientation {o}: scale mismatch at {bad[:5].tolist()}"
        bad = np.argwhere(host(q.codes) != oc)
        assert bad.size == 0, f"orientation {o}: code mismatch at {bad[:5].tolist()}"


@pytest.mark.parametrize("rounding", [lib.RNE, lib.SR])
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (320, 400, 128), (512, 768, 1024), (48, 1040, 96),
                                   (16, 16, 16), (272, 528, 4112)])
def test_fused_output_quantization_exact(cuda_device, rounding, M, N, K):
    """Several output tiles, ragged edge tiles, aligned and unaligned K, zero
    output rows (zero blocks); everything bit-exact with the oracle."""
    rng = np.random.default_rng(M + 3 * N + 5 * K + rounding)
    a, ac, asc = _exact_operand(rng, M, K, 0.5, zero_rows=range(3, M, 37))
    b, bc, bsc = _exact_operand(rng, N, K, 2.0 ** -10)
    ybits = _oracle_output(ac, asc, 0.5, bc, bsc, 2.0 ** -10)
    y32 = formats.bf16_to_f32(ybits)
    out_ts = np.float32(np.float32(np.max(np.abs(y32))) / np.float32(43008.0))
    _check_exact(a, b, ybits, out_ts, rounding, seed=1000 + M, offset=7)


def test_single_orientations_and_ragged_rows_exact(cuda_device):
    """Row-wise output alone allows any M; transposed output alone any N."""
    rng = np.random.default_rng(11)
    a, ac, asc = _exact_operand(rng, 300, 256, 0.25)
    b, bc, bsc = _exact_operand(rng, 272, 256, 2.0 ** -7)
    ybits = _oracle_output(ac, asc, 0.25, bc, bsc, 2.0 ** -7)
    _check_exact(a, b, ybits, 1e-4, lib.SR, 5, 1, row=True, col=False)
    a2, ac2, asc2 = _exact_operand(rng, 288, 128, 0.25)
    b2, bc2, bsc2 = _exact_operand(rng, 250, 128, 2.0 ** -7)
    ybits2 = _oracle_output(ac2, asc2, 0.25, bc2, bsc2, 2.0 ** -7)
    _check_exact(a2, b2, ybits2, 1e-4, lib.RNE, 5, 1, row=False, col=True)


@pytest.mark.parametrize("out_ts", [1e-30, 3.0e30, 2.0 ** -120])
def test_extreme_output_tensor_scales_exact(cuda_device, out_ts):
    """Tensor scales outside the fast path's range (flushed, saturated and
    general-path blocks)."""
    rng = np.random.default_rng(23)
    a, ac, asc = _exact_operand(rng, 64, 128, 1.0)
    b, bc, bsc = _exact_operand(rng, 48, 128, 1.0)
    ybits = _oracle_output(ac, asc, 1.0, bc, bsc, 1.0)
    for rounding in (lib.RNE, lib.SR):
        _check_exact(a, b, ybits, out_ts, rounding, 3, 3)


def test_nan_block_in_output(cuda_device):
    """A NaN operand scale (0xFF) poisons an output row.  The sign of the
    stored NaN is the hardware's, so for that row the test checks what the
    format fixes: NaN values, scale 0xFF and magnitude-0 codes in every block;
    every other row is bit-exact with the oracle."""
    rng = np.random.default_rng(31)
    a, ac, asc = _exact_operand(rng, 64, 64, 1.0)
    b, bc, bsc = _exact_operand(rng, 32, 64, 1.0)
    asc[9, 1] = 0xFF
    a = _device_operand(ac, asc, 1.0)
    ybits = _oracle_output(ac, asc, 1.0, bc, bsc, 1.0)
    ok_rows = np.delete(np.arange(64), 9)
    for rounding in (lib.RNE, lib.SR):
        y, amax, qr, qc = _run(a, b, 1e-3, rounding, 2, 0, True, True)
        got = _bits(y)
        assert np.all(np.isnan(formats.bf16_to_f32(got[9])))
        assert np.array_equal(got[ok_rows], ybits[ok_rows])
        assert np.isnan(host(amax)[0])
        # row-wise output: rows other than 9 exact (sampled with their true row ids)
        oc_full, os_full = quantize.quantize_blockscale(ybits, np.float32(1e-3), rounding, 2, 0, 0,
                                                        rows=ok_rows)
        assert np.array_equal(host(qr.scales)[ok_rows], os_full)
        assert np.array_equal(host(qr.codes)[ok_rows], oc_full)
        assert np.all(host(qr.scales)[9] == 0xFF) and np.all((host(qr.codes)[9] & 0x77) == 0)
        # transposed output: block 0 of every column holds row 9 -> NaN block; the others exact
        cs, cc = host(qc.scales), host(qc.codes)
        occ, ocs = quantize.quantize_blockscale(ybits, np.float32(1e-3), rounding, 2, 0, 1)
        assert np.all(cs[:, 0] == 0xFF) and np.all((cc[:, :8] & 0x77) == 0)
        assert np.array_equal(cs[:, 1:], ocs[:, 1:]) and np.array_equal(cc[:, 8:], occ[:, 8:])


@pytest.mark.parametrize("rounding", [lib.RNE, lib.SR])
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (320, 400, 128), (272, 528, 4112)])
def test_wide_range_operands_consistency(cuda_device, rounding, M, N, K):
    """Full E2M1 and UE5M3 ranges (accumulation order visible in the last
    bit): the bf16 output equals the plain bf16-output GEMM's, and the fused
    codes, scales and amax equal what the stand-alone quantizer writes for
    that stored output."""
    import torch

    rng = np.random.default_rng(M + 7 * N + K + rounding)
    a, _, _ = _wide_operand(rng, M, K, 0.5)
    b, _, _ = _wide_operand(rng, N, K, 2.0e-3)
    out_ts = np.float32(4.0 / 43008.0)
    y, amax, qr, qc = _run(a, b, out_ts, rounding, 1000 + M, 7, True, True)
    y_ref = torch.empty_like(y)
    lib.gemm_nt_bf16(a, b, y_ref)
    assert np.array_equal(_bits(y), _bits(y_ref)), "bf16 output differs from the plain bf16 GEMM's"
    ts = dev_scalar(out_ts)
    sr = lib.empty_quantized(M, N, ts)
    sc = lib.empty_quantized(N, M, ts)
    samax = dev_scalar(0.0)
    lib.quantize_blockscale(y_ref, ts, rounding, 1000 + M, 7, row=sr, col=sc, amax=samax)
    for fused, alone in ((qr, sr), (qc, sc)):
        assert np.array_equal(host(fused.codes), host(alone.codes))
        assert np.array_equal(host(fused.scales), host(alone.scales))
    assert host(amax)[0] == host(samax)[0]


def test_k_zero_output_is_zero(cuda_device):
    import torch

    a = lib.Quantized(torch.empty((32, 0), dtype=torch.uint8, device="cuda"),
                      torch.empty((32, 0), dtype=torch.uint8, device="cuda"), dev_scalar(1.0))
    b = lib.Quantized(torch.empty((48, 0), dtype=torch.uint8, device="cuda"),
                      torch.empty((48, 0), dtype=torch.uint8, device="cuda"), dev_scalar(1.0))
    y, amax, qr, qc = _run(a, b, 1.0, lib.RNE, 0, 0, True, True)
    assert not host(y.float()).any() and host(amax)[0] == 0.0
    assert not host(qr.codes).any() and not host(qr.scales).any()
    assert not host(qc.codes).any() and not host(qc.scales).any()
