"""Pins of the oracle's Philox4x32-10 stream and its stochastic-rounding layout.

[Philox] Salmon et al., SC'11, defines the generator; rocRAND ships an
independent open-source implementation (header-only, under the ROCm include
directory).  The test compiles a small host program against those headers and
compares its output with the oracle's for random counters and keys.  rocRAND's
engine exposes the raw counter through (seed, subsequence, offset): key = seed,
counter words 2-3 = subsequence, counter words 0-1 = offset / 4.
"""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def rocrand_philox():
    hipcc = _hipcc()
    inc = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if hipcc is None or not os.path.exists(inc):
        pytest.skip("hipcc or rocRAND headers not present")
    tmp = tempfile.mkdtemp(prefix="philox_kat_")
    exe = os.path.join(tmp, "philox_rocrand")
    subprocess.run([hipcc, "--cuda-host-only", "-O1",
                    os.path.join(HERE, "philox_rocrand_check.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(rows):
        text = "".join("%x %x %x %x %x %x\n" % tuple(r) for r in rows)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
        return [tuple(int(w, 16) for w in line.split()) for line in out.stdout.splitlines()]

    yield run
    shutil.rmtree(tmp, ignore_errors=True)


def test_philox_matches_rocrand(rocrand_philox):
    rng = np.random.default_rng(7)
    rows = rng.integers(0, 1 << 32, size=(400, 6), dtype=np.uint64)
    rows[:, 1] &= (1 << 30) - 1  # keep 4 * counter-low below 2^64 for rocRAND's offset
    rows[:3] = 0
    rows[1, 4:] = [0xFFFFFFFF, 0xFFFFFFFF]
    rows[2, 2:4] = [0xFFFFFFFF, 0xFFFFFFFF]
    ref = rocrand_philox(rows.tolist())
    assert len(ref) == len(rows)
    for i, r in enumerate(rows.tolist()):
        words = philox.philox4x32(tuple(np.uint64(w) for w in r[:4]), (r[4], r[5]))
        assert tuple(int(w) for w in words) == ref[i], (r, ref[i])


def test_philox_vectorized_matches_scalar_twin():
    rng = np.random.default_rng(8)
    ctr = rng.integers(0, 1 << 32, size=(4, 512), dtype=np.uint64)
    for key in [(0, 0), (1, 2), (0xFFFFFFFF, 0x12345678), (0xDEADBEEF, 0)]:
        vec = philox.philox4x32(tuple(ctr), key)
        for j in range(0, 512, 37):
            assert philox.philox4x32_scalar([int(c[j]) for c in ctr], key) == \
                tuple(int(w[j]) for w in vec)


def test_sr_bits_layout():
    """Element e of orientation o takes 16 bits of call n = e >> 3 with counter
    (n lo, n hi, offset, o): low half of word (e & 7) >> 1 for even e."""
    seed, offset = 0x0123456789ABCDEF, 77
    out_rows, out_cols = 3, 48
    for o in (0, 1):
        bits = philox.sr_bits(seed, offset, o, out_rows, out_cols)
        assert bits.shape == (out_rows, out_cols) and bits.dtype == np.uint16
        for i in range(out_rows):
            for j in range(out_cols):
                e = i * out_cols + j
                n = e >> 3
                w = philox.philox4x32_scalar([n & 0xFFFFFFFF, n >> 32, offset, o],
                                             [seed & 0xFFFFFFFF, seed >> 32])
                word = w[(e & 7) >> 1]
                assert bits[i, j] == ((word >> (16 * (e & 1))) & 0xFFFF)
    # row subsets use true coordinates
    full = philox.sr_bits(seed, offset, 0, 64, 32)
    sub = philox.sr_bits(seed, offset, 0, None, 32, rows=[5, 63, 0])
    np.testing.assert_array_equal(sub, full[[5, 63, 0]])


def test_sr_bits_large_counter_word():
    """n >= 2^32 lands in the second counter word."""
    cols = 1 << 20
    row = (1 << 35) // cols  # e = row * cols >= 2^35, n >= 2^32
    bits = philox.sr_bits(5, 0, 0, None, cols, rows=[row])[0, :8]
    n = (row * cols) >> 3
    w = philox.philox4x32_scalar([n & 0xFFFFFFFF, n >> 32, 0, 0], [5, 0])
    exp = [(w[k >> 1] >> (16 * (k & 1))) & 0xFFFF for k in range(8)]
    assert bits.tolist() == exp


def test_sr_bits_uniform():
    bits = philox.sr_bits(99, 3, 0, 1024, 1024).ravel().astype(np.int64)
    counts = np.bincount(bits >> 8, minlength=256)  # top byte
    expected = bits.size / 256
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    # 255 degrees of freedom: mean 255, sd ~22.6; 6 sd margin
    assert chi2 < 255 + 6 * 22.6, chi2
    # orientations and offsets give different streams
    assert not np.array_equal(philox.sr_bits(99, 3, 1, 4, 64), philox.sr_bits(99, 3, 0, 4, 64))
    assert not np.array_equal(philox.sr_bits(99, 4, 0, 4, 64), philox.sr_bits(99, 3, 0, 4, 64))
