"""Philox4x32-10 counter-based generator and the stochastic-rounding bit layout.

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this module.

The generator follows [Philox] (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11): a 128-bit counter (four 32-bit words)
and a 64-bit key (two words) pass through 10 rounds.  Each round multiplies
words 0 and 2 by the constants 0xD2511F53 and 0xCD9E8D57 (full 64-bit
products), and the new words are
    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0)).
Between rounds the key words are bumped by the Weyl constants 0x9E3779B9 and
0xBB67AE85 (mod 2^32).

The pages ([UE5M3] abstract) only say the backward gradients use stochastic
rounding.  Reading for the random bits, fixed so that they depend only on the
output coordinates and not on how a GPU maps threads:
  * a quantize call takes a 64-bit seed and a 32-bit offset from the caller;
  * the output orientation is o = 0 (row-wise) or 1 (the transposed output);
  * output element (i, j) of an (R_o, C_o) output has linear index
    e = i * C_o + j, and n = e >> 3;
  * counter = (n mod 2^32, n >> 32, offset, o), key = (seed mod 2^32, seed >> 32);
  * the four 32-bit outputs w[0..3] give eight 16-bit values; element e takes
    the low half of w[(e & 7) >> 1] when e is even and the high half when odd.
"""

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF
ROUNDS = 10


def philox4x32(counter, key, rounds=ROUNDS):
    """Vectorized Philox4x32-R.

    counter: tuple of four integer arrays (values < 2^32), broadcastable.
    key:     tuple of two integers (< 2^32).
    Returns a tuple of four uint64 arrays holding 32-bit words.
    """
    c0, c1, c2, c3 = (np.asarray(w, dtype=np.uint64) for w in counter)
    k0 = np.uint64(key[0] & MASK32)
    k1 = np.uint64(key[1] & MASK32)
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    mask = np.uint64(MASK32)
    shift = np.uint64(32)
    for r in range(rounds):
        if r > 0:
            k0 = np.uint64((int(k0) + W0) & MASK32)
            k1 = np.uint64((int(k1) + W1) & MASK32)
        p0 = m0 * c0  # < 2^64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> shift, p0 & mask
        hi1, lo1 = p1 >> shift, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox4x32_scalar(counter, key, rounds=ROUNDS):
    """Pure-Python scalar twin of philox4x32 (one counter, Python ints)."""
    c = [w & MASK32 for w in counter]
    k = [key[0] & MASK32, key[1] & MASK32]
    for r in range(rounds):
        if r > 0:
            k = [(k[0] + W0) & MASK32, (k[1] + W1) & MASK32]
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k[0], p1 & MASK32, (p0 >> 32) ^ c[3] ^ k[1], p0 & MASK32]
    return tuple(c)


def sr_bits(seed, offset, orientation, out_rows, out_cols, rows=None):
    """16-bit random values for every element of an (out_rows, out_cols) output.

    rows: optional array of output-row indices; then only those rows are
    produced (shape (len(rows), out_cols)), with their true coordinates.
    Returns a uint16 array.
    """
    if rows is None:
        rows = np.arange(out_rows, dtype=np.uint64)
    rows = np.asarray(rows, dtype=np.uint64)
    cols = np.arange(out_cols, dtype=np.uint64)
    e = rows[:, None] * np.uint64(out_cols) + cols[None, :]
    n = e >> np.uint64(3)
    ctr = (n & np.uint64(MASK32), n >> np.uint64(32),
           np.uint64(offset & MASK32), np.uint64(orientation))
    key = (seed & MASK32, (seed >> 32) & MASK32)
    words = philox4x32(ctr, key)
    lane = e & np.uint64(7)
    word_idx = lane >> np.uint64(1)
    w = np.select([word_idx == 0, word_idx == 1, word_idx == 2, word_idx == 3], words)
    half = (lane & np.uint64(1)) * np.uint64(16)
    return ((w >> half) & np.uint64(0xFFFF)).astype(np.uint16)
