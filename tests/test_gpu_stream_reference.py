"""GPU test of the streaming reference (a measurement aid with no method
arithmetic): every byte it writes equals the host's XOR of the input words,
with one output and with two, on a ragged size."""

import numpy as np
import pytest
import torch

import fp4_block_scaled_amax_amd as lib

pytestmark = pytest.mark.gpu


def expected(bits):
    w = bits.reshape(-1, 8).view(np.uint32).reshape(-1, 2, 4)  # per block: two 16-byte units
    h = np.bitwise_xor.reduce(w[:, 0, :], axis=1)
    g = np.bitwise_xor.reduce(w[:, 1, :], axis=1)
    x = h ^ g
    c0 = np.stack([h, g], axis=1).view(np.uint8).reshape(-1)
    c1 = np.stack([g, h], axis=1).view(np.uint8).reshape(-1)
    return c0, (x & 0xFF).astype(np.uint8), c1, ((x >> 8) & 0xFF).astype(np.uint8)


@pytest.mark.parametrize("rows,cols", [(48, 4112), (1024, 1024)])
def test_stream_reference_bytes(rows, cols):
    rng = np.random.default_rng(rows + cols)
    bits = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).cuda()
    r = (torch.zeros((rows, cols // 2), dtype=torch.uint8, device="cuda"),
         torch.zeros((rows, cols // 16), dtype=torch.uint8, device="cuda"))
    c = (torch.zeros((cols, rows // 2), dtype=torch.uint8, device="cuda"),
         torch.zeros((cols, rows // 16), dtype=torch.uint8, device="cuda"))
    e_c0, e_s0, e_c1, e_s1 = expected(bits)
    lib.stream_reference(x, r)
    torch.cuda.synchronize()
    assert np.array_equal(r[0].cpu().numpy().reshape(-1), e_c0)
    assert np.array_equal(r[1].cpu().numpy().reshape(-1), e_s0)
    assert int(c[0].cpu().sum()) == 0  # untouched with one output
    lib.stream_reference(x, r, c)
    torch.cuda.synchronize()
    assert np.array_equal(c[0].cpu().numpy().reshape(-1), e_c1)
    assert np.array_equal(c[1].cpu().numpy().reshape(-1), e_s1)
