"""Pins of the oracle's periodic tensor-scale refresh (closed-form cases).

[UE5M3] abstract: periodic tensor scaling replaces a current-tensor amax pass.
The refresh rule is the reading stated in oracle/tensor_scale.py.
"""

import numpy as np

from oracle import tensor_scale as T


def test_refresh_formula():
    amax, ts = T.update_tensor_scale(np.float32(43008.0), np.float32(5.0), 0, 1)
    assert amax == 0 and ts == np.float32(1.0)
    amax, ts = T.update_tensor_scale(np.float32(3.0), np.float32(5.0), 4, 2, max_safe=0.5)
    assert ts == np.float32(1.0)  # 3 / (6 * 0.5)


def test_period_gates_refresh():
    for step in range(1, 10):
        a, ts = T.update_tensor_scale(np.float32(7.0), np.float32(2.0), step, 4)
        if step % 4 == 0:
            assert a == 0 and ts == np.float32(np.float32(7.0) / np.float32(43008.0))
        else:
            assert a == np.float32(7.0) and ts == np.float32(2.0)
    a, ts = T.update_tensor_scale(np.float32(7.0), np.float32(2.0), 0, 0)
    assert a == np.float32(7.0) and ts == np.float32(2.0)  # period < 1: never


def test_zero_or_nonfinite_amax_keeps_scale():
    for bad in (0.0, np.nan, np.inf):
        a, ts = T.update_tensor_scale(np.float32(bad), np.float32(2.5), 0, 1)
        assert a == 0 and ts == np.float32(2.5)


def test_running_amax_fold():
    assert T.fold_amax(1.0, 2.0) == 2.0
    assert T.fold_amax(3.0, 2.0) == 3.0
    assert np.isnan(T.fold_amax(np.nan, 2.0)) and np.isnan(T.fold_amax(2.0, np.nan))


def test_max_safe_leaves_four_octaves():
    """The block holding the tensor's amax gets raw scale amax / (6 ts) =
    max_safe = 7168, i.e. 114688 / 16: four octaves below the largest UE5M3
    value, so a tensor that grows x8 before the next refresh still fits."""
    amax = np.float32(123.456)
    _, ts = T.update_tensor_scale(amax, np.float32(1.0), 0, 1)
    s_raw = np.float32(amax / np.float32(np.float32(6) * ts))
    assert abs(float(s_raw) - 7168.0) <= 7168.0 * 2 ** -22
    assert 8 * 7168.0 < 114688.0
