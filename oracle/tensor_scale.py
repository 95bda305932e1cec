"""Periodic tensor-scale refresh (oracle side).

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this module.

[UE5M3] abstract: the wider range of UE5M3 block scales permits *periodic*
tensor scaling, in place of a current-tensor amax pass before every
quantization.  The pages give no formula, period or window.  Reading:

  * every quantize call folds max|x| of its input into a running amax
    (max since the last refresh);
  * at step t, when period >= 1 and t % period == 0, the scale is refreshed:
    ts = amax_run / (6 * max_safe) if amax_run is finite and > 0 (otherwise
    ts keeps its value), and amax_run is reset to 0;
  * max_safe defaults to 7168 = 114688 / 16 (UE5M3 code 0xDE): the largest
    block of the tensor at refresh time gets the block scale 7168, which
    leaves four octaves of headroom below the largest UE5M3 value for
    tensors that grow before the next refresh;
  * bootstrap: before step 0 an amax-only pass fills amax_run, then the
    step-0 refresh sets the first ts.
All arithmetic is fp32: ts = float32(amax_run / float32(6 * max_safe)).
"""

import numpy as np

MAX_SAFE_DEFAULT = 7168.0


def update_tensor_scale(amax_run, ts, step, period, max_safe=MAX_SAFE_DEFAULT):
    """Returns (new_amax_run, new_ts) as float32."""
    amax_run = np.float32(amax_run)
    ts = np.float32(ts)
    if period < 1 or step % period != 0:
        return amax_run, ts
    if np.isfinite(amax_run) and amax_run > 0:
        denom = np.float32(np.float32(6.0) * np.float32(max_safe))
        ts = np.float32(amax_run / denom)
    return np.float32(0.0), ts


def fold_amax(amax_run, amax_new):
    """Running max with NaN propagation."""
    a, b = np.float32(amax_run), np.float32(amax_new)
    if np.isnan(a) or np.isnan(b):
        return np.float32(np.nan)
    return np.float32(max(a, b))
