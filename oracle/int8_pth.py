"""int8 per-token-head KV encoding (test infrastructure only).

The format holds, for every stored token and KV head, D signed 8-bit codes plus
one 4-byte float scale, separately for K and for V (FreeToken PR #898: the
description bullet on the per-token-head formats, whose scales a shared layer
looks up through its source; "End to end" gives D + 4 bytes per row).  The
pages do not print the recipe.  This oracle's reading, step by step:

1. x is the row of D bf16 values, exact in float32; amax = max_d |x_d|.
2. scale = fl32(amax / 127), one IEEE float32 division.
3. amax == 0: scale = 0 and every code is 0.  Otherwise
   q_d = clamp(round_half_even(fl32(x_d / scale)), -127, 127), again with an
   IEEE float32 division.  -128 is never produced (symmetric range).
4. A row decodes to q_d * scale, taken exactly in float64.

numpy's float32 division is the correctly rounded IEEE operation and
``np.rint`` rounds half to even, so the codes and scales here are the unique
results of the steps above.
"""

import numpy as np

QMAX = 127


def quantise_rows(x):
    """x: [..., D] float32 (bf16 values) -> (codes int8 [..., D], scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.divide(amax, np.float32(QMAX), dtype=np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), scale).astype(np.float32)
    r = np.divide(x, safe[..., None], dtype=np.float32)
    codes = np.clip(np.rint(r), -QMAX, QMAX)
    codes[zero] = 0
    return codes.astype(np.int8), scale.astype(np.float32)


def dequantise_rows(codes, scale):
    """Exact float64 value of each stored element: code * scale."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[..., None]
