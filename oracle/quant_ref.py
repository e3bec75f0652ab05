"""Plain reference for the low-bit latent cache -- TEST INFRASTRUCTURE ONLY.

At deployment the KV cache is quantised to about 6 bits per element and the
weights to FP8 (ai-library "DeepSeek-V2" notes, "Training and Inference
Efficiency", "Inference cost"); quantisation there is fine-grained, with the
scales computed online from the data and the products accumulated in high
precision (V3 read-through, 2kiu.com/news/6340724, section 4.4).

Reading taken here (the pages give no cache format): every cached row
[c^KV | k^R] is stored as 8-bit floats in the OCP E4M3 format (1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits, no infinities, largest finite
value 448, codes 0x7F / 0xFF are NaN) with one fp32 scale per row (per token):
    s = max_j |x_j| / 448   (s = 1 for an all-zero row)
    q_j = E4M3(x_j / s)     (round to nearest, ties to even; |x_j / s| <= 448)
    x_j ~ q_j * s
The scale and the division are fp32 operations (as the kernel performs them),
so that the codes, an integer result decided by floating point, are the same
on both sides.  Attention over such a cache is the plain latent attention
over the dequantised rows q_j * s.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (float64; NaN for 0x7F and 0xFF).

    Exponent field e, mantissa field m: e > 0 gives 2^(e-7) * (1 + m/8), e = 0
    gives the subnormal 2^-6 * (m/8)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), magnitudes
    above 448 saturated to 448, the sign kept (also on zero); NaN maps to 0x7F.

    The representable magnitudes are the decoded values of codes 0..126, in
    increasing order; the nearest one is picked, a tie going to the code
    whose last mantissa bit is 0."""
    x = np.asarray(x, dtype=np.float64)
    grid = e4m3_decode(np.arange(127))          # magnitudes of codes 0..126
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 126)   # grid[hi] >= a
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    # The sign bit is kept, also for values that round to zero (-0 is 0x80).
    code = pick.astype(np.int64) | np.where(np.signbit(x), 0x80, 0)
    return np.where(np.isnan(x), 0x7F, code).astype(np.uint8)


def quantize_rows(rows) -> tuple:
    """Per-row E4M3 quantisation of rows [..., width] (float32 values):
    returns (codes uint8 [..., width], scales float32 [...]) as described in
    the module docstring."""
    x = np.asarray(rows, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    r = (x / scale[..., None]).astype(np.float32)
    r = np.clip(r, -np.float32(E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(r), scale


def dequantize_rows(codes, scales) -> np.ndarray:
    """Rows q_j * s in float64."""
    return e4m3_decode(codes) * np.asarray(scales, np.float64)[..., None]
