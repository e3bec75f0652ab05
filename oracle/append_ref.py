"""Plain, slow, fp64 reference for the MLA cache append -- TEST INFRASTRUCTURE ONLY.

What one decode step adds to a layer's cache for the new token of each
request, in the pages' order:
  1. c^KV = W^DKV h, the joint K/V latent, W^DKV of shape d_c x d (V3
     read-through section 2.2, the KV-side listing and its parameter notes;
     zeeklog equation 9; V2 read-through section 2.2).
  2. RMSNorm of the compressed latent (ai-library "DeepSeek-V2" notes,
     "Model configuration": an RMSNorm follows the compressed latent vectors).
  3. k^R = RoPE(W^KR h), the decoupled key shared by every head, computed from
     h directly and rotated by the token's position (V3 read-through section
     2.3; V2 read-through section 2.4).  With YaRN (long-context extension,
     only on k^R: ai-library notes, "Long-Context Extension"; zeeklog, the
     YaRN paragraph: scale s = 40, alpha = 1, beta = 32, from 4K) the rotation
     frequencies are interpolated as in the published YaRN method (Peng et
     al., 2023, "NTK-by-parts").
  4. The row [c^KV | k^R] is what is cached (V3 read-through section 2.2,
     cache.append((c_kv, k_r)); section 2.4).

Readings where the pages are silent:
  * RMSNorm is x / sqrt(mean(x^2) + eps) * gamma with a caller-given gamma and
    eps; the pages give neither.
  * RoPE rotates consecutive pairs (x[2i], x[2i+1]) by the angle pos * f_i
    with f_i = base^(-2i/d) (the original rotary formulation; the pages only
    say every dimension is rotated by a position-dependent angle).  base is a
    parameter.
  * YaRN's attention-temperature factor (sqrt(t) = 0.0707 ln s + 1 on the
    zeeklog page) adjusts the softmax temperature; it belongs to the softmax
    scale of the decode step, not to the cached row, and is not applied here.

Library primitives used as single steps: numpy matmul, sqrt, cos, sin.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np


def down_project(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = W h for each request: h [B, d], W [n_out, d] -> [B, n_out] (the
    d_c x d down-projection W^DKV, or W^KR for the RoPE key)."""
    return np.asarray(h, np.float64) @ np.asarray(w, np.float64).T


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * weight."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, np.float64)


def rope_frequencies(d: int, base: float, yarn_scale: float = 1.0, yarn_alpha: float = 1.0,
                     yarn_beta: float = 32.0, yarn_original_len: int = 4096) -> np.ndarray:
    """Rotation frequency of each of the d/2 pairs, f_i = base^(-2i/d).

    With yarn_scale s != 1, YaRN's frequency interpolation: for pair i with
    wavelength lambda_i = 2 pi / f_i, r_i = L / lambda_i counts the rotations
    it completes over the original context L.  Pairs with r_i > beta (many
    rotations: local position information) keep f_i, pairs with r_i < alpha
    are interpolated to f_i / s, and in between the two are blended linearly
    in r: f'_i = (1 - g) f_i / s + g f_i, g = (r_i - alpha) / (beta - alpha).
    """
    i = np.arange(d // 2, dtype=np.float64)
    f = float(base) ** (-2.0 * i / d)
    if yarn_scale == 1.0:
        return f
    r = yarn_original_len * f / (2.0 * math.pi)
    g = np.clip((r - yarn_alpha) / (yarn_beta - yarn_alpha), 0.0, 1.0)
    return (1.0 - g) * f / yarn_scale + g * f


def rope(x: np.ndarray, pos, freqs: np.ndarray) -> np.ndarray:
    """Rotate consecutive pairs of x [..., d] by the angle pos * freqs[i]:
    (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).  pos is a scalar or has
    x's leading shape."""
    x = np.asarray(x, np.float64)
    pos = np.asarray(pos, np.float64)[..., None]
    ang = pos * np.asarray(freqs, np.float64)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def append_rows(h: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray, rms_weight: np.ndarray,
                rms_eps: float, positions: np.ndarray, rope_base: float,
                yarn_scale: float = 1.0, yarn_alpha: float = 1.0, yarn_beta: float = 32.0,
                yarn_original_len: int = 4096) -> np.ndarray:
    """The cached row [RMSNorm(W^DKV h) | RoPE(W^KR h, pos)] of each request's
    new token: h [B, d], w_dkv [d_c, d], w_kr [d_h^R, d], positions [B]
    -> rows [B, d_c + d_h^R] (fp64)."""
    c = rms_norm(down_project(h, w_dkv), rms_weight, rms_eps)
    freqs = rope_frequencies(np.asarray(w_kr).shape[0], rope_base, yarn_scale, yarn_alpha,
                             yarn_beta, yarn_original_len)
    k_r = rope(down_project(h, w_kr), np.asarray(positions), freqs)
    return np.concatenate([c, k_r], axis=1)


def append_into(cache: np.ndarray, rows: np.ndarray, positions: np.ndarray,
                page_table: Optional[np.ndarray] = None, page_size: int = 0) -> np.ndarray:
    """A copy of `cache` with row positions[b] of request b replaced by rows[b]
    (contiguous [B, max_len, row] or paged [pages, page_size, row] with page
    table [B, max_pages]): the cache.append of the V3 read-through, section
    2.2, at an explicit position."""
    out = np.array(cache, copy=True)
    for b, p in enumerate(np.asarray(positions)):
        p = int(p)
        if page_table is None:
            out[b, p] = rows[b]
        else:
            out[int(page_table[b, p // page_size]), p % page_size] = rows[b]
    return out
