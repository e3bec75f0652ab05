"""Pins for the cache-append oracle (oracle/append_ref.py), CPU only.

Each pin rests on something other than the oracle's own formula: hand-worked
rotations, identities every correct RoPE satisfies, YaRN's limiting cases and
the linearity of its ramp in the number of turns, RMSNorm's closed forms, and
brute-force scalar loops.  The planted-mistake
tests check that plausible errors (a swapped sin/cos, a wrong sign, a wrong
frequency exponent, a missing mean in RMSNorm, swapped halves of the row)
fail at least one pin.
"""

import math

import numpy as np
import pytest

import oracle
from oracle.append_ref import rope_frequencies


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def rope_pin_failures(rope_fn):
    """Failed pins of a candidate rope(x, pos, freqs) implementation."""
    fails = []
    # d = 2: f_0 = 1 for any base; position 1 turns (1,0) by 1 radian.
    f2 = rope_frequencies(2, 10000.0)
    got = rope_fn(np.array([1.0, 0.0]), 1, f2)
    if not np.allclose(got, [math.cos(1.0), math.sin(1.0)], atol=1e-15):
        fails.append("unit vector e0 at pos 1")
    got = rope_fn(np.array([0.0, 1.0]), 1, f2)
    if not np.allclose(got, [-math.sin(1.0), math.cos(1.0)], atol=1e-15):
        fails.append("unit vector e1 at pos 1")
    # d = 4, base 100: frequencies 1 and 100^(-1/2) = 0.1; position 2.
    f4 = rope_frequencies(4, 100.0)
    got = rope_fn(np.array([0.0, 0.0, 1.0, 0.0]), 2, f4)
    if not np.allclose(got, [0.0, 0.0, math.cos(0.2), math.sin(0.2)], atol=1e-15):
        fails.append("second pair at pos 2, base 100")
    rng = np.random.default_rng(3)
    d = 64
    f = rope_frequencies(d, 10000.0)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    if not np.allclose(rope_fn(q, 0, f), q, atol=0):
        fails.append("position 0 is the identity")
    # Relative position: <R_m q, R_n k> = <R_{m-n} q, k>.
    for m, n in [(7, 3), (1000, 999), (5, 123)]:
        lhs = rope_fn(q, m, f) @ rope_fn(k, n, f)
        rhs = rope_fn(q, m - n, f) @ k
        if abs(lhs - rhs) > 1e-10 * (1 + abs(lhs)):
            fails.append(f"relative position {m},{n}")
    # Rotations compose: R_b R_a = R_{a+b}; every pair keeps its length.
    x = rng.standard_normal(d)
    if not np.allclose(rope_fn(rope_fn(x, 11, f), 29, f), rope_fn(x, 40, f), atol=1e-12):
        fails.append("composition")
    y = rope_fn(x, 12345, f)
    if not np.allclose(y[0::2] ** 2 + y[1::2] ** 2, x[0::2] ** 2 + x[1::2] ** 2, atol=1e-12):
        fails.append("pair lengths")
    return fails


def test_rope_pins():
    assert rope_pin_failures(oracle.rope) == []


def test_rope_planted_mistakes_fail():
    def swapped(x, pos, freqs):  # sin and cos exchanged
        x = np.asarray(x, np.float64)
        ang = np.asarray(pos, np.float64)[..., None] * freqs
        c, s = np.sin(ang), np.cos(ang)
        out = np.empty_like(x)
        out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
        out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
        return out

    def wrong_sign(x, pos, freqs):  # rotates the other way
        return oracle.rope(x, -np.asarray(pos), freqs)

    def half_split(x, pos, freqs):  # pairs (i, i + d/2) instead of (2i, 2i+1)
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        ang = np.asarray(pos, np.float64)[..., None] * freqs
        c, s = np.cos(ang), np.sin(ang)
        out = np.empty_like(x)
        out[..., :d // 2] = x[..., :d // 2] * c - x[..., d // 2:] * s
        out[..., d // 2:] = x[..., :d // 2] * s + x[..., d // 2:] * c
        return out

    for bad in (swapped, wrong_sign, half_split):
        assert rope_pin_failures(bad), bad.__name__

    # A wrong exponent in the frequencies (base^(-i/d)) breaks the d = 4 pin.
    def wrong_freq_rope(x, pos, freqs):
        d = 2 * len(freqs)
        base = 100.0 if d == 4 else 10000.0
        return oracle.rope(x, pos, float(base) ** (-np.arange(d // 2) / d))
    assert rope_pin_failures(wrong_freq_rope)


def yarn_pin_failures(freq_fn) -> list:
    """Pins of YaRN's frequency interpolation (ai-library "DeepSeek-V2" notes,
    "Long-Context Extension"; zeeklog notes: s = 40, alpha = 1, beta = 32 from
    a 4K context) on freq_fn(d, base, s, alpha, beta, L): s = 1 is plain RoPE;
    pairs that turn more than beta times over the original context keep their
    frequency and those that turn fewer than alpha times are slowed by s; in
    between, the blend weight h = (f'/f - 1/s) / (1 - 1/s) is an affine
    function of the number of turns r (the ramp is linear in r), reaching 0 at
    r = alpha and 1 at r = beta.  Returns the failures."""
    bad = []
    d, base, s, a, b, L = 64, 10000.0, 40.0, 1.0, 32.0, 4096
    f = base ** (-2.0 * np.arange(d // 2) / d)
    if not np.array_equal(freq_fn(d, base, 1.0, a, b, L), f):
        bad.append("s = 1 changes the frequencies")
    fy = freq_fn(d, base, s, a, b, L)
    r = L * f / (2 * math.pi)  # rotations over the original context
    fast, slow = r > b, r < a
    mid = ~(fast | slow)
    assert fast.any() and slow.any() and mid.sum() >= 3
    if not np.array_equal(fy[fast], f[fast]):
        bad.append("fast pairs changed")
    if not np.allclose(fy[slow], f[slow] / s, rtol=1e-15):
        bad.append("slow pairs not divided by s")
    h = (fy / f - 1 / s) / (1 - 1 / s)
    hm, rm = h[mid], r[mid]
    # Affine in r: the line through the two extreme mid-band pairs predicts
    # every other one, and it meets 0 at alpha and 1 at beta.
    i0, i1 = np.argmin(rm), np.argmax(rm)
    slope = (hm[i1] - hm[i0]) / (rm[i1] - rm[i0])
    pred = hm[i0] + slope * (rm - rm[i0])
    if not np.allclose(hm, pred, rtol=0, atol=1e-12):
        bad.append("blend not linear in the number of turns")
    if not (abs(hm[i0] + slope * (a - rm[i0])) < 1e-12 and
            abs(hm[i0] + slope * (b - rm[i0]) - 1) < 1e-12):
        bad.append("ramp does not run from alpha to beta")
    return bad


def test_yarn_frequencies():
    assert yarn_pin_failures(rope_frequencies) == []


def test_yarn_planted_mistakes_fail():
    """Plausible slips in the ramp each fail a pin: blending the wavelengths
    or the log frequencies instead of the frequencies, a ramp in wavelength
    instead of turns, and the two ends of the ramp exchanged."""
    def blend_wavelength(d, base, s, a, b, L):
        f = rope_frequencies(d, base)
        if s == 1.0:
            return f
        r = L * f / (2 * math.pi)
        g = np.clip((r - a) / (b - a), 0, 1)
        lam = (1 - g) * (2 * math.pi * s / f) + g * (2 * math.pi / f)
        return 2 * math.pi / lam

    def blend_log(d, base, s, a, b, L):
        f = rope_frequencies(d, base)
        if s == 1.0:
            return f
        r = L * f / (2 * math.pi)
        g = np.clip((r - a) / (b - a), 0, 1)
        return np.exp((1 - g) * np.log(f / s) + g * np.log(f))

    def ramp_in_wavelength(d, base, s, a, b, L):
        f = rope_frequencies(d, base)
        if s == 1.0:
            return f
        lam_turns = L / (2 * math.pi / f)          # same r at the ends ...
        r = np.where((lam_turns > a) & (lam_turns < b), L / (2 * math.pi) * f ** 0.5,
                     lam_turns)                    # ... another measure inside
        g = np.clip((r - a) / (b - a), 0, 1)
        return (1 - g) * f / s + g * f

    def ends_exchanged(d, base, s, a, b, L):
        f = rope_frequencies(d, base)
        if s == 1.0:
            return f
        r = L * f / (2 * math.pi)
        g = np.clip((r - a) / (b - a), 0, 1)
        return g * f / s + (1 - g) * f

    for bad in (blend_wavelength, blend_log, ramp_in_wavelength, ends_exchanged):
        assert yarn_pin_failures(bad), bad.__name__


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------

def test_rms_norm_pins():
    # Hand example: x = (3, 4), mean square 12.5.
    got = oracle.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(got, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], atol=1e-15)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 512))
    # With unit weights the output's mean square is ms / (ms + eps).
    eps = 1e-3
    y = oracle.rms_norm(x, np.ones(512), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)
    # Scale invariance at eps = 0, and the weight multiplies elementwise.
    assert np.allclose(oracle.rms_norm(3.0 * x, np.ones(512), 0.0),
                       oracle.rms_norm(x, np.ones(512), 0.0), atol=1e-12)
    w = rng.standard_normal(512)
    assert np.allclose(oracle.rms_norm(x, w, eps), y * w, atol=1e-12)


def test_rms_norm_planted_mistake_fails():
    def no_mean(x, weight, eps):  # sum of squares instead of their mean
        x = np.asarray(x, np.float64)
        return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * weight
    got = no_mean(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert not np.allclose(got, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)])


# ----------------------------------------------------------------------------
# The appended row
# ----------------------------------------------------------------------------

def brute_row(h, w_dkv, w_kr, g, eps, pos, base):
    """Scalar loops, straight from the definitions (no numpy vectorisation)."""
    d_c, d_r, d = w_dkv.shape[0], w_kr.shape[0], len(h)
    c = [sum(float(w_dkv[n, k]) * float(h[k]) for k in range(d)) for n in range(d_c)]
    ms = sum(v * v for v in c) / d_c
    c = [c[n] / math.sqrt(ms + eps) * float(g[n]) for n in range(d_c)]
    kr = [sum(float(w_kr[n, k]) * float(h[k]) for k in range(d)) for n in range(d_r)]
    out = list(c)
    for i in range(d_r // 2):
        ang = pos * base ** (-2.0 * i / d_r)
        x0, x1 = kr[2 * i], kr[2 * i + 1]
        out += [x0 * math.cos(ang) - x1 * math.sin(ang), x0 * math.sin(ang) + x1 * math.cos(ang)]
    return np.array(out)


def test_append_rows_brute_force():
    rng = np.random.default_rng(11)
    B, d, d_c, d_r = 3, 24, 8, 4
    h = rng.standard_normal((B, d))
    w_dkv = rng.standard_normal((d_c, d)) / math.sqrt(d)
    w_kr = rng.standard_normal((d_r, d)) / math.sqrt(d)
    g = 1 + 0.1 * rng.standard_normal(d_c)
    pos = np.array([0, 5, 4095])
    rows = oracle.append_rows(h, w_dkv, w_kr, g, 1e-6, pos, 10000.0)
    assert rows.shape == (B, d_c + d_r)
    for b in range(B):
        ref = brute_row(h[b], w_dkv, w_kr, g, 1e-6, int(pos[b]), 10000.0)
        assert np.allclose(rows[b], ref, atol=1e-12)
    # The latent half is RMS-normalised (unit weights => mean square ~1) and
    # does not depend on the position; the key half does.
    r2 = oracle.append_rows(h, w_dkv, w_kr, g, 1e-6, pos + 1, 10000.0)
    assert np.array_equal(r2[:, :d_c], rows[:, :d_c])
    assert not np.allclose(r2[1:, d_c:], rows[1:, d_c:])
    # Swapping the halves (a plausible layout mistake) breaks the comparison.
    swapped = np.concatenate([rows[:, d_c:], rows[:, :d_c]], axis=1)
    assert not np.allclose(swapped[0], brute_row(h[0], w_dkv, w_kr, g, 1e-6, 0, 10000.0))


def test_append_rows_yarn_changes_only_the_slow_pairs():
    rng = np.random.default_rng(12)
    d, d_c, d_r = 32, 8, 64
    h = rng.standard_normal((1, d))
    w_dkv = rng.standard_normal((d_c, d))
    w_kr = rng.standard_normal((d_r, d))
    g = np.ones(d_c)
    pos = np.array([100000])
    plain = oracle.append_rows(h, w_dkv, w_kr, g, 1e-6, pos, 10000.0)
    yarn = oracle.append_rows(h, w_dkv, w_kr, g, 1e-6, pos, 10000.0, 40.0, 1.0, 32.0, 4096)
    f = rope_frequencies(d_r, 10000.0)
    fast = 4096 * f / (2 * math.pi) > 32.0
    key_p, key_y = plain[0, d_c:], yarn[0, d_c:]
    pairs_equal = np.isclose(key_p[0::2], key_y[0::2], atol=1e-12) & \
        np.isclose(key_p[1::2], key_y[1::2], atol=1e-12)
    assert np.all(pairs_equal[fast]) and not np.all(pairs_equal)
    assert np.array_equal(plain[0, :d_c], yarn[0, :d_c])


def test_append_into_contiguous_and_paged():
    rng = np.random.default_rng(13)
    B, L, row = 3, 16, 6
    cache = rng.standard_normal((B, L, row))
    rows = rng.standard_normal((B, row))
    pos = np.array([0, 7, 15])
    out = oracle.append_into(cache, rows, pos)
    for b in range(B):
        assert np.array_equal(out[b, pos[b]], rows[b])
        mask = np.ones(L, bool)
        mask[pos[b]] = False
        assert np.array_equal(out[b, mask], cache[b, mask])
    # Paged: 4-token pages, a permuted page table.
    ps, mp = 4, 4
    pt = rng.permutation(B * mp).reshape(B, mp).astype(np.int32)
    pool = rng.standard_normal((B * mp, ps, row))
    outp = oracle.append_into(pool, rows, pos, pt, ps)
    for b in range(B):
        page, off = pt[b, pos[b] // ps], pos[b] % ps
        assert np.array_equal(outp[page, off], rows[b])
    changed = np.argwhere(np.any(outp != pool, axis=2))
    assert len(changed) == B
