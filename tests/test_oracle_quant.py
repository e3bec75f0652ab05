"""Pins of the low-bit cache oracle (oracle.quant_ref): OCP E4M3 codes with one
fp32 scale per row (ai-library "DeepSeek-V2" notes, "Training and Inference
Efficiency" / "Inference cost": KV cache quantised for deployment; V3
read-through, section 4.4: scales computed online from the data).

Independent checks: values of named codes from the format definition, torch's
own float8_e4m3fn conversion (a separate implementation) on every code and on
random, midpoint and subnormal inputs, round trips, and the error bound of
round-to-nearest.  Planted mistakes (truncation, ties away from zero, the
240-max variant of the format, a wrong exponent bias) must each fail a pin.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.quant_ref as qr


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn) \
        .float().numpy().astype(np.float64)


def pin_named_codes():
    """Codes with values fixed by the format: 1.0 = 0x38 (exponent 7 = bias),
    2.0 = 0x40, 1.5 = 0x3C, 448 = 0x7E (largest finite), 2^-6 = 0x08 (smallest
    normal), 2^-9 = 0x01 (smallest subnormal), 7 * 2^-9 = 0x07, -1 = 0xB8,
    NaN = 0x7F."""
    table = {0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
             0x07: 7 * 2.0 ** -9, 0xB8: -1.0, 0x00: 0.0}
    for code, v in table.items():
        assert qr.e4m3_decode([code])[0] == v, hex(code)
        assert qr.e4m3_encode([v])[0] == code, hex(code)
    assert np.isnan(qr.e4m3_decode([0x7F, 0xFF])).all()


def pin_matches_torch():
    """Every code decodes as torch decodes it; random values (normal and
    subnormal ranges) and all midpoints between neighbouring codes encode as
    torch encodes them."""
    codes = np.arange(256)
    a, b = qr.e4m3_decode(codes), _torch_decode(codes)
    assert np.all((a == b) | (np.isnan(a) & np.isnan(b)))
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(50000) * 60, rng.standard_normal(20000) * 0.01,
                        rng.uniform(-448, 448, 20000)]).astype(np.float32)
    grid = qr.e4m3_decode(np.arange(127))
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    assert np.array_equal(qr.e4m3_encode(x), _torch_encode(x))


def pin_round_trip_and_order():
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(qr.e4m3_encode(qr.e4m3_decode(finite)), finite.astype(np.uint8))
    pos = qr.e4m3_decode(np.arange(127))
    assert np.all(np.diff(pos) > 0)


def pin_ties_to_even_and_saturation():
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39): 0x38;
    # 1.1875 halfway between 1.125 and 1.25 (0x3A, even): 0x3A.
    assert list(qr.e4m3_encode([1.0625, 1.1875, -1.0625])) == [0x38, 0x3A, 0xB8]
    assert list(qr.e4m3_encode([449.0, 1e6, -460.0])) == [0x7E, 0x7E, 0xFE]


def pin_quantize_rows():
    rng = np.random.default_rng(3)
    rows = (rng.standard_normal((64, 576)) * rng.uniform(0.01, 30, (64, 1))).astype(np.float32)
    rows[5] = 0.0
    codes, scales = oracle.quantize_rows(rows)
    assert codes.dtype == np.uint8 and scales.dtype == np.float32
    # Zero row: scale 1, every code zero.
    assert scales[5] == 1.0 and not codes[5].any()
    # The largest magnitude of each row maps to +-448.
    nz = np.arange(64) != 5
    i = np.argmax(np.abs(rows), axis=1)
    top = codes[np.arange(64), i][nz]
    assert np.all((top & 0x7F) == 0x7E)
    # Round to nearest: error at most half a step of the code grid, i.e.
    # 2^-4 relative in the normal range and 2^-10 * s below it.
    deq = oracle.dequantize_rows(codes, scales)
    r = np.abs(rows.astype(np.float64) / scales[:, None])
    err = np.abs(deq - rows) / scales[:, None]
    bound = np.where(r >= 2.0 ** -6, r * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


PINS = [("named_codes", pin_named_codes), ("matches_torch", pin_matches_torch),
        ("round_trip_and_order", pin_round_trip_and_order),
        ("ties_and_saturation", pin_ties_to_even_and_saturation),
        ("quantize_rows", pin_quantize_rows)]


@pytest.mark.parametrize("name,fn", PINS, ids=[n for n, _ in PINS])
def test_pin(name, fn):
    fn()


_orig_decode = qr.e4m3_decode
_orig_encode = qr.e4m3_encode


def _mut_truncate(x):
    x = np.asarray(x, np.float64)
    grid = _orig_decode(np.arange(127))
    a = np.minimum(np.abs(x), 448.0)
    idx = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 126)
    return (idx | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _mut_ties_away(x):
    x = np.asarray(x, np.float64)
    grid = _orig_decode(np.arange(127))
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    pick = np.where(a - grid[lo] < grid[hi] - a, lo, hi)
    return (pick | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _mut_bias8(codes):
    c = np.asarray(codes, dtype=np.int64)
    e, m = (c >> 3) & 0xF, c & 7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 8), np.ldexp(m / 8.0, -7))
    out = np.where(c & 0x80, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def _mut_max240(rows):
    x = np.asarray(rows, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(240.0), np.float32(1.0)).astype(np.float32)
    r = np.clip((x / scale[..., None]).astype(np.float32), -448, 448)
    return _orig_encode(r), scale


@pytest.mark.parametrize("target,mutant", [
    ("e4m3_encode", _mut_truncate), ("e4m3_encode", _mut_ties_away),
    ("e4m3_decode", _mut_bias8), ("quantize_rows", _mut_max240),
], ids=["truncate", "ties_away", "bias8", "max240"])
def test_planted_mistakes(monkeypatch, target, mutant):
    monkeypatch.setattr(qr, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    failed = []
    for name, fn in PINS:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    assert failed, "planted mistake caught by no pin"
