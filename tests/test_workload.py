"""Input generator: determinism, bfloat16 rounding, lengths and page tables."""

import numpy as np

from workload import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_case, round_to_bf16


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1 + 2^-7: ties go to even (1.0).
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -1.0 - 2 ** -8, 0.0, -0.0], np.float32)
    r = round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0 + 2 ** -6          # 1.01100000 ties to even -> 1.0110 (rounds up)
    assert r[2] == 1.0 + 2 ** -7          # above the tie rounds up
    assert r[3] == -1.0
    assert np.signbit(r[5]) and r[5] == 0


def test_bf16_specials():
    x = np.array([np.inf, -np.inf, np.nan, np.finfo(np.float32).max, 1e-40], np.float32)
    bits = f32_to_bf16_bits(x)
    assert bits[0] == 0x7F80 and bits[1] == 0xFF80
    assert np.isnan(bf16_bits_to_f32(bits[2:3]))[0]
    assert np.isinf(bf16_bits_to_f32(bits[3:4]))[0]       # past max finite bf16 -> inf
    back = bf16_bits_to_f32(bits[4:5])[0]
    assert back > 0 and abs(back - 1e-40) < 0.1e-40        # subnormals survive (coarsely)


def test_bf16_exhaustive_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(bits)
    ok = ~np.isnan(f)
    assert np.array_equal(f32_to_bf16_bits(f)[ok], bits[ok])


def test_determinism_and_seed_sensitivity():
    cfg = CONFIGS["tiny_f32"]
    a, b, c = make_case(cfg, 3), make_case(cfg, 3), make_case(cfg, 4)
    for name in ("q_c", "q_r", "cache", "w_uk", "w_uv"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
        assert not np.array_equal(getattr(a, name), getattr(c, name))


def test_bf16_case_values_are_representable():
    cfg = CONFIGS["dsv2_b16_t4096"].replace(batch=2, len_lo=37, len_hi=300, max_len=320)
    case = make_case(cfg, 0)
    for name in ("q_c", "q_r", "cache", "w_uk", "w_uv"):
        x = getattr(case, name)
        assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(x)), x)
    assert 1 / 512 * 0.8 < case.w_uk.var() < 1 / 512 * 1.2


def test_ragged_lengths_in_range():
    cfg = CONFIGS["ragged_b4_16k_32k"]
    for seed in (0, 1):
        rng = np.random.Generator(np.random.PCG64(seed))
        lens = rng.integers(cfg.len_lo, cfg.len_hi, size=cfg.batch, endpoint=True)
        assert ((lens >= 16384) & (lens <= 32768)).all()


def test_paged_case_structure():
    cfg = CONFIGS["paged_b128_t2048"].replace(batch=6, max_len=256, len_hi=256)
    case = make_case(cfg, 1, pad_value=np.nan)
    pt = case.page_table
    assert pt.shape == (6, 4) and pt.dtype == np.int32
    assert np.array_equal(np.sort(pt.ravel()), np.arange(24))
    assert ((case.seq_lens >= 1) & (case.seq_lens <= 256)).all()
    # Pages owned by a request hold finite rows; everything else is padding.
    used = np.zeros(case.cache.shape[:2], bool)
    for b in range(6):
        idx = case.logical_row_index(b)
        used.reshape(-1)[idx] = True
    assert np.isfinite(case.cache[used]).all()
    assert np.isnan(case.cache[~used]).all()


def test_seq_lens_override_keeps_stream():
    cfg = CONFIGS["dsv2_b16_t4096"].replace(batch=2, len_lo=5, len_hi=9, max_len=16)
    a = make_case(cfg, 7)
    b = make_case(cfg, 7, seq_lens=a.seq_lens)
    assert np.array_equal(a.q_c, b.q_c) and np.array_equal(a.w_uv, b.w_uv)
