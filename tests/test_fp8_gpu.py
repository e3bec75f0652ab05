"""GPU parity of the low-bit cache (OCP E4M3 rows with one fp32 scale per
row), through the C ABI, against the CPU oracle:

* mla_quantize_rows against oracle.quantize_rows: codes and scales bit for
  bit (the codes are integers decided in fp32 on both sides);
* decode over a quantised cache against oracle.latent_attention over
  oracle.dequantize_rows of the same codes and scales (fp64), within the
  usual tolerances (bf16: relative L2 <= 1e-2, max abs <= 2e-2; fp32 query and
  output: relative L2 <= 1e-5).
"""

import sys

import numpy as np
import pytest
import torch

import head_latent_attention_absorb_amd as mla
import oracle
from tests.gpu_util import assert_close, from_dev
from workload import CONFIGS, draw_latent_query, f32_to_bf16_bits, make_case

pytestmark = pytest.mark.gpu

DSV2 = CONFIGS["dsv2_b16_t4096"]
TINY = CONFIGS["tiny_f32"]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16(x):
    return torch.from_numpy(f32_to_bf16_bits(np.asarray(x, np.float32)).view(np.int16)) \
        .view(torch.bfloat16).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_rows_bit_exact(dtype):
    rng = np.random.default_rng(11)
    rows = (rng.standard_normal((300, 576)) * rng.uniform(1e-3, 50, (300, 1))).astype(np.float32)
    rows[7] = 0.0
    rows[8, :] = 0.0
    rows[8, 100] = -3.5
    rows[9] *= 1e-30                      # codes in the subnormal range
    if dtype == "bf16":
        from workload import round_to_bf16
        rows = round_to_bf16(rows)
        x = _bf16(rows)
    else:
        x = torch.from_numpy(rows).cuda()
    codes, scales = mla.quantize_rows(x)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.quantize_rows(rows)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != c_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def _fp8_case(cfg, seed, lens, paged=False):
    case = make_case(cfg, seed, seq_lens=np.asarray(lens, np.int32), pad_value=0.0)
    codes, scales = oracle.quantize_rows(case.cache)
    return case, codes, scales


def _device_cache(case, codes, scales):
    cfg = case.cfg
    lens = torch.from_numpy(case.seq_lens.astype(np.int32)).cuda()
    pt = torch.from_numpy(case.page_table).cuda() if case.page_table is not None else None
    return mla.latent_cache(torch.from_numpy(codes).cuda(), lens, cfg.d_rope, pt,
                            cfg.page_size, cfg.max_len if cfg.paged else None,
                            scales=torch.from_numpy(scales).cuda())


def _reference(case, codes, scales, q, heads=None):
    cfg = case.cfg
    deq = oracle.dequantize_rows(codes, scales)
    hs = np.arange(cfg.n_heads) if heads is None else np.asarray(heads)
    o = np.zeros((cfg.batch, cfg.n_heads, cfg.d_latent))
    lse = np.full((cfg.batch, cfg.n_heads), -np.inf)
    for b in range(cfg.batch):
        rows = oracle.gather_rows(deq, b, int(case.seq_lens[b]), case.page_table, cfg.page_size)
        o[b, hs], lse[b, hs] = oracle.latent_attention(q[b, hs], rows, cfg.d_latent, cfg.scale)
    return o, lse


@pytest.mark.parametrize("split", [0, 7])
def test_tiny_f32_query_over_fp8_cache(split):
    cfg = TINY.replace(batch=3, len_lo=1, len_hi=64)
    case, codes, scales = _fp8_case(cfg, 81, [64, 1, 40])
    dc = _device_cache(case, codes, scales)
    q = draw_latent_query(cfg, 81)
    o_lat, lse = mla.decode_attn(torch.from_numpy(q).cuda(), dc, cfg.scale, split_tokens=split)
    torch.cuda.synchronize()
    o_ref, lse_ref = _reference(case, codes, scales, q)
    assert_close(from_dev(o_lat), o_ref, "f32", "o_lat")
    assert_close(from_dev(lse), lse_ref, "f32", "lse")


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("split", [0, 64])
def test_bf16_query_over_fp8_cache(paged, split):
    if paged:
        cfg = DSV2.replace(batch=3, len_lo=1, len_hi=600, max_len=640, page_size=64)
    else:
        cfg = DSV2.replace(batch=3, len_lo=1, len_hi=600, max_len=608)
    case, codes, scales = _fp8_case(cfg, 82, [600, 3, 257])
    _log(f"[fp8] {'paged' if paged else 'contiguous'} split={split}")
    dc = _device_cache(case, codes, scales)
    q = draw_latent_query(cfg, 82)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc,
                           split_tokens=split)
    assert plan.kernel == 1  # the MFMA kernel, converting the codes in LDS
    o_lat, lse = mla.decode_attn(_bf16(q), dc, cfg.scale, plan=plan)
    torch.cuda.synchronize()
    heads = np.arange(0, 128, 7)
    o_ref, lse_ref = _reference(case, codes, scales, q, heads)
    assert_close(from_dev(o_lat)[:, heads], o_ref[:, heads], "bf16", "o_lat")
    assert_close(from_dev(lse)[:, heads], lse_ref[:, heads], "bf16", "lse")


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_append_into_fp8_cache(paged):
    """mla_cache_append into a low-bit cache: the appended rows dequantise to
    the oracle's rows (oracle.append_rows, fp64) within E4M3's rounding
    (half a code step: 2^-4 relative, 2^-10 * scale below the normal range,
    plus the fp32 arithmetic), the scale is the row's max|x| / 448 to fp32
    rounding, and no other row or scale changes."""
    from workload import make_append_case
    if paged:
        cfg = DSV2.replace(batch=4, max_len=256, len_lo=1, len_hi=256, page_size=64)
    else:
        cfg = DSV2.replace(batch=4, max_len=256, len_lo=1, len_hi=256)
    ac = make_append_case(cfg, 91)
    base = make_case(cfg, 91, pad_value=0.0)
    codes0, scales0 = oracle.quantize_rows(base.cache)
    dc = _device_cache(base, codes0, scales0)
    mla.cache_append(dc, _bf16(ac.h), _bf16(ac.w_dkv), _bf16(ac.w_kr), _bf16(ac.rms_weight),
                     torch.from_numpy(ac.positions).cuda(), rms_eps=1e-6, rope_base=10000.0)
    torch.cuda.synchronize()
    codes, scales = dc.data.cpu().numpy(), dc.scales.cpu().numpy()
    rows = oracle.append_rows(ac.h, ac.w_dkv, ac.w_kr, ac.rms_weight, 1e-6, ac.positions,
                              10000.0)
    touched = np.zeros(codes.shape[:2], bool)
    for b, pos in enumerate(ac.positions):
        if base.page_table is None:
            idx = (b, int(pos))
        else:
            idx = (int(base.page_table[b, pos // cfg.page_size]), int(pos % cfg.page_size))
        touched[idx] = True
        ref = rows[b]
        s_ref = np.float32(np.max(np.abs(ref)) / 448.0)
        assert abs(scales[idx] - s_ref) <= 1e-5 * s_ref, (b, scales[idx], s_ref)
        deq = oracle.dequantize_rows(codes[idx][None], scales[idx][None])[0]
        r = np.abs(ref / scales[idx])
        bound = (np.where(r >= 2.0 ** -6, r * 2.0 ** -4, 2.0 ** -10) + 1e-3) * scales[idx]
        assert np.all(np.abs(deq - ref) <= bound), b
    assert np.array_equal(codes[~touched], codes0[~touched])
    assert np.array_equal(scales[~touched], scales0[~touched])
