"""GPU parity of mla_cache_append (through the C ABI) against the CPU oracle
(oracle.append_rows / oracle.append_into, fp64).

Tolerances as for decode: bf16 storage -- relative L2 <= 1e-2 and max abs
<= 2e-2 on the appended rows; fp32 -- relative L2 <= 1e-5.  Every row the call
must not write is compared bitwise (the caches start filled with NaN or with
drawn rows).
"""

import sys

import numpy as np
import pytest
import torch

import head_latent_attention_absorb_amd as mla
import oracle
from tests.gpu_util import assert_close, from_dev, rel_l2
from workload import CONFIGS, f32_to_bf16_bits, make_append_case, make_case

pytestmark = pytest.mark.gpu

DSV2 = CONFIGS["dsv2_b16_t4096"]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(f32_to_bf16_bits(np.asarray(x, np.float32)).view(np.int16)) \
            .view(torch.bfloat16).cuda()
    return torch.from_numpy(np.asarray(x, np.float32)).cuda()


def _run(cfg, seed, *, cache_np=None, page_table=None, positions=None, yarn=None):
    """Append with the GPU; return (device cache after, host cache before,
    positions, oracle rows)."""
    ac = make_append_case(cfg, seed)
    if positions is not None:
        ac.positions = np.asarray(positions, np.int32)
    if cache_np is None:
        cache_np = make_case(cfg, seed, pad_value=np.nan).cache
    data = _dev(cache_np, cfg.dtype)
    lens = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")
    pt = torch.from_numpy(page_table).cuda() if page_table is not None else None
    cache = mla.latent_cache(data, lens, cfg.d_rope, pt, cfg.page_size,
                             cfg.max_len if pt is not None else None)
    y = dict(yarn_scale=1.0) if yarn is None else yarn
    mla.cache_append(cache, _dev(ac.h, cfg.dtype), _dev(ac.w_dkv, cfg.dtype),
                     _dev(ac.w_kr, cfg.dtype), _dev(ac.rms_weight, cfg.dtype),
                     torch.from_numpy(ac.positions).cuda(), rms_eps=1e-6, rope_base=10000.0, **y)
    torch.cuda.synchronize()
    rows = oracle.append_rows(ac.h, ac.w_dkv, ac.w_kr, ac.rms_weight, 1e-6, ac.positions,
                              10000.0, y.get("yarn_scale", 1.0), y.get("yarn_alpha", 1.0),
                              y.get("yarn_beta", 32.0), y.get("yarn_original_len", 4096))
    return from_dev(data), cache_np, ac.positions, rows


def _check(after, before, positions, rows, dtype, page_table=None, page_size=0):
    want = oracle.append_into(before, rows, positions, page_table, page_size)
    written = np.zeros(before.shape[:2], bool)
    got_rows, ref_rows = [], []
    for b, p in enumerate(positions):
        if page_table is None:
            idx = (b, int(p))
        else:
            idx = (int(page_table[b, p // page_size]), int(p % page_size))
        written[idx] = True
        got_rows.append(after[idx])
        ref_rows.append(want[idx])
    if len(got_rows):
        assert_close(np.array(got_rows), np.array(ref_rows), dtype, "appended rows")
    # Everything else is untouched, bit for bit (NaN padding included).
    b_rows = np.asarray(before, np.float64)[~written]
    a_rows = after[~written]
    if dtype == "bf16":
        b_rows = oracle_round(b_rows)
    assert np.array_equal(a_rows, b_rows, equal_nan=True)


def oracle_round(x):
    from workload import round_to_bf16
    return np.asarray(round_to_bf16(np.asarray(x, np.float32)), np.float64)


def test_tiny_f32_append():
    cfg = CONFIGS["tiny_f32"]
    _log(f"[append] tiny f32 d_model={cfg.hidden}")
    after, before, pos, rows = _run(cfg, 3)
    _check(after, before, pos, rows, "f32")
    assert rel_l2(after[0, pos[0]], rows[0]) <= 1e-5


@pytest.mark.parametrize("seed", [0, 1])
def test_dsv2_append_contiguous(seed):
    cfg = DSV2.replace(max_len=512, len_lo=1, len_hi=512)
    _log(f"[append] dsv2 B={cfg.batch} d_model={cfg.hidden} seed={seed}")
    after, before, pos, rows = _run(cfg, seed)
    _check(after, before, pos, rows, "bf16")


def test_dsv2_append_paged_b128():
    cfg = CONFIGS["paged_b128_t2048"]
    case = make_case(cfg, 5, seq_lens=np.ones(cfg.batch, np.int32), pad_value=np.nan)
    _log(f"[append] paged B={cfg.batch} page={cfg.page_size}")
    after, before, pos, rows = _run(cfg, 5, cache_np=case.cache, page_table=case.page_table)
    _check(after, before, pos, rows, "bf16", case.page_table, cfg.page_size)


def test_yarn_append_at_long_positions():
    """YaRN (s = 40, alpha = 1, beta = 32, from 4K) at positions beyond 100K,
    where an fp32 rotation angle would already be visibly wrong.  A 16-page
    pool aliased by a 131072-token page table keeps the cache small."""
    cfg = DSV2.replace(batch=2, max_len=131072, len_lo=1, len_hi=1, page_size=64)
    rng = np.random.default_rng(7)
    pool = np.full((16, 64, cfg.row), np.nan, np.float32)
    pt = rng.integers(0, 16, size=(2, cfg.max_pages)).astype(np.int32)
    positions = np.array([100003, 131071], np.int32)
    pt[1, positions[1] // 64] = (pt[0, positions[0] // 64] + 1) % 16  # distinct target pages
    yarn = dict(yarn_scale=40.0, yarn_alpha=1.0, yarn_beta=32.0, yarn_original_len=4096)
    _log("[append] yarn long positions")
    after, before, pos, rows = _run(cfg, 9, cache_np=pool, page_table=pt, positions=positions,
                                    yarn=yarn)
    _check(after, before, pos, rows, "bf16", pt, 64)
    # The key part really moved with YaRN: without it the same positions give
    # other values.
    plain = oracle.append_rows(*[getattr(make_append_case(cfg, 9), k) for k in
                                 ("h", "w_dkv", "w_kr", "rms_weight")], 1e-6, positions, 10000.0)
    assert not np.allclose(plain[:, cfg.d_latent:], rows[:, cfg.d_latent:], atol=1e-2)


def test_positions_outside_the_cache_write_nothing():
    cfg = DSV2.replace(batch=3, max_len=256, len_lo=1, len_hi=256)
    _log("[append] out-of-range positions")
    after, before, pos, rows = _run(cfg, 4, positions=[-1, 256, 100])
    # Only request 2's row is written; everything else is untouched.
    exp = oracle_round(before)
    exp[2, 100] = after[2, 100]
    assert np.array_equal(after, exp, equal_nan=True)
    assert_close(after[2, 100][None], rows[2][None], "bf16", "row")


def test_workspace_reuse_across_batches():
    """One workspace for calls of different batch sizes, never cleared: each
    call writes the same rows as with a fresh workspace (the workspace carries
    nothing from one call to the next)."""
    ws = torch.full((1 << 20,), 0x7F, dtype=torch.uint8, device="cuda")
    for batch in (16, 4, 16, 1):
        cfg = DSV2.replace(batch=batch, max_len=64, len_lo=1, len_hi=64)
        ac = make_append_case(cfg, 40 + batch)
        args = [_dev(ac.h, cfg.dtype), _dev(ac.w_dkv, cfg.dtype), _dev(ac.w_kr, cfg.dtype),
                _dev(ac.rms_weight, cfg.dtype), torch.from_numpy(ac.positions % 64).cuda()]
        lens = torch.zeros(batch, dtype=torch.int32, device="cuda")
        outs = []
        for w in (ws, None):
            data = torch.zeros((batch, 64, cfg.d_latent + cfg.d_rope), dtype=torch.bfloat16,
                               device="cuda")
            mla.cache_append(mla.latent_cache(data, lens, cfg.d_rope), *args, workspace=w)
            torch.cuda.synchronize()
            outs.append(data)
        _log(f"[append reuse] batch={batch}")
        assert torch.equal(outs[0], outs[1])
