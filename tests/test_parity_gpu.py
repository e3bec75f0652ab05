"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (fp32 accumulation everywhere): bf16 storage -- relative L2 error
<= 1e-2 and max abs error <= 2e-2; fp32 storage -- relative L2 error <= 1e-5.

References:
  * full decode step o  -> oracle.mla_decode_reference (unabsorbed, fp64)
  * q_cat (absorb)      -> oracle.absorb_query
  * o_lat, lse (decode) -> oracle.latent_attention, which the oracle pins equal
                           to the unabsorbed reference with identity W^UK/W^UV
  * o from o_lat        -> oracle.project_out
The decode and output steps are also tested on their own with seeded inputs
(draw_latent_query / draw_latent_output), never with values produced by the
HIP path.
"""

import sys

import numpy as np
import pytest
import torch

import head_latent_attention_absorb_amd as mla
import oracle
from tests.gpu_util import DevCase, assert_close, from_dev, max_abs, rel_l2
from workload import CONFIGS, draw_latent_output, draw_latent_query, make_case

pytestmark = pytest.mark.gpu

DSV2 = CONFIGS["dsv2_b16_t4096"]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16_dev(x: np.ndarray) -> torch.Tensor:
    from workload import f32_to_bf16_bits
    return torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def _latent_ref(case, q_cat: np.ndarray, requests=None, heads=None):
    """oracle.latent_attention per request on the given (seeded) absorbed query."""
    cfg = case.cfg
    B = cfg.batch
    reqs = range(B) if requests is None else requests
    hs = np.arange(cfg.n_heads) if heads is None else np.asarray(heads)
    o = np.zeros((B, cfg.n_heads, cfg.d_latent))
    lse = np.full((B, cfg.n_heads), -np.inf)
    for b in reqs:
        rows = oracle.gather_rows(case.cache, b, int(case.seq_lens[b]), case.page_table,
                                  cfg.page_size)
        o[b, hs], lse[b, hs] = oracle.latent_attention(q_cat[b, hs], rows, cfg.d_latent,
                                                       cfg.scale)
    return o, lse


def _decode_only(case, dc: DevCase, seed: int, split_tokens=0):
    q_np = draw_latent_query(case.cfg, seed)
    q_dev = _bf16_dev(q_np) if case.cfg.dtype == "bf16" else torch.from_numpy(q_np).cuda()
    o_lat, lse = mla.decode_attn(q_dev, dc.cache, case.cfg.scale, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return q_np, from_dev(o_lat), from_dev(lse)


# ----------------------------------------------------------------------------
# Tiny fp32 config: B=1, n_h=4, d_h=16, d_h^R=8, d_c=32, T=64, seeds 0-9
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(10))
def test_tiny_f32_full_chain(seed):
    cfg = CONFIGS["tiny_f32"]
    case = make_case(cfg, seed)
    _log(f"[tiny_f32] seed={seed}")
    q_cat, o_lat, lse, o = DevCase(case).run()
    o_ref, lse_ref = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache,
                                                 case.seq_lens, case.w_uk, case.w_uv, cfg.scale)
    assert_close(from_dev(o), o_ref, "f32", "o")
    assert_close(from_dev(lse), lse_ref, "f32", "lse")
    assert_close(from_dev(q_cat), oracle.absorb_query(case.q_c, case.q_r, case.w_uk), "f32",
                 "q_cat")


@pytest.mark.parametrize("split", [0, 1, 7, 64])
def test_tiny_f32_splits(split):
    cfg = CONFIGS["tiny_f32"]
    case = make_case(cfg, 3)
    _log(f"[tiny_f32 splits] split={split}")
    dc = DevCase(case)
    q_np, o_lat, lse = _decode_only(case, dc, 3, split_tokens=split)
    o_ref, lse_ref = _latent_ref(case, q_np)
    assert_close(o_lat, o_ref, "f32", "o_lat")
    assert_close(lse, lse_ref, "f32", "lse")


# ----------------------------------------------------------------------------
# DeepSeek-V2 dims at small sizes: several tiles, ragged tails, paging
# ----------------------------------------------------------------------------

SMALL = DSV2.replace(name="dsv2_small", batch=3, len_lo=1, len_hi=320, max_len=320)
SMALL_PAGED = DSV2.replace(name="dsv2_small_paged", batch=5, len_lo=1, len_hi=384,
                           max_len=384, page_size=64)


@pytest.mark.parametrize("cfg", [SMALL, SMALL_PAGED], ids=["contiguous", "paged"])
@pytest.mark.parametrize("split", [0, 32, 64, 96, 320])
def test_decode_small_bf16(cfg, split):
    lens = np.array([1, 37, 300, 384, 129][:cfg.batch], np.int32)
    lens = np.minimum(lens, cfg.max_len)
    case = make_case(cfg, 11, seq_lens=lens, pad_value=np.nan)
    _log(f"[decode small] {cfg.name} split={split} lens={lens.tolist()}")
    dc = DevCase(case)
    q_np, o_lat, lse = _decode_only(case, dc, 11, split_tokens=split)
    o_ref, lse_ref = _latent_ref(case, q_np)
    assert np.isfinite(o_lat).all() and np.isfinite(lse).all()
    assert_close(o_lat, o_ref, "bf16", "o_lat")
    assert_close(lse, lse_ref, "bf16", "lse")


@pytest.mark.parametrize("cfg", [SMALL, SMALL_PAGED], ids=["contiguous", "paged"])
def test_chain_small_bf16(cfg):
    case = make_case(cfg, 5)
    _log(f"[chain small] {cfg.name} lens={case.seq_lens.tolist()}")
    q_cat, o_lat, lse, o = DevCase(case).run()
    o_ref, lse_ref = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache, case.seq_lens,
                                                 case.w_uk, case.w_uv, cfg.scale,
                                                 case.page_table, cfg.page_size)
    assert_close(from_dev(o), o_ref, "bf16", "o")
    assert_close(from_dev(lse), lse_ref, "bf16", "lse")
    assert_close(from_dev(q_cat), oracle.absorb_query(case.q_c, case.q_r, case.w_uk), "bf16",
                 "q_cat")


@pytest.mark.parametrize("cfg", [SMALL, SMALL_PAGED], ids=["contiguous", "paged"])
def test_chain_small_bf16_fused(cfg):
    """absorb -> partials -> combine fused with W^UV against the oracle."""
    case = make_case(cfg, 5)
    _log(f"[chain small fused] {cfg.name} lens={case.seq_lens.tolist()}")
    _, o_lat, lse, o = DevCase(case).run_fused()
    o_ref, lse_ref = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache, case.seq_lens,
                                                 case.w_uk, case.w_uv, cfg.scale,
                                                 case.page_table, cfg.page_size)
    assert_close(from_dev(o), o_ref, "bf16", "o")
    assert_close(from_dev(lse), lse_ref, "bf16", "lse")


# 40 requests: past the batch where mla_decode_combine_out stops fusing.
MID_B40 = DSV2.replace(name="dsv2_b40_short", batch=40, len_lo=1, len_hi=160, max_len=160)


@pytest.mark.parametrize("cfg", [SMALL, SMALL_PAGED, MID_B40], ids=["contiguous", "paged", "b40"])
@pytest.mark.parametrize("split", [0, 64])
def test_combine_out_matches_separate_calls(cfg, split):
    """The tail in one call writes exactly mla_decode_combine's o_lat and lse,
    and an o that differs from mla_out_uv(o_lat) only by fp32 summation order
    (fused kernel up to 32 requests, the two calls beyond)."""
    case = make_case(cfg, 15)
    _log(f"[combine_out] {cfg.name} split={split}")
    dc = DevCase(case)
    q_np = draw_latent_query(cfg, 15)
    q_dev = _bf16_dev(q_np)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           split_tokens=split, d_head=cfg.d_head)
    ws = mla.workspace_for(plan, "cuda")
    mla.decode_partials(q_dev, dc.cache, cfg.scale, plan, ws)
    shape = (cfg.batch, cfg.n_heads, cfg.d_latent)
    o_lat1 = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse1 = torch.empty(shape[:2], dtype=torch.float32, device="cuda")
    mla.decode_combine(dc.cache, cfg.n_heads, plan, ws, o_lat1, lse1)
    o1 = mla.out_uv(o_lat1, dc.w_uv)
    o_lat2 = torch.empty_like(o_lat1)
    lse2 = torch.empty_like(lse1)
    o2 = mla.decode_combine_out(dc.cache, plan, ws, dc.w_uv, o_lat2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o_lat1, o_lat2) and torch.equal(lse1, lse2)
    a, b = from_dev(o1), from_dev(o2)
    # Both round an fp32 sum of the same bf16 products to bf16: at most one
    # bf16 step apart (2^-8 relative).
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6)
    o_ref, _ = _latent_ref(case, q_np)
    assert_close(from_dev(o_lat2), o_ref, "bf16", "o_lat")


# Many splits per request: 157 partitions of 32 tokens, so the merge spreads
# each request over 8 waves (two batches of loads each), and the short
# requests leave most of those waves without a used split.
MANY_SPLITS = DSV2.replace(name="dsv2_b3_many_splits", batch=3, len_lo=1, len_hi=5000,
                           max_len=5024)


@pytest.mark.parametrize("lens", [(1, 300, 5000), (5000, 33, 4097)], ids=["short_first", "long_first"])
def test_combine_many_splits(lens):
    cfg = MANY_SPLITS
    case = make_case(cfg, 21, seq_lens=np.array(lens, np.int32), pad_value=np.nan)
    _log(f"[many_splits] lens={lens}")
    dc = DevCase(case)
    q_np = draw_latent_query(cfg, 21)
    q_dev = _bf16_dev(q_np)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           split_tokens=32, d_head=cfg.d_head)
    assert plan.num_splits == 157
    ws = mla.workspace_for(plan, "cuda")
    mla.decode_partials(q_dev, dc.cache, cfg.scale, plan, ws)
    shape = (cfg.batch, cfg.n_heads, cfg.d_latent)
    o_lat1 = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse1 = torch.empty(shape[:2], dtype=torch.float32, device="cuda")
    mla.decode_combine(dc.cache, cfg.n_heads, plan, ws, o_lat1, lse1)
    o_lat2 = torch.empty_like(o_lat1)
    lse2 = torch.empty_like(lse1)
    mla.decode_combine_out(dc.cache, plan, ws, dc.w_uv, o_lat2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o_lat1, o_lat2) and torch.equal(lse1, lse2)
    heads = np.arange(0, 128, 9)
    o_ref, lse_ref = _latent_ref(case, q_np, heads=heads)
    assert_close(from_dev(o_lat1)[:, heads], o_ref[:, heads], "bf16", "o_lat")
    assert_close(from_dev(lse1)[:, heads], lse_ref[:, heads], "bf16", "lse")


@pytest.mark.parametrize("seed", [0, 4])
def test_tiny_f32_combine_out(seed):
    """fp32 storage takes the generic merge and projection behind the same call."""
    cfg = CONFIGS["tiny_f32"]
    case = make_case(cfg, seed)
    _, o_lat, lse, o = DevCase(case).run_fused(split_tokens=16)
    o_ref, lse_ref = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache,
                                                 case.seq_lens, case.w_uk, case.w_uv, cfg.scale)
    assert_close(from_dev(o), o_ref, "f32", "o")
    assert_close(from_dev(lse), lse_ref, "f32", "lse")


@pytest.mark.parametrize("batch", [1, 16, 33, 129, 200])
def test_absorb_q_bf16(batch):
    """Decode row counts: one M tile, a ragged second tile, a second chunk of
    one row, seven tiles over two chunks."""
    cfg = DSV2.replace(batch=batch, len_lo=1, len_hi=1, max_len=1)
    case = make_case(cfg, 2)
    dc = DevCase(case)
    q_cat = mla.absorb_q(dc.q_c, dc.q_r, dc.w_uk)
    torch.cuda.synchronize()
    assert_close(from_dev(q_cat), oracle.absorb_query(case.q_c, case.q_r, case.w_uk), "bf16",
                 "q_cat")


# Heads checked at prefill row counts (every row of them): both ends, and
# heads on either side of the groups of 8 that share an XCD.
_SAMPLED_HEADS = [0, 1, 7, 8, 9, 63, 64, 120, 126, 127]


@pytest.mark.parametrize("batch", [256, 300, 2085])
def test_absorb_q_bf16_many_rows(batch):
    """Prefill-sized row counts: the form that keeps a head's whole W^UK in
    LDS, with row runs split over workgroups and a ragged last run."""
    cfg = DSV2.replace(batch=batch, len_lo=1, len_hi=1, max_len=1)
    case = make_case(cfg, 5)
    dc = DevCase(case)
    _log(f"[absorb many rows] batch={batch}")
    q_cat = mla.absorb_q(dc.q_c, dc.q_r, dc.w_uk)
    torch.cuda.synchronize()
    hs = _SAMPLED_HEADS
    assert_close(from_dev(q_cat)[:, hs],
                 oracle.absorb_query(case.q_c[:, hs], case.q_r[:, hs], case.w_uk[hs]), "bf16",
                 "q_cat")


@pytest.mark.parametrize("batch", [256, 300, 2085])
def test_out_uv_bf16_many_rows(batch):
    cfg = DSV2.replace(batch=batch, len_lo=1, len_hi=1, max_len=1)
    case = make_case(cfg, 6)
    o_lat_np = draw_latent_output(cfg, 6)
    _log(f"[out_uv many rows] batch={batch}")
    o = mla.out_uv(_bf16_dev(o_lat_np), DevCase(case).w_uv)
    torch.cuda.synchronize()
    hs = _SAMPLED_HEADS
    assert_close(from_dev(o)[:, hs], oracle.project_out(o_lat_np[:, hs], case.w_uv[hs]), "bf16",
                 "o")


@pytest.mark.parametrize("batch", [1, 16, 33, 128, 200])
def test_out_uv_bf16(batch):
    cfg = DSV2.replace(batch=batch, len_lo=1, len_hi=1, max_len=1)
    case = make_case(cfg, 4)
    o_lat_np = draw_latent_output(cfg, 4)
    o = mla.out_uv(_bf16_dev(o_lat_np), DevCase(case).w_uv)
    torch.cuda.synchronize()
    assert_close(from_dev(o), oracle.project_out(o_lat_np, case.w_uv), "bf16", "o")


@pytest.mark.parametrize("batch", [1, 40])
def test_projections_other_widths_bf16(batch):
    """The bf16 projection kernels at widths other than DeepSeek-V2's: d_c = 256
    (two 128-column blocks of W^UK per head) for the absorption and d_h = 64
    (one 64-column block of W^UV) for the output, with one M tile and with two
    (the row-chunk form), against the oracle."""
    cfg = DSV2.replace(batch=batch, len_lo=1, len_hi=1, max_len=1, n_heads=24, d_latent=256)
    case = make_case(cfg, 8)
    dc = DevCase(case)
    _log(f"[projection widths] batch={batch} d_c=256")
    q_cat = mla.absorb_q(dc.q_c, dc.q_r, dc.w_uk)
    torch.cuda.synchronize()
    assert_close(from_dev(q_cat), oracle.absorb_query(case.q_c, case.q_r, case.w_uk), "bf16",
                 "q_cat")
    cfg_o = DSV2.replace(batch=batch, len_lo=1, len_hi=1, max_len=1, n_heads=24, d_head=64)
    case_o = make_case(cfg_o, 9)
    o_lat_np = draw_latent_output(cfg_o, 9)
    _log(f"[projection widths] batch={batch} d_h=64")
    o = mla.out_uv(_bf16_dev(o_lat_np), DevCase(case_o).w_uv)
    torch.cuda.synchronize()
    assert_close(from_dev(o), oracle.project_out(o_lat_np, case_o.w_uv), "bf16", "o")


@pytest.mark.parametrize("batch", [33, 65, 129, 200, 255])
def test_projections_row_chunks_match_one_tile(batch):
    """Above one M tile (32 rows) both projections stage chunks of rows in
    LDS (128 rows for absorption, 64 for the output); each row's product has
    the same operands and summation order as with one tile, so the first and
    the last rows of the batch, computed again as batches of their own (one
    tile), must come out bit for bit the same."""
    cfg = DSV2.replace(batch=batch, len_lo=1, len_hi=1, max_len=1)
    case = make_case(cfg, 7)
    dc = DevCase(case)
    o_lat = _bf16_dev(draw_latent_output(cfg, 7))
    _log(f"[projection row chunks] batch={batch}")
    q_cat = from_dev(mla.absorb_q(dc.q_c, dc.q_r, dc.w_uk))
    o = from_dev(mla.out_uv(o_lat, dc.w_uv))
    for lo, hi in ((0, 16), (batch - min(batch, 32) + 1, batch)):
        q_part = from_dev(mla.absorb_q(dc.q_c[lo:hi].contiguous(), dc.q_r[lo:hi].contiguous(),
                                       dc.w_uk))
        o_part = from_dev(mla.out_uv(o_lat[lo:hi].contiguous(), dc.w_uv))
        torch.cuda.synchronize()
        assert np.array_equal(q_cat[lo:hi], q_part), f"q_cat rows {lo}..{hi - 1}"
        assert np.array_equal(o[lo:hi], o_part), f"o rows {lo}..{hi - 1}"


# ----------------------------------------------------------------------------
# Edge cases and invariants
# ----------------------------------------------------------------------------

def test_zero_length_requests():
    cfg = SMALL
    lens = np.array([0, 40, 0], np.int32)
    case = make_case(cfg, 6, seq_lens=lens, pad_value=np.nan)
    dc = DevCase(case)
    q_np, o_lat, lse = _decode_only(case, dc, 6)
    assert np.all(o_lat[0] == 0) and np.all(o_lat[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    o_ref, lse_ref = _latent_ref(case, q_np, requests=[1])
    assert_close(o_lat[1], o_ref[1], "bf16", "o_lat[1]")


def test_zero_length_requests_fused():
    cfg = SMALL
    lens = np.array([0, 40, 0], np.int32)
    case = make_case(cfg, 6, seq_lens=lens, pad_value=np.nan)
    _, o_lat, lse, o = DevCase(case).run_fused()
    o = from_dev(o)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.all(np.isneginf(from_dev(lse)[[0, 2]]))
    o_ref, _ = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache, case.seq_lens,
                                           case.w_uk, case.w_uv, cfg.scale, requests=[1])
    assert_close(o[1], o_ref[1], "bf16", "o[1]")


def test_single_token_request_equals_row():
    """T = 1: the output is the cached latent itself, for every head."""
    cfg = SMALL.replace(batch=1)
    case = make_case(cfg, 8, seq_lens=np.array([1], np.int32))
    dc = DevCase(case)
    _, o_lat, _ = _decode_only(case, dc, 8)
    row = case.cache[0, 0, :cfg.d_latent]
    assert np.array_equal(o_lat[0], np.broadcast_to(row, o_lat[0].shape))


def test_page_permutation_is_bitwise_invariant():
    cfg = SMALL_PAGED
    case = make_case(cfg, 9)
    dc = DevCase(case)
    q_np, o1, l1 = _decode_only(case, dc, 9, split_tokens=64)
    # Move every page to a new physical slot.
    perm = np.random.default_rng(1).permutation(case.cache.shape[0])
    pool2 = np.empty_like(case.cache)
    pool2[perm] = case.cache
    case2 = make_case(cfg, 9)
    case2.cache = pool2
    case2.page_table = perm[case.page_table].astype(np.int32)
    _, o2, l2 = _decode_only(case2, DevCase(case2), 9, split_tokens=64)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_paged_equals_contiguous_bitwise():
    cfg = SMALL_PAGED
    case = make_case(cfg, 12)
    q_np, o_p, l_p = _decode_only(case, DevCase(case), 12, split_tokens=64)
    cont = np.zeros((cfg.batch, cfg.max_len, cfg.row), np.float32)
    for b in range(cfg.batch):
        n = int(case.seq_lens[b])
        cont[b, :n] = case.cache.reshape(-1, cfg.row)[case.logical_row_index(b)]
    case_c = make_case(cfg.replace(page_size=0), 12)
    case_c.cache = cont
    case_c.seq_lens = case.seq_lens
    case_c.page_table = None
    _, o_c, l_c = _decode_only(case_c, DevCase(case_c), 12, split_tokens=64)
    assert np.array_equal(o_p, o_c) and np.array_equal(l_p, l_c)


def test_request_independence_and_determinism():
    cfg = SMALL
    case = make_case(cfg, 13)
    dc = DevCase(case)
    # The default (length-balanced) plan is deterministic.
    _, o1, l1 = _decode_only(case, dc, 13)
    _, o2, l2 = _decode_only(case, dc, 13)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # Under one uniform split, request 0 alone gives bitwise the same result
    # as inside the batch.  (A balanced plan cuts partitions from the whole
    # batch's lengths, so there the rounding may differ.)
    _, o1, l1 = _decode_only(case, dc, 13, split_tokens=128)
    case1 = make_case(cfg.replace(batch=1), 13)
    case1.cache = case.cache[:1].copy()
    case1.seq_lens = case.seq_lens[:1].copy()
    q_full = draw_latent_query(cfg, 13)
    q_dev = _bf16_dev(q_full[:1])
    dc1 = DevCase(case1)
    o_lat, lse = mla.decode_attn(q_dev, dc1.cache, cfg.scale, split_tokens=128)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(o_lat)[0], o1[0])


@pytest.mark.parametrize("scale", [-0.0722, 0.0], ids=["negative", "zero"])
def test_scale_sign_and_zero(scale):
    """The softmax scale is a free parameter of the call.  A negative scale
    reverses the score order (the kernel's max must follow it) and zero gives
    uniform weights over every valid token, including a partial last tile."""
    cfg = SMALL.replace(softmax_scale=scale)
    lens = np.array([1, 45, 300], np.int32)
    case = make_case(cfg, 21, seq_lens=lens, pad_value=np.nan)
    _log(f"[scale] scale={scale} lens={lens.tolist()}")
    dc = DevCase(case)
    q_np, o_lat, lse = _decode_only(case, dc, 21, split_tokens=96)
    o_ref, lse_ref = _latent_ref(case, q_np)
    assert np.isfinite(o_lat).all() and np.isfinite(lse).all()
    assert_close(o_lat, o_ref, "bf16", "o_lat")
    assert_close(lse, lse_ref, "bf16", "lse")
    if scale == 0.0:
        for b, n in enumerate(lens):
            mean = case.cache[b, :n, :cfg.d_latent].astype(np.float64).mean(axis=0)
            assert max_abs(o_lat[b], np.broadcast_to(mean, o_lat[b].shape)) <= 2e-2
            assert np.allclose(lse[b], np.log(n), atol=1e-5)


def test_large_scores_rescale_path():
    """Scores that keep growing along the sequence (by ~30 in natural-log units
    over 300 tokens) push later tiles far past the running max, exercising the
    accumulator rescale; the result must still match at the stated bf16
    tolerances.  The softmax is then nearly one-hot, so o is close to single
    cached rows: the rows are scaled by 1/4 and the query by 4 more (every
    score unchanged), which keeps |o| at unit scale, where those tolerances
    are stated."""
    cfg = SMALL
    lens = np.array([300, 300, 300], np.int32)
    case = make_case(cfg, 14, seq_lens=lens)
    from workload import round_to_bf16
    q_np = round_to_bf16((draw_latent_query(cfg, 14) * 32.0).astype(np.float32))
    for b in range(cfg.batch):
        ramp = (np.arange(300, dtype=np.float32) / 1000.0)[:, None]
        case.cache[b, :300, :cfg.d_latent] += ramp * np.sign(q_np[b, 0, :cfg.d_latent])
    case.cache = round_to_bf16(case.cache * np.float32(0.25))
    dc = DevCase(case)
    o_lat, lse = mla.decode_attn(_bf16_dev(q_np), dc.cache, cfg.scale, split_tokens=320)
    torch.cuda.synchronize()
    o_ref, lse_ref = _latent_ref(case, q_np)
    # Head 0 of every request is the one whose scores ramp up.
    assert lse_ref[:, 0].min() > lse_ref[:, 1:].max() - 5
    assert np.abs(o_ref).max() < 1.5
    assert_close(from_dev(o_lat), o_ref, "bf16", "o_lat")
    assert_close(from_dev(lse), lse_ref, "bf16", "lse")


# ----------------------------------------------------------------------------
# Full-size configurations
# ----------------------------------------------------------------------------

def test_dsv2_b16_t4096_full():
    cfg = DSV2
    _log("[dsv2_b16_t4096] generating")
    case = make_case(cfg, 0)
    dc = DevCase(case)
    q_np, o_lat, lse = _decode_only(case, dc, 0)
    _log("[dsv2_b16_t4096] decode done; oracle on every request and head")
    o_ref, lse_ref = _latent_ref(case, q_np)
    r, m = assert_close(o_lat, o_ref, "bf16", "o_lat")
    assert_close(lse, lse_ref, "bf16", "lse")
    _log(f"[dsv2_b16_t4096] o_lat rel_l2={r:.2e} max_abs={m:.2e}")
    # Whole decode step on sampled (request, head) pairs against the unabsorbed form.
    _, _, _, o = dc.run()
    heads = [0, 37, 64, 127]
    reqs = [0, 9, 15]
    o_ref, _ = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache, case.seq_lens,
                                           case.w_uk, case.w_uv, cfg.scale,
                                           requests=reqs, heads=heads)
    got = from_dev(o)[np.ix_(reqs, heads)]
    assert_close(got, o_ref[np.ix_(reqs, heads)], "bf16", "o (sampled)")


def test_dsv2_b16_t4096_seed1_chain_sampled():
    cfg = DSV2
    case = make_case(cfg, 1)
    _, o_lat, lse, o = DevCase(case).run()
    heads = [3, 100]
    reqs = [4, 11]
    o_ref, lse_ref = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache, case.seq_lens,
                                                 case.w_uk, case.w_uv, cfg.scale,
                                                 requests=reqs, heads=heads)
    assert_close(from_dev(o)[np.ix_(reqs, heads)], o_ref[np.ix_(reqs, heads)], "bf16", "o")
    assert_close(from_dev(lse)[np.ix_(reqs, heads)], lse_ref[np.ix_(reqs, heads)], "bf16",
                 "lse")


def test_dsv2_b16_t4096_fused_chain_sampled():
    cfg = DSV2
    case = make_case(cfg, 0)
    _log("[dsv2_b16_t4096 fused] running")
    _, o_lat, lse, o = DevCase(case).run_fused()
    heads = [1, 64, 126]
    reqs = [0, 7, 15]
    o_ref, lse_ref = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache, case.seq_lens,
                                                 case.w_uk, case.w_uv, cfg.scale,
                                                 requests=reqs, heads=heads)
    assert_close(from_dev(o)[np.ix_(reqs, heads)], o_ref[np.ix_(reqs, heads)], "bf16", "o")
    assert_close(from_dev(lse)[np.ix_(reqs, heads)], lse_ref[np.ix_(reqs, heads)], "bf16",
                 "lse")


@pytest.mark.parametrize("seed", [0, 1])
def test_ragged_b4_long(seed):
    cfg = CONFIGS["ragged_b4_16k_32k"]
    case = make_case(cfg, seed, pad_value=np.nan)
    _log(f"[ragged_b4] seed={seed} lens={case.seq_lens.tolist()}")
    dc = DevCase(case)
    q_np, o_lat, lse = _decode_only(case, dc, seed)
    assert np.isfinite(o_lat).all()
    heads = np.arange(0, 128, 4)
    o_ref, lse_ref = _latent_ref(case, q_np, heads=heads)
    assert_close(o_lat[:, heads], o_ref[:, heads], "bf16", "o_lat")
    assert_close(lse[:, heads], lse_ref[:, heads], "bf16", "lse")
    _, _, _, o = dc.run()
    o_ref, _ = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache, case.seq_lens,
                                           case.w_uk, case.w_uv, cfg.scale, requests=[0, 3],
                                           heads=[5, 77])
    assert_close(from_dev(o)[np.ix_([0, 3], [5, 77])], o_ref[np.ix_([0, 3], [5, 77])], "bf16",
                 "o (sampled)")


@pytest.mark.parametrize("seed", [0, 1])
def test_paged_b128(seed):
    cfg = CONFIGS["paged_b128_t2048"]
    case = make_case(cfg, seed, pad_value=np.nan)
    _log(f"[paged_b128] seed={seed}")
    dc = DevCase(case)
    q_np, o_lat, lse = _decode_only(case, dc, seed)
    assert np.isfinite(o_lat).all()
    reqs = list(range(0, 128, 8)) + [int(np.argmin(case.seq_lens)), int(np.argmax(case.seq_lens))]
    o_ref, lse_ref = _latent_ref(case, q_np, requests=reqs)
    assert_close(o_lat[reqs], o_ref[reqs], "bf16", "o_lat")
    assert_close(lse[reqs], lse_ref[reqs], "bf16", "lse")
    _, _, _, o = dc.run()
    o_ref, _ = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache, case.seq_lens,
                                           case.w_uk, case.w_uv, cfg.scale, case.page_table,
                                           cfg.page_size, requests=reqs[:4], heads=[1, 90])
    assert_close(from_dev(o)[np.ix_(reqs[:4], [1, 90])], o_ref[np.ix_(reqs[:4], [1, 90])],
                 "bf16", "o (sampled)")


@pytest.mark.parametrize("layer", [0, 59])
def test_ctx128k_layer(layer):
    cfg = CONFIGS["ctx128k_b2_60l"]
    _log(f"[ctx128k] layer={layer} generating")
    case = make_case(cfg, 1000 + layer)
    dc = DevCase(case)
    q_np, o_lat, lse = _decode_only(case, dc, 1000 + layer)
    heads = [0, 31, 64, 127]
    _log(f"[ctx128k] layer={layer} oracle")
    o_ref, lse_ref = _latent_ref(case, q_np, heads=heads)
    assert_close(o_lat[:, heads], o_ref[:, heads], "bf16", "o_lat")
    assert_close(lse[:, heads], lse_ref[:, heads], "bf16", "lse")
    _, _, _, o = dc.run()
    o_ref, _ = oracle.mla_decode_reference(case.q_c, case.q_r, case.cache, case.seq_lens,
                                           case.w_uk, case.w_uv, cfg.scale, heads=[7, 99])
    assert_close(from_dev(o)[:, [7, 99]], o_ref[:, [7, 99]], "bf16", "o (sampled)")
