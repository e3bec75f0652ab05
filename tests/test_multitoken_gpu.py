"""GPU parity of the causal decode of several new tokens per request (the
verification pass of speculative decoding), through the C ABI, against
oracle.latent_attention_causal (fp64).

Tolerances as for single-token decode: bf16 storage -- relative L2 <= 1e-2 and
max abs <= 2e-2; fp32 -- relative L2 <= 1e-5.  Queries come from the seeded
draw_latent_query stream ([B * q_len, n_h, row] reshaped token-major), caches
from make_case; nothing is taken from the HIP path.
"""

import sys

import numpy as np
import pytest
import torch

import head_latent_attention_absorb_amd as mla
import oracle
from tests.gpu_util import DevCase, assert_close, from_dev
from workload import CONFIGS, draw_latent_query, f32_to_bf16_bits, make_case

pytestmark = pytest.mark.gpu

DSV2 = CONFIGS["dsv2_b16_t4096"]
TINY = CONFIGS["tiny_f32"]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _query(cfg, seed, q_len):
    q = draw_latent_query(cfg, seed, batch=cfg.batch * q_len)
    q = q.reshape(cfg.batch, q_len, cfg.n_heads, cfg.row)
    if cfg.dtype == "bf16":
        dev = torch.from_numpy(f32_to_bf16_bits(q).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        dev = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    return q, dev


def _reference(case, q, q_len, heads=None):
    cfg = case.cfg
    hs = np.arange(cfg.n_heads) if heads is None else np.asarray(heads)
    o = np.zeros((cfg.batch, q_len, cfg.n_heads, cfg.d_latent))
    lse = np.full((cfg.batch, q_len, cfg.n_heads), -np.inf)
    for b in range(cfg.batch):
        rows = oracle.gather_rows(case.cache, b, int(case.seq_lens[b]), case.page_table,
                                  cfg.page_size)
        ob, lb = oracle.latent_attention_causal(q[b][:, hs], rows, cfg.d_latent, cfg.scale)
        o[b][:, hs], lse[b][:, hs] = ob, lb
    return o, lse


def _check(o_lat, lse, o_ref, lse_ref, dtype, heads=None):
    if heads is not None:
        o_lat, lse = o_lat[:, :, heads], lse[:, :, heads]
        o_ref, lse_ref = o_ref[:, :, heads], lse_ref[:, :, heads]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), "tokens with no visible row"
    assert np.all(o_lat[empty] == 0)
    assert_close(o_lat, o_ref, dtype, "o_lat")
    assert_close(lse[~empty], lse_ref[~empty], dtype, "lse")


@pytest.mark.parametrize("split", [0, 5, 16])
@pytest.mark.parametrize("q_len", [2, 3])
def test_tiny_f32_causal(q_len, split):
    """Generic kernel: lengths 1..64 include requests shorter than q_len."""
    cfg = TINY.replace(batch=4, len_lo=1, len_hi=64)
    case = make_case(cfg, 30 + q_len, seq_lens=np.array([64, 1, 2, 37], np.int32))
    _log(f"[mq tiny] q_len={q_len} split={split}")
    dc = DevCase(case)
    q, q_dev = _query(cfg, 30 + q_len, q_len)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.float32, dc.cache,
                           split_tokens=split, q_len=q_len)
    assert plan.q_len == q_len and plan.kernel == 0
    o_lat, lse = mla.decode_attn(q_dev, dc.cache, cfg.scale, plan=plan)
    torch.cuda.synchronize()
    o_ref, lse_ref = _reference(case, q, q_len)
    _check(from_dev(o_lat), from_dev(lse), o_ref, lse_ref, "f32")


@pytest.mark.parametrize("cfg_name,split", [("contiguous", 0), ("contiguous", 64),
                                            ("paged", 0)])
@pytest.mark.parametrize("q_len", [2, 4])
def test_bf16_causal(q_len, cfg_name, split):
    """MFMA kernel: ragged lengths, a request shorter than q_len, several
    partitions; contiguous and paged caches."""
    if cfg_name == "paged":
        cfg = DSV2.replace(batch=4, len_lo=1, len_hi=700, max_len=768, page_size=64)
    else:
        cfg = DSV2.replace(batch=4, len_lo=1, len_hi=700, max_len=704)
    lens = np.array([700, 2, 333, 64], np.int32)
    case = make_case(cfg, 40 + q_len, seq_lens=lens, pad_value=np.nan)
    _log(f"[mq bf16] {cfg_name} q_len={q_len} split={split}")
    dc = DevCase(case)
    q, q_dev = _query(cfg, 40 + q_len, q_len)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           split_tokens=split, q_len=q_len)
    assert plan.q_len == q_len and plan.kernel in (1, 2)
    assert plan.head_groups == q_len * (1 if plan.kernel == 1 else 2)
    o_lat, lse = mla.decode_attn(q_dev, dc.cache, cfg.scale, plan=plan)
    torch.cuda.synchronize()
    heads = np.arange(0, 128, 5)
    o_ref, lse_ref = _reference(case, q, q_len, heads)
    _check(from_dev(o_lat), from_dev(lse), o_ref, lse_ref, "bf16", heads)


def test_each_token_is_a_shorter_single_token_decode():
    """Query token j of a q_len pass equals a plain decode of the same query
    over the first seq_len - (q_len - 1 - j) rows, bit for bit (same kernel,
    same partitions)."""
    cfg = DSV2.replace(batch=3, len_lo=100, len_hi=900, max_len=928)
    case = make_case(cfg, 50, seq_lens=np.array([900, 130, 513], np.int32))
    dc = DevCase(case)
    q_len = 3
    _, q_dev = _query(cfg, 50, q_len)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           split_tokens=128, q_len=q_len)
    o_lat, lse = mla.decode_attn(q_dev, dc.cache, cfg.scale, plan=plan)
    for j in range(q_len):
        lens_j = (dc.seq_lens - (q_len - 1 - j)).contiguous()
        cache_j = mla.latent_cache(dc.cache_data, lens_j, cfg.d_rope)
        plan_j = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16,
                                 cache_j, split_tokens=128)
        o1, l1 = mla.decode_attn(q_dev[:, j].contiguous(), cache_j, cfg.scale, plan=plan_j)
        torch.cuda.synchronize()
        assert torch.equal(o1, o_lat[:, j]) and torch.equal(l1, lse[:, j]), f"token {j}"


@pytest.mark.parametrize("batch", [3, 20])
def test_combine_out_with_several_tokens(batch):
    """The tail in one call (fused while batch * q_len <= 32) writes exactly the
    split combine's o_lat and lse, and o within one bf16 step of
    out_uv(o_lat); o_lat matches the oracle."""
    q_len = 2
    cfg = DSV2.replace(batch=batch, len_lo=1, len_hi=400, max_len=416)
    case = make_case(cfg, 60 + batch, pad_value=np.nan)
    _log(f"[mq combine_out] batch={batch}")
    dc = DevCase(case)
    q, q_dev = _query(cfg, 60 + batch, q_len)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           split_tokens=64, d_head=cfg.d_head, q_len=q_len)
    ws = mla.workspace_for(plan, "cuda")
    mla.decode_partials(q_dev, dc.cache, cfg.scale, plan, ws)
    shape = (batch, q_len, cfg.n_heads, cfg.d_latent)
    o_lat1 = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse1 = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    mla.decode_combine(dc.cache, cfg.n_heads, plan, ws, o_lat1, lse1)
    o1 = mla.out_uv(o_lat1.view(batch * q_len, cfg.n_heads, cfg.d_latent), dc.w_uv)
    o_lat2 = torch.empty_like(o_lat1)
    lse2 = torch.empty_like(lse1)
    o2 = mla.decode_combine_out(dc.cache, plan, ws, dc.w_uv, o_lat2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o_lat1, o_lat2) and torch.equal(lse1, lse2)
    a = from_dev(o1).reshape(batch, q_len, cfg.n_heads, cfg.d_head)
    b = from_dev(o2)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6)
    heads = np.arange(3, 128, 11)
    o_ref, lse_ref = _reference(case, q, q_len, heads)
    _check(from_dev(o_lat2), from_dev(lse2), o_ref, lse_ref, "bf16", heads)


def test_one_token_plan_matches_plain_plan():
    cfg = DSV2.replace(batch=2, len_lo=50, len_hi=300, max_len=320)
    case = make_case(cfg, 70)
    dc = DevCase(case)
    _, q_dev = _query(cfg, 70, 1)
    p1 = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache)
    pm = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                         q_len=1)
    assert (p1.split_tokens, p1.num_splits, p1.head_groups, p1.q_len, p1.workspace_bytes) == \
        (pm.split_tokens, pm.num_splits, pm.head_groups, pm.q_len, pm.workspace_bytes)
    a, la = mla.decode_attn(q_dev[:, 0].contiguous(), dc.cache, cfg.scale, plan=p1)
    b, lb = mla.decode_attn(q_dev, dc.cache, cfg.scale, plan=pm)
    torch.cuda.synchronize()
    assert torch.equal(a, b[:, 0]) and torch.equal(la, lb[:, 0])


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_prefill_chunk(paged):
    """A prompt chunk of 96 new tokens per request decoded at once (chunked
    prefill in the absorbed form): every token attends causally to the
    prefix and to the chunk up to itself.  Sampled tokens and heads against
    the oracle."""
    q_len = 96
    if paged:
        cfg = DSV2.replace(batch=2, len_lo=1, len_hi=640, max_len=640, page_size=64)
    else:
        cfg = DSV2.replace(batch=2, len_lo=1, len_hi=640, max_len=640)
    case = make_case(cfg, 77, seq_lens=np.array([640, 150], np.int32), pad_value=np.nan)
    _log(f"[prefill] {'paged' if paged else 'contiguous'} q_len={q_len}")
    dc = DevCase(case)
    q, q_dev = _query(cfg, 77, q_len)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           q_len=q_len)
    assert plan.kernel in (1, 2) and plan.head_groups == q_len * (1 if plan.kernel == 1 else 2)
    o_lat, lse = mla.decode_attn(q_dev, dc.cache, cfg.scale, plan=plan)
    torch.cuda.synchronize()
    o_lat, lse = from_dev(o_lat), from_dev(lse)
    toks = [0, 1, 47, 94, 95]
    heads = [0, 63, 127]
    for b in range(cfg.batch):
        rows = oracle.gather_rows(case.cache, b, int(case.seq_lens[b]), case.page_table,
                                  cfg.page_size)
        o_ref, lse_ref = oracle.latent_attention_causal(q[b][:, heads], rows, cfg.d_latent,
                                                        cfg.scale)
        got_o = o_lat[b][np.ix_(toks, heads)]
        assert_close(got_o, o_ref[toks], "bf16", f"o_lat request {b}")
        assert_close(lse[b][np.ix_(toks, heads)], lse_ref[toks], "bf16", f"lse request {b}")


@pytest.mark.parametrize("q_len", [1, 4])
def test_one_split_writes_output_directly(q_len):
    """One split per request: mla_decode_attn has the MFMA kernel normalise its
    rows and write o_lat and lse itself (no partials, no combine).  Lengths
    include 0 and requests shorter than q_len, whose tokens see nothing."""
    cfg = DSV2.replace(batch=5, len_lo=0, len_hi=700, max_len=704)
    lens = np.array([0, 700, 2, 129, 33], np.int32)
    case = make_case(cfg, 61 + q_len, seq_lens=lens)
    _log(f"[direct] q_len={q_len}")
    dc = DevCase(case)
    q, q_dev = _query(cfg, 61 + q_len, q_len)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           split_tokens=1024, q_len=q_len)
    assert plan.kernel == 1 and plan.num_splits == 1
    q_in = q_dev if q_len > 1 else q_dev[:, 0]
    ws = mla.workspace_for(plan, "cuda")
    o_lat, lse = mla.decode_attn(q_in, dc.cache, cfg.scale, plan=plan, workspace=ws)
    # The same plan through the separate partials and combine calls.
    mla.decode_partials(q_in, dc.cache, cfg.scale, plan, ws)
    o_lat2 = torch.empty_like(o_lat)
    lse2 = torch.empty_like(lse)
    mla.decode_combine(dc.cache, cfg.n_heads, plan, ws, o_lat2, lse2)
    torch.cuda.synchronize()
    o_ref, lse_ref = _reference(case, q, q_len)
    shape = (cfg.batch, q_len, cfg.n_heads)
    for o_dev, l_dev in ((o_lat, lse), (o_lat2, lse2)):
        _check(from_dev(o_dev).reshape(shape + (cfg.d_latent,)), from_dev(l_dev).reshape(shape),
               o_ref, lse_ref, "bf16")
