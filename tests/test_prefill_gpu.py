"""GPU parity of the unabsorbed chunk form (mla_prefill_expand, then
mla_prefill_attn), through the C ABI, against oracle.up_project and
oracle.mla_prefill_reference (fp64).

bf16 storage, tolerances as for decode: relative L2 <= 1e-2 and max abs <=
2e-2.  Inputs come from make_case (seeded); nothing is taken from the HIP
path.  Heads are sampled where the full set would keep the oracle busy for
minutes; every query token and key row of a sampled head is checked.
"""

import sys

import numpy as np
import pytest
import torch

import head_latent_attention_absorb_amd as mla
import oracle
from tests.gpu_util import DevCase, assert_close, from_dev
from workload import CONFIGS, make_case

pytestmark = pytest.mark.gpu

DSV2 = CONFIGS["dsv2_b16_t4096"]
HEADS = [0, 1, 31, 32, 77, 127]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _reference(case, heads):
    cfg = case.cfg
    q_len = cfg.q_len
    o = np.zeros((cfg.batch, q_len, cfg.n_heads, cfg.d_head))
    lse = np.full((cfg.batch, q_len, cfg.n_heads), -np.inf)
    for b in range(cfg.batch):
        rows = oracle.gather_rows(case.cache, b, int(case.seq_lens[b]))
        q_c = case.q_c[b].reshape(q_len, cfg.n_heads, cfg.d_head)
        q_r = case.q_r[b].reshape(q_len, cfg.n_heads, cfg.d_rope)
        o[b], lse[b] = oracle.mla_prefill_reference(
            q_c, q_r, rows[:, :cfg.d_latent], rows[:, cfg.d_latent:],
            case.w_uk, case.w_uv, cfg.scale, heads=heads)
    return o, lse


def test_expand_keys_and_values():
    cfg = DSV2.replace(batch=2, len_lo=1, len_hi=320, max_len=320)
    case = make_case(cfg, 71, seq_lens=np.array([300, 77], np.int32))
    _log("[prefill expand] lens (300, 77)")
    dc = DevCase(case)
    shape = (cfg.batch, cfg.n_heads, cfg.max_len, cfg.d_head)
    sentinel = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda")
    k_c, v = mla.prefill_expand(dc.cache, dc.w_uk, dc.w_uv, k_c=sentinel.clone(),
                                v=sentinel.clone())
    torch.cuda.synchronize()
    k_np, v_np = from_dev(k_c), from_dev(v)
    for b in range(cfg.batch):
        n = int(case.seq_lens[b])
        latent = oracle.gather_rows(case.cache, b, n)[:, :cfg.d_latent]
        k_ref, v_ref = oracle.up_project(latent, case.w_uk[HEADS], case.w_uv[HEADS])
        assert_close(k_np[b, HEADS, :n], k_ref, "bf16", f"k_c[{b}]")
        assert_close(v_np[b, HEADS, :n], v_ref, "bf16", f"v[{b}]")
        # Rows past the length are not written.
        assert (k_np[b, :, n:] == 7.0).all() and (v_np[b, :, n:] == 7.0).all()


@pytest.mark.parametrize("q_len,lens", [(150, (300, 100)), (300, (700, 290)), (64, (64, 1000)),
                                        (1, (5, 129))],
                         ids=["ragged_block_short_history", "two_blocks", "one_block",
                              "one_token"])
def test_prefill_attention(q_len, lens):
    """Ragged query blocks (150 queries: waves with part of a tile, a wave
    with none; 300 = 256 + 44), requests shorter than the chunk (their first
    tokens see nothing), tiles cut by the length."""
    cfg = DSV2.replace(batch=2, len_lo=1, len_hi=1024, max_len=1024, q_len=q_len)
    case = make_case(cfg, 72 + q_len, seq_lens=np.array(lens, np.int32))
    _log(f"[prefill attn] q_len={q_len} lens={lens}")
    dc = DevCase(case)
    q_c = dc.q_c.view(cfg.batch, q_len, cfg.n_heads, cfg.d_head)
    q_r = dc.q_r.view(cfg.batch, q_len, cfg.n_heads, cfg.d_rope)
    k_c, v = mla.prefill_expand(dc.cache, dc.w_uk, dc.w_uv)
    out, lse = mla.prefill_attn(q_c, q_r, dc.cache, k_c, v, cfg.scale)
    torch.cuda.synchronize()
    o_np, lse_np = from_dev(out), from_dev(lse)
    o_ref, lse_ref = _reference(case, HEADS)
    o_np, lse_np = o_np[:, :, HEADS], lse_np[:, :, HEADS]
    o_ref, lse_ref = o_ref[:, :, HEADS], lse_ref[:, :, HEADS]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_np), empty), "tokens with no visible row"
    assert np.all(o_np[empty] == 0)
    assert_close(o_np, o_ref, "bf16", "o")
    assert_close(lse_np[~empty], lse_ref[~empty], "bf16", "lse")


def test_prefill_matches_absorbed_chunk():
    """The two forms of the same chunk on the GPU: explicit keys and values
    against absorb -> several-token decode -> W^UV, every head."""
    q_len = 96
    cfg = DSV2.replace(batch=2, len_lo=1, len_hi=700, max_len=704, q_len=q_len)
    case = make_case(cfg, 81, seq_lens=np.array([700, 200], np.int32))
    dc = DevCase(case)
    B, nh = cfg.batch, cfg.n_heads
    q_c = dc.q_c.view(B, q_len, nh, cfg.d_head)
    q_r = dc.q_r.view(B, q_len, nh, cfg.d_rope)
    k_c, v = mla.prefill_expand(dc.cache, dc.w_uk, dc.w_uv)
    out, lse = mla.prefill_attn(q_c, q_r, dc.cache, k_c, v, cfg.scale)
    q_cat = mla.absorb_q(q_c.reshape(B * q_len, nh, cfg.d_head),
                         q_r.reshape(B * q_len, nh, cfg.d_rope), dc.w_uk)
    plan = mla.decode_plan(nh, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache, q_len=q_len)
    o_lat, lse2 = mla.decode_attn(q_cat.view(B, q_len, nh, -1), dc.cache, cfg.scale, plan=plan)
    out2 = mla.out_uv(o_lat.view(B * q_len, nh, cfg.d_latent), dc.w_uv)
    torch.cuda.synchronize()
    assert_close(from_dev(out), from_dev(out2).reshape(B, q_len, nh, cfg.d_head), "bf16", "o")
    assert_close(from_dev(lse), from_dev(lse2).reshape(B, q_len, nh), "bf16", "lse")


def test_prefill_c512_b4_t4096_sampled():
    """The benchmark's chunk: 4 requests of 4096 rows, the last 512 new."""
    cfg = CONFIGS["prefill_c512_b4_t4096"]
    case = make_case(cfg, 0)
    _log("[prefill attn] prefill_c512_b4_t4096 sampled heads")
    dc = DevCase(case)
    B, C, nh = cfg.batch, cfg.q_len, cfg.n_heads
    k_c, v = mla.prefill_expand(dc.cache, dc.w_uk, dc.w_uv)
    out, lse = mla.prefill_attn(dc.q_c.view(B, C, nh, cfg.d_head),
                                dc.q_r.view(B, C, nh, cfg.d_rope), dc.cache, k_c, v, cfg.scale)
    torch.cuda.synchronize()
    heads = [0, 127]
    o_ref, lse_ref = _reference(case, heads)
    assert_close(from_dev(out)[:, :, heads], o_ref[:, :, heads], "bf16", "o")
    assert_close(from_dev(lse)[:, :, heads], lse_ref[:, :, heads], "bf16", "lse")


@pytest.mark.parametrize("scale", [-0.0722, 0.0], ids=["negative", "zero"])
def test_prefill_scale_sign_and_zero(scale):
    """The kernel folds a positive scale into the exponent; a negative or zero
    scale takes the plain path."""
    q_len = 80
    cfg = DSV2.replace(batch=1, len_lo=1, len_hi=400, max_len=400, q_len=q_len)
    case = make_case(cfg, 91, seq_lens=np.array([400], np.int32))
    dc = DevCase(case)
    q_c = dc.q_c.view(1, q_len, cfg.n_heads, cfg.d_head)
    q_r = dc.q_r.view(1, q_len, cfg.n_heads, cfg.d_rope)
    k_c, v = mla.prefill_expand(dc.cache, dc.w_uk, dc.w_uv)
    out, lse = mla.prefill_attn(q_c, q_r, dc.cache, k_c, v, scale)
    torch.cuda.synchronize()
    heads = [0, 64, 127]
    rows = oracle.gather_rows(case.cache, 0, 400)
    o_ref, lse_ref = oracle.mla_prefill_reference(
        case.q_c[0], case.q_r[0], rows[:, :cfg.d_latent], rows[:, cfg.d_latent:], case.w_uk,
        case.w_uv, scale, heads=heads)
    assert_close(from_dev(out)[0][:, heads], o_ref[:, heads], "bf16", "o")
    assert_close(from_dev(lse)[0][:, heads], lse_ref[:, heads], "bf16", "lse")


def test_prefill_long_chunk_1024():
    """A 1024-token chunk (four query blocks) over 2048 rows, the longest
    chunk the absorbed plan takes, every token of sampled heads."""
    q_len = 1024
    cfg = DSV2.replace(batch=1, len_lo=1, len_hi=2048, max_len=2048, q_len=q_len)
    case = make_case(cfg, 93, seq_lens=np.array([2048], np.int32))
    _log("[prefill attn] 1024-token chunk")
    dc = DevCase(case)
    k_c, v = mla.prefill_expand(dc.cache, dc.w_uk, dc.w_uv)
    out, lse = mla.prefill_attn(dc.q_c.view(1, q_len, cfg.n_heads, cfg.d_head),
                                dc.q_r.view(1, q_len, cfg.n_heads, cfg.d_rope), dc.cache, k_c, v,
                                cfg.scale)
    torch.cuda.synchronize()
    heads = [5, 100]
    o_ref, lse_ref = _reference(case, heads)
    assert_close(from_dev(out)[:, :, heads], o_ref[:, :, heads], "bf16", "o")
    assert_close(from_dev(lse)[:, :, heads], lse_ref[:, :, heads], "bf16", "lse")
