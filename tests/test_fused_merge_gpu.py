"""GPU tests of the one-launch merge of mla_decode_attn.

When every workgroup of a multi-split plan fits on the device at once, the
splits of each (request, 128-row group) write their partial sums, meet at a
pair of counters in the workspace and merge each other's partials in the same
launch.  These tests check it against the oracle (oracle.latent_attention, the
fp64 latent-space softmax attention that the oracle pins to the unabsorbed
form) at the bf16 tolerances, against the two-phase path
(mla_decode_partials + mla_decode_combine, the same merge done by a separate
kernel: within two bf16 units in the last place of each other), for split
counts that take every batch shape of the merge (1, 2, 4, 8, 16, 40, 128 and
256 partitions per request), with empty, one-split and many-split requests
in one launch, and that the counters are zero again after every call.
"""

import sys

import numpy as np
import pytest
import torch

import head_latent_attention_absorb_amd as mla
import oracle
from tests.gpu_util import DevCase, assert_close, from_dev
from workload import CONFIGS, draw_latent_query, f32_to_bf16_bits, make_case

pytestmark = [pytest.mark.gpu,
              pytest.mark.skip(reason="the one-launch merge is switched off in the library "
                                      "until its partial volume shrinks (slower than the "
                                      "two-phase path at 128 heads per workgroup)")]

DSV2 = CONFIGS["dsv2_b16_t4096"]
BF16_ULP_REL = 2.0 ** -7


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def _counter_bytes(batch: int, head_groups: int) -> int:
    return (batch * head_groups * 8 + 255) // 256 * 256


def _case(name, batch, lo, hi, max_len, seed, lens=None):
    cfg = DSV2.replace(name=name, batch=batch, len_lo=lo, len_hi=hi, max_len=max_len)
    return make_case(cfg, seed, pad_value=np.nan,
                     seq_lens=None if lens is None else np.asarray(lens, np.int32))


def _run_both(case, split, seed):
    """(fused o_lat, lse, two-phase o_lat, lse, q, plan, workspace) on one query."""
    cfg = case.cfg
    dc = DevCase(case)
    q_np = draw_latent_query(cfg, seed)
    q = _bf16_dev(q_np)
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           split_tokens=split)
    ws = mla.workspace_for(plan, "cuda")
    o_f, l_f = mla.decode_attn(q, dc.cache, cfg.scale, plan=plan, workspace=ws)
    ws2 = mla.workspace_for(plan, "cuda")
    mla.decode_partials(q, dc.cache, cfg.scale, plan, ws2)
    o_t = torch.empty_like(o_f)
    l_t = torch.empty_like(l_f)
    mla.decode_combine(dc.cache, cfg.n_heads, plan, ws2, o_t, l_t)
    torch.cuda.synchronize()
    return from_dev(o_f), from_dev(l_f), from_dev(o_t), from_dev(l_t), q_np, plan, ws


def _oracle(case, q_np, heads):
    cfg = case.cfg
    o = np.zeros((cfg.batch, len(heads), cfg.d_latent))
    lse = np.full((cfg.batch, len(heads)), -np.inf)
    for b in range(cfg.batch):
        rows = oracle.gather_rows(case.cache, b, int(case.seq_lens[b]), case.page_table,
                                  cfg.page_size)
        o[b], lse[b] = oracle.latent_attention(q_np[b, heads], rows, cfg.d_latent, cfg.scale)
    return o, lse


# (name, batch, len_lo, len_hi, max_len, split_tokens): partitions per request
# max_len / split, the grid batch * that <= 256.
SHAPES = [
    ("p2", 8, 300, 640, 640, 320),        # 1 or 2 partitions
    ("p4", 8, 1000, 1280, 1280, 320),     # 4
    ("p8", 4, 2000, 2560, 2560, 320),     # 7 or 8
    ("p16", 2, 3900, 4096, 4096, 256),    # 16
    ("p40", 2, 1200, 1280, 1280, 32),     # 38 to 40: units per partition < 16
    ("p128", 1, 4000, 4096, 4096, 32),    # 125 to 128
    ("p256", 1, 8192, 8192, 8192, 32),    # 256: eight slots share each unit
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_fused_merge_against_oracle_and_two_phase(shape):
    name, batch, lo, hi, max_len, split = shape
    case = _case(f"fused_{name}", batch, lo, hi, max_len, seed=41)
    _log(f"[fused {name}] lens={case.seq_lens.tolist()} split={split}")
    o_f, l_f, o_t, l_t, q_np, plan, ws = _run_both(case, split, seed=41)
    assert plan.num_splits == (max_len + split - 1) // split
    assert np.isfinite(o_f).all() and np.isfinite(l_f).all()
    # The two merges differ only in fp32 rounding order before the bf16 output.
    assert np.all(np.abs(o_f - o_t) <= 2 * BF16_ULP_REL * np.abs(o_t) + 1e-30), \
        f"max diff {np.abs(o_f - o_t).max():.3e}"
    np.testing.assert_allclose(l_f, l_t, rtol=1e-5, atol=1e-5)
    heads = np.arange(0, 128, 9)
    o_ref, lse_ref = _oracle(case, q_np, heads)
    assert_close(o_f[:, heads], o_ref, "bf16", "o_lat")
    assert_close(l_f[:, heads], lse_ref, "bf16", "lse")
    cb = _counter_bytes(batch, plan.head_groups)
    assert int(ws[plan.workspace_bytes - cb:plan.workspace_bytes].count_nonzero()) == 0


def test_fused_mixed_lengths_one_launch():
    """Empty, one-partition and many-partition requests in one launch: the empty
    one is written by its first partition (o = 0, lse = -inf), one-partition
    requests are written directly, the others merged."""
    lens = [0, 1, 31, 33, 700, 4096, 2000, 257]
    case = _case("fused_mixed", 8, 1, 4096, 4096, seed=43, lens=lens)
    o_f, l_f, o_t, l_t, q_np, plan, ws = _run_both(case, 256, seed=43)
    assert plan.num_splits == 16
    assert np.all(o_f[0] == 0) and np.all(l_f[0] == -np.inf)
    assert np.all(np.abs(o_f - o_t) <= 2 * BF16_ULP_REL * np.abs(o_t) + 1e-30)
    np.testing.assert_allclose(l_f[1:], l_t[1:], rtol=1e-5, atol=1e-5)
    heads = np.arange(0, 128, 5)
    o_ref, lse_ref = _oracle(case, q_np, heads)
    assert_close(o_f[1:, heads], o_ref[1:], "bf16", "o_lat")
    assert_close(l_f[1:, heads], lse_ref[1:], "bf16", "lse")


def test_fused_repeated_calls_reset_counters():
    """Three calls on one workspace give the same bits, and each leaves the
    counter area zero (the next call relies on it)."""
    case = make_case(DSV2, 0)
    dc = DevCase(case)
    q = _bf16_dev(draw_latent_query(DSV2, 5))
    plan = mla.decode_plan(128, 512, 64, torch.bfloat16, dc.cache)
    assert plan.num_splits == 16
    ws = mla.workspace_for(plan, "cuda")
    cb = _counter_bytes(DSV2.batch, plan.head_groups)
    outs = []
    for i in range(3):
        o, lse = mla.decode_attn(q, dc.cache, DSV2.scale, plan=plan, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[plan.workspace_bytes - cb:plan.workspace_bytes].count_nonzero()) == 0
        outs.append((o.clone(), lse.clone()))
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_fused_wait_gives_up_and_marks_output():
    """A counter the splits can never satisfy (set from the host) ends every
    split's bounded wait: the row group's output is NaN, the kernel exits and
    the counters are zero again, so the next call is correct."""
    case = _case("fused_giveup", 2, 1024, 1024, 1024, seed=47)
    dc = DevCase(case)
    q_np = draw_latent_query(case.cfg, 47)
    q = _bf16_dev(q_np)
    plan = mla.decode_plan(128, 512, 64, torch.bfloat16, dc.cache, split_tokens=256)
    assert plan.num_splits == 4
    ws = mla.workspace_for(plan, "cuda")
    cb = _counter_bytes(2, plan.head_groups)
    counters = ws[plan.workspace_bytes - cb:].view(torch.int32)
    counters[0] = -(1 << 30)  # request 0's arrival count never reaches 4
    o, lse = mla.decode_attn(q, dc.cache, case.cfg.scale, plan=plan, workspace=ws)
    torch.cuda.synchronize()
    o0, l0 = from_dev(o), from_dev(lse)
    assert np.isnan(o0[0]).all() and np.isnan(l0[0]).all()
    assert np.isfinite(o0[1]).all()
    assert int(ws[plan.workspace_bytes - cb:plan.workspace_bytes].count_nonzero()) == 0
    o, lse = mla.decode_attn(q, dc.cache, case.cfg.scale, plan=plan, workspace=ws)
    torch.cuda.synchronize()
    heads = np.arange(0, 128, 16)
    o_ref, lse_ref = _oracle(case, q_np, heads)
    assert_close(from_dev(o)[:, heads], o_ref, "bf16", "o_lat after the give-up")


def test_workspace_bytes_matches_default_plan():
    data = torch.zeros((16, 4096, 576), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((16,), 4096, dtype=torch.int32, device="cuda")
    cache = mla.latent_cache(data, lens, 64)
    plan = mla.decode_plan(128, 512, 64, torch.bfloat16, cache)
    assert mla.decode_workspace_bytes(128, 512, 64, torch.bfloat16, 16, 4096) == \
        plan.workspace_bytes
    assert mla.decode_workspace_bytes(128, 512, 64, torch.bfloat16, -1, 4096) == 0
