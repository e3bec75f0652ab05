"""GPU parity of length-balanced split plans.

When the batch alone leaves compute units idle, the planner returns a plan
with split_tokens == 0: the decode kernel reads seq_lens on the device and
picks one partition length c for the call, the smallest multiple of 32
tokens at which the requests' partition counts ceil(len_b / c) add up to at
most one workgroup per compute unit (capped so that a paged partition
touches at most 64 pages).  Splitting a request's rows into partitions
changes only the rounding of the merged result (the merge is the softmax of
the concatenated scores regrouped by partition: DeepSeek-V2 read-through,
section 2.3, computes one weighted sum over the cached latents), so these
tests check:

* the outputs against the oracle (oracle.latent_attention, fp64) at the bf16
  tolerances, on batches of extreme length skew, empty requests, a paged
  cache and several query tokens per request;
* the same inputs under a uniform plan: the two agree within 2^-8 of the
  largest cached element (one bf16 rounding step of a probability, as between
  the kernel's two forms) and to relative L2 2e-3;
* the partition table the kernel leaves in the workspace against the rule
  above: c a multiple of 32, the counts within the target, c minimal, and
  every request's first partition the running sum of the counts before it.
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
HEADS = np.arange(0, 128, 9)


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def _round256(x: int) -> int:
    return (x + 255) // 256 * 256


def _table(plan, ws, batch: int, rows: int) -> np.ndarray:
    """The partition table of a balanced call: it follows the bf16 partial
    rows and the (lse, m) pairs of plan.partitions partitions."""
    off = _round256(plan.partitions * rows * 512 * 2) + _round256(plan.partitions * rows * 8)
    return ws[off:off + 4 * (batch + 2)].view(torch.int32).cpu().numpy()


def _check_table(tab: np.ndarray, lens: np.ndarray, plan, cus: int, c_cap: int):
    """c_cap: the longest partition allowed (max_len rounded up to 32 tokens;
    paged: at most 63 pages' worth)."""
    B = len(lens)
    c, offs, total = int(tab[0]), tab[1:1 + B].astype(np.int64), int(tab[1 + B])
    counts = -(-lens.astype(np.int64) // c)
    target = max(1, cus // plan.head_groups)
    assert 32 <= c <= c_cap and c % 32 == 0, (c, c_cap)
    assert total == counts.sum() <= plan.partitions
    assert np.array_equal(offs, np.concatenate([[0], np.cumsum(counts)[:-1]]))
    if total > target:
        # only when even the longest partition allowed leaves too many
        assert c == c_cap, (c, total, target)
    elif c > 32:
        # one granule shorter would exceed the target
        assert (-(-lens.astype(np.int64) // (c - 32))).sum() > target, (c, total, target)
    return c, counts


def _oracle(case, q_np, heads, q_len):
    cfg = case.cfg
    o = np.zeros((cfg.batch, q_len, len(heads), cfg.d_latent))
    lse = np.full((cfg.batch, q_len, len(heads)), -np.inf)
    for b in range(cfg.batch):
        rows = oracle.gather_rows(case.cache, b, int(case.seq_lens[b]), case.page_table,
                                  cfg.page_size)
        qb = q_np[b].reshape(q_len, cfg.n_heads, -1)[:, heads]
        o[b], lse[b] = oracle.latent_attention_causal(qb, rows, cfg.d_latent, cfg.scale)
    return o, lse


CASES = [
    # (name, cfg overrides, lengths, q_len)
    ("skew_one_long", dict(batch=16, max_len=4096), [4096] + [1] * 15, 1),
    ("skew_with_empty", dict(batch=8, max_len=4096), [0, 4096, 0, 5, 33, 0, 1, 2047], 1),
    ("ragged_long", dict(batch=4, max_len=32768), [32768, 16384, 20001, 17], 1),
    ("paged_b128", dict(batch=128, max_len=2048, page_size=64), None, 1),
    # near the largest balanced batch on 256 compute units (batch x head
    # groups must stay below the CU count): four lengths per planner lane
    ("b200_ragged", dict(batch=200, max_len=1024), None, 1),
    ("paged_skew", dict(batch=5, max_len=8192, page_size=64), [8192, 1, 64, 4000, 0], 1),
    ("two_tokens", dict(batch=3, max_len=4096), [4096, 2, 333], 2),
    # 24-token pages cap a partition at 1504 tokens (63 pages' worth, whatever
    # the alignment); eight query tokens leave a target of 32 partitions, so
    # the cap binds: c is the cap and the count exceeds the target
    ("paged_cap_binds", dict(batch=2, max_len=30720, page_size=24), [30720, 30000], 8),
]


@pytest.mark.parametrize("case_def", CASES, ids=[c[0] for c in CASES])
def test_balanced_plan_parity(case_def):
    name, over, lens, q_len = case_def
    cfg = DSV2.replace(name=name, len_lo=1, len_hi=over["max_len"], **over)
    case = make_case(cfg, 71, pad_value=np.nan,
                     seq_lens=None if lens is None else np.asarray(lens, np.int32))
    _log(f"[balanced] {name} B={cfg.batch} q_len={q_len} "
         f"lens[:8]={case.seq_lens[:8].tolist()}")
    dc = DevCase(case)
    q_np = np.stack([draw_latent_query(cfg, 71 + j) for j in range(q_len)], axis=1)
    q = _bf16_dev(q_np.reshape(cfg.batch, q_len, cfg.n_heads, -1))
    q_in = q if q_len > 1 else q[:, 0]
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           q_len=q_len)
    assert plan.balanced, plan
    rows = q_len * cfg.n_heads
    ws = mla.workspace_for(plan, "cuda")
    mla.decode_partials(q_in, dc.cache, cfg.scale, plan, ws)
    lead = (cfg.batch, q_len) if q_len > 1 else (cfg.batch,)
    o_lat = torch.empty(lead + (cfg.n_heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(lead + (cfg.n_heads,), dtype=torch.float32, device="cuda")
    mla.decode_combine(dc.cache, cfg.n_heads, plan, ws, o_lat, lse)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    c_cap = -(-cfg.max_len // 32) * 32
    if cfg.page_size:
        c_cap = min(c_cap, 63 * cfg.page_size // 32 * 32)
    c, counts = _check_table(_table(plan, ws, cfg.batch, rows), case.seq_lens, plan, cus, c_cap)
    _log(f"[balanced] {name}: c={c} partitions={int(counts.sum())} of {plan.partitions}")
    if name in ("ragged_long", "paged_b128"):
        # the configurations' shapes (B=4 at 16K-32K, paged B=128): the cut
        # fills the compute units (one workgroup per CU per head group)
        target = cus // plan.head_groups
        assert counts.sum() >= 0.9 * target, (int(counts.sum()), target)
    if cfg.page_size:
        # a partition touches at most 64 pages
        assert c <= 63 * cfg.page_size

    o = from_dev(o_lat).reshape(cfg.batch, q_len, cfg.n_heads, -1)
    l = from_dev(lse).reshape(cfg.batch, q_len, cfg.n_heads)
    o_ref, lse_ref = _oracle(case, q_np.reshape(cfg.batch, rows, -1), HEADS, q_len)
    assert_close(o[:, :, HEADS], o_ref, "bf16", f"o_lat ({name})")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(l[:, :, HEADS]), fin)
    assert_close(l[:, :, HEADS][fin], lse_ref[fin], "bf16", f"lse ({name})")
    # empty requests: o = 0, lse = -inf on every head
    empty = case.seq_lens == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(l[empty]))

    # The same inputs under a uniform plan.
    uplan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                            split_tokens=256, q_len=q_len)
    assert not uplan.balanced
    o_u, l_u = mla.decode_attn(q_in, dc.cache, cfg.scale, plan=uplan)
    torch.cuda.synchronize()
    o_u = from_dev(o_u).reshape(o.shape)
    l_u = from_dev(l_u).reshape(l.shape)
    row_max = float(np.nanmax(np.abs(case.cache)))
    assert np.abs(o - o_u).max() <= 2.0 ** -8 * row_max
    assert np.linalg.norm(o - o_u) <= 2e-3 * max(np.linalg.norm(o_u), 1e-30)
    f = np.isfinite(l_u)
    assert np.array_equal(f, np.isfinite(l))
    np.testing.assert_allclose(l[f], l_u[f], rtol=1e-5, atol=1e-5)


def test_balanced_all_empty_and_fused_tail():
    """Every request empty: nothing to attend to, o_lat = 0 and lse = -inf; and
    the fused combine + W^UV tail over a skewed balanced plan matches the
    separate combine and projection."""
    cfg = DSV2.replace(name="empty", batch=4, max_len=1024, len_lo=0, len_hi=0)
    case = make_case(cfg, 5, seq_lens=np.zeros(4, np.int32))
    dc = DevCase(case)
    q_cat = mla.absorb_q(dc.q_c, dc.q_r, dc.w_uk)
    o_lat, lse = mla.decode_attn(q_cat, dc.cache, cfg.scale)
    torch.cuda.synchronize()
    assert torch.all(o_lat == 0) and torch.all(torch.isneginf(lse))

    cfg = DSV2.replace(name="skew_fused", batch=6, max_len=4096, len_lo=1, len_hi=4096)
    case = make_case(cfg, 6, seq_lens=np.asarray([4096, 1, 3, 0, 100, 2], np.int32))
    dc = DevCase(case)
    q_cat, o_lat_f, lse_f, o_f = dc.run_fused()
    _, o_lat_s, lse_s, o_s = dc.run()
    assert torch.equal(o_lat_f, o_lat_s)
    assert torch.equal(lse_f, lse_s)
    d = (o_f.float() - o_s.float()).abs().max().item()
    assert d <= 2.0 ** -7 * max(o_s.float().abs().max().item(), 1e-30), d
