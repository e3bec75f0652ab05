"""GPU parity of the decode kernel's two forms on the same inputs.

The MFMA decode kernel runs with 128 query rows per workgroup (plan->kernel
1) or 64 (plan->kernel 2: the two waves of a head block split the 576-long
score contraction and the 512-wide latent output in halves and add their
partial scores in LDS).  The planner picks the 64-row form for several
splits of at most 256 tokens; here both forms are forced on the same seeded
inputs and each is checked against the oracle (oracle.latent_attention, the
fp64 latent-space attention the oracle pins to the unabsorbed form) at the
bf16 tolerances, and against each other.  The two differ only in the fp32
rounding order of the scores (the 64-row form adds two half sums); that can
flip the bf16 rounding of a probability to its neighbour, a relative change
of 2^-8 that moves the output by at most 2^-8 p_j |row_j| / l, so the forms
agree within 2^-8 of the largest cached element in absolute terms, and to
relative L2 2e-3 overall.
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


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def _forced(plan, kernel):
    """The same split plan in the other form (rows per workgroup 128 or 64)."""
    groups = plan.q_len * 128 // (128 if kernel == 1 else 64)
    return mla.Plan(plan.split_tokens, plan.num_splits, kernel, groups, plan.q_len,
                    plan.workspace_bytes, plan.partitions)


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
    # (name, cfg overrides, lengths, split, q_len)
    ("ragged_split64", dict(batch=4, max_len=1024), [1024, 3, 700, 65], 64, 1),
    ("b16_split256", dict(batch=16, max_len=1024), None, 256, 1),
    ("paged_split128", dict(batch=6, max_len=1024, page_size=64),
     [1024, 1, 511, 700, 64, 900], 128, 1),
    ("two_tokens_split96", dict(batch=3, max_len=640), [640, 2, 333], 96, 2),
]


@pytest.mark.parametrize("case_def", CASES, ids=[c[0] for c in CASES])
def test_64_and_128_row_forms(case_def):
    name, over, lens, split, q_len = case_def
    cfg = DSV2.replace(name=name, len_lo=1, len_hi=over["max_len"], **over)
    case = make_case(cfg, 61, pad_value=np.nan,
                     seq_lens=None if lens is None else np.asarray(lens, np.int32))
    _log(f"[forms] {name} lens={case.seq_lens.tolist()} split={split} q_len={q_len}")
    dc = DevCase(case)
    q_np = np.stack([draw_latent_query(cfg, 61 + j) for j in range(q_len)], axis=1)
    q = _bf16_dev(q_np.reshape(cfg.batch, q_len, cfg.n_heads, -1))
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           split_tokens=split, q_len=q_len)
    outs = {}
    for kernel in (1, 2):
        pl = _forced(plan, kernel)
        o, lse = mla.decode_attn(q if q_len > 1 else q[:, 0], dc.cache, cfg.scale, plan=pl)
        torch.cuda.synchronize()
        outs[kernel] = (from_dev(o).reshape(cfg.batch, q_len, cfg.n_heads, -1),
                        from_dev(lse).reshape(cfg.batch, q_len, cfg.n_heads))
    heads = np.arange(0, 128, 11)
    o_ref, lse_ref = _oracle(case, q_np.reshape(cfg.batch, q_len * cfg.n_heads, -1), heads,
                             q_len)
    for kernel in (1, 2):
        o, lse = outs[kernel]
        assert_close(o[:, :, heads], o_ref, "bf16", f"o_lat (kernel {kernel})")
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse[:, :, heads]), fin)
        assert_close(lse[:, :, heads][fin], lse_ref[fin], "bf16", f"lse (kernel {kernel})")
    (o1, l1), (o2, l2) = outs[1], outs[2]
    d = np.abs(o1 - o2)
    row_max = float(np.nanmax(np.abs(case.cache)))
    assert d.max() <= 2.0 ** -8 * row_max, f"forms differ by {d.max():.3e}"
    assert np.linalg.norm(o1 - o2) <= 2e-3 * np.linalg.norm(o1)
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2))
    np.testing.assert_allclose(l1[fin], l2[fin], rtol=1e-5, atol=1e-5)
