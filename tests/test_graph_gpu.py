"""The decode step captured into a HIP graph through torch's graph API and
replayed, in both call patterns: absorb -> mla_decode_attn -> W^UV, and
absorb -> partials -> combine + W^UV.  Every replay must give the eager
result bit for bit, with eager work and synchronisations between the
replays, and a replay after the inputs (query values, then request lengths)
change in place must follow them.
No call of the step allocates, synchronises or clears memory, so the step is
capturable as is."""

import sys

import numpy as np
import pytest
import torch

import head_latent_attention_absorb_amd as mla
from tests.gpu_util import DevCase
from workload import CONFIGS, make_case

pytestmark = pytest.mark.gpu

DSV2 = CONFIGS["dsv2_b16_t4096"]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("form", ["decode_attn", "partials_combine_out"])
def test_step_graph_replays_match_eager(form):
    cfg = DSV2.replace(batch=6, len_lo=1, len_hi=1500, max_len=1536)
    case = make_case(cfg, 101, seq_lens=np.array([1500, 1, 700, 0, 1024, 33], np.int32))
    other = make_case(cfg, 102, seq_lens=case.seq_lens)
    _log(f"[graph] {form}: B=6 ragged lengths, 3 replays")
    dc, dc2 = DevCase(case), DevCase(other)
    B, nh = cfg.batch, cfg.n_heads
    plan = mla.decode_plan(nh, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache)
    ws = mla.workspace_for(plan, "cuda")
    q_c, q_r = dc.q_c.clone(), dc.q_r.clone()
    q_cat = torch.empty((B, nh, cfg.row), dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty((B, nh, cfg.d_latent), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, nh), dtype=torch.float32, device="cuda")
    o = torch.empty((B, nh, cfg.d_head), dtype=torch.bfloat16, device="cuda")

    assert plan.num_splits > 1 and plan.balanced

    def step():
        mla.absorb_q(q_c, q_r, dc.w_uk, out=q_cat)
        if form == "decode_attn":
            mla.decode_attn(q_cat, dc.cache, cfg.scale, plan, o_lat, lse, ws)
            mla.out_uv(o_lat, dc.w_uv, out=o)
        else:
            mla.decode_partials(q_cat, dc.cache, cfg.scale, plan, ws)
            mla.decode_combine_out(dc.cache, plan, ws, dc.w_uv, o_lat, lse, out=o)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), o_lat.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        o.zero_(); o_lat.zero_(); lse.zero_()
        # Eager work between replays: the other case's step on its own buffers.
        _, ol2, _ = DevCase.run(dc2)[:3]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(o_lat, ref[1]), f"replay {rep}"
        assert torch.equal(torch.nan_to_num(lse, neginf=-1e30), torch.nan_to_num(ref[2], neginf=-1e30))
    # New query values in the captured input buffers.
    q_c.copy_(dc2.q_c)
    q_r.copy_(dc2.q_r)
    g.replay()
    torch.cuda.synchronize()
    got = o.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(got, o)
    assert not torch.equal(got, ref[0])
    # New lengths in the captured length buffer: the balanced plan's
    # partitions are cut on the device at every call, so the replay follows.
    dc.seq_lens.copy_(torch.tensor([1536, 2, 2, 1536, 900, 1], dtype=torch.int32))
    g.replay()
    torch.cuda.synchronize()
    got, got_lat = o.clone(), o_lat.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(got, o) and torch.equal(got_lat, o_lat)
