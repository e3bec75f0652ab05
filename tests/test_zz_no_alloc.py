"""mla_decode_attn_noalloc (the decode call whose workspace is the library's
static device array, for callers that cannot allocate) against
mla_decode_attn with a caller workspace: the same kernels on the same inputs,
so the outputs must be the same bits.  Two calls in a row, the second with a
smaller batch and shorter lengths (the array keeps the first call's
contents), then a plan whose workspace exceeds the array, which is refused
with nothing launched."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import head_latent_attention_absorb_amd as mla
from tests.gpu_util import DevCase
from workload import CONFIGS, draw_latent_query, f32_to_bf16_bits, make_case

pytestmark = pytest.mark.gpu

DSV2 = CONFIGS["dsv2_b16_t4096"]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16_dev(x):
    return torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def _both(cfg, seed, lens, split=0):
    case = make_case(cfg, seed, seq_lens=np.asarray(lens, np.int32))
    dc = DevCase(case)
    q = _bf16_dev(draw_latent_query(cfg, seed))
    plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, torch.bfloat16, dc.cache,
                           split_tokens=split)
    assert plan.workspace_bytes <= int(mla.lib().mla_decode_noalloc_max_bytes())
    o_ref, l_ref = mla.decode_attn(q, dc.cache, cfg.scale, plan=plan)
    out = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    o, l = mla.decode_attn_noalloc(q, dc.cache, cfg.scale, plan=plan, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, l, o_ref, l_ref, plan


def test_noalloc_matches_decode_attn_twice():
    # First: the B=16 DeepSeek-V2 shape at T=4096 (the default plan:
    # length-balanced, 512-token partitions).
    _log("[noalloc] B=16 T=4096")
    o, l, o_ref, l_ref, plan = _both(DSV2, 3, [4096] * 16)
    assert plan.num_splits > 1
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    # Second, smaller: B=3, ragged lengths, one of them empty, 128-token splits.
    cfg = DSV2.replace(batch=3, max_len=1024)
    _log("[noalloc] B=3 ragged")
    o, l, o_ref, l_ref, plan = _both(cfg, 4, [1000, 0, 77], split=128)
    assert torch.equal(o, o_ref)
    assert torch.equal(torch.nan_to_num(l, neginf=-1e30), torch.nan_to_num(l_ref, neginf=-1e30))


def test_noalloc_rejects_a_plan_beyond_its_array():
    cfg = DSV2.replace(batch=16, max_len=4096)
    case = make_case(cfg, 5, seq_lens=np.full(16, 4096, np.int32))
    dc = DevCase(case)
    # 32-token splits: 128 splits of 16 requests need about 268 MB of workspace.
    plan = mla.decode_plan(128, 512, 64, torch.bfloat16, dc.cache, split_tokens=32)
    assert plan.workspace_bytes > int(mla.lib().mla_decode_noalloc_max_bytes())
    q = _bf16_dev(draw_latent_query(cfg, 5))
    out = torch.zeros((16, 128, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        mla.decode_attn_noalloc(q, dc.cache, cfg.scale, plan=plan, out=out)
    assert e.value.status == 4  # MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(out.count_nonzero()) == 0
