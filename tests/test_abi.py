"""The C ABI: the library loads, exports every symbol include/*.h declares, and
rejects bad arguments before launching anything."""

import ctypes
import glob
import os
import re

import numpy as np
import pytest
import torch

import head_latent_attention_absorb_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(mla_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_library_loads_and_exports_every_declared_symbol():
    L = mla.lib()
    names = _declared_functions()
    assert {"mla_absorb_q", "mla_decode_attn", "mla_out_uv", "mla_decode_plan"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/ but not exported"
    assert L.mla_abi_version() == 6


def test_status_strings():
    L = mla.lib()
    for code in range(8):
        s = L.mla_status_str(code).decode()
        assert s.startswith("MLA_")
    assert L.mla_status_str(99).decode() == "MLA_ERR_UNKNOWN"


def test_struct_sizes_match_header():
    # mla_dims_t: 5 x int32; mla_cache_t: 3 pointers, 2 int32, int64; plan: 5 int32, size_t, int32.
    assert ctypes.sizeof(mla.Dims) == 20
    assert ctypes.sizeof(mla.CacheDesc) == 56
    assert ctypes.sizeof(mla.Plan) == 40
    # mla_rope_t: 4 floats and an int32.
    assert ctypes.sizeof(mla.Rope) == 20


def _dims(**kw):
    d = dict(n_heads=128, d_head=128, d_rope=64, d_latent=512, dtype=mla.MLA_BF16)
    d.update(kw)
    return mla.Dims(d["n_heads"], d["d_head"], d["d_rope"], d["d_latent"], d["dtype"])


# Host-side argument checks run before any device query, so they work on a
# machine without a GPU.

def test_null_and_bad_dims_rejected_on_host():
    L = mla.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.mla_absorb_q(None, 1, fake, fake, fake, fake, None) == 1          # NULL dims
    assert L.mla_absorb_q(ctypes.byref(_dims(dtype=7)), 1, fake, fake, fake, fake, None) == 3
    assert L.mla_absorb_q(ctypes.byref(_dims(n_heads=0)), 1, fake, fake, fake, fake, None) == 2
    assert L.mla_absorb_q(ctypes.byref(_dims(d_latent=4096)), 1, fake, fake, fake, fake,
                          None) == 2
    assert L.mla_absorb_q(ctypes.byref(_dims()), -1, fake, fake, fake, fake, None) == 2
    assert L.mla_absorb_q(ctypes.byref(_dims()), 0, None, None, None, None, None) == 0
    assert L.mla_absorb_q(ctypes.byref(_dims()), 2, None, fake, fake, fake, None) == 1
    assert L.mla_absorb_q(ctypes.byref(_dims()), 2, ctypes.c_void_p(0x1004), fake, fake, fake,
                          None) == 5
    assert L.mla_out_uv(ctypes.byref(_dims()), 2, fake, None, fake, None) == 1
    cache = mla.CacheDesc(0x1000, 0x2000, 0x3000, 0, 64, 1)  # paged without page_size
    assert L.mla_decode_attn(ctypes.byref(_dims()), 1, fake, ctypes.byref(cache), 1.0, None,
                             fake, None, fake, 1 << 20, None) == 2
    cache = mla.CacheDesc(0x1000, 0x2000, None, 0, 64, 0)
    assert L.mla_decode_attn(ctypes.byref(_dims()), 1, None, ctypes.byref(cache), 1.0, None,
                             fake, None, fake, 1 << 20, None) == 1
    # Fused combine + W^UV: NULL or misaligned projection operands.
    assert L.mla_decode_combine_out(ctypes.byref(_dims()), 1, ctypes.byref(cache), None, fake,
                                    1 << 20, None, fake, fake, None, None) == 1
    assert L.mla_decode_combine_out(ctypes.byref(_dims()), 1, ctypes.byref(cache), None, fake,
                                    1 << 20, fake, None, fake, None, None) == 1
    assert L.mla_decode_combine_out(ctypes.byref(_dims()), 1, ctypes.byref(cache), None, fake,
                                    1 << 20, ctypes.c_void_p(0x1002), fake, fake, None,
                                    None) == 5
    assert L.mla_decode_combine_out(ctypes.byref(_dims()), 0, ctypes.byref(cache), None, None,
                                    0, None, None, None, None, None) == 0


def test_cache_append_host_checks():
    L = mla.lib()
    fake = ctypes.c_void_p(0x1000)
    rope = mla.Rope(10000.0, 1.0, 1.0, 32.0, 4096)
    cache = mla.CacheDesc(0x1000, 0x2000, None, 0, 64, 0)
    d = _dims()
    ws = 1 << 20
    # Workspace size: 16 slices of fp32 sums per request on the MFMA path.
    assert L.mla_cache_append_workspace_bytes(ctypes.byref(d), 16, 5120) >= 16 * 16 * 576 * 4
    assert L.mla_cache_append_workspace_bytes(None, 16, 5120) == 0

    def call(**kw):
        a = dict(dims=ctypes.byref(d), batch=2, d_model=5120, h=fake, w_dkv=fake, w_kr=fake,
                 g=fake, eps=1e-6, rope=ctypes.byref(rope), pos=fake,
                 cache=ctypes.byref(cache), ws=fake, ws_bytes=ws)
        a.update(kw)
        return L.mla_cache_append(a["dims"], a["batch"], a["d_model"], a["h"], a["w_dkv"],
                                  a["w_kr"], a["g"], a["eps"], a["rope"], a["pos"], a["cache"],
                                  a["ws"], a["ws_bytes"], None)

    assert call(batch=0, h=None, w_dkv=None, w_kr=None, g=None, pos=None) == 0
    assert call(h=None) == 1
    assert call(pos=None) == 1
    assert call(rope=None) == 1
    assert call(d_model=0) == 2
    assert call(eps=-1.0) == 2
    assert call(eps=float("nan")) == 2
    assert call(dims=ctypes.byref(_dims(d_rope=63))) == 2
    bad_rope = mla.Rope(0.0, 1.0, 1.0, 32.0, 4096)
    assert call(rope=ctypes.byref(bad_rope)) == 2
    bad_yarn = mla.Rope(10000.0, 40.0, 32.0, 1.0, 4096)  # beta <= alpha
    assert call(rope=ctypes.byref(bad_yarn)) == 2
    no_len = mla.Rope(10000.0, 40.0, 1.0, 32.0, 0)
    assert call(rope=ctypes.byref(no_len)) == 2
    assert call(h=ctypes.c_void_p(0x1008)) == 5
    assert call(ws_bytes=16) == 4
    assert call(ws=None) == 4


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_no_device_is_reported_without_gpu():
    L = mla.lib()
    fake = ctypes.c_void_p(0x1000)
    st = L.mla_absorb_q(ctypes.byref(_dims()), 1, fake, fake, fake, fake, None)
    assert st == 7
    # The workspace size needs the device's compute-unit count: 0 without one.
    assert L.mla_decode_workspace_bytes(ctypes.byref(_dims()), 16, 4096) == 0


def test_decode_workspace_bytes_rejects_bad_arguments():
    L = mla.lib()
    assert L.mla_decode_workspace_bytes(None, 16, 4096) == 0
    assert L.mla_decode_workspace_bytes(ctypes.byref(_dims(n_heads=0)), 16, 4096) == 0
    assert L.mla_decode_workspace_bytes(ctypes.byref(_dims()), -1, 4096) == 0
    assert L.mla_decode_workspace_bytes(ctypes.byref(_dims()), 16, -1) == 0


# ----------------------------------------------------------------------------
# Device-side checks (need the GPU for the device query)
# ----------------------------------------------------------------------------

@pytest.mark.gpu
def test_plan_shapes_and_workspace_errors():
    L = mla.lib()
    B, T = 16, 4096
    data = torch.zeros((B, T, 576), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    cache = mla.latent_cache(data, lens, 64)
    plan = mla.decode_plan(128, 512, 64, torch.bfloat16, cache)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # Several splits per request: the 64-row form, two row groups per request,
    # and 16 requests x 2 groups leave compute units idle: a length-balanced
    # plan with room for one workgroup per compute unit.
    assert plan.kernel == 2 and plan.head_groups == 2
    assert plan.split_tokens == 0 and plan.balanced
    assert plan.partitions == cus // 2 and plan.num_splits == min(plan.partitions, T // 32)
    # bf16 partial outputs plus fp32 (lse, m) pairs, plus the partition table
    assert plan.workspace_bytes >= plan.partitions * 128 * (512 * 2 + 8) + 4 * (B + 2)
    # The exported size query returns this plan's workspace.
    assert mla.decode_workspace_bytes(128, 512, 64, torch.bfloat16, B, T) == plan.workspace_bytes
    # A split length asked for gives a uniform plan.
    up = mla.decode_plan(128, 512, 64, torch.bfloat16, cache, split_tokens=512)
    assert (up.split_tokens, up.num_splits, up.partitions) == (512, T // 512, B * T // 512)
    assert not up.balanced
    q = torch.zeros((B, 128, 576), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, 128, 512), dtype=torch.bfloat16, device="cuda")
    ws = mla.workspace_for(plan, "cuda")
    d = _dims()
    desc = cache.desc()
    st = L.mla_decode_attn(ctypes.byref(d), B, q.data_ptr(), ctypes.byref(desc), 0.07,
                           ctypes.byref(plan), out.data_ptr(), None, ws.data_ptr(),
                           plan.workspace_bytes - 1, None)
    assert st == 4
    st = L.mla_decode_attn(ctypes.byref(d), B, q.data_ptr() + 2, ctypes.byref(desc), 0.07,
                           ctypes.byref(plan), out.data_ptr(), None, ws.data_ptr(),
                           plan.workspace_bytes, None)
    assert st == 5
    # A plan whose split count does not match its split length is rejected.
    bad = mla.Plan(plan.split_tokens, plan.num_splits - 1, plan.kernel, plan.head_groups,
                   plan.q_len, plan.workspace_bytes, plan.partitions)
    st = L.mla_decode_attn(ctypes.byref(d), B, q.data_ptr(), ctypes.byref(desc), 0.07,
                           ctypes.byref(bad), out.data_ptr(), None, ws.data_ptr(),
                           plan.workspace_bytes, None)
    assert st == 2
    # So is a plan whose query count was changed by hand (its head groups and
    # workspace no longer match), and a query count out of range.
    bad = mla.Plan(plan.split_tokens, plan.num_splits, plan.kernel, plan.head_groups,
                   2, plan.workspace_bytes, plan.partitions)
    st = L.mla_decode_attn(ctypes.byref(d), B, q.data_ptr(), ctypes.byref(desc), 0.07,
                           ctypes.byref(bad), out.data_ptr(), None, ws.data_ptr(),
                           plan.workspace_bytes, None)
    assert st == 2
    # And a balanced plan whose capacity was changed by hand.
    bad = mla.Plan(plan.split_tokens, plan.num_splits, plan.kernel, plan.head_groups,
                   plan.q_len, plan.workspace_bytes, plan.partitions + 1)
    st = L.mla_decode_attn(ctypes.byref(d), B, q.data_ptr(), ctypes.byref(desc), 0.07,
                           ctypes.byref(bad), out.data_ptr(), None, ws.data_ptr(),
                           plan.workspace_bytes, None)
    assert st == 2
    p2 = mla.Plan()
    for q_len in (0, 1025):
        assert L.mla_decode_plan_mq(ctypes.byref(d), B, q_len, ctypes.byref(desc), 0,
                                    ctypes.byref(p2)) == 2
    torch.cuda.synchronize()


@pytest.mark.gpu
def test_generic_and_mfma_plans_selected_by_dims():
    data = torch.zeros((2, 64, 40), dtype=torch.float32, device="cuda")
    lens = torch.full((2,), 64, dtype=torch.int32, device="cuda")
    cache = mla.latent_cache(data, lens, 8)
    assert mla.decode_plan(4, 32, 8, torch.float32, cache).kernel == 0
    data = torch.zeros((2, 64, 576), dtype=torch.bfloat16, device="cuda")
    cache = mla.latent_cache(data, lens, 64)
    assert mla.decode_plan(128, 512, 64, torch.bfloat16, cache).kernel == 1
    assert mla.decode_plan(96, 512, 64, torch.bfloat16, cache).kernel == 0
    assert mla.decode_plan(128, 512, 64, torch.bfloat16, cache, split_tokens=33).split_tokens == 64


def test_prefill_host_checks():
    """mla_prefill_expand / mla_prefill_attn reject bad arguments on the host
    (before any device query), and report the missing device last."""
    L = mla.lib()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    d = ctypes.byref(_dims())
    cache = mla.CacheDesc(0x1000, 0x2000, None, 0, 64, 0)
    c = ctypes.byref(cache)
    E = L.mla_prefill_expand
    assert E(None, 1, c, fake, fake, fake, fake, None) == 1
    assert E(ctypes.byref(_dims(d_head=64)), 1, c, fake, fake, fake, fake, None) == 2
    assert E(ctypes.byref(_dims(dtype=mla.MLA_F32)), 1, c, fake, fake, fake, fake, None) == 3
    paged = mla.CacheDesc(0x1000, 0x2000, 0x3000, 16, 64, 4)
    assert E(d, 1, ctypes.byref(paged), fake, fake, fake, fake, None) == 2
    fp8 = mla.CacheDesc(0x1000, 0x2000, None, 0, 64, 0)
    fp8.scales = 0x4000
    fp8.row_format = mla.MLA_ROWS_FP8
    assert E(d, 1, ctypes.byref(fp8), fake, fake, fake, fake, None) == 3
    assert E(d, -1, c, fake, fake, fake, fake, None) == 2
    assert E(d, 0, c, None, None, None, None, None) == 0
    assert E(d, 1, c, None, fake, fake, fake, None) == 1
    assert E(d, 1, c, fake, fake, odd, fake, None) == 5
    assert E(d, 1, c, fake, fake, fake, fake, None) == 7
    A = L.mla_prefill_attn
    args = (fake, fake, c, fake, fake, ctypes.c_float(0.07), fake)
    assert A(d, 1, 0, *args, None, None) == 2        # q_len 0
    assert A(d, 1, 65, *args, None, None) == 2       # q_len past max_len
    assert A(d, 0, 8, *args, None, None) == 0
    assert A(d, 1, 8, None, fake, c, fake, fake, ctypes.c_float(0.07), fake, None, None) == 1
    assert A(d, 1, 8, *args, ctypes.c_void_p(0x1002), None) == 5   # lse not 4-byte aligned
    assert A(d, 1, 8, *args, None, None) == 7
