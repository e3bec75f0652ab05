#!/usr/bin/env python3
"""Benchmark: MLA absorbed decode on one MI355X (default: DeepSeek-V2 shape B=16, T=4096).

A step is one whole decode step of one layer on one batch of synthetic input:
    mla_absorb_q -> mla_decode_partials -> mla_decode_combine_out
(the last merges the split partials and applies W^UV in one kernel; it does
exactly what mla_decode_combine followed by mla_out_uv does; with one split
per request the step is mla_absorb_q -> mla_decode_attn -> mla_out_uv, the
decode kernel writing o_lat itself).  For the
60-layer workload a step is the 60 layers back to back, each with its own
weights and cache.  Inputs are resident in HBM before the timed region.  A
single-layer step uses the next entry of a rotating pool of independently
seeded (cache, W^UK, W^UV, q) sets totalling > 512 MB, twice the 256 MB
Infinity Cache, so the cache bytes really come from HBM.

Beside the step, the attention alone (mla_decode_attn: the decode kernel and
the split combine, one C call) is timed back to back over the same inputs and
set against its roofline.

Prints ONE JSON line on stdout (everything else goes to stderr).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import head_latent_attention_absorb_amd as mla  # noqa: E402
from workload import CONFIGS, f32_to_bf16_bits, make_append_case, make_case  # noqa: E402

METRIC = "MLA decode tokens/s and latent-cache HBM GB/s (% roofline), B=16 T=4096"
WORKLOAD = "dsv2_b16_t4096"
WORKLOADS = ("dsv2_b16_t4096", "ragged_b4_16k_32k", "paged_b128_t2048", "ctx128k_b2_60l",
             "mtp2_b16_t4096", "fp8_b16_t4096", "prefill_c512_b4_t4096",
             "prefill_unabsorbed_c512_b4_t4096")
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_partials_dsv2_b16_t4096_counters.json")
KERNEL_SOURCE = os.path.join(ROOT, "head_latent_attention_absorb_amd", "csrc", "decode_mfma.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


class Entry:
    """One input set (one layer of one batch) resident on the GPU, drawn with
    the same seeded generator as the parity tests."""

    def __init__(self, cfg, seed):
        case = make_case(cfg, seed)
        self.case = case
        self.q_c = to_dev(case.q_c)
        self.q_r = to_dev(case.q_r)
        self.w_uk = to_dev(case.w_uk)
        self.w_uv = to_dev(case.w_uv)
        self.cache_t = to_dev(case.cache)
        self.scales = None
        if cfg.cache_format == "fp8":
            # The low-bit cache: the drawn rows quantised on the GPU (E4M3
            # codes and one fp32 scale per row); the bf16 copy is dropped.
            self.cache_t, self.scales = mla.quantize_rows(self.cache_t)
        self.lens = torch.from_numpy(case.seq_lens.astype(np.int32)).cuda()
        self.page_table = (torch.from_numpy(case.page_table).cuda()
                           if case.page_table is not None else None)
        self.cache = mla.latent_cache(self.cache_t, self.lens, cfg.d_rope, self.page_table,
                                      cfg.page_size, cfg.max_len if cfg.paged else None,
                                      scales=self.scales)
        self.tokens = int(case.seq_lens.sum())
        self.nbytes = sum(t.numel() * t.element_size()
                          for t in (self.q_c, self.q_r, self.w_uk, self.w_uv, self.cache_t,
                                    self.scales) if t is not None)
        # Inputs of the cache append (the step before the decode path): the new
        # token's hidden state, W^DKV, W^KR and the RMSNorm weight.
        ac = make_append_case(cfg, seed)
        self.h = to_dev(ac.h)
        self.w_dkv = to_dev(ac.w_dkv)
        self.w_kr = to_dev(ac.w_kr)
        self.rms_weight = to_dev(ac.rms_weight)
        self.positions = torch.from_numpy(ac.positions).cuda()


class DeviceEntry:
    """The same distributions drawn on the GPU from a seeded torch generator
    (contiguous caches only): used for the 60-layer 128K workload, whose
    18 GB of cache would take minutes to draw on the host.  Timing only."""

    def __init__(self, cfg, seed):
        assert not cfg.paged and cfg.len_lo == cfg.len_hi
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        B, nh, dh, dr, dc = cfg.batch, cfg.n_heads, cfg.d_head, cfg.d_rope, cfg.d_latent

        def randn(shape, std=1.0):
            return (torch.randn(shape, generator=g, device="cuda") * std).to(torch.bfloat16)

        self.q_c = randn((B, nh, dh))
        self.q_r = randn((B, nh, dr))
        self.w_uk = randn((nh, dh, dc), dc ** -0.5)
        self.w_uv = randn((nh, dc, dh), dc ** -0.5)
        self.cache_t = torch.empty((B, cfg.max_len, dc + dr), dtype=torch.bfloat16,
                                   device="cuda")
        for b in range(B):  # one request at a time bounds the fp32 temporary
            self.cache_t[b] = randn((cfg.max_len, dc + dr))
        self.lens = torch.full((B,), cfg.len_lo, dtype=torch.int32, device="cuda")
        self.cache = mla.latent_cache(self.cache_t, self.lens, cfg.d_rope)
        self.tokens = B * cfg.len_lo
        self.nbytes = sum(t.numel() * t.element_size()
                          for t in (self.q_c, self.q_r, self.w_uk, self.w_uv, self.cache_t))


def kernel_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counters_for(sha: str):
    """The committed rocprofv3 PMC counters of the decode kernel, or {} when
    absent or taken on a different kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return {}
    with open(COUNTERS_FILE) as f:
        c = json.load(f)
    return c if c.get("kernel_source_sha") == sha else {}


def cpu_baseline(entry: Entry, cfg, n_requests: int, min_seconds: float = 8.0):
    """The oracle on a bounded sample of the same workload, on the host cores:
    its absorbed form in fp32 (the method itself on the CPU: absorb, latent
    attention, W^UV, numpy BLAS) as the reported value, and beside it the same
    absorbed form in fp64 and the unabsorbed fp64 form that parity is graded
    against.  Each leg repeats whole passes over the sample until min_seconds
    have elapsed."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = None
    case = entry.case
    reqs = list(range(n_requests))
    args = (case.q_c, case.q_r, case.cache, case.seq_lens, case.w_uk, case.w_uv, cfg.scale)

    def leg(fn):
        passes = 0
        t0 = time.perf_counter()
        while True:
            fn()
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                return passes * n_requests / dt, passes, dt

    kw = dict(page_table=case.page_table, page_size=cfg.page_size, requests=reqs)
    v32, p32, t32 = leg(lambda: oracle.mla_decode_absorbed(*args, dtype=np.float32, **kw))
    v64a, p64a, t64a = leg(lambda: oracle.mla_decode_absorbed(*args, **kw))
    v64u, p64u, t64u = leg(lambda: oracle.mla_decode_reference(
        *args, case.page_table, cfg.page_size, requests=reqs))
    return {
        "value": v32,
        "unit": "tokens/s",
        "cores": int(blas_threads or os.cpu_count()),
        "kind": "oracle",
        "sample": (f"absorbed oracle in fp32 (numpy BLAS), {n_requests} of {cfg.batch} "
                   f"requests x all {cfg.n_heads} heads x T={cfg.max_len}, one layer, "
                   f"{p32} passes in {t32:.2f} s"),
        "cpu_count": os.cpu_count(),
        "blas_threads": blas_threads,
        "absorbed_fp64_tokens_per_s": v64a,
        "unabsorbed_fp64_tokens_per_s": v64u,
        "legs": (f"absorbed fp64: {p64a} passes in {t64a:.2f} s; unabsorbed fp64 (the parity "
                 f"reference): {p64u} passes in {t64u:.2f} s"),
    }


def copy_calibration(n_bytes: int = 256 << 20, copies: int = 6):
    """Plain device-to-device copies of a known size.  Under rocprofv3 --pmc the
    ratio of FETCH_SIZE (or WRITE_SIZE) per copy dispatch to n_bytes is the factor
    that turns those counters into bytes for the decode kernel."""
    src = [torch.full((n_bytes,), i, dtype=torch.uint8, device="cuda") for i in range(2)]
    dst = [torch.empty(n_bytes, dtype=torch.uint8, device="cuda") for _ in range(3)]
    torch.cuda.synchronize()
    for i in range(copies):
        dst[i % 3].copy_(src[i % 2])
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n_bytes, "copies": copies}), flush=True)


def percentiles(x):
    x = np.asarray(x)
    return {"p10": float(np.percentile(x, 10)), "p50": float(np.percentile(x, 50)),
            "p90": float(np.percentile(x, 90))}


def run_unabsorbed(args, cfg, name):
    """The chunk in the unabsorbed form: one step = mla_prefill_expand (explicit
    keys and values of every cached row) + mla_prefill_attn (causal attention
    of the q_len new tokens over them), per request batch.  Same inputs, pool
    rotation, timing and JSON line as the absorbed workloads; the roofline is
    prefill_attn_kernel's MFMA one."""
    B, nh, ql = cfg.batch, cfg.n_heads, cfg.q_len
    dh, dr, dc = cfg.d_head, cfg.d_rope, cfg.d_latent
    log(f"[bench] generating inputs for {name}")
    pool = [Entry(cfg, 0)]
    n_pool = max(1, math.ceil(args.pool_mb * 1e6 / pool[0].nbytes))
    for i in range(1, n_pool):
        pool.append(Entry(cfg, i))
    pool_mb = sum(e.nbytes for e in pool) / 1e6
    log(f"[bench] pool: {n_pool} entries, {pool_mb:.0f} MB")
    dev = "cuda"
    kv_shape = (B, nh, cfg.max_len, dh)
    k_c = torch.empty(kv_shape, dtype=torch.bfloat16, device=dev)
    v = torch.empty(kv_shape, dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, ql, nh, dh), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, ql, nh), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def views(e):
        return e.q_c.view(B, ql, nh, dh), e.q_r.view(B, ql, nh, dr)

    def step(i, ev=None):
        e = pool[i % n_pool]
        q_c, q_r = views(e)
        if ev is not None:
            ev[0].record(stream)
        mla.prefill_expand(e.cache, e.w_uk, e.w_uv, k_c=k_c, v=v)
        if ev is not None:
            ev[1].record(stream)
        mla.prefill_attn(q_c, q_r, e.cache, k_c, v, cfg.scale, out=out, lse=lse)
        if ev is not None:
            ev[2].record(stream)

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_start.record(stream)
    for i in range(args.steps):
        step(i)
    e_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e_start.elapsed_time(e_end) / args.steps
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    bounds[0].record(stream)
    for i in range(args.steps):
        step(i)
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    step_us = [bounds[i].elapsed_time(bounds[i + 1]) * 1e3 for i in range(args.steps)]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    phase = np.array([[ev[k].elapsed_time(ev[k + 1]) for k in range(2)] for ev in evs])
    expand_us, attn_phase_us = (float(x) for x in phase.mean(axis=0) * 1e3)
    log(f"[bench] step {ms_per_step*1e3:.1f} us: expand {expand_us:.1f}, attn {attn_phase_us:.1f}")
    # The attention kernel alone, back to back over the expanded keys/values
    # of the last step (the roofline's time).
    def attn_only(i):
        q_c, q_r = views(pool[i % n_pool])
        mla.prefill_attn(q_c, q_r, pool[i % n_pool].cache, k_c, v, cfg.scale, out=out, lse=lse)
    attn_us = timed(attn_only, args.steps)
    expand_b2b_us = timed(lambda i: mla.prefill_expand(
        pool[i % n_pool].cache, pool[i % n_pool].w_uk, pool[i % n_pool].w_uv, k_c=k_c, v=v),
        args.steps)
    log(f"[bench] prefill_attn back to back: {attn_us:.1f} us; expand back to back: "
        f"{expand_b2b_us:.1f} us")

    tokens = sum(pool[i % n_pool].tokens for i in range(args.steps)) / args.steps
    # Query-key pairs: token j of a request sees len - q_len + j + 1 rows.
    visible = ql * tokens - B * ql * (ql - 1) / 2
    attn_flops = 2.0 * nh * (dh + dr + dh) * visible
    expand_flops = 2.0 * nh * tokens * dc * 2 * dh
    kv_bytes = 2 * nh * tokens * dh * 2
    cache_bytes = tokens * (dc + dr) * 2
    w_bytes = 2 * nh * dh * dc * 2
    io_bytes = B * ql * nh * (dh + dr + dh) * 2 + B * ql * nh * 4
    # Step: the cache, weights, queries and outputs once, and the explicit keys
    # and values written once and read once (the form's own round trip).
    step_bytes = cache_bytes + w_bytes + io_bytes + 2 * kv_bytes
    step_flops = attn_flops + expand_flops
    t_roof_us = max(step_bytes / (HBM_PEAK_GBPS * 1e9),
                    step_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
    attn_bytes = kv_bytes + B * cfg.max_len * dr * 2 + io_bytes
    attn_tflops = attn_flops / (attn_us * 1e-6) / 1e12
    result = {
        "metric": f"MLA decode tokens/s and latent-cache HBM GB/s (% roofline), {name}",
        "value": B * ql / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": name, "batch": B, "seq_len": cfg.max_len,
            "seq_len_range": [cfg.len_lo, cfg.len_hi], "n_heads": nh, "d_head": dh,
            "d_latent": dc, "d_rope": dr, "cache": "contiguous", "layers_per_step": 1,
            "rotating_pool_mb": round(pool_mb), "query_tokens_per_request": ql,
            "form": "unabsorbed (explicit keys and values)", "parallelism": "single-gpu",
        },
        "step_us": percentiles(step_us),
        "step_roofline_us": t_roof_us,
        "step_pct_roofline": 100.0 * t_roof_us / (ms_per_step * 1e3),
        "kernels_us": {"prefill_expand": expand_us, "prefill_attn": attn_phase_us,
                       "prefill_attn_back_to_back": attn_us,
                       "prefill_expand_back_to_back": expand_b2b_us},
        "expand_tflops": expand_flops / (expand_b2b_us * 1e-6) / 1e12,
        "roofline": {
            "kernel": "prefill_attn_kernel (mla_prefill_attn)",
            "bound": "mfma",
            "achieved": attn_tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
            "alg_flops_per_launch": attn_flops,
            "alg_bytes_per_launch": attn_bytes,
            "launch_us": attn_us,
        },
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=WORKLOAD, choices=WORKLOADS)
    ap.add_argument("--pool-mb", type=int, default=640,
                    help="total bytes of the rotating input pool (>= 512 MB defeats the MALL)")
    ap.add_argument("--cpu-requests", type=int, default=16,
                    help="requests in the CPU oracle sample (0 skips it; default workload only)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--seq-len", type=int, default=0,
                    help="every request at this many cached rows instead of the workload's "
                         "lengths (single-layer contiguous workloads; a sweep of it splits "
                         "the decode kernel's time into per-step and fixed costs)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a HIP graph instead of plain calls")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 256 MiB device copies (a known-size kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(one GPU holds the whole batch; see the project notes on sharding). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    name = args.workload
    cfg = CONFIGS[name]
    if args.seq_len > 0:
        if cfg.paged or cfg.layers > 1 or cfg.form == "unabsorbed":
            print("--seq-len applies to single-layer contiguous workloads", file=sys.stderr)
            sys.exit(2)
        cfg = cfg.replace(len_lo=args.seq_len, len_hi=args.seq_len, max_len=args.seq_len)
    if cfg.form == "unabsorbed":
        run_unabsorbed(args, cfg, name)
        return
    B, nh, row = cfg.batch, cfg.n_heads, cfg.row
    # Query tokens per request: the verification workload decodes the last
    # q_len positions of every request at once; the absorb and the output
    # projection then see B * q_len query rows.
    ql = cfg.q_len
    lead = (B,) if ql == 1 else (B, ql)
    layered = cfg.layers > 1
    log(f"[bench] generating inputs for {name}")
    if layered:
        # One step = every layer once, each with its own weights and cache.
        pool = [DeviceEntry(cfg, 1000 + l) for l in range(cfg.layers)]
    else:
        pool = [Entry(cfg, 0)]
        n_pool = max(1, math.ceil(args.pool_mb * 1e6 / pool[0].nbytes))
        for i in range(1, n_pool):
            pool.append(Entry(cfg, i))
    n_pool = len(pool)
    pool_mb = sum(e.nbytes for e in pool) / 1e6
    log(f"[bench] {'layers' if layered else 'pool'}: {n_pool} entries, {pool_mb:.0f} MB")

    dev = "cuda"
    plan = mla.decode_plan(nh, cfg.d_latent, cfg.d_rope, torch.bfloat16, pool[0].cache,
                           split_tokens=args.split_tokens, d_head=cfg.d_head, q_len=ql)
    log(f"[bench] {plan}")
    ws = mla.workspace_for(plan, dev)
    append_ws = torch.empty(max(256, int(mla.lib().mla_cache_append_workspace_bytes(
        mla.make_dims(1, 1, cfg.d_rope, cfg.d_latent, torch.bfloat16), B, cfg.hidden))),
        dtype=torch.uint8, device=dev)
    q_cat = torch.empty(lead + (nh, row), dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty(lead + (nh, cfg.d_latent), dtype=torch.bfloat16, device=dev)
    lse = torch.empty(lead + (nh,), dtype=torch.float32, device=dev)
    o = torch.empty(lead + (nh, cfg.d_head), dtype=torch.bfloat16, device=dev)
    q_rows = q_cat.view(B * ql, nh, row)
    direct = plan.direct
    form = f"{128 if plan.kernel == 1 else 64} query rows per workgroup"
    stream = torch.cuda.current_stream()

    def layer(e: Entry, ev=None):
        if ev is not None:
            ev[0].record(stream)
        mla.absorb_q(e.q_c.view(B * ql, nh, cfg.d_head), e.q_r.view(B * ql, nh, cfg.d_rope),
                     e.w_uk, out=q_rows)
        if ev is not None:
            ev[1].record(stream)
        if direct:
            # One split per request: mla_decode_attn's decode kernel writes
            # o_lat and lse itself, then the per-head W^UV product.
            mla.decode_attn(q_cat, e.cache, cfg.scale, plan, o_lat, lse, ws)
            if ev is not None:
                ev[2].record(stream)
            mla.out_uv(o_lat.view(B * ql, nh, cfg.d_latent), e.w_uv,
                       out=o.view(B * ql, nh, cfg.d_head))
        else:
            mla.decode_partials(q_cat, e.cache, cfg.scale, plan, ws)
            if ev is not None:
                ev[2].record(stream)
            mla.decode_combine_out(e.cache, plan, ws, e.w_uv, o_lat, lse, out=o)
        if ev is not None:
            ev[3].record(stream)

    def entries(i):
        return pool if layered else [pool[i % n_pool]]

    # --graph: single-layer workloads replay each pool entry's step from a HIP
    # graph (captured once, after the warmup).  Measured slower than plain
    # calls on MI355X (54.5 vs 53.1 us at B=16): the gaps between the three
    # dependent kernels are on the GPU side, so plain calls are the default.
    graphs = None

    def step(i):
        if graphs is not None:
            graphs[i % n_pool].replay()
            return
        for e in entries(i):
            layer(e)

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us per call

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    eager_ms = None
    if not layered and args.graph:
        eager_ms = timed(step, args.steps) / 1e3
        graphs = []
        for e in pool:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layer(e)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        log(f"[bench] eager step {eager_ms*1e3:.1f} us; timing graph replays")

    # Timed region: exactly --steps whole steps, between device synchronisations.
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_start.record(stream)
    for i in range(args.steps):
        step(i)
    e_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e_start.elapsed_time(e_end) / args.steps

    # The same steps again with an event between steps: the spread of step
    # times.
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    bounds[0].record(stream)
    for i in range(args.steps):
        step(i)
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    step_us = [bounds[i].elapsed_time(bounds[i + 1]) * 1e3 for i in range(args.steps)]
    kernels_us = {}
    if not layered:
        # And once more with events between the kernels: per-kernel times (the
        # event records add a little to each).  This pass also runs the cache
        # append of the step's new token first (the step before the decode
        # path, not part of the step timed above); the step's ~100 MB between
        # two appends keep its weights out of the last-level cache.
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            e = pool[i % n_pool]
            evs[i][0].record(stream)
            mla.cache_append(e.cache, e.h, e.w_dkv, e.w_kr, e.rms_weight, e.positions,
                             workspace=append_ws)
            layer(e, evs[i][1:])
        torch.cuda.synchronize()
        phase = np.array([[ev[k].elapsed_time(ev[k + 1]) for k in range(4)] for ev in evs])
        append_us, absorb_us, partials_us, tail_us = (float(x) for x in phase.mean(axis=0) * 1e3)
        if direct:
            kernels_us = {"absorb_q": absorb_us, "decode_attn_direct": partials_us,
                          "out_uv": tail_us, "cache_append": append_us}
        else:
            kernels_us = {"absorb_q": absorb_us, "decode_partials": partials_us,
                          "decode_combine_out": tail_us, "cache_append": append_us}
        log(f"[bench] step {ms_per_step*1e3:.1f} us: absorb {absorb_us:.1f}, "
            f"{'decode (direct)' if direct else 'partials'} {partials_us:.1f}, "
            f"{'out_uv' if direct else 'combine+out_uv'} {tail_us:.1f}")
    else:
        log(f"[bench] step ({cfg.layers} layers) {ms_per_step*1e3:.1f} us")

    # The decode kernel alone, launched back to back on the same stream over
    # the same inputs: its average launch duration, free of the event records
    # that split the phases above.  This is the roofline's time.  With one
    # split the kernel runs in the form that writes o_lat directly (through
    # mla_decode_attn, which then launches nothing else).
    n_dec = args.steps * (cfg.layers if layered else 1)
    if direct:
        decode_us = timed(lambda i: mla.decode_attn(
            q_cat, pool[i % n_pool].cache, cfg.scale, plan, o_lat, lse, ws), n_dec)
    else:
        decode_us = timed(lambda i: mla.decode_partials(
            q_cat, pool[i % n_pool].cache, cfg.scale, plan, ws), n_dec)
    log(f"[bench] decode kernel back to back: {decode_us:.1f} us per launch ({form})")

    # mla_decode_attn (the decode kernel, then the split combine unless one
    # split), back to back, per step: one C call per layer.
    def attn(i):
        for e in entries(i):
            mla.decode_attn(q_cat, e.cache, cfg.scale, plan, o_lat, lse, ws)
    attn_us = timed(attn, args.steps)
    log(f"[bench] mla_decode_attn back to back: {attn_us:.1f} us per step")

    # Algorithmic work per step (split partials excluded), averaged over the
    # entries the timed steps used.
    layers_per_step = cfg.layers if layered else 1
    tokens = (sum(e.tokens for e in pool) if layered
              else sum(pool[i % n_pool].tokens for i in range(args.steps)) / args.steps)
    tokens_layer = tokens / layers_per_step
    # Cached bytes per token: bf16 rows, or E4M3 rows plus one fp32 scale.
    row_bytes = row + 4 if cfg.cache_format == "fp8" else row * 2
    cache_bytes = tokens * row_bytes
    q_bytes = layers_per_step * B * ql * nh * row * 2
    olat_bytes = layers_per_step * B * ql * nh * (cfg.d_latent * 2 + 4)
    # Query token j of a request sees ql - 1 - j rows fewer than the request
    # holds (causal among the new tokens).
    visible = ql * tokens - layers_per_step * B * ql * (ql - 1) / 2
    flops = 2.0 * nh * (row + cfg.d_latent) * visible
    attn_bytes = cache_bytes + q_bytes + olat_bytes
    t_roof_attn_us = max(attn_bytes / (HBM_PEAK_GBPS * 1e9),
                         flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
    # The decode kernel's algorithmic bytes: the cache and the query (its
    # split partials are not algorithmic); in the direct form also o_lat and
    # lse, which it writes itself.
    k2_bytes = (attn_bytes if direct else cache_bytes + q_bytes) / layers_per_step
    k2_gbps = k2_bytes / (decode_us * 1e-6) / 1e9
    k2_tflops = flops / layers_per_step / (decode_us * 1e-6) / 1e12
    # The decode kernel's bound: HBM, unless its products take longer at the
    # MFMA peak (several query tokens per request raise the flops per byte).
    k2_mfma_bound = (flops / layers_per_step / (MFMA_BF16_PEAK_TFLOPS * 1e12) >
                     k2_bytes / (HBM_PEAK_GBPS * 1e9))
    # Whole step: the cache, both up-projection weights, the query in and the
    # output out, each moved once.
    w_bytes = layers_per_step * 2 * nh * cfg.d_head * cfg.d_latent * 2
    io_bytes = layers_per_step * B * ql * (nh * (cfg.d_head + cfg.d_rope) * 2 +
                                           nh * cfg.d_head * 2)
    step_bytes = cache_bytes + w_bytes + io_bytes
    step_flops = flops + layers_per_step * 2.0 * 2 * B * ql * nh * cfg.d_head * cfg.d_latent
    t_roof_us = max(step_bytes / (HBM_PEAK_GBPS * 1e9),
                    step_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
    sha = kernel_sha()
    default_shape = name == WORKLOAD and args.seq_len == 0
    counters = counters_for(sha) if default_shape else {}

    result = {
        "metric": METRIC if default_shape else
                  f"MLA decode tokens/s and latent-cache HBM GB/s (% roofline), {name}"
                  + (f", every request at {args.seq_len} rows" if args.seq_len else ""),
        # Tokens decoded per second: every query token of every request (the
        # verification workload decodes q_len per request and step).
        "value": B * ql / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": name, "batch": B, "seq_len": cfg.max_len,
            "seq_len_range": [cfg.len_lo, cfg.len_hi], "n_heads": nh,
            "d_head": cfg.d_head, "d_latent": cfg.d_latent, "d_rope": cfg.d_rope,
            "cache": (f"paged, {cfg.page_size}-token pages" if cfg.paged else "contiguous") +
                     (", E4M3 rows + fp32 row scales" if cfg.cache_format == "fp8" else ""),
            "layers_per_step": layers_per_step,
            "rotating_pool_mb": round(pool_mb), "split_tokens": plan.split_tokens,
            "num_splits": plan.num_splits, "query_tokens_per_request": ql,
            "parallelism": "single-gpu",
        },
        "step_us": percentiles(step_us),
        "launch": "hip graph per step (three kernels)" if graphs is not None else "eager calls",
        "eager_ms_per_step": eager_ms,
        "step_roofline_us": t_roof_us,
        "step_pct_roofline": 100.0 * t_roof_us / (ms_per_step * 1e3),
        "attn": {
            "what": ("mla_decode_attn, one split: the decode kernel writes o_lat and lse "
                     "directly" if direct else
                     "mla_decode_attn = decode kernel + split combine (one C call), back to back"),
            "us_per_step": attn_us,
            "roofline_us": t_roof_attn_us,
            "pct_roofline": 100.0 * t_roof_attn_us / attn_us,
            "alg_bytes": attn_bytes,
            "latent_cache_GBps": cache_bytes / (attn_us * 1e-6) / 1e9,
        },
        "latent_cache_GBps": cache_bytes / layers_per_step / (decode_us * 1e-6) / 1e9,
        "tokens_per_layer": tokens_layer,
        "kernels_us": dict(kernels_us, decode_kernel_back_to_back=decode_us),
        "roofline": {
            "kernel": (f"decode_mfma_kernel (mla_decode_attn, one split, direct output, {form})"
                       if direct else f"decode_mfma_kernel (mla_decode_partials, {form})"),
            "bound": "mfma" if k2_mfma_bound else "hbm",
            "achieved": k2_tflops if k2_mfma_bound else k2_gbps,
            "peak": MFMA_BF16_PEAK_TFLOPS if k2_mfma_bound else HBM_PEAK_GBPS,
            "unit": "TFLOP/s" if k2_mfma_bound else "GB/s",
            "frac": (k2_tflops / MFMA_BF16_PEAK_TFLOPS if k2_mfma_bound
                     else k2_gbps / HBM_PEAK_GBPS),
            "achieved_GBps": k2_gbps,
            # Counter-measured (rocprofv3 --pmc, same kernel source only):
            # HBM bytes per launch (FETCH_SIZE, WRITE_SIZE scaled by a plain
            # copy's), the MFMA busy fraction (rocprofv3's MfmaUtil) and the
            # MFMA flops the SQ counted.
            "traffic": counters.get("hbm_bytes_per_launch"),
            "mfma_util": counters.get("mfma", {}).get("mfma_util"),
            "mfma_flops_counted": counters.get("mfma", {}).get("mfma_flops_counted"),
            "alg_bytes_per_launch": k2_bytes,
            "launch_us": decode_us,
            "mfma_tflops": k2_tflops,
            "kernel_source_sha": sha,
        },
    }
    if not layered:
        # The cache append: every weight element of [W^DKV; W^KR] read once,
        # plus h, the RMSNorm weight and the written rows.
        ap_bytes = (row * cfg.hidden + B * cfg.hidden + cfg.d_latent + B * row) * 2 + B * 4
        result["cache_append"] = {
            "what": ("mla_cache_append (projection + RMSNorm + RoPE + row write) of one new "
                     "token per request, per step"),
            "us": kernels_us["cache_append"],
            "alg_bytes": ap_bytes,
            "roofline_us": ap_bytes / (HBM_PEAK_GBPS * 1e9) * 1e6,
            "achieved_GBps": ap_bytes / (kernels_us["cache_append"] * 1e-6) / 1e9,
            "timing": "events around the call inside the per-kernel pass",
        }
    if args.cpu_requests > 0 and default_shape:
        log(f"[bench] cpu baseline: oracle on {args.cpu_requests} requests")
        result["cpu_baseline"] = cpu_baseline(pool[0], cfg, args.cpu_requests)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
