"""Helpers for GPU parity tests: upload seeded cases, run the HIP path through
the C ABI, and compare with the oracle (float64, CPU)."""

from __future__ import annotations

import numpy as np
import torch

import head_latent_attention_absorb_amd as mla
from workload import Case

# Tolerances for bf16 storage with fp32 accumulation, and for fp32 storage.
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 2e-2
F32_REL_L2 = 1e-5


def gpu_available() -> bool:
    return torch.cuda.is_available()


def to_dev(case: Case, name: str, device="cuda") -> torch.Tensor:
    x = getattr(case, name)
    if case.cfg.dtype == "bf16":
        bits = case.bits(name)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class DevCase:
    """A case resident on the GPU plus its cache descriptor."""

    def __init__(self, case: Case, device="cuda"):
        cfg = case.cfg
        self.case = case
        self.q_c = to_dev(case, "q_c", device)
        self.q_r = to_dev(case, "q_r", device)
        self.w_uk = to_dev(case, "w_uk", device)
        self.w_uv = to_dev(case, "w_uv", device)
        self.cache_data = to_dev(case, "cache", device)
        self.seq_lens = torch.from_numpy(case.seq_lens.astype(np.int32)).to(device)
        self.page_table = (torch.from_numpy(case.page_table).to(device)
                           if case.page_table is not None else None)
        self.cache = mla.latent_cache(self.cache_data, self.seq_lens, cfg.d_rope,
                                      self.page_table, cfg.page_size,
                                      cfg.max_len if cfg.paged else None)

    def run(self, split_tokens: int = 0):
        """absorb -> decode -> out_uv; returns device tensors (q_cat, o_lat, lse, o)."""
        cfg = self.case.cfg
        q_cat = mla.absorb_q(self.q_c, self.q_r, self.w_uk)
        o_lat, lse = mla.decode_attn(q_cat, self.cache, cfg.scale, split_tokens=split_tokens)
        o = mla.out_uv(o_lat, self.w_uv)
        torch.cuda.synchronize()
        return q_cat, o_lat, lse, o

    def run_fused(self, split_tokens: int = 0):
        """absorb -> decode partials -> combine fused with W^UV; returns device
        tensors (q_cat, o_lat, lse, o)."""
        cfg = self.case.cfg
        B = cfg.batch
        q_cat = mla.absorb_q(self.q_c, self.q_r, self.w_uk)
        plan = mla.decode_plan(cfg.n_heads, cfg.d_latent, cfg.d_rope, q_cat.dtype, self.cache,
                               split_tokens=split_tokens, d_head=cfg.d_head)
        ws = mla.workspace_for(plan, q_cat.device)
        mla.decode_partials(q_cat, self.cache, cfg.scale, plan, ws)
        o_lat = torch.empty((B, cfg.n_heads, cfg.d_latent), dtype=q_cat.dtype,
                            device=q_cat.device)
        lse = torch.empty((B, cfg.n_heads), dtype=torch.float32, device=q_cat.device)
        o = mla.decode_combine_out(self.cache, plan, ws, self.w_uv, o_lat, lse)
        torch.cuda.synchronize()
        return q_cat, o_lat, lse, o


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def assert_close(got, ref, dtype: str, what: str):
    r = rel_l2(got, ref)
    m = max_abs(got, ref)
    if dtype == "bf16":
        assert r <= BF16_REL_L2 and m <= BF16_MAX_ABS, f"{what}: rel_l2={r:.3e} max_abs={m:.3e}"
    else:
        assert r <= F32_REL_L2, f"{what}: rel_l2={r:.3e} max_abs={m:.3e}"
    return r, m
