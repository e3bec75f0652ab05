"""Seeded input generator for MLA absorbed decode workloads.

Every tensor is drawn from one numpy PCG64 stream per (config, seed) in a
fixed order: lengths, page permutation, q^C, q^R, c^KV, k^R, W^UK, W^UV.
bfloat16 configurations round each drawn fp32 value to bfloat16 with
round-to-nearest-even; the rounded values are what both the GPU path (as raw
bf16 bits) and the oracle (upcast to float) consume.

The shapes follow the MLA description of DeepSeek-V2: a latent c^KV of width
d_c and a shared, already-rotated RoPE key k^R of width d_h^R are cached per
token, stored as one row ``[c^KV | k^R]`` (DeepSeek-V3 read-through,
2kiu.com/news/6340724, section 2.2: the cache keeps exactly the latent and the
RoPE key).  Paged caches are a storage choice of this library, not of the
pages.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np


# ----------------------------------------------------------------------------
# bfloat16 bit handling (storage format only, no attention arithmetic)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    NaN maps to a quiet NaN with the input's sign; values that round past the
    largest finite bfloat16 become infinity, as IEEE rounding requires.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        sign = ((u[nan] >> 16) & 0x8000).astype(np.uint16)
        r[nan] = sign | np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------
# Workload configurations
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    batch: int
    n_heads: int
    d_head: int
    d_rope: int
    d_latent: int
    dtype: str               # "f32" or "bf16": storage type of every input
    len_lo: int              # request lengths ~ U{len_lo..len_hi} (inclusive)
    len_hi: int
    max_len: int             # contiguous row stride, or max_pages * page_size
    page_size: int = 0       # 0 => contiguous cache
    layers: int = 1
    softmax_scale: Optional[float] = None   # None => 1/sqrt(d_head + d_rope)
    d_model: int = 0         # hidden width d of the cache append; 0 => n_heads * d_head
    q_len: int = 1           # query tokens per request (several: speculative verification)
    cache_format: str = "native"  # "fp8": E4M3 rows with one fp32 scale per row
    # "unabsorbed": the chunk runs with explicit keys and values (benchmark only;
    # the drawn inputs are the same)
    form: str = "absorbed"

    @property
    def row(self) -> int:
        """Cached elements per token per layer: d_c + d_h^R."""
        return self.d_latent + self.d_rope

    @property
    def paged(self) -> bool:
        return self.page_size > 0

    @property
    def max_pages(self) -> int:
        return self.max_len // self.page_size if self.paged else 0

    @property
    def scale(self) -> float:
        if self.softmax_scale is not None:
            return float(self.softmax_scale)
        return 1.0 / math.sqrt(self.d_head + self.d_rope)

    @property
    def hidden(self) -> int:
        return self.d_model if self.d_model > 0 else self.n_heads * self.d_head

    def replace(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


# d = 5120: the hidden width in the zeeklog page's worked cache example.
_DSV2 = dict(n_heads=128, d_head=128, d_rope=64, d_latent=512, d_model=5120)

CONFIGS: Dict[str, WorkloadConfig] = {
    # Tiny fp32 decode: B=1, n_h=4, d_h=16, d_h^R=8, d_c=32, T=64.
    "tiny_f32": WorkloadConfig("tiny_f32", batch=1, n_heads=4, d_head=16, d_rope=8,
                               d_latent=32, dtype="f32", len_lo=64, len_hi=64,
                               max_len=64),
    # DeepSeek-V2 single-layer decode: B=16, every request at T=4096, contiguous.
    "dsv2_b16_t4096": WorkloadConfig("dsv2_b16_t4096", batch=16, dtype="bf16",
                                     len_lo=4096, len_hi=4096, max_len=4096, **_DSV2),
    # Long-context ragged batch: B=4, lengths U{16384..32768}.
    "ragged_b4_16k_32k": WorkloadConfig("ragged_b4_16k_32k", batch=4, dtype="bf16",
                                        len_lo=16384, len_hi=32768, max_len=32768,
                                        **_DSV2),
    # High-batch paged cache: B=128, lengths U{1..2048}, 64-token pages.
    "paged_b128_t2048": WorkloadConfig("paged_b128_t2048", batch=128, dtype="bf16",
                                       len_lo=1, len_hi=2048, max_len=2048,
                                       page_size=64, **_DSV2),
    # Speculative verification: B=16, T=4096, the last 2 positions of every
    # request decoded at once (causal between them).
    "mtp2_b16_t4096": WorkloadConfig("mtp2_b16_t4096", batch=16, dtype="bf16",
                                     len_lo=4096, len_hi=4096, max_len=4096, q_len=2,
                                     **_DSV2),
    # Chunked prefill in the absorbed form: 4 prompts of 4096 tokens whose last
    # 512 rows are the chunk being processed (causal within it).
    "prefill_c512_b4_t4096": WorkloadConfig("prefill_c512_b4_t4096", batch=4, dtype="bf16",
                                            len_lo=4096, len_hi=4096, max_len=4096,
                                            q_len=512, **_DSV2),
    # The same chunk in the unabsorbed form (explicit keys and values).
    "prefill_unabsorbed_c512_b4_t4096": WorkloadConfig(
        "prefill_unabsorbed_c512_b4_t4096", batch=4, dtype="bf16", len_lo=4096, len_hi=4096,
        max_len=4096, q_len=512, form="unabsorbed", **_DSV2),
    # The default shape over the low-bit cache: the same drawn rows, quantised
    # to E4M3 with one scale per row.
    "fp8_b16_t4096": WorkloadConfig("fp8_b16_t4096", batch=16, dtype="bf16",
                                    len_lo=4096, len_hi=4096, max_len=4096,
                                    cache_format="fp8", **_DSV2),
    # 128K-context decode: B=2, T=131072, 60 independently seeded layers.
    "ctx128k_b2_60l": WorkloadConfig("ctx128k_b2_60l", batch=2, dtype="bf16",
                                     len_lo=131072, len_hi=131072, max_len=131072,
                                     layers=60, **_DSV2),
}


# ----------------------------------------------------------------------------
# Cases
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Case:
    """One seeded draw of a workload.

    Float tensors hold float32 values that are exactly representable in the
    config's storage dtype.  ``cache`` is ``[B, max_len, d_c+d_h^R]`` for a
    contiguous cache and ``[num_pages, page_size, d_c+d_h^R]`` for a paged one;
    rows that no request owns hold ``pad_value``.
    """

    cfg: WorkloadConfig
    seed: int
    seq_lens: np.ndarray            # [B] int32
    page_table: Optional[np.ndarray]  # [B, max_pages] int32, or None
    q_c: np.ndarray                 # [B, n_h, d_h] ([B, q_len, n_h, d_h] if q_len > 1)
    q_r: np.ndarray                 # [B, n_h, d_h^R] (likewise)
    cache: np.ndarray               # see class docstring
    w_uk: np.ndarray                # [n_h, d_h, d_c]
    w_uv: np.ndarray                # [n_h, d_c, d_h]

    def bits(self, name: str) -> np.ndarray:
        """bf16 bit pattern (uint16) of a float tensor of a bf16 case."""
        if self.cfg.dtype != "bf16":
            raise ValueError("bits() is only defined for bf16 cases")
        return f32_to_bf16_bits(getattr(self, name))

    def logical_row_index(self, b: int) -> np.ndarray:
        """Flat row indices (into cache.reshape(-1, row)) of request b's tokens."""
        n = int(self.seq_lens[b])
        t = np.arange(n, dtype=np.int64)
        if self.page_table is None:
            return b * self.cfg.max_len + t
        ps = self.cfg.page_size
        return self.page_table[b, t // ps].astype(np.int64) * ps + (t % ps)


def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        x = round_to_bf16(x)
    return x


def make_case(cfg: WorkloadConfig, seed: int, *, pad_value: float = 0.0,
              seq_lens: Optional[np.ndarray] = None) -> Case:
    """Draw one case of ``cfg`` from PCG64(seed).

    Draw order: lengths, page permutation, q^C, q^R, c^KV, k^R, W^UK, W^UV.
    q^C, q^R, c^KV and k^R are N(0, 1); W^UK and W^UV are N(0, 1/d_c).
    ``seq_lens`` overrides the drawn lengths (the draw still happens, so the
    rest of the stream is unchanged).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, nh, dh, dr, dc = cfg.batch, cfg.n_heads, cfg.d_head, cfg.d_rope, cfg.d_latent

    lens = rng.integers(cfg.len_lo, cfg.len_hi, size=B, endpoint=True).astype(np.int32)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32).copy()
        if lens.shape != (B,):
            raise ValueError("seq_lens must have shape [batch]")
    if (lens < 0).any() or (lens > cfg.max_len).any():
        raise ValueError("request lengths must lie in [0, max_len]")

    page_table = None
    if cfg.paged:
        if cfg.max_len % cfg.page_size:
            raise ValueError("max_len must be a multiple of page_size")
        n_pages = B * cfg.max_pages
        page_table = rng.permutation(n_pages).astype(np.int32).reshape(B, cfg.max_pages)

    # With several query tokens per request, q^C and q^R hold them token-major
    # ([B, q_len, n_h, .]); one token keeps the [B, n_h, .] shape.
    lead = (B,) if cfg.q_len == 1 else (B, cfg.q_len)
    q_c = _draw(rng, lead + (nh, dh), 1.0, cfg.dtype)
    q_r = _draw(rng, lead + (nh, dr), 1.0, cfg.dtype)
    total = int(lens.sum())
    c_kv = _draw(rng, (total, dc), 1.0, cfg.dtype)
    k_r = _draw(rng, (total, dr), 1.0, cfg.dtype)
    w_std = 1.0 / math.sqrt(dc)
    w_uk = _draw(rng, (nh, dh, dc), w_std, cfg.dtype)
    w_uv = _draw(rng, (nh, dc, dh), w_std, cfg.dtype)

    if cfg.paged:
        cache = np.full((B * cfg.max_pages, cfg.page_size, cfg.row), pad_value, np.float32)
    else:
        cache = np.full((B, cfg.max_len, cfg.row), pad_value, np.float32)
    case = Case(cfg, seed, lens, page_table, q_c, q_r, cache, w_uk, w_uv)

    flat = cache.reshape(-1, cfg.row)
    start = 0
    for b in range(B):
        n = int(lens[b])
        idx = case.logical_row_index(b)
        flat[idx, :dc] = c_kv[start:start + n]
        flat[idx, dc:] = k_r[start:start + n]
        start += n
    return case


def draw_latent_query(cfg: WorkloadConfig, seed: int, batch: Optional[int] = None) -> np.ndarray:
    """Seeded stand-in for an absorbed query [B, n_h, d_c + d_h^R], used to
    test the decode step on its own.  The latent part is N(0, d_h / d_c) (the
    variance an absorbed query has when q^C ~ N(0,1) and W^UK ~ N(0, 1/d_c));
    the RoPE part is N(0, 1).  Rounded to bf16 for bf16 configs."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED0001))
    B = cfg.batch if batch is None else batch
    lat = _draw(rng, (B, cfg.n_heads, cfg.d_latent), math.sqrt(cfg.d_head / cfg.d_latent),
                cfg.dtype)
    rope = _draw(rng, (B, cfg.n_heads, cfg.d_rope), 1.0, cfg.dtype)
    return np.concatenate([lat, rope], axis=2)


def draw_latent_output(cfg: WorkloadConfig, seed: int, batch: Optional[int] = None) -> np.ndarray:
    """Seeded stand-in for a latent-space attention output [B, n_h, d_c],
    N(0, 1), used to test the W^UV projection on its own."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED0002))
    B = cfg.batch if batch is None else batch
    return _draw(rng, (B, cfg.n_heads, cfg.d_latent), 1.0, cfg.dtype)


@dataclasses.dataclass
class AppendCase:
    """Inputs of one cache append: the new token's hidden state per request
    and the projections that make its cached row."""
    cfg: WorkloadConfig
    seed: int
    h: np.ndarray           # [B, d_model]
    w_dkv: np.ndarray       # [d_c, d_model]
    w_kr: np.ndarray        # [d_h^R, d_model]
    rms_weight: np.ndarray  # [d_c]
    positions: np.ndarray   # int32 [B], in [0, max_len)


def make_append_case(cfg: WorkloadConfig, seed: int) -> AppendCase:
    """Draw one append case from PCG64(seed ^ 0x5EED0003).

    Draw order: positions, h, W^DKV, W^KR, RMSNorm weight.  h is N(0, 1) (the
    normalised attention input); W^DKV and W^KR are N(0, 1/d); the RMSNorm
    weight is N(1, 0.1^2); positions are uniform in [0, max_len).
    """
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED0003))
    B, d = cfg.batch, cfg.hidden
    positions = rng.integers(0, cfg.max_len, size=B).astype(np.int32)
    h = _draw(rng, (B, d), 1.0, cfg.dtype)
    w_std = 1.0 / math.sqrt(d)
    w_dkv = _draw(rng, (cfg.d_latent, d), w_std, cfg.dtype)
    w_kr = _draw(rng, (cfg.d_rope, d), w_std, cfg.dtype)
    g = rng.standard_normal(cfg.d_latent) * 0.1 + 1.0
    rms_weight = round_to_bf16(g.astype(np.float32)) if cfg.dtype == "bf16" else \
        g.astype(np.float32)
    return AppendCase(cfg, seed, h, w_dkv, w_kr, rms_weight, positions)
