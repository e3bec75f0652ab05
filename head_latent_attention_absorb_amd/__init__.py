"""MI355X-native MLA absorbed decode: thin Python binding over libmla_absorb.so.

Every call marshals torch tensors (device memory and the current HIP stream)
into the C ABI declared in include/mla_absorb.h; all arithmetic happens in the
library's gfx950 kernels.  There is no CPU or PyTorch fallback: if the
library is missing or the device is not a gfx950, calls raise.

Decode step of one layer (DeepSeek-V2 read-through, 2kiu.com/news/6085339,
section 2.3):
    q_cat = absorb_q(q_c, q_r, w_uk)                # [q_lat | q^R]
    o_lat, lse = decode_attn(q_cat, cache, scale)   # latent-space attention
    o = out_uv(o_lat, w_uv)                         # W^UV applied last
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmla_absorb.so")

MLA_F32, MLA_BF16 = 0, 1
MLA_ROWS_NATIVE, MLA_ROWS_FP8 = 0, 1


class Dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("max_len", ctypes.c_int32), ("num_pages", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("row_format", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("split_tokens", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("head_groups", ctypes.c_int32),
                ("q_len", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t),
                ("partitions", ctypes.c_int32)]

    @property
    def balanced(self) -> bool:
        """Partitions sized on the device from the lengths (split_tokens 0)."""
        return self.split_tokens == 0

    @property
    def direct(self) -> bool:
        """One uniform split per request: the decode kernel writes o_lat itself."""
        return self.split_tokens > 0 and self.num_splits == 1 and self.kernel >= 1

    def __repr__(self):
        return (f"Plan(split_tokens={self.split_tokens}, num_splits={self.num_splits}, "
                f"kernel={ {0: 'generic', 1: 'mfma-128rows', 2: 'mfma-64rows'}.get(self.kernel, self.kernel)}, "
                f"head_groups={self.head_groups}, q_len={self.q_len}, "
                f"workspace_bytes={self.workspace_bytes}, partitions={self.partitions})")


class Rope(ctypes.Structure):
    """mla_rope_t: RoPE base and optional YaRN interpolation of the key."""
    _fields_ = [("base", ctypes.c_float), ("yarn_scale", ctypes.c_float),
                ("yarn_alpha", ctypes.c_float), ("yarn_beta", ctypes.c_float),
                ("yarn_original_len", ctypes.c_int32)]


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmla_absorb.so (built by ``head_latent_attention_absorb_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -m head_latent_attention_absorb_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.mla_status_str.restype = ctypes.c_char_p
    L.mla_status_str.argtypes = [ctypes.c_int]
    L.mla_abi_version.restype = i32
    L.mla_absorb_q.restype = ctypes.c_int
    L.mla_absorb_q.argtypes = [ctypes.POINTER(Dims), i32, vp, vp, vp, vp, vp]
    L.mla_decode_plan.restype = ctypes.c_int
    L.mla_decode_plan.argtypes = [ctypes.POINTER(Dims), i32, ctypes.POINTER(CacheDesc), i32,
                                  ctypes.POINTER(Plan)]
    L.mla_decode_plan_mq.restype = ctypes.c_int
    L.mla_decode_plan_mq.argtypes = [ctypes.POINTER(Dims), i32, i32, ctypes.POINTER(CacheDesc),
                                     i32, ctypes.POINTER(Plan)]
    L.mla_decode_workspace_bytes.restype = sz
    L.mla_decode_workspace_bytes.argtypes = [ctypes.POINTER(Dims), i32, i32]
    L.mla_decode_attn.restype = ctypes.c_int
    L.mla_decode_attn.argtypes = [ctypes.POINTER(Dims), i32, vp, ctypes.POINTER(CacheDesc),
                                  ctypes.c_float, ctypes.POINTER(Plan), vp, vp, vp, sz, vp]
    L.mla_decode_attn_noalloc.restype = ctypes.c_int
    L.mla_decode_attn_noalloc.argtypes = [ctypes.POINTER(Dims), i32, vp,
                                          ctypes.POINTER(CacheDesc), ctypes.c_float,
                                          ctypes.POINTER(Plan), vp, vp, vp]
    L.mla_decode_noalloc_max_bytes.restype = sz
    L.mla_decode_noalloc_max_bytes.argtypes = []
    L.mla_decode_partials.restype = ctypes.c_int
    L.mla_decode_partials.argtypes = [ctypes.POINTER(Dims), i32, vp, ctypes.POINTER(CacheDesc),
                                      ctypes.c_float, ctypes.POINTER(Plan), vp, sz, vp]
    L.mla_decode_combine.restype = ctypes.c_int
    L.mla_decode_combine.argtypes = [ctypes.POINTER(Dims), i32, ctypes.POINTER(CacheDesc),
                                     ctypes.POINTER(Plan), vp, sz, vp, vp, vp]
    L.mla_decode_combine_out.restype = ctypes.c_int
    L.mla_decode_combine_out.argtypes = [ctypes.POINTER(Dims), i32, ctypes.POINTER(CacheDesc),
                                         ctypes.POINTER(Plan), vp, sz, vp, vp, vp, vp, vp]
    L.mla_quantize_rows.restype = ctypes.c_int
    L.mla_quantize_rows.argtypes = [ctypes.c_int64, i32, i32, vp, vp, vp, vp]
    L.mla_out_uv.restype = ctypes.c_int
    L.mla_out_uv.argtypes = [ctypes.POINTER(Dims), i32, vp, vp, vp, vp]
    L.mla_cache_append_workspace_bytes.restype = sz
    L.mla_cache_append_workspace_bytes.argtypes = [ctypes.POINTER(Dims), i32, i32]
    L.mla_cache_append.restype = ctypes.c_int
    L.mla_cache_append.argtypes = [ctypes.POINTER(Dims), i32, i32, vp, vp, vp, vp,
                                   ctypes.c_float, ctypes.POINTER(Rope), vp,
                                   ctypes.POINTER(CacheDesc), vp, sz, vp]
    L.mla_prefill_expand.restype = ctypes.c_int
    L.mla_prefill_expand.argtypes = [ctypes.POINTER(Dims), i32, ctypes.POINTER(CacheDesc), vp,
                                     vp, vp, vp, vp]
    L.mla_prefill_attn.restype = ctypes.c_int
    L.mla_prefill_attn.argtypes = [ctypes.POINTER(Dims), i32, i32, vp, vp,
                                   ctypes.POINTER(CacheDesc), vp, vp, ctypes.c_float, vp, vp, vp]
    _lib = L
    return L


def _check(fn: str, status: int):
    if status != 0:
        raise MLAError(fn, status, lib().mla_status_str(status).decode())


_DT = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _require(t: torch.Tensor, name: str, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


@dataclasses.dataclass
class LatentCache:
    """One layer's latent cache on the device.

    data: contiguous [B, max_len, d_latent + d_rope] or paged
          [num_pages, page_size, d_latent + d_rope]
    seq_lens: int32 [B]; page_table: int32 [B, max_len // page_size] or None.
    scales: for a low-bit cache, fp32 [B, max_len] or [num_pages, page_size]
          (one per row) with data holding uint8 E4M3 codes; None otherwise.
    """

    data: torch.Tensor
    seq_lens: torch.Tensor
    d_rope: int
    page_table: Optional[torch.Tensor] = None
    page_size: int = 0
    max_len: int = 0
    scales: Optional[torch.Tensor] = None

    def desc(self) -> CacheDesc:
        d = CacheDesc()
        d.data = self.data.data_ptr()
        d.seq_lens = self.seq_lens.data_ptr()
        d.page_table = self.page_table.data_ptr() if self.page_table is not None else None
        d.page_size = self.page_size if self.page_table is not None else 0
        d.max_len = self.max_len if self.page_table is not None else self.data.shape[1]
        d.num_pages = self.data.shape[0] if self.page_table is not None else 0
        if self.scales is not None:
            d.scales = self.scales.data_ptr()
            d.row_format = MLA_ROWS_FP8
        return d

    def batch(self) -> int:
        return int(self.seq_lens.shape[0])


def make_dims(n_heads: int, d_head: int, d_rope: int, d_latent: int, dtype) -> Dims:
    return Dims(n_heads, d_head, d_rope, d_latent,
                _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype))


def absorb_q(q_c: torch.Tensor, q_r: torch.Tensor, w_uk: torch.Tensor,
             out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q_cat[b,i] = [W^UK_i^T q^C[b,i] | q^R[b,i]]  -> [B, n_h, d_c + d_h^R]."""
    B, nh, dh = q_c.shape
    dr = q_r.shape[2]
    dc = w_uk.shape[2]
    dims = make_dims(nh, dh, dr, dc, _dtype_code(q_c))
    _require(q_r, "q_r", (B, nh, dr), q_c.dtype, q_c.device)
    _require(w_uk, "w_uk", (nh, dh, dc), q_c.dtype, q_c.device)
    _require(q_c, "q_c", (B, nh, dh), q_c.dtype, q_c.device)
    if out is None:
        out = torch.empty((B, nh, dc + dr), dtype=q_c.dtype, device=q_c.device)
    _require(out, "out", (B, nh, dc + dr), q_c.dtype, q_c.device)
    _check("mla_absorb_q", lib().mla_absorb_q(ctypes.byref(dims), B, _ptr(q_c), _ptr(q_r),
                                              _ptr(w_uk), _ptr(out), _stream(stream)))
    return out


def decode_plan(n_heads: int, d_latent: int, d_rope: int, dtype, cache: LatentCache,
                split_tokens: int = 0, d_head: int = 1, q_len: int = 1) -> Plan:
    """Split-KV plan for `cache`; q_len > 1 plans the causal decode of the last
    q_len positions of every request at once (mla_decode_plan_mq).
    split_tokens > 0 asks for a uniform cut of that many tokens per partition;
    0 lets the library choose: on the MFMA kernel usually a length-balanced
    plan (Plan.balanced), whose partitions the decode kernel sizes from the
    device's seq_lens at every call."""
    dims = make_dims(n_heads, d_head, d_rope, d_latent, dtype)
    plan = Plan()
    desc = cache.desc()
    if q_len == 1:
        _check("mla_decode_plan", lib().mla_decode_plan(ctypes.byref(dims), cache.batch(),
                                                        ctypes.byref(desc), split_tokens,
                                                        ctypes.byref(plan)))
    else:
        _check("mla_decode_plan_mq", lib().mla_decode_plan_mq(
            ctypes.byref(dims), cache.batch(), int(q_len), ctypes.byref(desc), split_tokens,
            ctypes.byref(plan)))
    return plan


def _query_shape(q_cat: torch.Tensor, plan: Optional[Plan]):
    """(B, q_len, n_h, row) of a [B, n_h, row] or [B, q_len, n_h, row] query,
    checked against the plan's q_len."""
    if q_cat.dim() == 3:
        B, nh, row = q_cat.shape
        q_len = 1
    elif q_cat.dim() == 4:
        B, q_len, nh, row = q_cat.shape
    else:
        raise ValueError(f"q_cat must be [B, n_h, row] or [B, q_len, n_h, row], got "
                         f"{tuple(q_cat.shape)}")
    if plan is not None and int(plan.q_len) != q_len:
        raise ValueError(f"q_cat holds {q_len} query tokens per request, the plan "
                         f"{int(plan.q_len)}")
    return B, q_len, nh, row


def _lead(B: int, q_len: int, token_axis: bool):
    """Leading output shape: [B] for a [B, n_h, ...] query, [B, q_len] for a
    [B, q_len, n_h, ...] one (a token axis is required when q_len > 1)."""
    if q_len > 1 and not token_axis:
        raise ValueError(f"the plan has {q_len} query tokens: outputs need a token axis")
    return (B, q_len) if token_axis else (B,)


def workspace_for(plan: Plan, device) -> torch.Tensor:
    """A device workspace of plan.workspace_bytes (256-byte aligned)."""
    n = max(int(plan.workspace_bytes), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode_workspace_bytes(n_heads: int, d_latent: int, d_rope: int, dtype, batch: int,
                           max_len: int) -> int:
    """mla_decode_workspace_bytes: workspace bytes of the default plan for
    `batch` requests of at most `max_len` rows (one query token each, a
    contiguous cache of native rows); 0 when the arguments are invalid."""
    dims = make_dims(n_heads, 1, d_rope, d_latent, dtype)
    return int(lib().mla_decode_workspace_bytes(ctypes.byref(dims), batch, max_len))


def decode_attn(q_cat: torch.Tensor, cache: LatentCache, softmax_scale: float,
                plan: Optional[Plan] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None, split_tokens: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Latent-space decode attention; returns (o_lat [B,n_h,d_c], lse [B,n_h] fp32).
    With a [B, q_len, n_h, row] query (and a plan for q_len), the last q_len
    positions of each request attend causally: o_lat [B,q_len,n_h,d_c],
    lse [B,q_len,n_h]."""
    B, q_len, nh, row = _query_shape(q_cat, plan)
    if cache.data.shape[2] != row:
        raise ValueError(f"cache row width {cache.data.shape[2]} != q_cat width {row}")
    d_rope = int(cache.d_rope)
    d_latent = row - d_rope
    dev = q_cat.device
    _require(cache.seq_lens, "seq_lens", (B,), torch.int32, dev)
    if cache.scales is None and cache.data.dtype != q_cat.dtype:
        raise TypeError("cache and q_cat dtypes differ")
    if cache.scales is not None and cache.data.dtype != torch.uint8:
        raise TypeError("a low-bit cache holds uint8 E4M3 codes")
    dims = make_dims(nh, 1, d_rope, d_latent, _dtype_code(q_cat))
    desc = cache.desc()
    if plan is None:
        plan = decode_plan(nh, d_latent, d_rope, q_cat.dtype, cache, split_tokens, q_len=q_len)
    if workspace is None:
        workspace = workspace_for(plan, dev)
    lead = _lead(B, q_len, q_cat.dim() == 4)
    if out is None:
        out = torch.empty(lead + (nh, d_latent), dtype=q_cat.dtype, device=dev)
    if lse is None:
        lse = torch.empty(lead + (nh,), dtype=torch.float32, device=dev)
    _require(out, "out", lead + (nh, d_latent), q_cat.dtype, dev)
    _require(lse, "lse", lead + (nh,), torch.float32, dev)
    _check("mla_decode_attn", lib().mla_decode_attn(
        ctypes.byref(dims), B, _ptr(q_cat), ctypes.byref(desc), float(softmax_scale),
        ctypes.byref(plan), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def decode_attn_noalloc(q_cat: torch.Tensor, cache: LatentCache, softmax_scale: float,
                        plan: Optional[Plan] = None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, stream=None,
                        split_tokens: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode_attn_noalloc: decode_attn with the library's static device
    workspace (no workspace argument; the C call allocates nothing).  Pass
    `out` and `lse` to keep the whole call allocation-free."""
    B, q_len, nh, row = _query_shape(q_cat, plan)
    if cache.data.shape[2] != row:
        raise ValueError(f"cache row width {cache.data.shape[2]} != q_cat width {row}")
    d_rope = int(cache.d_rope)
    d_latent = row - d_rope
    dev = q_cat.device
    _require(cache.seq_lens, "seq_lens", (B,), torch.int32, dev)
    dims = make_dims(nh, 1, d_rope, d_latent, _dtype_code(q_cat))
    desc = cache.desc()
    if plan is None:
        plan = decode_plan(nh, d_latent, d_rope, q_cat.dtype, cache, split_tokens, q_len=q_len)
    lead = _lead(B, q_len, q_cat.dim() == 4)
    if out is None:
        out = torch.empty(lead + (nh, d_latent), dtype=q_cat.dtype, device=dev)
    if lse is None:
        lse = torch.empty(lead + (nh,), dtype=torch.float32, device=dev)
    _require(out, "out", lead + (nh, d_latent), q_cat.dtype, dev)
    _require(lse, "lse", lead + (nh,), torch.float32, dev)
    _check("mla_decode_attn_noalloc", lib().mla_decode_attn_noalloc(
        ctypes.byref(dims), B, _ptr(q_cat), ctypes.byref(desc), float(softmax_scale),
        ctypes.byref(plan), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def decode_partials(q_cat: torch.Tensor, cache: LatentCache, softmax_scale: float,
                    plan: Plan, workspace: torch.Tensor, stream=None) -> None:
    """First phase of decode_attn: per-split partials into `workspace`."""
    B, _, nh, row = _query_shape(q_cat, plan)
    d_rope = int(cache.d_rope)
    dims = make_dims(nh, 1, d_rope, row - d_rope, _dtype_code(q_cat))
    desc = cache.desc()
    _check("mla_decode_partials", lib().mla_decode_partials(
        ctypes.byref(dims), B, _ptr(q_cat), ctypes.byref(desc), float(softmax_scale),
        ctypes.byref(plan), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def decode_combine(cache: LatentCache, n_heads: int, plan: Plan, workspace: torch.Tensor,
                   out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """Second phase of decode_attn: merge the partials into out (and lse);
    out is [B, n_h, d_c], or [B, q_len, n_h, d_c] with a plan for q_len."""
    B = cache.batch()
    d_rope = int(cache.d_rope)
    d_latent = out.shape[-1]
    _require(out, "out", _lead(B, int(plan.q_len), out.dim() == 4) + (n_heads, d_latent),
             out.dtype, out.device)
    dims = make_dims(n_heads, 1, d_rope, d_latent, _dtype_code(out))
    desc = cache.desc()
    _check("mla_decode_combine", lib().mla_decode_combine(
        ctypes.byref(dims), B, ctypes.byref(desc), ctypes.byref(plan), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))


def decode_combine_out(cache: LatentCache, plan: Plan, workspace: torch.Tensor,
                       w_uv: torch.Tensor, out_lat: torch.Tensor,
                       lse: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """decode_combine then out_uv in one call: merges the partials into out_lat
    (and lse) and returns o[b,i,h] = sum_c o_lat[b,i,c] W^UV[i,c,h] (with a
    leading q_len axis after B when the plan has several query tokens)."""
    B = cache.batch()
    nh, dc, dh = w_uv.shape
    d_rope = int(cache.d_rope)
    dims = make_dims(nh, dh, d_rope, dc, _dtype_code(out_lat))
    lead = _lead(B, int(plan.q_len), out_lat.dim() == 4)
    _require(out_lat, "out_lat", lead + (nh, dc), w_uv.dtype, w_uv.device)
    if out is None:
        out = torch.empty(lead + (nh, dh), dtype=w_uv.dtype, device=w_uv.device)
    _require(out, "out", lead + (nh, dh), w_uv.dtype, w_uv.device)
    desc = cache.desc()
    _check("mla_decode_combine_out", lib().mla_decode_combine_out(
        ctypes.byref(dims), B, ctypes.byref(desc), ctypes.byref(plan), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(w_uv), _ptr(out), _ptr(out_lat),
        _ptr(lse), _stream(stream)))
    return out


def out_uv(o_lat: torch.Tensor, w_uv: torch.Tensor, out: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """o[b,i,h] = sum_c o_lat[b,i,c] W^UV[i,c,h] -> [B, n_h, d_h]."""
    B, nh, dc = o_lat.shape
    dh = w_uv.shape[2]
    dims = make_dims(nh, dh, 0, dc, _dtype_code(o_lat))
    _require(w_uv, "w_uv", (nh, dc, dh), o_lat.dtype, o_lat.device)
    if out is None:
        out = torch.empty((B, nh, dh), dtype=o_lat.dtype, device=o_lat.device)
    _require(out, "out", (B, nh, dh), o_lat.dtype, o_lat.device)
    _check("mla_out_uv", lib().mla_out_uv(ctypes.byref(dims), B, _ptr(o_lat), _ptr(w_uv),
                                          _ptr(out), _stream(stream)))
    return out


def latent_cache(data: torch.Tensor, seq_lens: torch.Tensor, d_rope: int,
                 page_table: Optional[torch.Tensor] = None, page_size: int = 0,
                 max_len: Optional[int] = None,
                 scales: Optional[torch.Tensor] = None) -> LatentCache:
    """Describe a contiguous ([B, max_len, row]) or paged ([pages, page_size, row])
    cache; with `scales` (one fp32 per row) `data` is a low-bit cache of uint8
    E4M3 codes (see quantize_rows)."""
    if scales is not None:
        if data.dtype != torch.uint8 or scales.dtype != torch.float32:
            raise TypeError("a low-bit cache is uint8 codes with float32 scales")
        if tuple(scales.shape) != tuple(data.shape[:2]):
            raise ValueError(f"scales: expected shape {tuple(data.shape[:2])}, got "
                             f"{tuple(scales.shape)}")
    if page_table is None:
        return LatentCache(data, seq_lens, int(d_rope), None, 0, int(data.shape[1]), scales)
    ml = int(max_len) if max_len is not None else int(page_table.shape[1]) * page_size
    return LatentCache(data, seq_lens, int(d_rope), page_table, page_size, ml, scales)


def quantize_rows(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                  scales: Optional[torch.Tensor] = None, stream=None):
    """Low-bit cache rows: x [..., width] (fp32 or bf16) -> (uint8 E4M3 codes
    [..., width], fp32 scales [...]) with scale = max|row| / 448 and codes
    E4M3(x / scale) (mla_quantize_rows)."""
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    width = int(x.shape[-1])
    n_rows = x.numel() // width if width > 0 else 0
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _require(out, "out", tuple(x.shape), torch.uint8, x.device)
    _require(scales, "scales", tuple(x.shape[:-1]), torch.float32, x.device)
    _check("mla_quantize_rows", lib().mla_quantize_rows(n_rows, width, _dtype_code(x),
                                                        _ptr(x), _ptr(out), _ptr(scales),
                                                        _stream(stream)))
    return out, scales


def cache_append(cache: LatentCache, h: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor,
                 rms_weight: torch.Tensor, positions: torch.Tensor, rms_eps: float = 1e-6,
                 rope_base: float = 10000.0, yarn_scale: float = 1.0, yarn_alpha: float = 1.0,
                 yarn_beta: float = 32.0, yarn_original_len: int = 4096,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Write row positions[b] of request b of `cache`:
    [RMSNorm(W^DKV h[b]) | RoPE(W^KR h[b], positions[b])] (see mla_cache_append)."""
    B, d_model = h.shape
    d_c = w_dkv.shape[0]
    d_r = w_kr.shape[0]
    dev = h.device
    _require(w_dkv, "w_dkv", (d_c, d_model), h.dtype, dev)
    _require(w_kr, "w_kr", (d_r, d_model), h.dtype, dev)
    _require(rms_weight, "rms_weight", (d_c,), h.dtype, dev)
    _require(positions, "positions", (B,), torch.int32, dev)
    _require(h, "h", (B, d_model), h.dtype, dev)
    if cache.data.shape[2] != d_c + d_r or (
            cache.data.dtype != (torch.uint8 if cache.scales is not None else h.dtype)):
        raise ValueError("cache row must be [d_latent + d_rope] of h's dtype "
                         "(or of E4M3 codes for a low-bit cache)")
    dims = make_dims(1, 1, d_r, d_c, _dtype_code(h))
    need = int(lib().mla_cache_append_workspace_bytes(ctypes.byref(dims), B, d_model))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    rope = Rope(float(rope_base), float(yarn_scale), float(yarn_alpha), float(yarn_beta),
                int(yarn_original_len))
    desc = cache.desc()
    _check("mla_cache_append", lib().mla_cache_append(
        ctypes.byref(dims), B, d_model, _ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(rms_weight),
        float(rms_eps), ctypes.byref(rope), _ptr(positions), ctypes.byref(desc),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


# ----------------------------------------------------------------------------
# A chunk of new tokens in the unabsorbed form
# ----------------------------------------------------------------------------

def prefill_expand(cache: LatentCache, w_uk: torch.Tensor, w_uv: torch.Tensor,
                   k_c: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                   stream=None):
    """Explicit keys and values of every cached row (rows past each request's
    length are left as they are): k_c[b,i,t] = W^UK_i c_t, v[b,i,t] = c_t W^UV_i,
    both [B, n_h, max_len, d_h] bf16.  Contiguous native bf16 cache only."""
    nh, dh, dc = w_uk.shape
    B, max_len = cache.batch(), cache.data.shape[1]
    dims = make_dims(nh, dh, cache.d_rope, dc, w_uk.dtype)
    dev = w_uk.device
    _require(w_uv, "w_uv", (nh, dc, dh), w_uk.dtype, dev)
    shape = (B, nh, max_len, dh)
    if k_c is None:
        k_c = torch.empty(shape, dtype=w_uk.dtype, device=dev)
    if v is None:
        v = torch.empty(shape, dtype=w_uk.dtype, device=dev)
    _require(k_c, "k_c", shape, w_uk.dtype, dev)
    _require(v, "v", shape, w_uk.dtype, dev)
    desc = cache.desc()
    _check("mla_prefill_expand", lib().mla_prefill_expand(
        ctypes.byref(dims), B, ctypes.byref(desc), _ptr(w_uk), _ptr(w_uv), _ptr(k_c), _ptr(v),
        _stream(stream)))
    return k_c, v


def prefill_attn(q_c: torch.Tensor, q_r: torch.Tensor, cache: LatentCache, k_c: torch.Tensor,
                 v: torch.Tensor, softmax_scale: float, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, stream=None):
    """Causal attention of the last q_len positions of each request over the
    explicit keys [k_c ; k^R] and values: q_c [B, q_len, n_h, d_h], q_r [B, q_len,
    n_h, d_h^R] -> (out [B, q_len, n_h, d_h], lse [B, q_len, n_h])."""
    B, q_len, nh, dh = q_c.shape
    dr = q_r.shape[3]
    dc = cache.data.shape[2] - dr
    dims = make_dims(nh, dh, dr, dc, q_c.dtype)
    dev = q_c.device
    _require(q_r, "q_r", (B, q_len, nh, dr), q_c.dtype, dev)
    max_len = cache.data.shape[1]
    _require(k_c, "k_c", (B, nh, max_len, dh), q_c.dtype, dev)
    _require(v, "v", (B, nh, max_len, dh), q_c.dtype, dev)
    if out is None:
        out = torch.empty((B, q_len, nh, dh), dtype=q_c.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, q_len, nh), dtype=torch.float32, device=dev)
    _require(out, "out", (B, q_len, nh, dh), q_c.dtype, dev)
    _require(lse, "lse", (B, q_len, nh), torch.float32, dev)
    desc = cache.desc()
    _check("mla_prefill_attn", lib().mla_prefill_attn(
        ctypes.byref(dims), B, q_len, _ptr(q_c), _ptr(q_r), ctypes.byref(desc), _ptr(k_c),
        _ptr(v), ctypes.c_float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse
