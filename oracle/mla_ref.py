"""Plain, slow, fp64 reference for MLA decode -- TEST INFRASTRUCTURE ONLY.

Nothing here is blocked, fused or reordered beyond what the definitions say.
Library primitives used as single steps: numpy matmul / einsum, exp, log.

Notation (from the zeeklog notes, equations 9-11, and the V2 read-through,
sections 2.3-2.4):
  n_h heads, d_h content width per head, d_h^R RoPE width, d_c latent width.
  Cached per token j: c_j = c^KV_j in R^{d_c} and k^R_j in R^{d_h^R}, stored as
  one row [c_j | k^R_j].
  W^UK[i] is head i's d_h x d_c up-projection block (k^C_{j,i} = W^UK[i] c_j);
  W^UV[i] is stored as d_c x d_h so that v_{j,i}[h] = sum_c W^UV[i,c,h] c_j[c].
  (The pages give both up-projections as (n_h d_h) x d_c matrices, V3
  read-through section 2.2; storing W^UV transposed is this library's layout
  reading, not something the pages state.)
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# Cache accounting
# ----------------------------------------------------------------------------

def cache_elems_per_token_mha(n_heads: int, d_head: int) -> int:
    """Elements cached per token per layer by standard MHA: one k and one v per
    head, 2 n_h d_h (zeeklog, MHA paragraph after the attention equation;
    V2 read-through section 2.1)."""
    return 2 * n_heads * d_head


def cache_elems_per_token_mla(d_latent: int, d_rope: int) -> int:
    """Elements cached per token per layer by MLA: the latent plus the shared
    RoPE key, d_c + d_h^R (zeeklog cache table; ai-library "Multi-Head Latent
    Attention")."""
    return d_latent + d_rope


def kv_cache_bytes(seq_len: int, n_layers: int, per_token_per_layer: int,
                   dtype_bytes: int = 2) -> int:
    """Bytes of KV cache held by one request: tokens x layers x elements per
    token per layer x bytes per element (V2 read-through section 2.1, the
    per-request cache estimate)."""
    return seq_len * n_layers * per_token_per_layer * dtype_bytes


# ----------------------------------------------------------------------------
# Cache access
# ----------------------------------------------------------------------------

def gather_rows(cache: np.ndarray, b: int, seq_len: int,
                page_table: Optional[np.ndarray] = None,
                page_size: int = 0) -> np.ndarray:
    """Return request b's cached rows 0..seq_len-1 as float64 [seq_len, row].

    Contiguous cache: ``cache[b, t]``.  Paged cache: logical token t lives in
    physical page ``page_table[b, t // page_size]`` at slot ``t % page_size``.
    Paging is a storage layout of this library; the pages do not discuss it.
    """
    if page_table is None:
        rows = cache[b, :seq_len]
    else:
        t = np.arange(seq_len)
        rows = cache[page_table[b, t // page_size], t % page_size]
    return np.asarray(rows, dtype=np.float64)


# ----------------------------------------------------------------------------
# Primary (unabsorbed) form
# ----------------------------------------------------------------------------

def up_project(latent: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray
               ) -> Tuple[np.ndarray, np.ndarray]:
    """Explicit up-projection of cached latents (zeeklog equations 10-11; the
    latent KV module in the V2 read-through section 2.2).

    latent [T, d_c], w_uk [n_h, d_h, d_c], w_uv [n_h, d_c, d_h]
    returns k_c [n_h, T, d_h] with k_c[i, j] = W^UK[i] @ c_j,
            v   [n_h, T, d_h] with v[i, j, h] = sum_c W^UV[i, c, h] c_j[c].
    """
    latent = np.asarray(latent, np.float64)
    # k_c[i] = latent @ W^UK[i]^T  ([T, d_c] x [d_c, d_h]);  v[i] = latent @ W^UV[i]
    k_c = np.matmul(latent[None], np.transpose(np.asarray(w_uk, np.float64), (0, 2, 1)))
    v = np.matmul(latent[None], np.asarray(w_uv, np.float64))
    return k_c, v


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Textbook single-query attention per head (zeeklog, the MHA equation
    o_{t,i} = sum_j softmax_j(q_{t,i}^T k_{j,i} * scale) v_{j,i}).

    q [n_h, d_q], k [n_h, T, d_q], v [n_h, T, d_v] -> (o [n_h, d_v], lse [n_h]).
    The softmax subtracts the per-head maximum before exponentiating (a
    numerical device; the result is the same real number).  lse is the natural
    log of sum_j exp(s_j).  T = 0 gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n_h, T = k.shape[0], k.shape[1]
    if T == 0:
        return np.zeros((n_h, v.shape[2])), np.full(n_h, -np.inf)
    s = scale * np.matmul(k, q[:, :, None])[:, :, 0]        # s[i, j] = scale * q_i . k_{i,j}
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    o = np.matmul(p[:, None, :], v)[:, 0, :]                 # o_i = sum_j p[i, j] v_{i,j}
    lse = (m + np.log(z))[:, 0]
    return o, lse


def mla_decode_reference(q_c: np.ndarray, q_r: np.ndarray, cache: np.ndarray,
                         seq_lens: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
                         scale: float, page_table: Optional[np.ndarray] = None,
                         page_size: int = 0, requests=None, heads=None
                         ) -> Tuple[np.ndarray, np.ndarray]:
    """MLA decode, unabsorbed: the parity reference.

    For each request b and head i, with the request's cached rows
    [c_j | k^R_j], j < len_b (the current token is already appended; the
    query attends positions 1..t, zeeklog, decode paragraphs):
      1. k^C_{j,i} = W^UK[i] c_j and v_{j,i} = W^UV[i]-contract c_j  (eq. 10-11)
      2. q = [q^C_{b,i}; q^R_{b,i}], k_j = [k^C_{j,i}; k^R_j]; k^R is the same
         for every head (ai-library "Multi-Head Latent Attention";
         V3 read-through section 2.3, k = [k_c; k_r])
      3. o_{b,i} = softmax attention with the given scale.
    The scale is a parameter: the pages state 1/sqrt(d_h) only for MHA and
    omit MLA's equations 14-19 (zeeklog); callers pass 1/sqrt(d_h + d_h^R).

    q_c [B, n_h, d_h], q_r [B, n_h, d_h^R], w_uk [n_h, d_h, d_c],
    w_uv [n_h, d_c, d_h]; cache as in ``gather_rows``.
    ``requests`` / ``heads`` restrict the work to a subset (others stay 0).
    Returns (o [B, n_h, d_h], lse [B, n_h]) in float64.
    """
    B, n_h, d_h = q_c.shape
    d_c = w_uk.shape[2]
    o = np.zeros((B, n_h, w_uv.shape[2]))
    lse = np.full((B, n_h), -np.inf)
    req = range(B) if requests is None else requests
    hs = np.arange(n_h) if heads is None else np.asarray(heads)
    w_uk_h = np.asarray(w_uk, np.float64)[hs]
    w_uv_h = np.asarray(w_uv, np.float64)[hs]
    for b in req:
        rows = gather_rows(cache, b, int(seq_lens[b]), page_table, page_size)
        latent, k_rope = rows[:, :d_c], rows[:, d_c:]
        k_c, v = up_project(latent, w_uk_h, w_uv_h)
        T = rows.shape[0]
        k = np.concatenate([k_c, np.broadcast_to(k_rope, (len(hs), T, k_rope.shape[1]))],
                           axis=2)
        q = np.concatenate([np.asarray(q_c[b, hs], np.float64),
                            np.asarray(q_r[b, hs], np.float64)], axis=1)
        o_b, lse_b = softmax_attention(q, k, v, scale)
        o[b, hs] = o_b
        lse[b, hs] = lse_b
    return o, lse


# ----------------------------------------------------------------------------
# Secondary (absorbed) form -- the method, step by step
# ----------------------------------------------------------------------------

def absorb_query(q_c: np.ndarray, q_r: np.ndarray, w_uk: np.ndarray,
                 dtype=np.float64) -> np.ndarray:
    """Absorb W^UK into the query: q_lat,i = W^UK[i]^T q^C_i, so that
    q^C_i . (W^UK[i] c) = q_lat,i . c (V2 read-through section 2.3;
    V3 read-through section 2.3).  Returns q_cat = [q_lat | q^R]
    [B, n_h, d_c + d_h^R], mirroring the cached row [c | k^R].
    ``dtype`` is the arithmetic type (float64, the parity reference, unless a
    caller times the method in float32)."""
    q_lat = np.einsum("bih,ihc->bic", np.asarray(q_c, dtype), np.asarray(w_uk, dtype))
    return np.concatenate([q_lat, np.asarray(q_r, dtype)], axis=2)


def latent_attention(q_cat: np.ndarray, rows: np.ndarray, d_latent: int, scale: float,
                     dtype=np.float64) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of one request against its cached rows in latent space.

    q_cat [n_h, d_c + d_h^R], rows [T, d_c + d_h^R].
    s_{i,j} = scale * q_cat_i . row_j (the 576-wide dot product covers both the
    absorbed content part and the RoPE part), p = softmax_j, and the weighted
    sum stays in latent space: o_lat_i = sum_j p_{i,j} c_j (V2 read-through
    section 2.3: the weighted sum is done on the latent, projected back last).
    Returns (o_lat [n_h, d_c], lse [n_h]); T = 0 gives zeros and -inf.
    ``dtype`` is the arithmetic type (float64 unless a caller times float32).
    """
    q_cat = np.asarray(q_cat, dtype)
    rows = np.asarray(rows, dtype)
    n_h = q_cat.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((n_h, d_latent)), np.full(n_h, -np.inf)
    s = scale * (q_cat @ rows.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    o_lat = (e / z) @ rows[:, :d_latent]
    return o_lat, (m + np.log(z))[:, 0]


def latent_attention_causal(q_cat: np.ndarray, rows: np.ndarray, d_latent: int,
                            scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Several new tokens of one request decoded at once, each attending
    causally (speculative-decoding verification: the extra prediction depths
    propose q_len - 1 further tokens and the main model checks all of them in
    one pass; V3 read-through, section 4.1, and the causal attention over
    positions 1..t of the zeeklog MHA equation).

    q_cat [q_len, n_h, d_c + d_h^R]: the queries of the request's last q_len
    positions, whose rows are already among `rows` [T, d_c + d_h^R].  New token
    j sits at position T - q_len + j and attends to rows 0 .. T - q_len + j,
    i.e. latent_attention over the first T - q_len + j + 1 rows (none when
    that count is <= 0).  Returns (o_lat [q_len, n_h, d_c], lse [q_len, n_h]).
    """
    q_cat = np.asarray(q_cat, np.float64)
    q_len, n_h = q_cat.shape[:2]
    T = np.asarray(rows).shape[0]
    o_lat = np.zeros((q_len, n_h, d_latent))
    lse = np.full((q_len, n_h), -np.inf)
    for j in range(q_len):
        visible = T - q_len + j + 1
        o_lat[j], lse[j] = latent_attention(q_cat[j], np.asarray(rows)[:max(visible, 0)],
                                            d_latent, scale)
    return o_lat, lse


def mla_prefill_reference(q_c: np.ndarray, q_r: np.ndarray, latent: np.ndarray,
                          k_rope: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
                          scale: float, heads=None) -> Tuple[np.ndarray, np.ndarray]:
    """A chunk of new tokens of one request in the primary (unabsorbed) form:
    the cached latents are up-projected to per-head keys and values (zeeklog
    equations 10-11), each key gets the shared k^R (ai-library "Multi-Head
    Latent Attention"; V3 read-through section 2.3, k = [k_c; k_r]), and each
    new token attends causally with the textbook softmax (zeeklog MHA
    equation, positions 1..t).  The V2 read-through (section 2.3) notes that
    the absorbed form is the one that pays off at decode; for a long chunk of
    queries the explicit keys and values are computed once and shared.

    latent [T, d_c], k_rope [T, d_h^R]: the request's cached rows, the chunk's
    own rows included.  q_c [q_len, n_h, d_h], q_r [q_len, n_h, d_h^R]: token
    j sits at position T - q_len + j and sees rows 0 .. T - q_len + j.
    ``heads`` restricts the work to a subset (others stay 0 / -inf).
    Returns (o [q_len, n_h, d_h], lse [q_len, n_h]) in float64.
    """
    q_c = np.asarray(q_c, np.float64)
    q_r = np.asarray(q_r, np.float64)
    q_len, n_h = q_c.shape[:2]
    hs = np.arange(n_h) if heads is None else np.asarray(heads)
    T = np.asarray(latent).shape[0]
    k_c, v = up_project(latent, np.asarray(w_uk)[hs], np.asarray(w_uv)[hs])
    k = np.concatenate([k_c, np.broadcast_to(np.asarray(k_rope, np.float64),
                                             (len(hs), T, np.asarray(k_rope).shape[1]))],
                       axis=2)
    o = np.zeros((q_len, n_h, v.shape[2]))
    lse = np.full((q_len, n_h), -np.inf)
    for j in range(q_len):
        visible = max(T - q_len + j + 1, 0)
        q = np.concatenate([q_c[j, hs], q_r[j, hs]], axis=1)
        o[j, hs], lse[j, hs] = softmax_attention(q, k[:, :visible], v[:, :visible], scale)
    return o, lse


def project_out(o_lat: np.ndarray, w_uv: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Apply W^UV after the latent-space sum: o_i[h] = sum_c W^UV[i,c,h] o_lat_i[c]
    (V2 read-through section 2.3; zeeklog equation 11 moved past the sum).
    o_lat [B, n_h, d_c] -> o [B, n_h, d_h], computed in ``dtype``."""
    return np.einsum("bic,ich->bih", np.asarray(o_lat, dtype), np.asarray(w_uv, dtype))


def mla_decode_absorbed(q_c, q_r, cache, seq_lens, w_uk, w_uv, scale,
                        page_table=None, page_size=0, requests=None, dtype=np.float64):
    """MLA decode in absorbed form: absorb_query -> latent_attention per request
    -> project_out.  Returns (o [B,n_h,d_h], o_lat [B,n_h,d_c], lse [B,n_h],
    q_cat [B,n_h,d_c+d_h^R]), computed in ``dtype`` (float64 by default)."""
    d_c = w_uk.shape[2]
    q_cat = absorb_query(q_c, q_r, w_uk, dtype)
    B, n_h = q_cat.shape[:2]
    o_lat = np.zeros((B, n_h, d_c), dtype)
    lse = np.full((B, n_h), -np.inf, dtype)
    for b in (range(B) if requests is None else requests):
        rows = gather_rows(cache, b, int(seq_lens[b]), page_table, page_size)
        o_lat[b], lse[b] = latent_attention(q_cat[b], rows, d_c, scale, dtype)
    return project_out(o_lat, w_uv, dtype), o_lat, lse, q_cat


def default_scale(d_head: int, d_rope: int) -> float:
    """1/sqrt(d_h + d_h^R): the MHA rule 1/sqrt(dot-product length) (zeeklog MHA
    equation) applied to MLA's concatenated query/key width."""
    return 1.0 / math.sqrt(d_head + d_rope)
