"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin is written as a function so that ``test_planted_mistakes`` can run
the whole set against deliberately broken copies of the oracle and show that
every planted mistake is caught by at least one pin.

Sources are cited by page title and section (see oracle/__init__.py).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.mla_ref as ref
from workload import CONFIGS, make_case

HERE = os.path.dirname(os.path.abspath(__file__))
TINY = CONFIGS["tiny_f32"]


def _rand_problem(seed, B=2, n_h=3, d_h=4, d_r=2, d_c=5, lens=(6, 3)):
    rng = np.random.default_rng(seed)
    q_c = rng.standard_normal((B, n_h, d_h))
    q_r = rng.standard_normal((B, n_h, d_r))
    T = max(lens)
    cache = rng.standard_normal((B, T, d_c + d_r))
    w_uk = rng.standard_normal((n_h, d_h, d_c)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((n_h, d_c, d_h)) / math.sqrt(d_c)
    return q_c, q_r, cache, np.array(lens, np.int32), w_uk, w_uv


def _relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ----------------------------------------------------------------------------
# Pin functions (each raises AssertionError when the oracle is wrong)
# ----------------------------------------------------------------------------

def brute_force_decode(q_c, q_r, cache, lens, w_uk, w_uv, scale):
    """Scalar loops straight from the definitions: k^C = W^UK c, v = W^UV c
    (zeeklog eq. 10-11), score over [q^C; q^R] . [k^C; k^R] (ai-library
    'Multi-Head Latent Attention'), softmax over positions 1..t, weighted sum
    of v (zeeklog MHA equation).  No max subtraction: inputs are tiny."""
    B, n_h, d_h = q_c.shape
    d_c = w_uk.shape[2]
    d_r = q_r.shape[2]
    out = np.zeros((B, n_h, d_h))
    for b in range(B):
        T = int(lens[b])
        for i in range(n_h):
            scores = []
            for j in range(T):
                s = 0.0
                for h in range(d_h):
                    kc = 0.0
                    for c in range(d_c):
                        kc += w_uk[i][h][c] * cache[b][j][c]
                    s += q_c[b][i][h] * kc
                for r in range(d_r):
                    s += q_r[b][i][r] * cache[b][j][d_c + r]
                scores.append(scale * s)
            w = [math.exp(x) for x in scores]
            z = sum(w)
            for h in range(d_h):
                acc = 0.0
                for j in range(T):
                    v = 0.0
                    for c in range(d_c):
                        v += w_uv[i][c][h] * cache[b][j][c]
                    acc += (w[j] / z) * v
                out[b][i][h] = acc
    return out


def pin_brute_force(seed=0):
    q_c, q_r, cache, lens, w_uk, w_uv = _rand_problem(seed)
    scale = 0.37
    o, _ = ref.mla_decode_reference(q_c, q_r, cache, lens, w_uk, w_uv, scale)
    o_bf = brute_force_decode(q_c, q_r, cache, lens, w_uk, w_uv, scale)
    assert _relerr(o, o_bf) < 1e-12


def pin_sdpa(seed=1):
    """MHA special case: with K = [W^UK c; k^R] and V = W^UV c built explicitly,
    torch's scaled_dot_product_attention (fp64, CPU, explicit scale) is an
    independent implementation of the softmax attention step."""
    q_c, q_r, cache, lens, w_uk, w_uv = _rand_problem(seed, lens=(7, 7))
    scale = 0.29
    d_c = w_uk.shape[2]
    o, _ = ref.mla_decode_reference(q_c, q_r, cache, lens, w_uk, w_uv, scale)
    c = torch.from_numpy(cache[:, :, :d_c])                       # [B, T, d_c]
    kr = torch.from_numpy(cache[:, :, d_c:])                      # [B, T, d_r]
    wk = torch.from_numpy(w_uk)                                   # [n_h, d_h, d_c]
    wv = torch.from_numpy(w_uv)                                   # [n_h, d_c, d_h]
    k_c = torch.matmul(c[:, None], wk.transpose(1, 2).contiguous()[None])   # [B, n_h, T, d_h]
    v = torch.matmul(c[:, None], wv[None])                                  # [B, n_h, T, d_h]
    n_h = w_uk.shape[0]
    k = torch.cat([k_c, kr[:, None].expand(-1, n_h, -1, -1)], dim=-1)
    q = torch.cat([torch.from_numpy(q_c), torch.from_numpy(q_r)], dim=-1)[:, :, None]
    o_t = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[:, :, 0]
    assert _relerr(o, o_t.numpy()) < 1e-12


def pin_selection_up_projection():
    """With 0/1 selection matrices the up-projection has an exact closed form:
    W^UK[i, h, c] = [c == a_i(h)] gives k^C_{j,i}[h] = c_j[a_i(h)], and
    W^UV[i, c, h] = [c == b_i(h)] gives v_{j,i}[h] = c_j[b_i(h)].  d_h = d_c and
    non-involutive permutations make a transposed operand visible."""
    rng = np.random.default_rng(5)
    n_h, d_c, T = 3, 6, 4
    latent = rng.standard_normal((T, d_c))
    a = np.array([np.roll(np.arange(d_c), i + 1) for i in range(n_h)])
    bsel = np.array([np.roll(np.arange(d_c), -(i + 2)) for i in range(n_h)])
    w_uk = np.zeros((n_h, d_c, d_c))
    w_uv = np.zeros((n_h, d_c, d_c))
    for i in range(n_h):
        for h in range(d_c):
            w_uk[i, h, a[i, h]] = 1.0
            w_uv[i, bsel[i, h], h] = 1.0
    k_c, v = ref.up_project(latent, w_uk, w_uv)
    for i in range(n_h):
        assert np.array_equal(k_c[i], latent[:, a[i]])
        assert np.array_equal(v[i], latent[:, bsel[i]])


def pin_absorbed_equals_unabsorbed(seed):
    """V2 read-through section 6, second step: the absorbed and unabsorbed
    paths must agree to rounding error; a large gap means a wrong product
    order or head split."""
    case = make_case(TINY, seed)
    args = (case.q_c, case.q_r, case.cache, case.seq_lens, case.w_uk, case.w_uv, TINY.scale)
    o_ref, lse_ref = ref.mla_decode_reference(*args)
    o_abs, _, lse_abs, _ = ref.mla_decode_absorbed(*args)
    assert _relerr(o_abs, o_ref) < 1e-12
    assert _relerr(lse_abs, lse_ref) < 1e-12


def pin_single_token():
    """T = 1: the softmax weight is exactly 1, so o_i = W^UV[i]-contract c_0;
    with a selection W^UV, o_i[h] = c_0[b_i(h)] and lse = s_0."""
    rng = np.random.default_rng(11)
    n_h, d_h, d_r, d_c = 2, 3, 2, 5
    q_c = rng.standard_normal((1, n_h, d_h))
    q_r = rng.standard_normal((1, n_h, d_r))
    cache = rng.standard_normal((1, 1, d_c + d_r))
    w_uk = rng.standard_normal((n_h, d_h, d_c))
    w_uv = np.zeros((n_h, d_c, d_h))
    sel = [[4, 0, 2], [1, 3, 0]]
    for i in range(n_h):
        for h in range(d_h):
            w_uv[i, sel[i][h], h] = 1.0
    o, lse = ref.mla_decode_reference(q_c, q_r, cache, np.array([1]), w_uk, w_uv, 0.5)
    for i in range(n_h):
        assert np.allclose(o[0, i], cache[0, 0, sel[i]], rtol=1e-14, atol=1e-14)
        s0 = 0.5 * (q_c[0, i] @ (w_uk[i] @ cache[0, 0, :d_c]) + q_r[0, i] @ cache[0, 0, d_c:])
        assert abs(lse[0, i] - s0) < 1e-12


def pin_zero_scale_mean():
    """Scale 0 makes every score 0: the softmax is uniform, o is W^UV applied
    to the mean latent and lse = log T (closed form)."""
    q_c, q_r, cache, lens, w_uk, w_uv = _rand_problem(3, lens=(5, 2))
    o, lse = ref.mla_decode_reference(q_c, q_r, cache, lens, w_uk, w_uv, 0.0)
    d_c = w_uk.shape[2]
    for b in range(2):
        mean_c = cache[b, :lens[b], :d_c].mean(axis=0)
        for i in range(w_uk.shape[0]):
            expect = np.array([sum(w_uv[i, c, h] * mean_c[c] for c in range(d_c))
                               for h in range(w_uv.shape[2])])
            assert np.allclose(o[b, i], expect, rtol=1e-12, atol=1e-13)
        assert np.allclose(lse[b], math.log(lens[b]), rtol=0, atol=1e-12)


def pin_equal_rows():
    """All cached rows equal: o is W^UV-contract c whatever the query, and
    lse = s + log T."""
    rng = np.random.default_rng(4)
    q_c, q_r, _, _, w_uk, w_uv = _rand_problem(4, lens=(6, 6))
    row = rng.standard_normal(w_uk.shape[2] + q_r.shape[2])
    cache = np.broadcast_to(row, (2, 6, row.size)).copy()
    o, lse = ref.mla_decode_reference(q_c, q_r, cache, np.array([6, 6]), w_uk, w_uv, 0.8)
    o1, lse1 = ref.mla_decode_reference(q_c, q_r, cache[:, :1], np.array([1, 1]), w_uk,
                                        w_uv, 0.8)
    assert _relerr(o, o1) < 1e-13
    assert np.allclose(lse, lse1 + math.log(6), atol=1e-12)


def pin_rope_query_zero():
    """q^R = 0 removes the position path: the result must not depend on k^R
    (kernel-level form of the 'zero the position path' check, V2 read-through
    section 5.2)."""
    q_c, q_r, cache, lens, w_uk, w_uv = _rand_problem(6)
    d_c = w_uk.shape[2]
    q_r0 = np.zeros_like(q_r)
    o1, _ = ref.mla_decode_reference(q_c, q_r0, cache, lens, w_uk, w_uv, 0.6)
    cache2 = cache.copy()
    cache2[:, :, d_c:] = np.random.default_rng(9).standard_normal(cache2[:, :, d_c:].shape) * 5
    o2, _ = ref.mla_decode_reference(q_c, q_r0, cache2, lens, w_uk, w_uv, 0.6)
    assert _relerr(o1, o2) < 1e-13
    # ... and with q^R != 0 it must depend on k^R.
    o3, _ = ref.mla_decode_reference(q_c, q_r, cache, lens, w_uk, w_uv, 0.6)
    o4, _ = ref.mla_decode_reference(q_c, q_r, cache2, lens, w_uk, w_uv, 0.6)
    assert _relerr(o3, o4) > 1e-3


def pin_shared_rope_shift():
    """k^R is shared by every head: adding one vector delta to every cached k^R
    shifts all of head i's scores by scale * q^R_i . delta, which leaves o
    unchanged and moves lse by exactly that amount."""
    q_c, q_r, cache, lens, w_uk, w_uv = _rand_problem(7)
    d_c = w_uk.shape[2]
    delta = np.array([0.7, -1.3])
    cache2 = cache.copy()
    cache2[:, :, d_c:] += delta
    o1, l1 = ref.mla_decode_reference(q_c, q_r, cache, lens, w_uk, w_uv, 0.45)
    o2, l2 = ref.mla_decode_reference(q_c, q_r, cache2, lens, w_uk, w_uv, 0.45)
    assert _relerr(o1, o2) < 1e-12
    assert np.allclose(l2 - l1, 0.45 * (q_r @ delta), atol=1e-12)


def pin_planted_needle():
    """A row aligned with head i's absorbed query and scaled up takes all the
    softmax mass, so o_i -> W^UV[i] c_p (synthetic stand-in for the
    long-distance retrieval sweep, V2 read-through section 6, third step)."""
    rng = np.random.default_rng(8)
    n_h, d_h, d_r, d_c, T = 2, 4, 2, 6, 40
    q_c = rng.standard_normal((1, n_h, d_h))
    q_r = np.zeros((1, n_h, d_r))
    w_uk = rng.standard_normal((n_h, d_h, d_c))
    w_uv = rng.standard_normal((n_h, d_c, d_h))
    for depth in (0, T // 2, T - 1):
        cache = rng.standard_normal((1, T, d_c + d_r)) * 0.1
        head = 1
        u = w_uk[head].T @ q_c[0, head]
        cache[0, depth, :d_c] = 40.0 * u / np.linalg.norm(u)
        o, _ = ref.mla_decode_reference(q_c, q_r, cache, np.array([T]), w_uk, w_uv, 1.0)
        expect = w_uv[head].T @ cache[0, depth, :d_c]
        assert _relerr(o[0, head], expect) < 1e-6


def pin_paged_gather():
    """A paged cache holding the same logical rows gives the identical result
    (page table resolution in gather_rows)."""
    q_c, q_r, cache, lens, w_uk, w_uv = _rand_problem(10, lens=(7, 5))
    ps = 2
    max_pages = 4
    perm = np.random.default_rng(3).permutation(2 * max_pages).reshape(2, max_pages)
    pool = np.full((2 * max_pages, ps, cache.shape[2]), np.nan)
    for b in range(2):
        for t in range(int(lens[b])):
            pool[perm[b, t // ps], t % ps] = cache[b, t]
    o1, l1 = ref.mla_decode_reference(q_c, q_r, cache, lens, w_uk, w_uv, 0.5)
    o2, l2 = ref.mla_decode_reference(q_c, q_r, pool, lens, w_uk, w_uv, 0.5, perm, ps)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_large_scores_finite():
    """Scores of order 1e3 must not overflow (softmax subtracts the max)."""
    q_c, q_r, cache, lens, w_uk, w_uv = _rand_problem(12)
    o, lse = ref.mla_decode_reference(q_c * 300, q_r * 300, cache, lens, w_uk, w_uv, 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


ALL_PINS = [
    ("brute_force", pin_brute_force),
    ("sdpa", pin_sdpa),
    ("selection_up_projection", pin_selection_up_projection),
    ("absorbed_equals_unabsorbed", lambda: pin_absorbed_equals_unabsorbed(0)),
    ("single_token", pin_single_token),
    ("zero_scale_mean", pin_zero_scale_mean),
    ("equal_rows", pin_equal_rows),
    ("rope_query_zero", pin_rope_query_zero),
    ("shared_rope_shift", pin_shared_rope_shift),
    ("planted_needle", pin_planted_needle),
    ("paged_gather", pin_paged_gather),
    ("large_scores_finite", pin_large_scores_finite),
]


# ----------------------------------------------------------------------------
# Tests
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_pin(name, fn):
    fn()


@pytest.mark.parametrize("seed", range(10))
def test_absorbed_equals_unabsorbed_tiny(seed):
    pin_absorbed_equals_unabsorbed(seed)


def test_brute_force_several_seeds():
    for s in range(3):
        pin_brute_force(s)


def test_latent_form_is_unabsorbed_with_identity_weights():
    """With d_h = d_c and W^UK[i] = W^UV[i] = I, the unabsorbed reference is
    exactly the latent-space attention (q^C plays q_lat, v = c), which pins the
    secondary latent_attention used for intermediate parity."""
    rng = np.random.default_rng(21)
    n_h, d_c, d_r, T = 3, 8, 4, 9
    q_lat = rng.standard_normal((1, n_h, d_c))
    q_r = rng.standard_normal((1, n_h, d_r))
    cache = rng.standard_normal((1, T, d_c + d_r))
    eye = np.broadcast_to(np.eye(d_c), (n_h, d_c, d_c)).copy()
    o, lse = ref.mla_decode_reference(q_lat, q_r, cache, np.array([T]), eye, eye, 0.3)
    q_cat = np.concatenate([q_lat[0], q_r[0]], axis=1)
    o_lat, lse2 = ref.latent_attention(q_cat, cache[0], d_c, 0.3)
    assert _relerr(o_lat, o[0]) < 1e-13
    assert _relerr(lse2, lse[0]) < 1e-13


def test_empty_request():
    q_c, q_r, cache, _, w_uk, w_uv = _rand_problem(2)
    o, lse = ref.mla_decode_reference(q_c, q_r, cache, np.array([0, 3]), w_uk, w_uv, 0.5)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.isfinite(lse[1]).all()
    o2, o_lat, lse2, _ = ref.mla_decode_absorbed(q_c, q_r, cache, np.array([0, 3]), w_uk,
                                                 w_uv, 0.5)
    assert np.all(o_lat[0] == 0) and np.all(np.isneginf(lse2[0]))


# --- cache accounting (check (b) of the build's oracle properties) ------------

def _golden():
    with open(os.path.join(HERE, "golden", "cache_accounting.json")) as f:
        g = json.load(f)
    return g["dims"], {e["id"]: e for e in g["entries"]}


def test_cache_accounting_matches_pages():
    dims, e = _golden()
    nh, dh, dc, dr, L = (dims[k] for k in ("n_heads", "d_head", "d_latent", "d_rope",
                                           "n_layers"))
    mha = oracle.cache_elems_per_token_mha(nh, dh)
    mla = oracle.cache_elems_per_token_mla(dc, dr)
    assert mha == e["mha_per_token_per_layer"]["value"]
    assert mla == e["mla_per_token_per_layer"]["value"]
    assert mha // dc == e["latent_only_reduction_factor"]["value"]
    assert math.isclose(mha * L, e["mha_per_token_60_layers_approx"]["value"],
                        rel_tol=e["mha_per_token_60_layers_approx"]["rel_tol"])
    assert math.isclose(mla * L, e["mla_per_token_60_layers_approx"]["value"],
                        rel_tol=e["mla_per_token_60_layers_approx"]["rel_tol"])
    assert abs(mha / mla - e["mla_over_mha_60_layers_inverse"]["value"]) <= \
        e["mla_over_mha_60_layers_inverse"]["abs_tol"]
    assert mla / dh == e["mla_in_units_of_d_head_per_layer"]["value"]
    assert mla / (2 * dh) == e["gqa_groups_equivalent"]["value"]
    gib = 2 ** 30
    assert oracle.kv_cache_bytes(131072, L, mha) / gib == \
        e["mha_bytes_128k_60_layers_bf16_gib"]["value"]
    assert oracle.kv_cache_bytes(131072, L, mla) / gib == \
        e["mla_bytes_128k_60_layers_bf16_gib"]["value"]
    assert mha * 2 == e["bf16_bytes_per_token_per_layer_mha"]["value"]


def test_cache_rows_hold_exactly_latent_plus_rope():
    """The cache object of every workload holds d_c + d_h^R elements per token
    (V2 read-through section 5.1: the cache must hold only c_kv and the RoPE
    key; a row of 2 n_h d_h would mean the up-projected k, v were cached)."""
    for cfg in CONFIGS.values():
        assert cfg.row == oracle.cache_elems_per_token_mla(cfg.d_latent, cfg.d_rope)
        assert cfg.row < oracle.cache_elems_per_token_mha(cfg.n_heads, cfg.d_head)
    case = make_case(TINY, 0)
    rows = oracle.gather_rows(case.cache, 0, int(case.seq_lens[0]))
    assert rows.shape == (64, 40)


# --- planted mistakes: every broken oracle must fail some pin ----------------

def _fails_some_pin():
    failed = []
    for name, fn in ALL_PINS:
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


def _mut_drop_rope(q_c, q_r, cache, seq_lens, w_uk, w_uv, scale, page_table=None,
                   page_size=0, requests=None, heads=None):
    d_c = w_uk.shape[2]
    B, n_h, _ = q_c.shape
    o = np.zeros((B, n_h, w_uv.shape[2]))
    lse = np.full((B, n_h), -np.inf)
    for b in range(B):
        rows = ref.gather_rows(cache, b, int(seq_lens[b]), page_table, page_size)
        k_c, v = ref.up_project(rows[:, :d_c], w_uk, w_uv)
        o[b], lse[b] = ref.softmax_attention(np.asarray(q_c[b], float), k_c, v, scale)
    return o, lse


def _mut_transposed_uk(latent, w_uk, w_uv):
    latent = np.asarray(latent, np.float64)
    return (np.matmul(latent[None], np.asarray(w_uk, np.float64)),
            np.matmul(latent[None], np.asarray(w_uv, np.float64)))


def _mut_softmax_over_heads(q, k, v, scale):
    s = scale * np.matmul(k, q[:, :, None])[:, :, 0]
    e = np.exp(s - s.max(axis=0, keepdims=True))
    p = e / e.sum(axis=0, keepdims=True)
    return np.matmul(p[:, None, :], v)[:, 0, :], np.log(e.sum(axis=1))


_orig_softmax_attention = ref.softmax_attention


def _mut_sign_flip(q, k, v, scale):
    return _orig_softmax_attention(-q, k, v, scale)


def _mut_absorb_no_rope(q_c, q_r, w_uk, dtype=np.float64):
    q_lat = np.einsum("bih,ihc->bic", np.asarray(q_c, dtype), np.asarray(w_uk, dtype))
    return np.concatenate([q_lat, np.zeros_like(np.asarray(q_r, dtype))], axis=2)


@pytest.mark.parametrize("target,mutant", [
    ("mla_decode_reference", _mut_drop_rope),
    ("up_project", _mut_transposed_uk),
    ("softmax_attention", _mut_softmax_over_heads),
    ("softmax_attention", _mut_sign_flip),
    ("absorb_query", _mut_absorb_no_rope),
], ids=["drop_rope", "transposed_w_uk", "softmax_over_heads", "sign_flip",
        "absorb_drops_rope"])
def test_planted_mistakes(monkeypatch, target, mutant):
    monkeypatch.setattr(ref, target, mutant)
    failed = _fails_some_pin()
    assert failed, f"planted mistake in {target} was caught by no pin"
