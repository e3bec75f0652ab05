"""Pins of oracle.mla_prefill_reference (a chunk of new tokens in the primary,
unabsorbed form) against things other than itself:

* the absorbed form (absorb_query -> latent_attention_causal -> project_out),
  a different factorisation pinned on its own (V2 read-through section 2.3:
  absorption leaves the scores and outputs unchanged);
* one new token: the unabsorbed decode reference;
* scalar loops over heads, keys and values on a tiny case;
* causality;
* planted mistakes, each of which one of the pins above must catch.
"""

import math

import numpy as np
import pytest

import oracle


def _case(seed, T=23, q_len=5, n_h=3, d_h=4, d_r=2, d_c=6):
    rng = np.random.default_rng(seed)
    latent = rng.standard_normal((T, d_c))
    k_rope = rng.standard_normal((T, d_r))
    q_c = rng.standard_normal((q_len, n_h, d_h))
    q_r = rng.standard_normal((q_len, n_h, d_r))
    w_uk = rng.standard_normal((n_h, d_h, d_c)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((n_h, d_c, d_h)) / math.sqrt(d_c)
    return q_c, q_r, latent, k_rope, w_uk, w_uv, 1.0 / math.sqrt(d_h + d_r)


def _absorbed(q_c, q_r, latent, k_rope, w_uk, w_uv, scale):
    rows = np.concatenate([latent, k_rope], axis=1)
    q_cat = oracle.absorb_query(q_c, q_r, w_uk)
    o_lat, lse = oracle.latent_attention_causal(q_cat, rows, latent.shape[1], scale)
    return oracle.project_out(o_lat, w_uv), lse


def _loops(q_c, q_r, latent, k_rope, w_uk, w_uv, scale):
    T = latent.shape[0]
    q_len, n_h, d_h = q_c.shape
    o = np.zeros((q_len, n_h, d_h))
    lse = np.full((q_len, n_h), -np.inf)
    for j in range(q_len):
        vis = T - q_len + j + 1
        for i in range(n_h):
            s = []
            for t in range(max(vis, 0)):
                acc = 0.0
                for h in range(d_h):
                    k = sum(w_uk[i, h, c] * latent[t, c] for c in range(latent.shape[1]))
                    acc += q_c[j, i, h] * k
                for r in range(k_rope.shape[1]):
                    acc += q_r[j, i, r] * k_rope[t, r]
                s.append(scale * acc)
            if not s:
                continue
            m = max(s)
            z = sum(math.exp(x - m) for x in s)
            lse[j, i] = m + math.log(z)
            for h in range(d_h):
                o[j, i, h] = sum(math.exp(s[t] - m) / z *
                                 sum(w_uv[i, c, h] * latent[t, c] for c in range(latent.shape[1]))
                                 for t in range(len(s)))
    return o, lse


@pytest.mark.parametrize("seed", range(4))
def test_equals_absorbed_form(seed):
    args = _case(seed)
    o, lse = oracle.mla_prefill_reference(*args)
    o_a, lse_a = _absorbed(*args)
    np.testing.assert_allclose(o, o_a, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_a, rtol=0, atol=1e-12)


def test_one_token_equals_decode_reference():
    q_c, q_r, latent, k_rope, w_uk, w_uv, scale = _case(7, q_len=1)
    o, lse = oracle.mla_prefill_reference(q_c, q_r, latent, k_rope, w_uk, w_uv, scale)
    cache = np.concatenate([latent, k_rope], axis=1)[None]
    o_d, lse_d = oracle.mla_decode_reference(q_c, q_r, cache, np.array([latent.shape[0]]),
                                             w_uk, w_uv, scale)
    np.testing.assert_allclose(o[0], o_d[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], lse_d[0], rtol=0, atol=1e-12)


def test_scalar_loops_with_short_history():
    # T < q_len: the first tokens see nothing (o = 0, lse = -inf).
    args = _case(11, T=3, q_len=5)
    o, lse = oracle.mla_prefill_reference(*args)
    o_l, lse_l = _loops(*args)
    assert np.isneginf(lse[:2]).all() and (o[:2] == 0).all()
    np.testing.assert_allclose(o, o_l, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lse_l))
    np.testing.assert_allclose(lse[2:], lse_l[2:], rtol=0, atol=1e-12)


def test_causality():
    q_c, q_r, latent, k_rope, w_uk, w_uv, scale = _case(3)
    T, q_len = latent.shape[0], q_c.shape[0]
    o, _ = oracle.mla_prefill_reference(q_c, q_r, latent, k_rope, w_uk, w_uv, scale)
    j = 2
    pos = T - q_len + j
    lat2 = latent.copy()
    lat2[pos + 1:] += 5.0
    o2, _ = oracle.mla_prefill_reference(q_c, q_r, lat2, k_rope, w_uk, w_uv, scale)
    np.testing.assert_array_equal(o[:j + 1], o2[:j + 1])
    assert not np.allclose(o[j + 1:], o2[j + 1:])
    lat3 = latent.copy()
    lat3[pos] += 5.0
    o3, _ = oracle.mla_prefill_reference(q_c, q_r, lat3, k_rope, w_uk, w_uv, scale)
    assert not np.allclose(o[j], o3[j])


def test_head_subset():
    args = _case(5)
    o, lse = oracle.mla_prefill_reference(*args)
    o_s, lse_s = oracle.mla_prefill_reference(*args, heads=[0, 2])
    np.testing.assert_array_equal(o_s[:, [0, 2]], o[:, [0, 2]])
    assert (o_s[:, 1] == 0).all() and np.isneginf(lse_s[:, 1]).all()


# Planted mistakes: plausible slips in the unabsorbed form.  Each must be
# caught by the absorbed-form pin.
def _mut_off_by_one(q_c, q_r, latent, k_rope, w_uk, w_uv, scale):
    return oracle.mla_prefill_reference(q_c, q_r, latent[:-1], k_rope[:-1], w_uk, w_uv, scale)


def _mut_no_rope(q_c, q_r, latent, k_rope, w_uk, w_uv, scale):
    return oracle.mla_prefill_reference(q_c, q_r, latent, np.zeros_like(k_rope), w_uk, w_uv,
                                        scale)


def _mut_swapped_heads(q_c, q_r, latent, k_rope, w_uk, w_uv, scale):
    return oracle.mla_prefill_reference(q_c, q_r, latent, k_rope, w_uk, w_uv[::-1], scale)


def _mut_reversed_tokens(q_c, q_r, latent, k_rope, w_uk, w_uv, scale):
    return oracle.mla_prefill_reference(q_c[::-1], q_r[::-1], latent, k_rope, w_uk, w_uv, scale)


@pytest.mark.parametrize("mut", [_mut_off_by_one, _mut_no_rope, _mut_swapped_heads,
                                 _mut_reversed_tokens])
def test_planted_mistakes_are_caught(mut):
    args = _case(9)
    o_m, _ = mut(*args)
    o_a, _ = _absorbed(*args)
    assert not np.allclose(o_m, o_a, rtol=0, atol=1e-6)
