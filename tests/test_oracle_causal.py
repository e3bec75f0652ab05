"""Pins of the oracle's several-new-token decode (oracle.latent_attention_causal):
verification of tokens proposed by the extra prediction depths (DeepSeek-V3
technical report read-through, 2kiu.com/news/6340724, section 4.1), each new
token attending causally to the positions up to its own (zeeklog MHA
equation: attention over positions 1..t).

Each pin checks the oracle against something other than itself: scalar loops
written from the definition, torch's scaled_dot_product_attention with an
explicit mask, reductions to the single-token oracle, and causality
invariants.  Planted mistakes (wrong mask alignment, off-by-one, no mask) must
each fail a pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.mla_ref as ref


def _problem(seed, q_len=3, n_h=2, row=7, d_c=5, T=6):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((q_len, n_h, row)), rng.standard_normal((T, row)), d_c


def _relerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def brute_force(q, rows, d_c, scale):
    """Scalar loops: new token j is at position T - q_len + j (0-based) and sees
    positions 0..T - q_len + j; plain softmax without max subtraction (inputs
    are small)."""
    q_len, n_h, width = q.shape
    T = rows.shape[0]
    o = np.zeros((q_len, n_h, d_c))
    lse = np.full((q_len, n_h), -np.inf)
    for j in range(q_len):
        last = T - q_len + j            # position of the new token itself
        for i in range(n_h):
            w = []
            for t in range(0, last + 1):
                s = 0.0
                for c in range(width):
                    s += q[j][i][c] * rows[t][c]
                w.append(math.exp(scale * s))
            if not w:
                continue
            z = sum(w)
            lse[j][i] = math.log(z)
            for c in range(d_c):
                acc = 0.0
                for t in range(len(w)):
                    acc += w[t] * rows[t][c]
                o[j][i][c] = acc / z
    return o, lse


def pin_brute_force():
    for seed, (q_len, T) in enumerate([(3, 6), (1, 4), (4, 4), (2, 9)]):
        q, rows, d_c = _problem(seed, q_len=q_len, T=T)
        o, lse = oracle.latent_attention_causal(q, rows, d_c, 0.41)
        o_bf, lse_bf = brute_force(q, rows, d_c, 0.41)
        assert _relerr(o, o_bf) < 1e-12 and _relerr(lse, lse_bf) < 1e-12


def pin_sdpa_masked():
    """torch SDPA (fp64, CPU) with the boolean mask allowed[j, t] = t <= T - q_len + j:
    an independent softmax-attention implementation with the mask spelt out."""
    q, rows, d_c = _problem(11, q_len=4, n_h=3, T=10)
    q_len, n_h, _ = q.shape
    T = rows.shape[0]
    o, _ = oracle.latent_attention_causal(q, rows, d_c, 0.3)
    allowed = torch.tensor([[t <= T - q_len + j for t in range(T)] for j in range(q_len)])
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                    # [1, n_h, q_len, row]
    kt = torch.from_numpy(rows)[None, None].expand(1, n_h, T, -1)
    vt = torch.from_numpy(rows[:, :d_c])[None, None].expand(1, n_h, T, -1)
    ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed,
                                                          scale=0.3)
    assert _relerr(o, ot[0].permute(1, 0, 2).numpy()) < 1e-12


def pin_single_token_and_last_token():
    """q_len = 1 is the single-token oracle; the last new token sees every row."""
    q, rows, d_c = _problem(3, q_len=1, T=5)
    o, lse = oracle.latent_attention_causal(q, rows, d_c, 0.5)
    o1, lse1 = oracle.latent_attention(q[0], rows, d_c, 0.5)
    assert _relerr(o[0], o1) < 1e-14 and _relerr(lse[0], lse1) < 1e-14
    q, rows, d_c = _problem(4, q_len=3, T=7)
    o, lse = oracle.latent_attention_causal(q, rows, d_c, 0.5)
    o1, lse1 = oracle.latent_attention(q[-1], rows, d_c, 0.5)
    assert _relerr(o[-1], o1) < 1e-14 and _relerr(lse[-1], lse1) < 1e-14


def pin_causality():
    """Rows after a token's position do not change its output; a row at or
    before it does."""
    q, rows, d_c = _problem(5, q_len=3, T=8)
    T, q_len = rows.shape[0], q.shape[0]
    o, _ = oracle.latent_attention_causal(q, rows, d_c, 0.7)
    for j in range(q_len):
        last = T - q_len + j
        later = rows.copy()
        later[last + 1:] += 3.0
        o2, _ = oracle.latent_attention_causal(q, later, d_c, 0.7)
        assert np.array_equal(o2[j], o[j])
        own = rows.copy()
        own[last] += 3.0
        o3, _ = oracle.latent_attention_causal(q, own, d_c, 0.7)
        assert not np.allclose(o3[j], o[j])


def pin_short_history():
    """Fewer rows than new tokens: the first tokens see nothing (zeros, -inf)."""
    q, rows, d_c = _problem(6, q_len=4, T=2)
    o, lse = oracle.latent_attention_causal(q, rows, d_c, 0.5)
    # T - q_len + j + 1 visible rows: -1, 0, 1, 2.
    assert np.all(o[:2] == 0) and np.all(np.isneginf(lse[:2]))
    o1, lse1 = oracle.latent_attention(q[3], rows, d_c, 0.5)
    assert _relerr(o[3], o1) < 1e-14 and _relerr(lse[3], lse1) < 1e-14


PINS = [("brute_force", pin_brute_force), ("sdpa_masked", pin_sdpa_masked),
        ("single_and_last_token", pin_single_token_and_last_token),
        ("causality", pin_causality), ("short_history", pin_short_history)]


@pytest.mark.parametrize("name,fn", PINS, ids=[n for n, _ in PINS])
def test_pin(name, fn):
    fn()


_orig_latent_attention = ref.latent_attention


def _causal_with(visible_fn):
    def mutant(q_cat, rows, d_latent, scale):
        q_cat = np.asarray(q_cat, np.float64)
        q_len, n_h = q_cat.shape[:2]
        T = np.asarray(rows).shape[0]
        o = np.zeros((q_len, n_h, d_latent))
        lse = np.full((q_len, n_h), -np.inf)
        for j in range(q_len):
            v = visible_fn(T, q_len, j)
            o[j], lse[j] = _orig_latent_attention(q_cat[j], np.asarray(rows)[:max(v, 0)],
                                                  d_latent, scale)
        return o, lse
    return mutant


@pytest.mark.parametrize("mutant", [
    _causal_with(lambda T, q_len, j: T - q_len + j),        # excludes the token itself
    _causal_with(lambda T, q_len, j: j + 1),                # mask aligned to the first row
    _causal_with(lambda T, q_len, j: T),                    # no mask among the new tokens
    _causal_with(lambda T, q_len, j: T - j),                # reversed token order
], ids=["off_by_one", "top_left_alignment", "no_mask", "reversed"])
def test_planted_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(oracle, "latent_attention_causal", mutant)
    failed = []
    for name, fn in PINS:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    assert failed, "planted mistake caught by no pin"
