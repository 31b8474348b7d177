"""Pins of the attention oracle to facts that do not come from the oracle.

The oracle computes softmax attention as "Modern GPU Programming For MLSys -
书籍总结", part IV (sections 5.1-5.3) describes it: a score product, a
softmax over the keys of each query row (with an optional causal mask), a
value product, and grouped-query heads.  Each ``pin_attn_*`` takes an
``oracle.Oracle`` and raises AssertionError when the oracle disagrees with:
  - a library special case: torch's scaled_dot_product_attention and
    logsumexp in float64 on the CPU, with the mask written out as a boolean
    matrix;
  - closed forms: a zero query gives the mean of the visible value rows and
    lse = log(number of visible keys); a score gap of thousands makes the
    softmax exactly one-hot, so the output row is exactly one value row;
  - invariants: grouped-query heads equal their key/value heads repeated;
    a causal row equals unmasked attention over its visible prefix; scaling
    a query by 2 and the scale by 1/2 changes nothing; permuting the keys
    with their values changes nothing; the magnitude output is the output of
    |V|; strided views read the same values as dense copies;
  - the stable form: scores near +-3000 (which overflow exp without the
    max shift) still match float64 SDPA.
``tests/test_oracle.py`` runs every pin on the real oracle and
``tests/test_oracle_mutations.py`` plants mistakes in copies of oracle.c.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(a: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _qkv(B, Hq, Hkv, Sq, Sk, D, seed, spread=1.0):
    g = torch.Generator().manual_seed(seed)
    Q = (spread * torch.randn(B, Hq, Sq, D, generator=g)).bfloat16()
    K = torch.randn(B, Hkv, Sk, D, generator=g).bfloat16()
    V = torch.randn(B, Hkv, Sk, D, generator=g).bfloat16()
    return bf16_bits(Q), bf16_bits(K), bf16_bits(V)


def _visible(Sq, Sk, causal):
    """Boolean [Sq, Sk]: key j visible to query i (bottom-right causal)."""
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    return (j <= i + (Sk - Sq)) if causal else np.ones((Sq, Sk), bool)


def _sdpa64(Q, K, V, scale, causal):
    """float64 SDPA + logsumexp on the decoded values, GQA by repetition.
    Rows with no visible key are left NaN here (SDPA has no value for them)."""
    q = torch.from_numpy(bits_to_f64(Q))
    k = torch.from_numpy(bits_to_f64(K))
    v = torch.from_numpy(bits_to_f64(V))
    g = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    vis = torch.from_numpy(_visible(q.shape[2], k.shape[2], causal))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=vis, scale=scale)
    s = scale * (q @ k.transpose(-1, -2))
    s = s.masked_fill(~vis, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy(), vis.numpy()


def pin_attn_sdpa_float64(orc):
    cases = [
        # B, Hq, Hkv, Sq, Sk, D, causal, seed
        (2, 3, 3, 17, 17, 16, False, 1),
        (1, 4, 2, 9, 23, 64, True, 2),      # Sq < Sk: bottom-right alignment
        (2, 4, 1, 31, 31, 32, True, 3),     # Sq == Sk, GQA 4:1
        (1, 2, 2, 1, 40, 16, True, 4),      # decode-like: one query sees all
        (1, 6, 3, 12, 5, 16, False, 5),
    ]
    for B, Hq, Hkv, Sq, Sk, D, causal, seed in cases:
        Q, K, V = _qkv(B, Hq, Hkv, Sq, Sk, D, seed)
        scale = 1.0 / math.sqrt(D)
        O, _, lse = orc.attention_fwd(Q, K, V, scale, causal)
        ref, ref_lse, _ = _sdpa64(Q, K, V, scale, causal)
        assert np.allclose(O, ref, rtol=1e-12, atol=1e-12), (B, Hq, Hkv, Sq, Sk, D, causal)
        assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12), (B, Hq, Hkv, Sq, Sk, D, causal)


def pin_attn_empty_rows(orc):
    """Causal with Sq > Sk: the first Sq - Sk rows see no key; Sk == 0 too."""
    Q, K, V = _qkv(1, 2, 1, 10, 4, 16, 11)
    O, Om, lse = orc.attention_fwd(Q, K, V, 0.25, True)
    assert (O[:, :, :6] == 0).all() and (Om[:, :, :6] == 0).all()
    assert np.isneginf(lse[:, :, :6]).all()
    ref, ref_lse, _ = _sdpa64(Q, K, V, 0.25, True)
    assert np.allclose(O[:, :, 6:], ref[:, :, 6:], rtol=1e-12, atol=1e-12)
    assert np.allclose(lse[:, :, 6:], ref_lse[:, :, 6:], rtol=1e-12, atol=1e-12)
    Q, K, V = _qkv(1, 1, 1, 3, 0, 16, 12)
    O, _, lse = orc.attention_fwd(Q, K, V, 0.25, False)
    assert (O == 0).all() and np.isneginf(lse).all()


def pin_attn_uniform_closed_form(orc):
    """q = 0: every visible score is 0, so o(i) is the exact mean of the
    visible value rows and lse(i) = log(count)."""
    for Sq, Sk, causal in ((7, 13, True), (13, 7, True), (9, 9, False), (9, 9, True)):
        rng = np.random.default_rng(Sq * 100 + Sk)
        D = 8
        Q = np.zeros((1, 1, Sq, D), np.uint16)
        Vi = rng.integers(-50, 51, size=(1, 1, Sk, D))
        V = bf16_bits(torch.from_numpy(Vi.astype(np.float32)).bfloat16())
        K = bf16_bits(torch.randn(1, 1, Sk, D, generator=torch.Generator().manual_seed(5)).bfloat16())
        O, _, lse = orc.attention_fwd(Q, K, V, 0.7, causal)
        vis = _visible(Sq, Sk, causal)
        for i in range(Sq):
            n = int(vis[i].sum())
            if n == 0:
                assert (O[0, 0, i] == 0).all() and np.isneginf(lse[0, 0, i])
                continue
            for d in range(D):
                want = float(Fraction(int(Vi[0, 0, :n, d].sum()), n))
                assert O[0, 0, i, d] == want, (Sq, Sk, causal, i, d)
            assert lse[0, 0, i] == math.log(n)


def pin_attn_one_hot(orc):
    """q(i) = 64 e_a(i), k(j) = 64 e_b(j), scale 1: the matching key scores
    4096 and every other 0, so exp(-4096) = 0 and the softmax is exactly
    one-hot (o(i) = v(j*), lse = 4096); rows whose key is masked or absent
    fall back to the uniform mean."""
    D, Sq, Sk = 16, 12, 10
    rng = np.random.default_rng(21)
    a = rng.permutation(D)[:Sq]
    b = rng.permutation(D)[:Sk]
    Qf = np.zeros((1, 1, Sq, D), np.float32)
    Kf = np.zeros((1, 1, Sk, D), np.float32)
    Qf[0, 0, np.arange(Sq), a] = 64.0
    Kf[0, 0, np.arange(Sk), b] = 64.0
    Vi = rng.integers(-20, 21, size=(1, 1, Sk, D)).astype(np.float32)
    enc = lambda x: bf16_bits(torch.from_numpy(x).bfloat16())
    for causal in (False, True):
        O, _, lse = orc.attention_fwd(enc(Qf), enc(Kf), enc(Vi), 1.0, causal)
        vis = _visible(Sq, Sk, causal)
        for i in range(Sq):
            hit = [j for j in range(Sk) if b[j] == a[i] and vis[i, j]]
            n = int(vis[i].sum())
            if hit:
                assert np.array_equal(O[0, 0, i], Vi[0, 0, hit[0]].astype(np.float64))
                assert lse[0, 0, i] == 4096.0
            elif n:
                want = Vi[0, 0, vis[i]].astype(np.float64).sum(0) / n
                assert np.allclose(O[0, 0, i], want, rtol=0, atol=1e-13)
            else:
                assert (O[0, 0, i] == 0).all()


def pin_attn_gqa_repeat(orc):
    Q, K, V = _qkv(2, 6, 2, 11, 14, 16, 31)
    for causal in (False, True):
        O, Om, lse = orc.attention_fwd(Q, K, V, 0.3, causal)
        Kr = np.repeat(K, 3, axis=1)
        Vr = np.repeat(V, 3, axis=1)
        O2, Om2, lse2 = orc.attention_fwd(Q, Kr, Vr, 0.3, causal)
        assert np.array_equal(O, O2) and np.array_equal(Om, Om2) and np.array_equal(lse, lse2)


def pin_attn_causal_prefix(orc):
    """A causal row i equals unmasked attention over keys 0 .. i + Sk - Sq."""
    Sq, Sk = 6, 9
    Q, K, V = _qkv(1, 2, 2, Sq, Sk, 16, 41)
    O, _, lse = orc.attention_fwd(Q, K, V, 0.2, True)
    for i in range(Sq):
        n = i + Sk - Sq + 1
        o1, _, l1 = orc.attention_fwd(np.ascontiguousarray(Q[:, :, i:i + 1]),
                                      np.ascontiguousarray(K[:, :, :n]),
                                      np.ascontiguousarray(V[:, :, :n]), 0.2, False)
        assert np.array_equal(O[:, :, i], o1[:, :, 0]) and np.array_equal(lse[:, :, i], l1[:, :, 0])


def pin_attn_scale_power_of_two(orc):
    """scale * (2q) . k with scale halved is the same product exactly."""
    Q, K, V = _qkv(1, 2, 1, 8, 8, 32, 51)
    O, _, lse = orc.attention_fwd(Q, K, V, 0.25, True)
    Q2 = bf16_bits(torch.from_numpy(2.0 * bits_to_f64(Q)).bfloat16())
    O2, _, lse2 = orc.attention_fwd(Q2, K, V, 0.125, True)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)
    O3, _, _ = orc.attention_fwd(Q2, K, V, 0.25, True)
    assert not np.allclose(O, O3)


def pin_attn_key_permutation(orc):
    Q, K, V = _qkv(1, 2, 2, 5, 19, 16, 61)
    O, _, lse = orc.attention_fwd(Q, K, V, 0.3, False)
    perm = np.random.default_rng(3).permutation(19)
    O2, _, lse2 = orc.attention_fwd(Q, np.ascontiguousarray(K[:, :, perm]),
                                    np.ascontiguousarray(V[:, :, perm]), 0.3, False)
    assert np.allclose(O, O2, rtol=0, atol=1e-13) and np.allclose(lse, lse2, rtol=0, atol=1e-13)


def pin_attn_magnitude(orc):
    """Omag = sum_j p_j |v(j, d)| is the output of the same softmax over |V|."""
    Q, K, V = _qkv(1, 3, 1, 7, 12, 16, 71)
    _, Om, _ = orc.attention_fwd(Q, K, V, 0.3, True)
    Vabs = V & np.uint16(0x7FFF)
    O2, _, _ = orc.attention_fwd(Q, K, Vabs, 0.3, True)
    assert np.array_equal(Om, O2)


def pin_attn_large_scores(orc):
    """Scores of order +-3000: exp overflows unless the row maximum is
    subtracted first; the stable result matches float64 SDPA."""
    Q, K, V = _qkv(1, 2, 2, 9, 9, 64, 81, spread=60.0)
    O, _, lse = orc.attention_fwd(Q, K, V, 1.0, True)
    ref, ref_lse, _ = _sdpa64(Q, K, V, 1.0, True)
    assert np.isfinite(O).all()
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-9)


def pin_attn_strided_views(orc):
    """[B, S, H, D] storage read through permuted views, and a view with an
    element stride of 2 along D, give the dense results."""
    Q, K, V = _qkv(2, 4, 2, 6, 10, 16, 91)
    O, _, lse = orc.attention_fwd(Q, K, V, 0.3, True)
    Qs = np.ascontiguousarray(Q.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    Ks = np.ascontiguousarray(K.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    Vs = np.ascontiguousarray(V.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    O2, _, lse2 = orc.attention_fwd(Qs, Ks, Vs, 0.3, True)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)
    wide = np.full(Q.shape[:3] + (32,), 0x7FC0, np.uint16)  # NaN between the elements
    wide[..., ::2] = Q
    O3, _, lse3 = orc.attention_fwd(wide[..., ::2], K, V, 0.3, True)
    assert np.array_equal(O, O3) and np.array_equal(lse, lse3)


def pin_attn_sampled_rows(orc):
    Q, K, V = _qkv(2, 4, 2, 7, 9, 16, 101)
    O, Om, lse = orc.attention_fwd(Q, K, V, 0.3, True)
    rows = np.array([[0, 0, 0], [1, 3, 6], [0, 2, 4], [1, 1, 1]], np.int64)
    o, om, l = orc.attention_fwd_at(Q, K, V, 0.3, True, rows)
    for t, (b, h, i) in enumerate(rows):
        assert np.array_equal(o[t], O[b, h, i]) and np.array_equal(om[t], Om[b, h, i])
        assert l[t] == lse[b, h, i]


ATTN_PINS = [
    pin_attn_sdpa_float64, pin_attn_empty_rows, pin_attn_uniform_closed_form, pin_attn_one_hot,
    pin_attn_gqa_repeat, pin_attn_causal_prefix, pin_attn_scale_power_of_two,
    pin_attn_key_permutation, pin_attn_magnitude, pin_attn_large_scores, pin_attn_strided_views,
    pin_attn_sampled_rows,
]
