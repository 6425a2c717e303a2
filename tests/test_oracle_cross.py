"""Pins of the text cross-attention oracle and of the text cache model
(RTR-DiT notes, Key Designs 1: text injected through cross attention; Key
Designs 4: a fixed-length cross-attention cache re-initialised on a switch)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import TextKV


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("Tq,Lt", [(37, 77), (64, 1), (5, 300)])
def test_cross_matches_sdpa(Tq, Lt):
    """Pin: torch scaled_dot_product_attention (float64, no mask)."""
    H, d = 3, 16
    q, k, v = _rand((Tq, H, d), 1), _rand((Lt, H, d), 2), _rand((Lt, H, d), 3)
    o, lse = oracle.attn_cross(q, k, v)
    t = lambda x: torch.tensor(x).permute(1, 0, 2)  # [H, T, d]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v)).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    s = np.einsum("thd,shd->hts", q, k) / np.sqrt(d)
    m = s.max(-1)
    np.testing.assert_allclose(lse, m + np.log(np.exp(s - m[..., None]).sum(-1)), rtol=1e-12)


def test_cross_closed_forms():
    Tq, Lt, H, d = 20, 9, 2, 8
    q, k = _rand((Tq, H, d), 4), _rand((Lt, H, d), 5)
    # one text token: every query returns its value
    v1 = _rand((1, H, d), 6)
    o, _ = oracle.attn_cross(q, k[:1], v1)
    np.testing.assert_allclose(o, np.broadcast_to(v1, (Tq, H, d)), atol=1e-14)
    # constant values: output equals the constant
    vc = np.ones((Lt, H, d)) * 0.37
    o, _ = oracle.attn_cross(q, k, vc)
    np.testing.assert_allclose(o, 0.37, atol=1e-14)
    # permuting the text tokens (K and V together) changes nothing
    v = _rand((Lt, H, d), 7)
    perm = np.random.default_rng(8).permutation(Lt)
    np.testing.assert_allclose(oracle.attn_cross(q, k[perm], v[perm])[0], oracle.attn_cross(q, k, v)[0],
                               atol=1e-13)
    # against the (pinned) full form: text as frame 0, the queries as frame 1
    # whose own keys and values are zero, so each frame-1 row sees the text
    # plus Lt keys of logit 0 and value 0
    kk = np.concatenate([k, np.zeros((Lt, H, d))], axis=0)
    vv = np.concatenate([v, np.zeros((Lt, H, d))], axis=0)
    qq = np.concatenate([np.zeros((Lt, H, d)), q[:Lt]], axis=0)
    o_full, _ = oracle.attn_block_causal(qq, kk, vv, Lt)
    # o = sum_text e^s v / (sum_text e^s + Lt), and the cross oracle is the
    # same expression without the Lt extra keys
    s = np.einsum("thd,shd->hts", q[:Lt], k) / np.sqrt(d)
    e = np.exp(s)
    expect = np.einsum("hts,shd->thd", e, v) / (e.sum(-1) + Lt).T[..., None]
    np.testing.assert_allclose(o_full[Lt:], expect, rtol=1e-10, atol=1e-12)
    oc, _ = oracle.attn_cross(q[:Lt], k, v)
    np.testing.assert_allclose(oc, np.einsum("hts,shd->thd", e, v) / e.sum(-1).T[..., None], rtol=1e-10)


def test_text_cache_schedule():
    """Pin: a hand-written set/clear schedule."""
    tc = TextKV(8)
    assert tc.tokens() == 0 and tc.generation == 0
    a = _rand((5, 1, 4), 9)
    tc.set(a, a + 1)
    assert tc.tokens() == 5 and tc.generation == 1
    a[0] = 0  # the cache holds a copy
    assert not np.all(tc.k[0] == 0)
    tc.set(_rand((8, 1, 4), 10), _rand((8, 1, 4), 11))
    assert tc.tokens() == 8 and tc.generation == 2
    tc.clear()
    assert tc.tokens() == 0 and tc.generation == 2
    with pytest.raises(ValueError):
        tc.set(_rand((9, 1, 4), 12), _rand((9, 1, 4), 13))
    with pytest.raises(ValueError):
        tc.set(_rand((0, 1, 4), 12), _rand((0, 1, 4), 13))
