"""Pins of the float64 attention gradients against things other than themselves.

The gradients are the derivative of the Attn equation (RTR-DiT notes, "DiT as
Real-Time Rerenderer ...", Key Designs 2).  They are pinned to central finite
differences of the (separately pinned) forward oracle, to torch.autograd on a
literal float64 forward written here, and to invariants that follow from the
softmax: rows of dS sum to zero, so dK sums to zero over keys and dQ ignores a
common shift of all keys; rows of P sum to one, so dV sums to the summed dO.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.attention_bwd import attn_block_causal_bwd, attn_bwd_cols, attn_bwd_rows


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _inputs(T, H, d, seed):
    return [_rand((T, H, d), seed + t) for t in range(4)]


@pytest.mark.parametrize("T,H,d,kpf", [(7, 2, 4, 3), (6, 1, 3, 1), (5, 1, 4, 8)])
def test_gradients_match_central_differences(T, H, d, kpf):
    """Pin: central differences of L = sum(O * G), O from the forward oracle.
    Covers a ragged last frame (7 = 3+3+1), token causality (k = 1) and the
    unmasked case (k > T)."""
    q, k, v, g = _inputs(T, H, d, 10)
    dq, dk, dv = attn_block_causal_bwd(q, k, v, g, kpf)
    eps = 1e-6

    def loss(qq, kk, vv):
        o, _ = oracle.attn_block_causal(qq, kk, vv, kpf)
        return float(np.sum(o * g))

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("T,kpf", [(40, 6), (33, 33), (24, 1)])
def test_gradients_match_autograd(T, kpf):
    """Pin: torch.autograd (float64, CPU) through softmax(Q K^T / sqrt(d) + M) V
    written out here."""
    H, d = 2, 16
    q, k, v, g = _inputs(T, H, d, 20)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = torch.where(j // kpf <= i // kpf, 0.0, float("-inf")).double()
    s = torch.einsum("thd,shd->hts", tq, tk) / d ** 0.5 + mask
    o = torch.einsum("hts,shd->thd", torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(g))
    dq, dk, dv = attn_block_causal_bwd(q, k, v, g, kpf)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_gradient_invariants():
    """Pin: closed-form consequences of the softmax, per head."""
    T, H, d, kpf = 50, 3, 8, 7
    q, k, v, g = _inputs(T, H, d, 30)
    dq, dk, dv = attn_block_causal_bwd(q, k, v, g, kpf)
    # rows of dS sum to zero -> sum over keys of dK is zero
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    # rows of P sum to one -> sum over keys of dV equals sum over queries of dO
    np.testing.assert_allclose(dv.sum(axis=0), g.sum(axis=0), atol=1e-11)
    # a common shift of every key leaves P, hence dQ and dV, unchanged
    shift = _rand((1, H, d), 31)
    dq2, _, dv2 = attn_block_causal_bwd(q, k + shift, v, g, kpf)
    np.testing.assert_allclose(dq2, dq, atol=1e-10)
    np.testing.assert_allclose(dv2, dv, atol=1e-10)
    # token 0 of frame 0 with k = 1 sees only itself: P = 1 there, dS = 0, dQ = 0
    dq1, _, _ = attn_block_causal_bwd(q, k, v, g, 1)
    assert np.all(dq1[0] == 0.0)
    # keys of the last frame are seen only by rows of the last frame
    last = (T - 1) // kpf * kpf
    g2 = g.copy()
    g2[last:] = 0.0
    _, dk2, dv2 = attn_block_causal_bwd(q, k, v, g2, kpf)
    assert np.all(dk2[last:] == 0.0) and np.all(dv2[last:] == 0.0)


def test_gradients_scale_argument():
    """An explicit scale equal to 1/sqrt(d) gives the same gradients; another
    scale equals the default applied to Q pre-multiplied accordingly (dK and dV
    exactly, dQ times the factor by the chain rule)."""
    T, H, d, kpf = 20, 1, 8, 5
    q, k, v, g = _inputs(T, H, d, 40)
    a = attn_block_causal_bwd(q, k, v, g, kpf)
    b = attn_block_causal_bwd(q, k, v, g, kpf, scale=1 / np.sqrt(d))
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-14, atol=1e-15)
    f = 0.37 * np.sqrt(d)                  # scale 0.37 == default scale on f * q
    dq, dk, dv = attn_block_causal_bwd(q, k, v, g, kpf, scale=0.37)
    dq2, dk2, dv2 = attn_block_causal_bwd(f * q, k, v, g, kpf)
    np.testing.assert_allclose(dk, dk2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dv2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq, f * dq2, rtol=1e-12, atol=1e-13)


def test_rows_and_cols_variants_equal_dense():
    T, H, d, kpf = 61, 2, 8, 9
    q, k, v, g = _inputs(T, H, d, 50)
    dq, dk, dv = attn_block_causal_bwd(q, k, v, g, kpf)
    rows = [0, 5, 8, 9, 30, 53, 54, 60]
    np.testing.assert_allclose(attn_bwd_rows(q, k, v, g, kpf, rows, [1, 0]),
                               dq[rows][:, [1, 0]], rtol=1e-12, atol=1e-13)
    cols = [0, 8, 9, 17, 40, 54, 60]
    ck, cv = attn_bwd_cols(q, k, v, g, kpf, cols, [1], group=7)
    np.testing.assert_allclose(ck, dk[cols][:, [1]], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(cv, dv[cols][:, [1]], rtol=1e-12, atol=1e-13)


def test_stream_step_bwd_equals_full_form_with_earlier_rows_silent():
    """Pin: a streaming step over [prefix frames | chunk] is the full form's
    last chunk; with dO zero on the prefix frames' own rows, the full-form
    gradients of the chunk rows and of every key are the step's gradients."""
    from oracle.attention_bwd import attn_stream_step_bwd
    kpf, H, d, Pf, C = 4, 2, 8, 3, 2
    T = (Pf + C) * kpf
    q, k, v, g = _inputs(T, H, d, 60)
    g[:Pf * kpf] = 0.0
    dq, dk, dv = attn_block_causal_bwd(q, k, v, g, kpf)
    c = slice(Pf * kpf, T)
    sq, sk, sv, spk, spv = attn_stream_step_bwd(k[:Pf * kpf], v[:Pf * kpf], q[c], k[c], v[c], g[c], kpf)
    np.testing.assert_allclose(sq, dq[c], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sk, dk[c], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sv, dv[c], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(spk, dk[:Pf * kpf], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(spv, dv[:Pf * kpf], rtol=1e-11, atol=1e-12)


def test_stream_step_bwd_central_differences():
    """Pin: central differences of sum(O * G) through the (pinned) streaming
    forward oracle, for the chunk's q, k, v and for the cached prefix."""
    from oracle.attention_bwd import attn_stream_step_bwd
    kpf, H, d, C, P = 3, 1, 4, 2, 5
    pk, pv = _rand((P, H, d), 70), _rand((P, H, d), 71)
    q, k, v, g = _inputs(C * kpf, H, d, 72)
    grads = attn_stream_step_bwd(pk, pv, q, k, v, g, kpf)
    args = [pk, pv, q, k, v]
    eps = 1e-6

    def loss(a):
        o, _ = oracle.attn_stream_step(a[0], a[1], a[2], a[3], a[4], kpf)
        return float(np.sum(o * g))

    for which, grad in ((2, grads[0]), (3, grads[1]), (4, grads[2]), (0, grads[3]), (1, grads[4])):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            ap = [x.copy() for x in args]
            am = [x.copy() for x in args]
            ap[which][idx] += eps
            am[which][idx] -= eps
            num[idx] = (loss(ap) - loss(am)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_cross_bwd_central_differences():
    """Pin: central differences of sum(O * G) through the (pinned) text
    cross-attention oracle, for q and the text keys and values."""
    from oracle.attention_bwd import attn_cross_bwd
    Tq, Lt, H, d = 5, 4, 2, 3
    q, kt, vt, g = _rand((Tq, H, d), 80), _rand((Lt, H, d), 81), _rand((Lt, H, d), 82), _rand((Tq, H, d), 83)
    grads = attn_cross_bwd(q, kt, vt, g)
    args = [q, kt, vt]
    eps = 1e-6

    def loss(a):
        o, _ = oracle.attn_cross(a[0], a[1], a[2])
        return float(np.sum(o * g))

    for which in range(3):
        num = np.zeros_like(grads[which])
        for idx in np.ndindex(*num.shape):
            ap = [x.copy() for x in args]
            am = [x.copy() for x in args]
            ap[which][idx] += eps
            am[which][idx] -= eps
            num[idx] = (loss(ap) - loss(am)) / (2 * eps)
        np.testing.assert_allclose(grads[which], num, rtol=1e-6, atol=1e-8)


def test_cross_bwd_autograd_and_invariants():
    """Pin: torch.autograd in float64 through softmax(Q K^T * scale) V written
    out here, an explicit scale; and the softmax invariants (the text keys'
    gradients sum to zero, the text values' gradients sum to the summed dO)."""
    from oracle.attention_bwd import attn_cross_bwd
    Tq, Lt, H, d = 30, 17, 2, 8
    q, kt, vt, g = _rand((Tq, H, d), 84), _rand((Lt, H, d), 85), _rand((Lt, H, d), 86), _rand((Tq, H, d), 87)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, kt, vt))
    s = torch.einsum("thd,shd->hts", tq, tk) * 0.3
    o = torch.einsum("hts,shd->thd", torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(g))
    dq, dk, dv = attn_cross_bwd(q, kt, vt, g, scale=0.3)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    np.testing.assert_allclose(dv.sum(axis=0), g.sum(axis=0), atol=1e-11)
