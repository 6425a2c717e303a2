"""Plain float64 reference for frame-block-causal attention (test infrastructure only).

Source: "DiT as Real-Time Rerenderer: Streaming Video Stylization with
Autoregressive Diffusion Transformer" (RTR-DiT notes), Key Designs 2, the
Attn(Q, K, V) equation: Attn = softmax(Q K^T / sqrt(d) + M) V with
M_ij = 0 when floor(j / k) <= floor(i / k) and -inf otherwise, where d is the
head dimension and k the number of spatial tokens per latent frame.  The notes
flag the printed equation as restored from a garbled cache; this module uses
the restored form as printed (i = query index, j = key index: a token sees every
token of its own latent frame and of all earlier frames).

Key Designs 1 of the same page makes the reference one extra latent frame placed
before the first frame, so it is simply frame 0 of the sequence here.

Layout: every tensor is token-major [tokens, heads, head_dim]; inputs of any
float dtype are upcast to float64 before any arithmetic.  LSE is the natural
log of the softmax denominator including the running max, shape [heads, rows].

Nothing here is blocked, fused or reordered beyond what the equation states:
the dense functions build S = Q K^T * scale, add M, take a max-subtracted
softmax along keys and multiply by V.  The *_rows variants evaluate the same
expression for a chosen set of query rows (one row at a time) so that very
large shapes can be sampled.
"""

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else float(scale)


def visible(i, j, k):
    """Mask predicate of the Attn equation: key j is visible to query i iff
    floor(j / k) <= floor(i / k).  Works elementwise on integer arrays."""
    return (np.asarray(j) // k) <= (np.asarray(i) // k)


def _mask_matrix(Tq, Tk, k, q_offset=0):
    """M of the Attn equation as a dense [Tq, Tk] float64 matrix (0 or -inf).
    Query row r has sequence index q_offset + r."""
    i = np.arange(Tq)[:, None] + q_offset
    j = np.arange(Tk)[None, :]
    return np.where(visible(i, j, k), 0.0, -np.inf)


def _softmax_attend(s, v):
    """softmax over the last axis of s (rows x keys, may hold -inf), times v.
    Returns (out [rows, d], lse [rows])."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    denom = np.sum(e, axis=1, keepdims=True)
    p = e / denom
    return p @ v, (m + np.log(denom))[:, 0]


def attn_block_causal(q, k, v, tokens_per_frame, scale=None):
    """Full-sequence form (training / teacher forcing), dense and literal.

    q, k, v: [T, H, d].  tokens_per_frame >= T gives the bidirectional teacher
    (no mask at all).  Returns (o [T, H, d] float64, lse [H, T] float64).
    Memory is O(T^2) per head: meant for T up to a few thousand.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, d = q.shape
    sc = _default_scale(d, scale)
    M = _mask_matrix(T, T, tokens_per_frame)
    o = np.empty((T, H, d))
    lse = np.empty((H, T))
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * sc + M
        o[:, h, :], lse[h] = _softmax_attend(s, v[:, h, :])
    return o, lse


def attn_brute_force(q, k, v, tokens_per_frame, scale=None):
    """The same quantity with explicit per-query, per-key Python loops and the
    mask applied as a condition; for tiny inputs only.  Returns (o, lse)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, d = q.shape
    sc = _default_scale(d, scale)
    o = np.zeros((T, H, d))
    lse = np.zeros((H, T))
    for h in range(H):
        for i in range(T):
            logits = []
            for j in range(T):
                if (j // tokens_per_frame) <= (i // tokens_per_frame):
                    dot = 0.0
                    for c in range(d):
                        dot += q[i, h, c] * k[j, h, c]
                    logits.append((j, dot * sc))
            mx = max(t for _, t in logits)
            weights = [(j, math.exp(t - mx)) for j, t in logits]
            denom = sum(w for _, w in weights)
            for j, w in weights:
                for c in range(d):
                    o[i, h, c] += (w / denom) * v[j, h, c]
            lse[h, i] = mx + math.log(denom)
    return o, lse


def attn_rows(q, k, v, tokens_per_frame, rows, heads=None, scale=None):
    """Full-sequence form evaluated for selected query rows only (any T).

    Each selected row i uses the keys j with floor(j/k) <= floor(i/k), i.e. the
    mask applied by selection.  Returns (o [len(rows), len(heads), d],
    lse [len(heads), len(rows)]).
    """
    T, H, d = q.shape
    heads = list(range(H)) if heads is None else list(heads)
    sc = _default_scale(d, scale)
    jj = np.arange(k.shape[0])
    o = np.empty((len(rows), len(heads), d))
    lse = np.empty((len(heads), len(rows)))
    for a, h in enumerate(heads):
        kh = _f64(k[:, h, :])
        vh = _f64(v[:, h, :])
        for b, i in enumerate(rows):
            sel = visible(i, jj, tokens_per_frame)
            s = (_f64(q[i, h, :]) @ kh[sel].T)[None, :] * sc
            out, l = _softmax_attend(s, vh[sel])
            o[b, a] = out[0]
            lse[a, b] = l[0]
    return o, lse


def _stream_keys(prefix_k, prefix_v, chunk_k, chunk_v):
    pk = _f64(prefix_k)
    pv = _f64(prefix_v)
    return (np.concatenate([pk, _f64(chunk_k)], axis=0),
            np.concatenate([pv, _f64(chunk_v)], axis=0),
            pk.shape[0])


def attn_stream_step(prefix_k, prefix_v, q, k, v, tokens_per_frame, scale=None):
    """Streaming form for one chunk, dense and literal.

    prefix_k/prefix_v: [P, H, d], the cached keys/values in logical order
    (anchored reference frame(s) first, then the rolling window oldest to
    newest; P may be 0).  q, k, v: [C*k, H, d], the current chunk's own tokens.
    Query row r of the chunk lies in chunk frame floor(r/k) and sees every
    prefix key plus the chunk keys of chunk frames <= its own: the Attn mask
    with the chunk placed right after the prefix, whose own queries are absent.
    Returns (o [C*k, H, d], lse [H, C*k]).
    """
    q = _f64(q)
    Tq, H, d = q.shape
    kk, vv, P = _stream_keys(prefix_k, prefix_v, k, v)
    sc = _default_scale(d, scale)
    kf = tokens_per_frame
    # Prefix keys are always visible; chunk keys obey the frame mask with
    # chunk-local indices.
    M = np.concatenate([np.zeros((Tq, P)), _mask_matrix(Tq, kk.shape[0] - P, kf)], axis=1)
    o = np.empty((Tq, H, d))
    lse = np.empty((H, Tq))
    for h in range(H):
        s = (q[:, h, :] @ kk[:, h, :].T) * sc + M
        o[:, h, :], lse[h] = _softmax_attend(s, vv[:, h, :])
    return o, lse


def attn_stream_rows(prefix_k, prefix_v, q, k, v, tokens_per_frame, rows, heads=None,
                     scale=None):
    """attn_stream_step for selected chunk query rows only (any size)."""
    Tq, H, d = q.shape
    heads = list(range(H)) if heads is None else list(heads)
    P = prefix_k.shape[0]
    sc = _default_scale(d, scale)
    jc = np.arange(k.shape[0])
    o = np.empty((len(rows), len(heads), d))
    lse = np.empty((len(heads), len(rows)))
    for a, h in enumerate(heads):
        pk = _f64(prefix_k[:, h, :])
        pv = _f64(prefix_v[:, h, :])
        ck = _f64(k[:, h, :])
        cv = _f64(v[:, h, :])
        for b, i in enumerate(rows):
            sel = visible(i, jc, tokens_per_frame)
            keys = np.concatenate([pk, ck[sel]], axis=0)
            vals = np.concatenate([pv, cv[sel]], axis=0)
            s = (_f64(q[i, h, :]) @ keys.T)[None, :] * sc
            out, l = _softmax_attend(s, vals)
            o[b, a] = out[0]
            lse[a, b] = l[0]
    return o, lse


def attn_cross(q, k_text, v_text, scale=None):
    """Cross-attention of video tokens to text tokens (RTR-DiT notes, Key
    Designs 1: text is encoded by T5 and injected through cross attention),
    dense and literal:
    softmax(Q K^T * scale) V with no mask -- every query sees every text token.

    q: [Tq, H, d]; k_text, v_text: [Lt, H, d], Lt >= 1.
    Returns (o [Tq, H, d], lse [H, Tq]).
    """
    q, kk, vv = _f64(q), _f64(k_text), _f64(v_text)
    Tq, H, d = q.shape
    sc = _default_scale(d, scale)
    o = np.empty((Tq, H, d))
    lse = np.empty((H, Tq))
    for h in range(H):
        o[:, h, :], lse[h] = _softmax_attend((q[:, h, :] @ kk[:, h, :].T) * sc, vv[:, h, :])
    return o, lse
