"""Plain float64 gradients of frame-block-causal attention (test infrastructure only).

Source: "DiT as Real-Time Rerenderer: Streaming Video Stylization with
Autoregressive Diffusion Transformer" (RTR-DiT notes).  Key Designs 2 defines
Attn(Q, K, V) = softmax(Q K^T / sqrt(d) + M) V with the frame mask M; Key
Designs 3 and "Loss & Training" post-train the causal generator with Self
Forcing + DMD, whose generator gradient passes back through every such
attention.  The pages do not print the backward pass, so this module is the
derivative of the Attn equation written out (reading: the exact gradient of
the forward definition, nothing approximated).

With S = Q K^T * scale + M, P = softmax_rows(S), O = P V and an upstream
gradient dO of a scalar loss:

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(dP * P))        (softmax Jacobian, row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q

rowsum(dP * P) for row i equals dO_i . O_i.  Masked entries have P = 0, so they
contribute nothing to any gradient.

Layout as the forward oracle: token-major [tokens, heads, head_dim]; inputs are
upcast to float64 before any arithmetic.  The dense function builds the full
[T, T] matrices per head (T up to a few thousand); the *_rows / *_cols variants
give the same quantities for chosen query rows (dQ) or key columns (dK, dV) at
any T, evaluating the same expressions for those rows or columns only.
"""

import math

import numpy as np

from .attention import visible


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _scale(d, scale):
    return 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else float(scale)


def _probs(s):
    """Row softmax of s (may hold -inf where masked)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attn_block_causal_bwd(q, k, v, do, tokens_per_frame, scale=None):
    """Gradients of the full-sequence form, dense and literal.

    q, k, v, do: [T, H, d].  Returns (dq, dk, dv), each [T, H, d] float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    T, H, d = q.shape
    sc = _scale(d, scale)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    M = np.where(visible(i, j, tokens_per_frame), 0.0, -np.inf)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for h in range(H):
        P = _probs((q[:, h] @ k[:, h].T) * sc + M)
        dv[:, h] = P.T @ do[:, h]
        dP = do[:, h] @ v[:, h].T
        dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
        dq[:, h] = sc * (dS @ k[:, h])
        dk[:, h] = sc * (dS.T @ q[:, h])
    return dq, dk, dv


def attn_bwd_rows(q, k, v, do, tokens_per_frame, rows, heads=None, scale=None):
    """dQ for selected query rows, any T.  Row i uses the keys it sees
    (floor(j/k) <= floor(i/k)).  Returns dq [len(rows), len(heads), d]."""
    T, H, d = q.shape
    heads = list(range(H)) if heads is None else list(heads)
    sc = _scale(d, scale)
    jj = np.arange(k.shape[0])
    out = np.empty((len(rows), len(heads), d))
    for a, h in enumerate(heads):
        kh, vh = _f64(k[:, h]), _f64(v[:, h])
        for b, i in enumerate(rows):
            sel = visible(i, jj, tokens_per_frame)
            p = _probs((_f64(q[i, h]) @ kh[sel].T) * sc)
            dp = vh[sel] @ _f64(do[i, h])
            ds = p * (dp - np.dot(dp, p))
            out[b, a] = sc * (ds @ kh[sel])
    return out


def attn_bwd_cols(q, k, v, do, tokens_per_frame, cols, heads=None, scale=None, group=512):
    """dK and dV for selected key columns, any T.

    Key j is seen by every query i with floor(i/k) >= floor(j/k).  Each such
    row needs its own softmax over all the keys it sees (for P_ij) and
    rowsum(dP * P) (= dO_i . O_i), so the rows are evaluated exactly as in
    attn_bwd_rows, `group` rows at a time to bound memory, and their terms
    summed over i.  Returns (dk, dv), each [len(cols), len(heads), d].
    """
    T, H, d = q.shape
    heads = list(range(H)) if heads is None else list(heads)
    sc = _scale(d, scale)
    kf = tokens_per_frame
    cols = np.asarray(cols)
    first = (int(cols.min()) // kf) * kf          # first row that sees any selected key
    dk = np.zeros((len(cols), len(heads), d))
    dv = np.zeros((len(cols), len(heads), d))
    jj = np.arange(k.shape[0])
    for a, h in enumerate(heads):
        kh, vh = _f64(k[:, h]), _f64(v[:, h])
        for r0 in range(first, T, group):
            ii = np.arange(r0, min(T, r0 + group))
            vis = visible(ii[:, None], jj[None, :], kf)
            s = np.where(vis, (_f64(q[ii, h]) @ kh.T) * sc, -np.inf)
            P = _probs(s)
            dP = _f64(do[ii, h]) @ vh.T
            Dr = np.sum(dP * P, axis=1, keepdims=True)
            Pc = P[:, cols]
            dSc = Pc * (dP[:, cols] - Dr)
            dv[:, a] += Pc.T @ _f64(do[ii, h])
            dk[:, a] += sc * (dSc.T @ _f64(q[ii, h]))
    return dk, dv


def attn_stream_step_bwd(prefix_k, prefix_v, q, k, v, do, tokens_per_frame, scale=None):
    """Gradients of one streaming step (the attention a chunk runs against the
    cached prefix), dense and literal.

    prefix_k/prefix_v: [P, H, d] cached keys/values (anchored reference, then
    the window); q, k, v, do: [C*k, H, d] for the chunk.  Chunk row r sees every
    prefix key and the chunk keys of chunk frames <= its own (tokens_per_frame
    sets the mask unit).  Returns (dq, dk, dv, dk_prefix, dv_prefix), float64.
    """
    pk, pv = _f64(prefix_k), _f64(prefix_v)
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Tq, H, d = q.shape
    P = pk.shape[0]
    sc = _scale(d, scale)
    i = np.arange(Tq)[:, None]
    j = np.arange(Tq)[None, :]
    M = np.concatenate([np.zeros((Tq, P)),
                        np.where(visible(i, j, tokens_per_frame), 0.0, -np.inf)], axis=1)
    kk = np.concatenate([pk, k], axis=0)
    vv = np.concatenate([pv, v], axis=0)
    dq = np.empty_like(q)
    dkk = np.empty_like(kk)
    dvv = np.empty_like(vv)
    for h in range(H):
        Pm = _probs((q[:, h] @ kk[:, h].T) * sc + M)
        dvv[:, h] = Pm.T @ do[:, h]
        dP = do[:, h] @ vv[:, h].T
        dS = Pm * (dP - np.sum(dP * Pm, axis=1, keepdims=True))
        dq[:, h] = sc * (dS @ kk[:, h])
        dkk[:, h] = sc * (dS.T @ q[:, h])
    return dq, dkk[P:], dvv[P:], dkk[:P], dvv[:P]


def attn_cross_bwd(q, k_text, v_text, do, scale=None):
    """Gradients of the text cross-attention (Key Designs 1: the text condition
    enters through cross attention; the generator's post-training sends its
    gradient back through it as through the self-attention), dense and
    literal.  Every query sees every text token, so the mask is empty.

    q, do: [Tq, H, d]; k_text, v_text: [Lt, H, d].
    Returns (dq, dk_text, dv_text), float64.
    """
    q, kk, vv, do = _f64(q), _f64(k_text), _f64(v_text), _f64(do)
    Tq, H, d = q.shape
    sc = _scale(d, scale)
    dq, dk, dv = np.empty_like(q), np.empty_like(kk), np.empty_like(vv)
    for h in range(H):
        P = _probs((q[:, h] @ kk[:, h].T) * sc)
        dv[:, h] = P.T @ do[:, h]
        dP = do[:, h] @ vv[:, h].T
        dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
        dq[:, h] = sc * (dS @ kk[:, h])
        dk[:, h] = sc * (dS.T @ q[:, h])
    return dq, dk, dv
