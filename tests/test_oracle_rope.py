"""Pins of the temporal rotary encoding and of the reference position that
follows the rolling window (see oracle/rope.py for the readings)."""

import numpy as np

import oracle
from oracle import ListKV, REF_REPLACE
from oracle.rope import reference_shift, rope_rotate


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rotation_closed_forms():
    T, H, d, P = 7, 2, 16, 5
    x = _rand((T, H, d), 1)
    pos = np.arange(T) * 3 - 4
    y = rope_rotate(x, pos, P)
    # norms of every pair (hence of every token) are kept; untouched dims are equal
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(y[:, :, 2 * P:], x[:, :, 2 * P:])
    # composition: R(a) R(b) = R(a + b); R(0) = identity; R(-a) inverts
    np.testing.assert_allclose(rope_rotate(rope_rotate(x, pos, P), pos + 5, P), rope_rotate(x, 2 * pos + 5, P),
                               atol=1e-12)
    np.testing.assert_allclose(rope_rotate(x, np.zeros(T), P), x, atol=0)
    np.testing.assert_allclose(rope_rotate(y, -pos, P), x, atol=1e-12)
    # a hand value: pair 0 rotates by the position itself (frequency 1)
    e = np.zeros((1, 1, d))
    e[0, 0, 0] = 1.0
    r = rope_rotate(e, [np.pi / 2], P)
    np.testing.assert_allclose(r[0, 0, :2], [0.0, 1.0], atol=1e-15)


def test_scores_depend_on_position_difference_only():
    H, d, P = 1, 8, 4
    q, k = _rand((1, H, d), 2), _rand((1, H, d), 3)
    s = lambda m, n: float(np.sum(rope_rotate(q, [m], P) * rope_rotate(k, [n], P)))
    for m, n in [(5, 2), (105, 102), (-7, -10)]:
        np.testing.assert_allclose(s(m, n), s(3, 0), rtol=1e-10)


def test_reference_follows_the_window():
    """A rollout whose frames repeat with period 1: once the window is full, the
    step's output must not depend on how far the rollout has gone, because the
    reference is re-placed in front of the oldest visible frame and every other
    key keeps its position relative to the chunk."""
    k, H, d, W, C, P, R = 4, 1, 8, 3, 2, 3, 1
    kv = ListKV(W)
    ref_raw = _rand((R, k, H, d), 4)
    ref_rot = rope_rotate(ref_raw.reshape(-1, H, d), np.repeat(np.arange(R), k), P).reshape(R, k, H, d)
    kv.reset_ref(REF_REPLACE, ref_rot, _rand((R, k, H, d), 5), keep_recent=-1)
    fk, fv, fq = _rand((k, H, d), 6), _rand((k, H, d), 7), _rand((k, H, d), 8)

    def step(follow=True):
        base = kv.next_frame_id                 # chunk frame c has id base + c
        pos = lambda fid: np.full(k, fid + R)   # temporal position of a frame
        cq = np.concatenate([rope_rotate(fq, pos(base + c), P) for c in range(C)])
        ck = np.concatenate([rope_rotate(fk, pos(base + c), P) for c in range(C)])
        cv = np.concatenate([fv] * C)
        oldest = (kv.frame_ids()[0] if kv.frame_ids() else base) + R
        shift = reference_shift(oldest, R) if follow else 0
        pk, pv = kv.prefix(k, H, d)
        pk = pk.copy()
        pk[:R * k] = rope_rotate(pk[:R * k], np.full(R * k, shift), P)
        o, _ = oracle.attn_stream_step(pk, pv, cq, ck, cv, k)
        kv.append(ck.reshape(C, k, H, d), cv.reshape(C, k, H, d))
        return o

    outs = [step() for _ in range(8)]
    for o in outs[3:]:
        np.testing.assert_allclose(o, outs[2], rtol=1e-10, atol=1e-12)
    # without the shift the reference drifts away and the outputs change
    assert not np.allclose(step(follow=False), outs[2], atol=1e-6)


def test_pair_frequencies_hand_values():
    """Pairs i >= 1 rotate at position * base^(-i / pairs) -- the usual rotary
    frequencies base^(-2i / n) over the n = 2 * pairs rotated dimensions.  With
    base 16 and 4 pairs the frequencies are 1, 1/2, 1/4, 1/8; at position 4 pi
    the angles are 4 pi, 2 pi, pi and pi / 2, so the unit vector (1, 0) of each
    pair goes to (1, 0), (1, 0), (-1, 0) and (0, 1); at position 2 pi / 3 pair 1
    turns by pi / 3, to (1/2, sqrt(3)/2)."""
    from oracle import rope as R
    P, d = 4, 10
    e = np.zeros((1, 1, d))
    e[0, 0, 0:2 * P:2] = 1.0
    e[0, 0, 2 * P:] = 7.0  # not rotated
    r = R.rope_rotate(e, [4 * np.pi], P, base=16.0)[0, 0]
    want = [1.0, 0.0, 1.0, 0.0, -1.0, 0.0, 0.0, 1.0, 7.0, 7.0]
    np.testing.assert_allclose(r, want, atol=1e-12)
    r = R.rope_rotate(e, [2 * np.pi / 3], P, base=16.0)[0, 0]
    np.testing.assert_allclose(r[2:4], [0.5, np.sqrt(3.0) / 2.0], atol=1e-12)
    # the second element of a pair rotates towards minus the first: (0, 1) at pi / 2 -> (-1, 0)
    f = np.zeros((1, 1, d))
    f[0, 0, 7] = 1.0
    r = R.rope_rotate(f, [4 * np.pi], P, base=16.0)[0, 0]
    np.testing.assert_allclose(r[6:8], [-1.0, 0.0], atol=1e-12)


def _placement_case(R_frames, W, fill, base_id, seed):
    """Stream step with the reference re-encoded by the oracle's placement
    against the full-form oracle over [reference frames | window frames |
    chunk frames] encoded at consecutive positions 0, 1, 2, ... (the reference
    one frame before the first frame it precedes, Key Designs 1), on the chunk
    rows."""
    from oracle import rope as R
    rng = np.random.default_rng(seed)
    k, H, d, C, P = 3, 2, 8, 2, 3
    n = lambda *s: rng.standard_normal(s)
    raw_ref_k, ref_v = n(R_frames, k, H, d), n(R_frames, k, H, d)
    # frames in generation order; frame id f is encoded at position f + offset
    offset = 5
    nfr = base_id + C
    fk, fv, fq = n(nfr, k, H, d), n(nfr, k, H, d), n(nfr, k, H, d)
    enc = lambda x, p: R.rope_rotate(x, np.full(x.shape[0], p), P)
    win_ids = list(range(base_id - fill, base_id))
    chunk_ids = list(range(base_id, base_id + C))
    oldest = (win_ids[0] if win_ids else base_id) + offset
    # streaming form: cached window keys encoded at their own positions; the
    # reference, stored at positions 0..R-1, re-encoded in front of the oldest
    ref0 = np.concatenate([enc(raw_ref_k[r], r) for r in range(R_frames)])
    ref_placed = R.rope_rotate(ref0, np.full(ref0.shape[0], R.reference_shift(oldest, R_frames)), P)
    pk = np.concatenate([ref_placed] + [enc(fk[f], f + offset) for f in win_ids])
    pv = np.concatenate([ref_v.reshape(-1, H, d)] + [fv[f] for f in win_ids])
    cq = np.concatenate([enc(fq[f], f + offset) for f in chunk_ids])
    ck = np.concatenate([enc(fk[f], f + offset) for f in chunk_ids])
    cv = np.concatenate([fv[f] for f in chunk_ids])
    o, lse = oracle.attn_stream_step(pk, pv, cq, ck, cv, k)
    # full form over the short sequence at consecutive positions from 0
    seq = [(raw_ref_k[r], ref_v[r], None) for r in range(R_frames)]
    seq += [(fk[f], fv[f], fq[f]) for f in win_ids + chunk_ids]
    K = np.concatenate([enc(s[0], p) for p, s in enumerate(seq)])
    V = np.concatenate([s[1] for s in seq])
    Q = np.concatenate([enc(s[2], p) if s[2] is not None else np.zeros((k, H, d))
                        for p, s in enumerate(seq)])
    fo, flse = oracle.attn_block_causal(Q, K, V, k)
    rows = slice(len(seq) * k - C * k, len(seq) * k)
    # reference frames beyond the first are separate frames of the full form,
    # which changes only the reference rows; every chunk row sees all of them
    np.testing.assert_allclose(o, fo[rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, flse[:, rows], rtol=1e-10, atol=1e-12)


def test_reference_placement_empty_window_first_chunk():
    _placement_case(R_frames=1, W=3, fill=0, base_id=0, seed=11)
    _placement_case(R_frames=2, W=3, fill=0, base_id=0, seed=12)


def test_reference_placement_after_a_switch_and_a_rolled_window():
    # empty window later in the stream (a switch that keeps no frame)
    _placement_case(R_frames=1, W=3, fill=0, base_id=7, seed=13)
    # a rolled window: frames 4..6 cached, chunk 7..8
    _placement_case(R_frames=1, W=3, fill=3, base_id=7, seed=14)
    _placement_case(R_frames=2, W=3, fill=2, base_id=9, seed=15)
