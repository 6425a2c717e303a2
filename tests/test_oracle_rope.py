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
