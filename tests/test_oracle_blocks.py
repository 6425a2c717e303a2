"""Pins for the chunk-level mask and several anchored references.

Chunk-level causality (the streaming VACE notes: fixed-size chunks, each
attending to itself and to earlier frames) is the streaming step of the Attn
equation (RTR-DiT notes, Key Designs 2) with a block of frames as the mask
unit, i.e. oracle.attn_stream_step with tokens_per_frame = block tokens.  It is
pinned here to the separately pinned unmasked cross-attention oracle over the
exact key set each row must see.  Several references (RTR-DiT notes, an
improvement direction: anchoring more than one reference) are extra frames
at the front of the cache prefix."""

import numpy as np
import pytest

import oracle
from oracle import ListKV, REF_KEEP, REF_REPLACE


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("C,B", [(3, 3), (3, 2), (4, 2), (2, 5)])
def test_blocked_step_equals_cross_over_visible_keys(C, B):
    k, H, d, P = 6, 2, 8, 13
    pk, pv = _rand((P, H, d), 1), _rand((P, H, d), 2)
    q, ck, cv = _rand((C * k, H, d), 3), _rand((C * k, H, d), 4), _rand((C * k, H, d), 5)
    blk = min(B, C) * k
    o, lse = oracle.attn_stream_step(pk, pv, q, ck, cv, blk)
    for r in range(C * k):
        end = (r // blk + 1) * blk          # chunk keys of blocks <= the row's block
        end = min(end, C * k)
        keys = np.concatenate([pk, ck[:end]])
        vals = np.concatenate([pv, cv[:end]])
        ro, rl = oracle.attn_cross(q[r:r + 1], keys, vals)
        np.testing.assert_allclose(o[r], ro[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, r], rl[:, 0], rtol=1e-12)


def test_whole_chunk_block_is_unmasked_over_prefix_and_chunk():
    k, H, d, C = 5, 1, 4, 3
    pk, pv = _rand((2 * k, H, d), 6), _rand((2 * k, H, d), 7)
    q, ck, cv = _rand((C * k, H, d), 8), _rand((C * k, H, d), 9), _rand((C * k, H, d), 10)
    o, _ = oracle.attn_stream_step(pk, pv, q, ck, cv, C * k)
    ro, _ = oracle.attn_cross(q, np.concatenate([pk, ck]), np.concatenate([pv, cv]))
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-13)


def test_several_references_lead_the_prefix():
    """Hand schedule: 3 references then 2 window frames; a switch to 1
    reference keeps the newest frame; KEEP keeps the references."""
    k, H, d = 2, 1, 1
    kv = ListKV(2)
    refs = np.arange(3 * k).reshape(3, k, H, d) + 100.0
    kv.reset_ref(REF_REPLACE, refs, -refs, keep_recent=-1)
    for f in range(3):
        fr = np.full((1, k, H, d), float(f))
        kv.append(fr, -fr)
    pk, pv = kv.prefix(k, H, d)
    expect = [100, 101, 102, 103, 104, 105, 1, 1, 2, 2]
    assert pk[:, 0, 0].tolist() == expect and pv[:, 0, 0].tolist() == [-x for x in expect]
    assert kv.ref_frames() == 3
    kv.reset_ref(REF_REPLACE, refs[:1] + 50, refs[:1] + 50, keep_recent=1)
    pk, _ = kv.prefix(k, H, d)
    assert pk[:, 0, 0].tolist() == [150, 151, 2, 2] and kv.ref_frames() == 1
    kv.reset_ref(REF_KEEP, keep_recent=-1)
    assert kv.prefix(k, H, d)[0][:, 0, 0].tolist() == [150, 151, 2, 2]
