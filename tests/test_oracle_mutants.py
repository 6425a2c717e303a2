"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutant below is a plausible slip in the float64 oracle -- a flipped mask
comparison, transposed mask indices, a wrong scale, a dropped LSE term, the
wrong end of the window evicted, a keep-recent slice that keeps everything for
keep = 0.  The test patches it in and checks that the pins in test_oracle.py
notice.
"""

import numpy as np
import pytest

import oracle.attention as A
import oracle.listkv as L
from tests import test_oracle as pins


def _fails(fn, *args):
    try:
        with np.errstate(all="ignore"):
            fn(*args)
    except Exception:  # AssertionError or a numeric failure both count
        return True
    return False


def _strict_mask(i, j, k):
    return (np.asarray(j) // k) < (np.asarray(i) // k)


def _transposed_mask(i, j, k):
    return (np.asarray(i) // k) <= (np.asarray(j) // k)


def _wrong_scale(d, scale):
    return 1.0 / d


def _lse_without_max(s, v):
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    den = np.sum(e, axis=1, keepdims=True)
    return (e / den) @ v, np.log(den)[:, 0]


def _no_normalise(s, v):
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    den = np.sum(e, axis=1, keepdims=True)
    return e @ v, (m + np.log(den))[:, 0]


ATTN_MUTANTS = [
    ("visible", _strict_mask),
    ("visible", _transposed_mask),
    ("_default_scale", _wrong_scale),
    ("_softmax_attend", _lse_without_max),
    ("_softmax_attend", _no_normalise),
]

ATTN_PINS = [
    (pins.test_mask_matches_hand_table, ("mask_k3_T7.txt",)),
    (pins.test_k1_is_token_causal_attention, (37, 2, 16)),
    (pins.test_lse_matches_library_logsumexp, ()),
    (pins.test_closed_form_frame_label_mean, (5, 7)),
    (pins.test_causality_is_bitwise, ()),
]


@pytest.mark.parametrize("name,fn", ATTN_MUTANTS, ids=lambda x: getattr(x, "__name__", x))
def test_attention_mutant_is_caught(monkeypatch, name, fn):
    # sanity: all pins pass on the real oracle
    for pin, args in ATTN_PINS:
        assert not _fails(pin, *args)
    monkeypatch.setattr(A, name, fn)
    assert any(_fails(pin, *args) for pin, args in ATTN_PINS)


def _append_evict_newest(self, k_frames, v_frames):
    for f in range(len(k_frames)):
        self.window.append((self.next_frame_id, k_frames[f], v_frames[f]))
        self.next_frame_id += 1
        while len(self.window) > self.W:
            self.window.pop()


_orig_reset = L.ListKV.reset_ref


def _reset_negative_slice(self, mode, k_ref=None, v_ref=None, keep_recent=1):
    win = list(self.window)
    _orig_reset(self, mode, k_ref, v_ref, keep_recent=-1)
    if keep_recent >= 0:
        self.window = win[-keep_recent:]


def _reset_keeps_oldest(self, mode, k_ref=None, v_ref=None, keep_recent=1):
    win = list(self.window)
    _orig_reset(self, mode, k_ref, v_ref, keep_recent=-1)
    if keep_recent >= 0:
        self.window = win[:keep_recent]


@pytest.mark.parametrize("name,fn", [("append", _append_evict_newest),
                                     ("reset_ref", _reset_negative_slice),
                                     ("reset_ref", _reset_keeps_oldest)],
                         ids=lambda x: getattr(x, "__name__", x))
def test_listkv_mutant_is_caught(monkeypatch, name, fn):
    assert not _fails(pins.test_listkv_matches_hand_schedule)
    monkeypatch.setattr(L.ListKV, name, fn)
    assert _fails(pins.test_listkv_matches_hand_schedule)


# Position-aware reference (oracle/rope.py): a placement one frame off, and
# the two plausible slips in the pair frequencies.
import oracle.rope as RP  # noqa: E402
from tests import test_oracle_rope as rope_pins  # noqa: E402


def _shift_one_late(oldest_position, ref_frames):
    return int(oldest_position) - int(ref_frames) + 1


def _angles_two_i(positions, pairs, base):
    i = np.arange(pairs, dtype=np.float64)
    return np.asarray(positions, dtype=np.float64)[:, None] * np.power(float(base), -2 * i / pairs)[None, :]


def _angles_positive(positions, pairs, base):
    i = np.arange(pairs, dtype=np.float64)
    return np.asarray(positions, dtype=np.float64)[:, None] * np.power(float(base), i / pairs)[None, :]


ROPE_PINS = [
    (rope_pins.test_rotation_closed_forms, ()),
    (rope_pins.test_pair_frequencies_hand_values, ()),
    (rope_pins.test_reference_placement_empty_window_first_chunk, ()),
    (rope_pins.test_reference_placement_after_a_switch_and_a_rolled_window, ()),
]


@pytest.mark.parametrize("name,fn", [("reference_shift", _shift_one_late),
                                     ("rope_angles", _angles_two_i),
                                     ("rope_angles", _angles_positive)],
                         ids=lambda x: getattr(x, "__name__", x))
def test_rope_mutant_is_caught(monkeypatch, name, fn):
    for pin, args in ROPE_PINS:
        assert not _fails(pin, *args)
    monkeypatch.setattr(RP, name, fn)
    assert any(_fails(pin, *args) for pin, args in ROPE_PINS)
