"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
rejects bad arguments before touching the device, and its host-side ring
metadata matches the oracle's literal list window under random schedules.

No call here reaches a kernel launch: argument checks fail first, and the
metadata paths used (in-place commit, reference KEEP/CLEAR/in-place REPLACE,
state snapshots) never touch the device.
"""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from causal_attention_frame_amd import rtr
from oracle import ListKV, REF_CLEAR, REF_KEEP, REF_REPLACE

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "rtr_attn.h")
FAKE = 0x7F0000000000          # a 16-byte aligned address that is never dereferenced
MB = 1 << 20


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(rtr_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 12
    L = rtr.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(rtr._SIGNATURES), "binding and header disagree"
    assert rtr.rtr_version() == 100


def test_binding_arity_matches_header():
    """Every prototype in the header takes as many arguments as the ctypes
    binding declares for it."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decls = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(rtr_\w+)\s*\(([^;]*?)\)\s*;", text, flags=re.M | re.S)
    assert len(decls) == len(rtr._SIGNATURES)
    for name, args in decls:
        n = 0 if args.strip() in ("", "void") else len(args.split(","))
        assert n == len(rtr._SIGNATURES[name][1]), name


def test_status_strings():
    L = rtr.lib()
    for code in (0, -1, -2, -3, -4):
        assert L.rtr_status_string(code)
    assert L.rtr_status_string(-99) == b"unknown status"


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE + MB, v=FAKE + 2 * MB, o=FAKE + 3 * MB, lse=None, T=64, H=2, d=128,
             kpf=16, ind=rtr.RTR_BF16, outd=rtr.RTR_BF16, scale=0.0, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return rtr.lib().rtr_attn_block_causal(a["q"], a["k"], a["v"], a["o"], a["lse"], a["T"],
                                           a["H"], a["d"], a["kpf"], a["ind"], a["outd"],
                                           a["scale"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), rtr.RTR_EINVAL),
    (dict(T=1 << 31), rtr.RTR_EINVAL),
    (dict(H=0), rtr.RTR_EINVAL),
    (dict(kpf=0), rtr.RTR_EINVAL),
    (dict(d=96), rtr.RTR_EUNSUPPORTED),
    (dict(d=256), rtr.RTR_EUNSUPPORTED),
    (dict(ind=7), rtr.RTR_EINVAL),
    (dict(ind=rtr.RTR_F32, outd=rtr.RTR_BF16), rtr.RTR_EUNSUPPORTED),
    (dict(q=None), rtr.RTR_EINVAL),
    (dict(o=None), rtr.RTR_EINVAL),
    (dict(k=FAKE + MB + 2), rtr.RTR_EINVAL),          # misaligned
    (dict(lse=FAKE + 4 * MB + 4), rtr.RTR_EINVAL),    # misaligned lse
    (dict(o=FAKE + 64), rtr.RTR_EINVAL),              # o overlaps q
    (dict(lse=FAKE + 3 * MB), rtr.RTR_EINVAL),        # lse overlaps o
    (dict(scale=float("inf")), rtr.RTR_EINVAL),
    (dict(ws=FAKE + 8 * MB + 8, ws_bytes=MB), rtr.RTR_EINVAL),  # misaligned workspace
    (dict(ws=FAKE + 2 * MB, ws_bytes=MB), rtr.RTR_EINVAL),      # workspace overlaps v
])
def test_block_causal_rejects_before_launch(kw, code):
    assert _attn(**kw) == code
    assert rtr.lib().rtr_last_error()


def test_workspace_size_args():
    L = rtr.lib()
    n = ctypes.c_size_t(7)
    assert L.rtr_attn_workspace_size(64, rtr.RTR_BF16, ctypes.byref(n)) == rtr.RTR_OK and n.value == 0
    assert L.rtr_attn_workspace_size(128, rtr.RTR_F32, ctypes.byref(n)) == rtr.RTR_OK and n.value == 0
    assert L.rtr_attn_workspace_size(96, rtr.RTR_BF16, ctypes.byref(n)) == rtr.RTR_EUNSUPPORTED
    assert L.rtr_attn_workspace_size(128, 9, ctypes.byref(n)) == rtr.RTR_EINVAL
    assert L.rtr_attn_workspace_size(128, rtr.RTR_BF16, None) == rtr.RTR_EINVAL


def test_block_causal_empty_is_noop():
    assert _attn(T=0, q=None, k=None, v=None, o=None) == rtr.RTR_OK


def _cache(W=4, R=1, kpf=8, H=2, d=64, dtype=rtr.RTR_BF16, N=None):
    fb = kpf * H * d * (2 if dtype == rtr.RTR_BF16 else 4)
    base = FAKE
    return rtr.KVCache(base, base + 64 * fb + 4096, base + 128 * fb + 8192,
                       base + 130 * fb + 12288, W, R, kpf, H, d, dtype, ring_slots=N)


@pytest.mark.parametrize("args,code", [
    (dict(W=-1), rtr.RTR_EUNSUPPORTED),
    (dict(W=rtr.RTR_MAX_WINDOW + 1), rtr.RTR_EUNSUPPORTED),
    (dict(R=rtr.RTR_MAX_REF + 1), rtr.RTR_EUNSUPPORTED),
    (dict(kpf=0), rtr.RTR_EINVAL),
    (dict(d=80), rtr.RTR_EUNSUPPORTED),
    (dict(W=4, N=3), rtr.RTR_EUNSUPPORTED),             # fewer ring slots than window frames
    (dict(W=4, N=rtr.RTR_MAX_WINDOW + 1), rtr.RTR_EUNSUPPORTED),
])
def test_create_rejects(args, code):
    with pytest.raises(rtr.RtrError) as e:
        _cache(**args)
    assert e.value.code == code


def test_create_rejects_overlapping_buffers():
    with pytest.raises(rtr.RtrError) as e:
        rtr.KVCache(FAKE, FAKE + 128, FAKE + 100 * MB, FAKE + 200 * MB, 4, 1, 8, 2, 64, rtr.RTR_BF16)
    assert e.value.code == rtr.RTR_EINVAL


def _state(kv):
    return rtr.rtr_kv_get_state(kv).as_dict()


def test_failed_calls_change_nothing():
    kv = _cache(W=3)
    rtr.rtr_kv_commit_inplace(kv, 5)
    rtr.rtr_kv_reset_ref(kv, rtr.RTR_REF_REPLACE, None, None, 1, -1)
    before = _state(kv)
    L = rtr.lib()
    h = kv.handle
    assert L.rtr_kv_append_evict(h, None, FAKE, 1, None) == rtr.RTR_EINVAL
    assert L.rtr_kv_append_evict(h, FAKE + 3, FAKE + 64 * MB, 1, None) == rtr.RTR_EINVAL
    assert L.rtr_kv_append_evict(h, FAKE, FAKE + 64 * MB, 1, None) == rtr.RTR_EINVAL  # overlaps ring
    assert L.rtr_kv_append_evict(h, FAKE, FAKE, -1, None) == rtr.RTR_EINVAL
    assert L.rtr_kv_reset_ref(h, 9, None, None, 1, 1, None) == rtr.RTR_EINVAL
    assert L.rtr_kv_reset_ref(h, rtr.RTR_REF_REPLACE, None, None, 2, 1, None) == rtr.RTR_EINVAL
    assert L.rtr_kv_reset_ref(h, rtr.RTR_REF_REPLACE, FAKE + 900 * MB, None, 1, 1, None) == rtr.RTR_EINVAL
    assert L.rtr_kv_reset_ref(h, rtr.RTR_REF_KEEP, None, None, 0, -2, None) == rtr.RTR_EINVAL
    assert L.rtr_attn_stream_step(h, FAKE + 900 * MB, FAKE + 901 * MB, FAKE + 902 * MB,
                                  FAKE + 903 * MB, None, 0, 0, 0.0, None, 0, None) == rtr.RTR_EUNSUPPORTED
    assert L.rtr_attn_stream_step(h, FAKE + 900 * MB, FAKE + 901 * MB, FAKE + 902 * MB,
                                  FAKE, None, 1, 0, 0.0, None, 0, None) == rtr.RTR_EINVAL  # o over ring
    assert L.rtr_attn_stream_step(h, FAKE + 900 * MB, FAKE + 901 * MB, FAKE + 902 * MB,
                                  FAKE + 903 * MB, None, 1, 0, 0.0, FAKE + 1024, MB,
                                  None) == rtr.RTR_EINVAL  # workspace over the ring
    assert L.rtr_attn_stream_step_blocked(h, FAKE + 900 * MB, FAKE + 901 * MB, FAKE + 902 * MB,
                                          FAKE + 903 * MB, None, 1, 0, 0, 0.0, None, 0,
                                          None) == rtr.RTR_EINVAL  # block_frames 0
    assert L.rtr_attn_stream_step(h, None, FAKE + 901 * MB, FAKE + 902 * MB,
                                  FAKE + 903 * MB, None, 1, 0, 0.0, None, 0, None) == rtr.RTR_EINVAL
    assert L.rtr_attn_stream_step(None, FAKE, FAKE, FAKE, FAKE, None, 1, 0, 0.0,
                                  None, 0, None) == rtr.RTR_EINVAL
    bad = rtr.rtr_kv_get_state(kv)
    bad.count = 2
    bad.frame_id[1] = bad.frame_id[0]          # ids must increase
    with pytest.raises(rtr.RtrError):
        rtr.rtr_kv_set_state(kv, bad)
    bad = rtr.rtr_kv_get_state(kv)
    bad.window_frames = 5
    with pytest.raises(rtr.RtrError):
        rtr.rtr_kv_set_state(kv, bad)
    assert _state(kv) == before


def test_reference_replace_needs_capacity():
    kv = _cache(R=0)
    with pytest.raises(rtr.RtrError) as e:
        rtr.rtr_kv_reset_ref(kv, rtr.RTR_REF_REPLACE, None, None, 1, 1)
    assert e.value.code == rtr.RTR_ESTATE


# ------------------------------------------------------------ ring vs ListKV
_op = st.one_of(
    st.tuples(st.just("append"), st.integers(0, 9)),
    st.tuples(st.just("reset"), st.sampled_from([REF_KEEP, REF_REPLACE, REF_CLEAR]),
              st.integers(-1, 6)),
)


def _check_against(kv, ref):
    s = _state(kv)
    assert s["count"] == len(ref.window)
    assert s["frame_id"] == ref.frame_ids()
    assert s["next_frame_id"] == ref.next_frame_id
    assert s["ref_frames"] == ref.ref_frames()
    assert s["ref_generation"] == ref.ref_generation
    N = s["ring_slots"]
    # physical slots: distinct, in range, a ring walk from head over the N slots
    assert len(set(s["slot"])) == len(s["slot"])
    assert all(0 <= x < max(N, 1) for x in s["slot"])
    assert s["slot"] == [(s["head"] + p) % N for p in range(s["count"])] if N else s["slot"] == []


@settings(max_examples=300, deadline=None)
@given(W=st.integers(0, 7), spare=st.integers(0, 3), ops=st.lists(_op, max_size=40))
def test_ring_metadata_matches_listkv(W, spare, ops):
    """The window (ids, order, eviction) follows the list oracle for any number
    of ring slots N = W + spare; an append of at most `spare` frames writes no
    slot of the window before it, so it can run beside a step of that window."""
    kv = _cache(W=W, N=W + spare)
    ref = ListKV(W)
    z = np.zeros((1, 1, 1, 1))
    for op in ops:
        if op[0] == "append":
            n = op[1]
            before = set(_state(kv)["slot"])
            predicted = rtr.rtr_kv_next_slots(kv, n)
            if n <= spare:
                assert not before & {p for p in predicted if p >= 0}
            rtr.rtr_kv_commit_inplace(kv, n)
            ref.append(np.zeros((n, 1, 1, 1)), np.zeros((n, 1, 1, 1)))
            s = _state(kv)
            # each surviving new frame sits where next_slots said it would
            survivors = [p for p in predicted if p >= 0]
            assert len(survivors) == min(n, W)
            if survivors:
                assert s["slot"][-len(survivors):] == survivors
            assert predicted[:n - len(survivors)] == [-1] * (n - len(survivors))
        else:
            _, mode, keep = op
            rtr.rtr_kv_reset_ref(kv, mode, None, None, 1, keep)
            ref.reset_ref(mode, z, z, keep_recent=keep)
        _check_against(kv, ref)


def test_ring_matches_hand_schedule_file():
    from tests.test_oracle import _read_schedule, MODES
    W, ops = _read_schedule()
    kv = _cache(W=W)
    for op, ids, ref_gen in ops:
        if op[0] == "append":
            rtr.rtr_kv_commit_inplace(kv, int(op[1]))
        else:
            rtr.rtr_kv_reset_ref(kv, MODES[op[1]], None, None, 1, int(op[2]))
        s = _state(kv)
        assert s["frame_id"] == ids
        assert (s["ref_generation"] if s["ref_frames"] else 0) == ref_gen


@pytest.mark.parametrize("N", [5, 8])
def test_state_roundtrip_resume(N):
    a = _cache(W=5, N=N)
    rtr.rtr_kv_commit_inplace(a, 7)
    rtr.rtr_kv_reset_ref(a, rtr.RTR_REF_REPLACE, None, None, 1, 2)
    rtr.rtr_kv_commit_inplace(a, 4)
    snap = rtr.rtr_kv_get_state(a)
    b = _cache(W=5, N=N)
    rtr.rtr_kv_set_state(b, snap)
    for kv in (a, b):
        rtr.rtr_kv_commit_inplace(kv, 3)
        rtr.rtr_kv_reset_ref(kv, rtr.RTR_REF_CLEAR, None, None, 1, 1)
        rtr.rtr_kv_commit_inplace(kv, 2)
    assert _state(a) == _state(b)
    # a snapshot of a cache with other ring slots is refused
    c = _cache(W=5, N=13 - N)
    with pytest.raises(rtr.RtrError) as e:
        rtr.rtr_kv_set_state(c, snap)
    assert e.value.code == rtr.RTR_ESTATE


def _bwd(**kw):
    a = dict(q=FAKE, k=FAKE + MB, v=FAKE + 2 * MB, o=FAKE + 3 * MB, lse=FAKE + 4 * MB,
             do=FAKE + 5 * MB, dq=FAKE + 6 * MB, dk=FAKE + 7 * MB, dv=FAKE + 8 * MB, T=64, H=2,
             d=128, kpf=16, dt=rtr.RTR_BF16, scale=0.0, ws=FAKE + 16 * MB, ws_bytes=16 * MB,
             stream=None)
    a.update(kw)
    return rtr.lib().rtr_attn_block_causal_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"],
                                               a["dq"], a["dk"], a["dv"], a["T"], a["H"], a["d"],
                                               a["kpf"], a["dt"], a["scale"], a["ws"],
                                               a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), rtr.RTR_EINVAL),
    (dict(H=0), rtr.RTR_EINVAL),
    (dict(kpf=0), rtr.RTR_EINVAL),
    (dict(d=64), rtr.RTR_EUNSUPPORTED),
    (dict(dt=rtr.RTR_F32), rtr.RTR_EUNSUPPORTED),
    (dict(dt=9), rtr.RTR_EINVAL),
    (dict(T=1 << 20, H=16), rtr.RTR_EUNSUPPORTED),     # T * H * d >= 2^31
    (dict(do=None), rtr.RTR_EINVAL),
    (dict(lse=None), rtr.RTR_EINVAL),
    (dict(dv=None), rtr.RTR_EINVAL),
    (dict(q=FAKE + 8), rtr.RTR_EINVAL),                 # misaligned
    (dict(lse=FAKE + 4 * MB + 2), rtr.RTR_EINVAL),      # misaligned lse
    (dict(dk=FAKE + 64), rtr.RTR_EINVAL),               # dk overlaps q
    (dict(dk=FAKE + 6 * MB + 64), rtr.RTR_EINVAL),      # dk overlaps dq
    (dict(ws=None), rtr.RTR_EINVAL),
    (dict(ws=FAKE + 16 * MB + 16), rtr.RTR_EINVAL),     # workspace not 256-byte aligned
    (dict(ws_bytes=100), rtr.RTR_EINVAL),               # workspace too small
    (dict(ws=FAKE + 5 * MB), rtr.RTR_EINVAL),           # workspace overlaps d_o
    (dict(scale=float("inf")), rtr.RTR_EINVAL),
])
def test_block_causal_bwd_rejects_before_launch(kw, code):
    assert _bwd(**kw) == code
    assert rtr.lib().rtr_last_error()


def test_bwd_workspace_size():
    n = rtr.rtr_attn_bwd_workspace_size(100, 3, 128)
    assert n == 3 * 4 * (256 + 2 * 8192)        # 4 tiles of 32 rows per head
    assert rtr.rtr_attn_bwd_workspace_size(0, 3, 128) == 0
    with pytest.raises(rtr.RtrError):
        rtr.rtr_attn_bwd_workspace_size(100, 3, 64)


def test_text_cache_metadata_and_rejections():
    """Host-side text cache: state changes without touching the device (the
    caller-wrote-it form of reset, and clear) and argument checks."""
    L = rtr.lib()
    h = ctypes.c_void_p()
    assert L.rtr_text_cache_create(ctypes.byref(h), FAKE, FAKE + MB, 0, 2, 128, rtr.RTR_BF16) == rtr.RTR_EINVAL
    assert L.rtr_text_cache_create(ctypes.byref(h), FAKE, FAKE + 64, 16, 2, 128, rtr.RTR_BF16) == rtr.RTR_EINVAL
    assert L.rtr_text_cache_create(ctypes.byref(h), FAKE, FAKE + MB, 16, 2, 96, rtr.RTR_BF16) == rtr.RTR_EUNSUPPORTED
    assert L.rtr_text_cache_create(ctypes.byref(h), FAKE, FAKE + MB, 16, 2, 128, rtr.RTR_BF16) == rtr.RTR_OK
    n, g = ctypes.c_int32(-1), ctypes.c_int64(-1)
    assert L.rtr_text_cache_state(h, ctypes.byref(n), ctypes.byref(g)) == 0 and (n.value, g.value) == (0, 0)
    # an empty cache has nothing to attend to
    assert L.rtr_attn_cross(h, FAKE + 2 * MB, FAKE + 3 * MB, None, 8, rtr.RTR_BF16, 0.0, None, 0,
                            None) == rtr.RTR_ESTATE
    # the caller wrote the condition into the cache buffers itself: no copy
    assert L.rtr_text_cache_reset(h, None, None, 12, None) == rtr.RTR_OK
    assert L.rtr_text_cache_reset(h, FAKE, FAKE + MB, 12, None) == rtr.RTR_OK   # same buffers: no copy
    assert L.rtr_text_cache_state(h, ctypes.byref(n), ctypes.byref(g)) == 0 and (n.value, g.value) == (12, 2)
    assert L.rtr_text_cache_reset(h, None, None, 17, None) == rtr.RTR_EINVAL    # over capacity
    assert L.rtr_text_cache_reset(h, FAKE + 2 * MB, None, 4, None) == rtr.RTR_EINVAL
    assert L.rtr_text_cache_reset(h, FAKE + 8, FAKE + 2 * MB, 4, None) == rtr.RTR_EINVAL  # overlaps the cache
    assert L.rtr_text_cache_state(h, ctypes.byref(n), ctypes.byref(g)) == 0 and (n.value, g.value) == (12, 2)
    # cross-attention argument checks
    assert L.rtr_attn_cross(h, FAKE + 2 * MB, FAKE + 2 * MB + 64, None, 8, rtr.RTR_BF16, 0.0, None, 0,
                            None) == rtr.RTR_EINVAL       # o overlaps q
    assert L.rtr_attn_cross(h, FAKE + 2 * MB, FAKE + 8, None, 8, rtr.RTR_BF16, 0.0, None, 0,
                            None) == rtr.RTR_EINVAL       # o overlaps the cache (and misaligned)
    assert L.rtr_attn_cross(h, FAKE + 2 * MB, FAKE + 3 * MB, None, -1, rtr.RTR_BF16, 0.0, None, 0,
                            None) == rtr.RTR_EINVAL
    assert L.rtr_attn_cross(h, FAKE + 2 * MB, FAKE + 3 * MB, None, 8, rtr.RTR_BF16, float("inf"), None, 0,
                            None) == rtr.RTR_EINVAL
    assert L.rtr_attn_cross(h, FAKE + 2 * MB, FAKE + 3 * MB, None, 0, rtr.RTR_BF16, 0.0, None, 0,
                            None) == rtr.RTR_OK           # no rows: no-op
    # clear
    assert L.rtr_text_cache_reset(h, None, None, 0, None) == rtr.RTR_OK
    assert L.rtr_text_cache_state(h, ctypes.byref(n), ctypes.byref(g)) == 0 and (n.value, g.value) == (0, 2)
    assert L.rtr_text_cache_destroy(h) == rtr.RTR_OK


def test_ref_rope_rejections():
    kv = _cache(W=3, R=1)
    L = rtr.lib()
    h = kv.handle
    fb = 8 * 2 * 64 * 2
    view = FAKE + 512 * MB
    assert L.rtr_kv_set_ref_rope(h, view, 0, 10000.0, 1) == rtr.RTR_EINVAL          # no pairs
    assert L.rtr_kv_set_ref_rope(h, view, 33, 10000.0, 1) == rtr.RTR_EINVAL         # > d / 2
    assert L.rtr_kv_set_ref_rope(h, view, 8, 1.0, 1) == rtr.RTR_EINVAL              # base
    assert L.rtr_kv_set_ref_rope(h, view, 8, 10000.0, -1) == rtr.RTR_EINVAL         # offset
    assert L.rtr_kv_set_ref_rope(h, view + 8, 8, 10000.0, 1) == rtr.RTR_EINVAL      # misaligned
    assert L.rtr_kv_set_ref_rope(h, FAKE + 16, 8, 10000.0, 1) == rtr.RTR_EINVAL     # overlaps the ring
    assert L.rtr_kv_set_ref_rope(h, view, 8, 10000.0, 1) == rtr.RTR_OK
    assert L.rtr_kv_set_ref_rope(h, None, 0, 0.0, 0) == rtr.RTR_OK                  # off
    kv0 = _cache(W=3, R=0)
    assert L.rtr_kv_set_ref_rope(kv0.handle, view, 8, 10000.0, 1) == rtr.RTR_ESTATE
    assert fb > 0


def _sbwd(kv, **kw):
    base = FAKE + 256 * MB
    a = dict(q=base, k=base + MB, v=base + 2 * MB, o=base + 3 * MB, lse=base + 4 * MB,
             do=base + 5 * MB, C=2, B=1, dq=base + 6 * MB, dk=base + 7 * MB, dv=base + 8 * MB,
             dkc=base + 9 * MB, dvc=base + 10 * MB, scale=0.0, ws=base + 16 * MB, ws_bytes=16 * MB,
             stream=None)
    a.update(kw)
    return rtr.lib().rtr_attn_stream_step_bwd(kv.handle, a["q"], a["k"], a["v"], a["o"], a["lse"],
                                              a["do"], a["C"], a["B"], a["dq"], a["dk"], a["dv"],
                                              a["dkc"], a["dvc"], a["scale"], a["ws"], a["ws_bytes"],
                                              a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(C=0), rtr.RTR_EUNSUPPORTED),
    (dict(C=rtr.RTR_MAX_CHUNK + 1), rtr.RTR_EUNSUPPORTED),
    (dict(B=0), rtr.RTR_EINVAL),
    (dict(q=None), rtr.RTR_EINVAL),
    (dict(lse=None), rtr.RTR_EINVAL),
    (dict(dv=None), rtr.RTR_EINVAL),
    (dict(dvc=None), rtr.RTR_EINVAL),                   # cache gradients come in pairs
    (dict(dk=FAKE + 256 * MB + 7 * MB + 8), rtr.RTR_EINVAL),   # misaligned
    (dict(lse=FAKE + 256 * MB + 4 * MB + 1), rtr.RTR_EINVAL),  # misaligned lse
    (dict(dq=FAKE + 64), rtr.RTR_EINVAL),               # dq overlaps the ring
    (dict(dkc=FAKE + 256 * MB + 6 * MB + 16), rtr.RTR_EINVAL),  # dk_cache overlaps dq
    (dict(ws=None), rtr.RTR_EINVAL),
    (dict(ws=FAKE + 256 * MB + 16 * MB + 16), rtr.RTR_EINVAL),  # not 256-byte aligned
    (dict(ws_bytes=100), rtr.RTR_EINVAL),
    (dict(ws=FAKE + 256 * MB + 5 * MB), rtr.RTR_EINVAL),       # overlaps d_o
    (dict(scale=float("inf")), rtr.RTR_EINVAL),
])
def test_stream_step_bwd_rejects_before_launch(kw, code):
    kv = _cache(W=3, R=1, d=128)
    rtr.rtr_kv_commit_inplace(kv, 2)
    assert _sbwd(kv, **kw) == code
    assert rtr.lib().rtr_last_error()


def test_stream_step_bwd_rejects_unsupported_caches():
    for kv in (_cache(W=3, R=1, d=64), _cache(W=3, R=1, d=128, dtype=rtr.RTR_F32)):
        assert _sbwd(kv) == rtr.RTR_EUNSUPPORTED
    assert rtr.lib().rtr_attn_stream_step_bwd(None, *([FAKE] * 6), 1, 1, *([FAKE] * 5), 0.0, FAKE,
                                              MB, None) == rtr.RTR_EINVAL


def test_cross_bwd_rejections():
    """Argument checks of rtr_attn_cross_bwd on a host-side text cache (no
    call reaches a launch)."""
    L = rtr.lib()
    H, d = 2, 128
    tc = rtr.TextCache(FAKE, FAKE + MB, 64, H, d, rtr.RTR_BF16)
    base = FAKE + 256 * MB
    a = dict(q=base, o=base + MB, lse=base + 2 * MB, do=base + 3 * MB, Tq=100, dq=base + 4 * MB,
             dk=base + 5 * MB, dv=base + 6 * MB, scale=0.0, ws=base + 16 * MB, ws_bytes=16 * MB)

    def call(h=tc.handle, **kw):
        x = dict(a)
        x.update(kw)
        return L.rtr_attn_cross_bwd(h, x["q"], x["o"], x["lse"], x["do"], x["Tq"], x["dq"], x["dk"],
                                    x["dv"], x["scale"], x["ws"], x["ws_bytes"], None)

    assert call() == rtr.RTR_ESTATE                       # no condition set
    assert L.rtr_text_cache_reset(tc.handle, None, None, 30, None) == rtr.RTR_OK
    assert call(h=None) == rtr.RTR_EINVAL
    assert call(Tq=-1) == rtr.RTR_EINVAL
    assert call(dv=None) == rtr.RTR_EINVAL                # text gradients come in pairs
    assert call(q=None) == rtr.RTR_EINVAL
    assert call(dq=None) == rtr.RTR_EINVAL
    assert call(dq=base + 4 * MB + 8) == rtr.RTR_EINVAL  # misaligned
    assert call(dk=FAKE + 64) == rtr.RTR_EINVAL          # overlaps the text keys
    assert call(dk=base + 4 * MB + 64) == rtr.RTR_EINVAL  # overlaps dq
    assert call(ws=None) == rtr.RTR_EINVAL
    assert call(ws_bytes=100) == rtr.RTR_EINVAL
    assert call(scale=float("inf")) == rtr.RTR_EINVAL
    assert call(Tq=0) == rtr.RTR_OK                       # no-op
    tc64 = rtr.TextCache(FAKE, FAKE + MB, 64, H, 64, rtr.RTR_BF16)
    L.rtr_text_cache_reset(tc64.handle, None, None, 30, None)
    assert call(h=tc64.handle) == rtr.RTR_EUNSUPPORTED


def test_step_rejects_a_chunk_in_a_slot_the_window_uses():
    """Zero-copy append: a chunk may sit in ring slots the window does not use
    (where rtr_kv_next_slots puts it), never in a slot in use or in the
    reference slot, for the step and for its backward."""
    W, kpf, H, d = 3, 8, 2, 128
    fb = kpf * H * d * 2
    kv = _cache(W=W, R=1, kpf=kpf, H=H, d=d)
    L = rtr.lib()
    h = kv.handle
    rtr.rtr_kv_reset_ref(kv, rtr.RTR_REF_REPLACE, None, None, 1, -1)
    rtr.rtr_kv_commit_inplace(kv, 2)                      # slots 0 and 1 in use, slot 2 free
    assert list(rtr.rtr_kv_next_slots(kv, 1)) == [2]
    k_ring, v_ring, k_ref = FAKE, FAKE + 64 * fb + 4096, FAKE + 128 * fb + 8192   # as _cache lays them out
    far = FAKE + 900 * MB

    def step(q=far, k=far + MB, v=far + 2 * MB):
        return L.rtr_attn_stream_step(h, q, k, v, far + 3 * MB, None, 1, 0, 0.0, None, 0, None)

    assert step(k=k_ring) == rtr.RTR_EINVAL                # slot 0 (oldest) in use
    assert step(v=v_ring + fb) == rtr.RTR_EINVAL           # slot 1 in use
    assert step(k=k_ring + fb + fb // 2) == rtr.RTR_EINVAL  # starts inside slot 1
    assert step(q=k_ring + fb) == rtr.RTR_EINVAL
    assert step(k=k_ref) == rtr.RTR_EINVAL                 # the reference slot
    assert "window slot" in L.rtr_last_error().decode()
    assert _sbwd(kv, k=k_ring + fb) == rtr.RTR_EINVAL
    assert _sbwd(kv, o=v_ring) == rtr.RTR_EINVAL
    assert _sbwd(kv, do=k_ref) == rtr.RTR_EINVAL
    # once the window is full, the reported slot is the oldest frame's
    rtr.rtr_kv_commit_inplace(kv, 1)
    assert list(rtr.rtr_kv_next_slots(kv, 1)) == [0]
    assert step(k=k_ring + 2 * fb) == rtr.RTR_EINVAL
    assert step(k=k_ring) == rtr.RTR_EINVAL
    assert _sbwd(kv, v=v_ring + 2 * fb) == rtr.RTR_EINVAL


def test_spare_ring_slots_take_a_chunk_before_its_step():
    """With ring slots beyond the window, the slots the next append takes are
    outside the full window, so a producer may write a chunk there and pass it
    to the step that reads it; the window's own slots are still refused
    (before anything is launched: these calls carry no device memory)."""
    W, N, kpf, H, d = 3, 5, 8, 2, 128
    fb = kpf * H * d * 2
    kv = _cache(W=W, R=1, kpf=kpf, H=H, d=d, N=N)
    L = rtr.lib()
    h = kv.handle
    rtr.rtr_kv_reset_ref(kv, rtr.RTR_REF_REPLACE, None, None, 1, -1)
    rtr.rtr_kv_commit_inplace(kv, 4)                      # full window: frames in slots 1, 2, 3
    assert _state(kv)["slot"] == [1, 2, 3]
    assert list(rtr.rtr_kv_next_slots(kv, 2)) == [4, 0]   # the spare slots, not the window's
    k_ring, v_ring = FAKE, FAKE + 64 * fb + 4096
    far = FAKE + 900 * MB

    def step(k, v, C):
        return L.rtr_attn_stream_step(h, far, k, v, far + 3 * MB, None, C, 0, 0.0, None, 0, None)

    # (a chunk in the spare slots passes these checks; tests/test_gpu_zero_copy.py runs such steps)
    assert step(k_ring + 1 * fb, v_ring + 4 * fb, 1) == rtr.RTR_EINVAL      # slot 1 is in use
    assert step(k_ring + 4 * fb, v_ring + 3 * fb, 1) == rtr.RTR_EINVAL      # slot 3 is in use
    rtr.rtr_kv_commit_inplace(kv, 2)
    assert _state(kv)["slot"] == [3, 4, 0]
