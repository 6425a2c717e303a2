"""Zero-copy append on the GPU (RTR-DiT notes, Key Designs 4: new frames are
appended, the oldest evicted once the window is full, the reference never).

A producer writes each chunk's K/V straight into the ring slots that
rtr_kv_next_slots reports and commits them with rtr_kv_commit_inplace.  While
the window has room, the chunk is written there first and the step reads it
from the ring; once the window is full, those slots hold the oldest frames
that the step still reads, so the chunk is written after the step.  Every
step is checked against the float64 oracle over the oracle's list window, and
the ring and reference bytes bit-exactly; a chunk placed over a slot in use is
rejected before anything is enqueued.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import ListKV, REF_REPLACE
from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from tests.gpu_util import assert_bf16_close, dev, host

pytestmark = pytest.mark.gpu


def _run(kpf, H, W, C, n_chunks, wid, N=None):
    d = 128
    N = W if N is None else N
    kr = torch.zeros((N, kpf, H, d), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    kf = torch.zeros((1, kpf, H, d), dtype=torch.bfloat16, device="cuda")
    vf = torch.zeros_like(kf)
    kv = rtr.rtr_kv_create_slots(kr, vr, kf, vf, W, N, 1, kpf, H, d, rtr.RTR_BF16)
    ref = ListKV(W)
    rk = gen.normal((1, kpf, H, d), "bf16", 0, wid, 0, gen.TAG_REFK)
    rv = gen.normal((1, kpf, H, d), "bf16", 0, wid, 0, gen.TAG_REFV)
    rtr.rtr_kv_reset_ref(kv, rtr.RTR_REF_REPLACE, dev(rk), dev(rv), 1, -1)
    ref.reset_ref(REF_REPLACE, rk.values, rv.values, keep_recent=-1)
    staged_first = written_after = 0
    for i in range(n_chunks):
        q = gen.normal((C * kpf, H, d), "bf16", 0, wid, i + 1, gen.TAG_Q)
        k = gen.normal((C * kpf, H, d), "bf16", 0, wid, i + 1, gen.TAG_K)
        v = gen.normal((C * kpf, H, d), "bf16", 0, wid, i + 1, gen.TAG_V)
        kd, vd = dev(k).view(C, kpf, H, d), dev(v).view(C, kpf, H, d)
        slots = rtr.rtr_kv_next_slots(kv, C)
        st = rtr.rtr_kv_get_state(kv).as_dict()
        in_use = set(st["slot"][:st["count"]])
        s0 = slots[0]
        free_run = (all(s >= 0 and s not in in_use for s in slots)
                    and slots == list(range(s0, s0 + C)))
        if free_run:
            # the slots are unused: write the chunk there and let the step read it from the ring
            kr[s0:s0 + C].copy_(kd)
            vr[s0:s0 + C].copy_(vd)
            step_k, step_v = kr[s0:s0 + C].view(C * kpf, H, d), vr[s0:s0 + C].view(C * kpf, H, d)
            staged_first += 1
        else:
            step_k, step_v = kd.view(C * kpf, H, d), vd.view(C * kpf, H, d)
            # a chunk over a slot the window still reads is refused
            busy = [s for s in slots if s in in_use]
            if busy:
                with pytest.raises(rtr.RtrError) as e:
                    rtr.rtr_attn_stream_step(kv, dev(q)[:kpf], kr[busy[0]], vd[0], 1)
                assert e.value.code == rtr.RTR_EINVAL
        o, lse = rtr.rtr_attn_stream_step(kv, dev(q), step_k, step_v, C, want_lse=True)
        if not free_run:
            # after the last step that reads the current window (same stream)
            for c, s in enumerate(slots):
                if s >= 0:
                    kr[s].copy_(kd[c])
                    vr[s].copy_(vd[c])
            written_after += 1
        rtr.rtr_kv_commit_inplace(kv, C)
        pk, pv = ref.prefix(kpf, H, d)
        ro, rl = oracle.attn_stream_step(pk, pv, q.values, k.values, v.values, kpf)
        assert_bf16_close(host(o), ro, f"chunk {i} output")
        assert_bf16_close(host(lse), rl, f"chunk {i} lse")
        ref.append(k.values.reshape(C, kpf, H, d), v.values.reshape(C, kpf, H, d))
        # ring state and bytes bit-exact against the list window
        torch.cuda.synchronize()
        st = rtr.rtr_kv_get_state(kv).as_dict()
        assert st["frame_id"] == ref.frame_ids()
        for p, (_, fk, fv) in enumerate(ref.window):
            s = st["slot"][p]
            assert np.array_equal(host(kr[s]), fk), f"chunk {i}: K bytes of slot {s}"
            assert np.array_equal(host(vr[s]), fv), f"chunk {i}: V bytes of slot {s}"
        assert np.array_equal(host(kf[0]), rk.values[0]) and np.array_equal(host(vf[0]), rv.values[0])
    kv.close()
    return staged_first, written_after


def test_zero_copy_append_two_frame_chunks():
    staged, after = _run(kpf=96, H=2, W=5, C=2, n_chunks=8, wid=301)
    assert staged >= 2 and after >= 2     # both orders ran


def test_zero_copy_append_wan_shape():
    staged, after = _run(kpf=1560, H=12, W=6, C=3, n_chunks=4, wid=302)
    assert staged >= 1 and after >= 1


def test_zero_copy_append_spare_slots_write_before_every_step():
    """A ring with C spare slots (rtr_kv_create_slots): once the window is full,
    the slots the next append takes are still outside it, so every chunk is
    written into the ring before its step and read from there."""
    staged, after = _run(kpf=96, H=2, W=4, C=2, n_chunks=8, wid=303, N=6)
    assert staged == 8 and after == 0
