"""The chunk append running beside the attention that reads the window (GPU).

With a ring of W + C slots (rtr_kv_create_slots), the append of chunk i writes
only slots outside the window that step i reads (RTR-DiT notes, Key Designs
4: the new frames enter, the oldest leave once the window is full), so it can
run on a second stream while step i's attention runs: it waits for the chunk's
upload and for step i-1 (which read the slots it overwrites), and step i+1
waits for it.  Every step's output is compared with the float64 oracle over
the list window it should see, and the ring bytes with the list window at the
end.  Both streams have the default priority.
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


@pytest.mark.parametrize("kpf,H,W,C,n_chunks", [(96, 2, 4, 2, 9), (1560, 12, 6, 3, 4)])
def test_append_overlapped_with_the_step(kpf, H, W, C, n_chunks):
    print(f"kpf={kpf} H={H} W={W} C={C}", flush=True)
    d, N, wid = 128, W + C, 310 + C
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
    torch.cuda.synchronize()

    sa = torch.cuda.current_stream()
    sb = torch.cuda.Stream()
    keep, expected = [], []
    ev_a_prev = None
    ev_c_prev = None
    for i in range(n_chunks):
        q = gen.normal((C * kpf, H, d), "bf16", 0, wid, i + 1, gen.TAG_Q)
        k = gen.normal((C * kpf, H, d), "bf16", 0, wid, i + 1, gen.TAG_K)
        v = gen.normal((C * kpf, H, d), "bf16", 0, wid, i + 1, gen.TAG_V)
        pk, pv = ref.prefix(kpf, H, d)
        expected.append(oracle.attn_stream_step(pk, pv, q.values, k.values, v.values, kpf))
        ref.append(k.values.reshape(C, kpf, H, d), v.values.reshape(C, kpf, H, d))
        with torch.cuda.stream(sa):
            qd, kd, vd = dev(q), dev(k), dev(v)
            ev_up = torch.cuda.Event()
            ev_up.record(sa)
            if ev_c_prev is not None:
                sa.wait_event(ev_c_prev)          # the step sees the previous chunk committed
            o, lse = rtr.rtr_attn_stream_step(kv, qd, kd, vd, C, want_lse=True, stream=sa)
            ev_a = torch.cuda.Event()
            ev_a.record(sa)
        # the append: after the upload and after the previous step, beside this step
        sb.wait_event(ev_up)
        if ev_a_prev is not None:
            sb.wait_event(ev_a_prev)
        rtr.rtr_kv_append_evict(kv, kd, vd, C, stream=sb)
        ev_c = torch.cuda.Event()
        ev_c.record(sb)
        keep.append((qd, kd, vd, o, lse))
        ev_a_prev, ev_c_prev = ev_a, ev_c
    torch.cuda.synchronize()

    for i, ((_, _, _, o, lse), (ro, rl)) in enumerate(zip(keep, expected)):
        assert_bf16_close(host(o), ro, f"chunk {i} output")
        assert_bf16_close(host(lse), rl, f"chunk {i} lse")
    st = rtr.rtr_kv_get_state(kv).as_dict()
    assert st["ring_slots"] == N
    assert st["frame_id"] == ref.frame_ids()
    for p, (_, fk, fv) in enumerate(ref.window):
        s = st["slot"][p]
        assert np.array_equal(host(kr[s]), fk), f"K bytes of slot {s}"
        assert np.array_equal(host(vr[s]), fv), f"V bytes of slot {s}"
    kv.close()
