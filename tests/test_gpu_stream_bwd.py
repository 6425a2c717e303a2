"""GPU parity of the streaming step's gradients (rtr_attn_stream_step_bwd,
through the C ABI) against the float64 oracle (oracle.attn_stream_step_bwd):
the chunk's dQ, dK, dV and the gradients of the cached keys and values, for
the Attn of one step over [reference | window | chunk] (RTR-DiT notes, Key
Designs 2 and 4).  The forward's o and lse come from the library's own
streaming step, as the entry point requires; the oracle recomputes everything
from the cache contents, q, k, v and dO."""

import numpy as np
import pytest
import torch

from oracle import ListKV, REF_REPLACE
from oracle.attention_bwd import attn_stream_step_bwd
from oracle.rope import reference_shift, rope_rotate
from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from tests.gpu_util import assert_grad_close, dev, guarded_empty, host

pytestmark = pytest.mark.gpu

D = 128


def _cache(kpf, H, W, R_cap):
    kr = torch.zeros((max(W, 1), kpf, H, D), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    kf = torch.zeros((max(R_cap, 1), kpf, H, D), dtype=torch.bfloat16, device="cuda")
    vf = torch.zeros_like(kf)
    return rtr.rtr_kv_create(kr, vr, kf, vf, W, R_cap, kpf, H, D), ListKV(W)


def _fill(kv, ref, kpf, H, R, n_past, seed):
    """Anchor R reference frames and commit n_past frames (the ring wraps
    when n_past > W, so logical and physical slot order differ)."""
    x = gen.stream_inputs(kpf, H, D, 1, max(n_past, 1), max(R, 1), "bf16", base_seed=seed, wid=90)
    if R:
        rk, rv = x["ref_k"], x["ref_v"]
        rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(rk), dev(rv), R, -1)
        ref.reset_ref(REF_REPLACE, rk.values, rv.values, keep_recent=-1)
    for f in range(n_past):
        fk, fv = x["ring_k"].values[f:f + 1], x["ring_v"].values[f:f + 1]
        rtr.rtr_kv_append_evict(kv, dev(gen.from_values(fk, "bf16")), dev(gen.from_values(fv, "bf16")), 1)
        ref.append(fk, fv)


def _step(kv, kpf, H, C, B, seed, cache_grads, guards=False):
    x = gen.stream_inputs(kpf, H, D, C, 1, 1, "bf16", base_seed=seed, wid=91)
    do = gen.normal((C * kpf, H, D), "bf16", seed, 91, 0, gen.TAG_DO)
    q, k, v, tdo = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(do)
    o, lse = rtr.rtr_attn_stream_step_blocked(kv, q, k, v, C, B, want_lse=True)
    checks = []
    outs = {}
    if guards:
        st = rtr.rtr_kv_get_state(kv)
        P = (st.ref_frames + st.count) * kpf
        for name, shape in (("dq", q.shape), ("dk", q.shape), ("dv", q.shape),
                            ("dk_cache", (P, H, D)), ("dv_cache", (P, H, D))):
            outs[name], chk = guarded_empty(shape, torch.bfloat16)
            checks.append(chk)
    got = rtr.rtr_attn_stream_step_bwd(kv, q, k, v, o, lse, tdo, C, B, want_cache_grads=cache_grads, **outs)
    torch.cuda.synchronize()
    for chk in checks:
        chk()
    return x, do, got


def _compare(got, ref_grads, cache_grads, what):
    names = ("dq", "dk", "dv", "dk_cache", "dv_cache")
    n = 5 if cache_grads else 3
    for name, g, r in list(zip(names, got, ref_grads))[:n]:
        if r.shape[0] == 0:
            continue
        assert_grad_close(host(g), r, f"{name} {what}")
    if not cache_grads:
        assert got[3] is None and got[4] is None


@pytest.mark.parametrize("kpf,H,W,R,n_past,C,B,cache_grads", [
    (96, 2, 3, 1, 5, 3, 1, True),     # frames straddle 32-row tiles; the ring has wrapped
    (96, 2, 4, 2, 2, 2, 2, True),     # two references, half-full window, whole-chunk block
    (40, 3, 2, 1, 2, 1, 1, False),    # 40-token frames: segments change inside a key tile
    (300, 1, 3, 1, 3, 2, 1, True),    # 256-key blocks of the prefix span two frames
    (64, 1, 2, 0, 0, 2, 1, True),     # empty cache: the full form over the chunk
    (33, 2, 2, 0, 3, 3, 2, True),     # window only, no reference; ragged tiles everywhere
])
def test_stream_bwd_matches_oracle(kpf, H, W, R, n_past, C, B, cache_grads):
    print(f"kpf={kpf} H={H} W={W} R={R} past={n_past} C={C} B={B} cache={cache_grads}", flush=True)
    kv, ref = _cache(kpf, H, W, max(R, 1))
    _fill(kv, ref, kpf, H, R, n_past, seed=kpf + 7 * C)
    x, do, got = _step(kv, kpf, H, C, B, seed=3 * kpf + B, cache_grads=cache_grads, guards=cache_grads)
    pk, pv = ref.prefix(kpf, H, D)
    r = attn_stream_step_bwd(pk, pv, x["q"].values, x["k"].values, x["v"].values, do.values,
                             min(B, C) * kpf)
    _compare(got, r, cache_grads, f"kpf={kpf} C={C} B={B}")
    kv.close()


def test_stream_bwd_deterministic_and_scale():
    kpf, H, W, C = 96, 2, 2, 2
    kv, ref = _cache(kpf, H, W, 1)
    _fill(kv, ref, kpf, H, 1, 2, seed=11)
    x = gen.stream_inputs(kpf, H, D, C, 1, 1, "bf16", base_seed=12, wid=92)
    do = gen.normal((C * kpf, H, D), "bf16", 12, 92, 0, gen.TAG_DO)
    q, k, v, tdo = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(do)
    o, lse = rtr.rtr_attn_stream_step_blocked(kv, q, k, v, C, 1, want_lse=True, scale=0.05)
    a = rtr.rtr_attn_stream_step_bwd(kv, q, k, v, o, lse, tdo, C, 1, want_cache_grads=True, scale=0.05)
    b = rtr.rtr_attn_stream_step_bwd(kv, q, k, v, o, lse, tdo, C, 1, want_cache_grads=True, scale=0.05)
    torch.cuda.synchronize()
    for s, t in zip(a, b):
        assert torch.equal(s.view(torch.int16), t.view(torch.int16))
    pk, pv = ref.prefix(kpf, H, D)
    r = attn_stream_step_bwd(pk, pv, x["q"].values, x["k"].values, x["v"].values, do.values, kpf,
                             scale=0.05)
    _compare(a, r, True, "scale 0.05")
    kv.close()


def test_stream_bwd_rotated_reference():
    """Position-aware reference: the step attends to the reference rotated to
    sit in front of the oldest window frame; dk_cache's reference rows are the
    gradient with respect to the stored (unrotated) keys, i.e. the gradient at
    the rotated keys rotated back by the same angle."""
    kpf, H, W, R, C, PAIRS, BASE = 64, 2, 3, 2, 2, 22, 10000.0
    kv, ref = _cache(kpf, H, W, R)
    view = torch.zeros((R, kpf, H, D), dtype=torch.bfloat16, device="cuda")
    rtr.rtr_kv_set_ref_rope(kv, view, PAIRS, BASE, R)
    _fill(kv, ref, kpf, H, R, 4, seed=21)
    x, do, got = _step(kv, kpf, H, C, 1, seed=22, cache_grads=True)
    ids = ref.frame_ids()
    shift = reference_shift(ids[0] + R, R)
    pk, pv = ref.prefix(kpf, H, D)
    pk = pk.copy()
    # the view the step reads is bf16: round the rotated keys as the library stores them
    rot = rope_rotate(pk[:R * kpf], np.full(R * kpf, shift), PAIRS, BASE)
    pk[:R * kpf] = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rot.astype(np.float32)))
    r = list(attn_stream_step_bwd(pk, pv, x["q"].values, x["k"].values, x["v"].values, do.values, kpf))
    r[3] = r[3].copy()
    r[3][:R * kpf] = rope_rotate(r[3][:R * kpf], np.full(R * kpf, -shift), PAIRS, BASE)
    _compare(got, r, True, "rotated reference")
    kv.close()


def test_stream_bwd_wan_shape_two_heads():
    """Wan-1.3B streaming shape (1,560 tokens per frame, reference + 6-frame
    window, 3-frame chunk) with 12 heads on the device; the dense oracle runs
    on heads 0 and 11 (heads are independent)."""
    kpf, H, W, C = 1560, 12, 6, 3
    kv, ref = _cache(kpf, H, W, 1)
    _fill(kv, ref, kpf, H, 1, 8, seed=31)
    x, do, got = _step(kv, kpf, H, C, 1, seed=32, cache_grads=True)
    heads = [0, H - 1]
    pk, pv = ref.prefix(kpf, H, D)
    sl = lambda a: np.ascontiguousarray(a[:, heads])
    r = attn_stream_step_bwd(sl(pk), sl(pv), sl(x["q"].values), sl(x["k"].values), sl(x["v"].values),
                             sl(do.values), kpf)
    _compare([g[:, heads] for g in got], r, True, "wan 1.3B")
    kv.close()


def test_stream_bwd_through_a_rollout():
    """The training-time order: each chunk runs its forward step, then its
    backward (before the chunk is committed), then the commit; a reference
    switch keeping one frame happens midway.  Every step's gradients,
    cache gradients included, match the oracle on the cache as it stood."""
    kpf, H, W, C = 64, 2, 3, 2
    kv, ref = _cache(kpf, H, W, 1)
    _fill(kv, ref, kpf, H, 1, 0, seed=41)
    for step in range(7):
        if step == 4:
            x0 = gen.stream_inputs(kpf, H, D, 1, 1, 1, "bf16", base_seed=99, wid=93)
            rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(x0["ref_k"]), dev(x0["ref_v"]), 1, 1)
            ref.reset_ref(REF_REPLACE, x0["ref_k"].values, x0["ref_v"].values, keep_recent=1)
        x, do, got = _step(kv, kpf, H, C, 1, seed=50 + step, cache_grads=True)
        pk, pv = ref.prefix(kpf, H, D)
        r = attn_stream_step_bwd(pk, pv, x["q"].values, x["k"].values, x["v"].values, do.values, kpf)
        _compare(got, r, True, f"step {step}")
        rtr.rtr_kv_append_evict(kv, dev(x["k"]).view(C, kpf, H, D), dev(x["v"]).view(C, kpf, H, D), C)
        ref.append(x["k"].values.reshape(C, kpf, H, D), x["v"].values.reshape(C, kpf, H, D))
    kv.close()


def test_stream_bwd_wan13b_every_element():
    """The timed backward workload (Wan-1.3B layer: 12 heads, 1,560-token
    frames, a 3-frame chunk over the reference and a full 6-frame window):
    every element of dQ, dK, dV and of the cache gradients against the dense
    oracle.  One launch of the dQ kernel covers the whole chunk here, so its
    workgroups take frame-paired row groups (frame 0 with frame 2, frame 1 on
    its own) and waves whose rows end before a key tile skip its products."""
    kpf, H, W, R, C = 1560, 12, 6, 1, 3
    print(f"kpf={kpf} H={H} W={W} R={R} C={C}", flush=True)
    kv, ref = _cache(kpf, H, W, R)
    _fill(kv, ref, kpf, H, R, W, seed=21)
    x, do, got = _step(kv, kpf, H, C, 1, seed=22, cache_grads=True)
    pk, pv = ref.prefix(kpf, H, D)
    r = attn_stream_step_bwd(pk, pv, x["q"].values, x["k"].values, x["v"].values, do.values, kpf)
    _compare(got, r, True, "Wan-1.3B step")
    kv.close()
