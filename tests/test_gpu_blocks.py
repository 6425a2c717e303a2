"""GPU parity of two widenings of the streaming step, through the C ABI:
several anchored references (up to RTR_MAX_REF frames at the front of the
cache) and the chunk-level mask (rtr_attn_stream_step_blocked: the chunk's
frames in blocks that see each other), against the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from oracle import ListKV, REF_REPLACE
from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from tests.gpu_util import assert_bf16_close, dev, host

pytestmark = pytest.mark.gpu


def _setup(kpf, H, d, W, R_cap):
    kr = torch.zeros((W, kpf, H, d), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    kf = torch.zeros((R_cap, kpf, H, d), dtype=torch.bfloat16, device="cuda")
    vf = torch.zeros_like(kf)
    return rtr.rtr_kv_create(kr, vr, kf, vf, W, R_cap, kpf, H, d), ListKV(W)


def _frames(n, kpf, H, d, seed, wid):
    x = gen.stream_inputs(kpf, H, d, 1, n, 1, "bf16", base_seed=seed, wid=wid)
    return x["ring_k"], x["ring_v"]


def _check_step(kv, ref, kpf, H, d, C, B, seed, ws=None):
    x = gen.stream_inputs(kpf, H, d, C, 1, 1, "bf16", base_seed=seed, wid=61)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    if B == 1 and ws is None:
        o, lse = rtr.rtr_attn_stream_step(kv, q, k, v, C, want_lse=True)
    else:
        o, lse = rtr.rtr_attn_stream_step_blocked(kv, q, k, v, C, B, want_lse=True, workspace=ws)
    pk, pv = ref.prefix(kpf, H, d)
    ro, rl = oracle.attn_stream_step(pk, pv, x["q"].values, x["k"].values, x["v"].values, min(B, C) * kpf)
    torch.cuda.synchronize()
    assert_bf16_close(host(o), ro, f"o C={C} B={B}")
    assert_bf16_close(host(lse), rl, f"lse C={C} B={B}")
    return k, v, x


@pytest.mark.parametrize("R", [2, 3, 4])
def test_several_references(R):
    kpf, H, d, W, C = 96, 2, 128, 4, 3
    kv, ref = _setup(kpf, H, d, W, 4)
    rk, rv = _frames(R, kpf, H, d, seed=R, wid=60)
    rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(rk), dev(rv), R, -1)
    ref.reset_ref(REF_REPLACE, rk.values, rv.values, keep_recent=-1)
    wk, wv = _frames(W, kpf, H, d, seed=10 + R, wid=60)
    rtr.rtr_kv_append_evict(kv, dev(wk), dev(wv), W)
    ref.append(wk.values, wv.values)
    k, v, x = _check_step(kv, ref, kpf, H, d, C, 1, seed=20 + R)
    assert rtr.rtr_kv_get_state(kv).as_dict()["ref_frames"] == R
    # commit, then switch to a single new reference keeping the newest frame
    rtr.rtr_kv_append_evict(kv, k, v, C)
    ref.append(x["k"].values.reshape(C, kpf, H, d), x["v"].values.reshape(C, kpf, H, d))
    nk, nv = _frames(1, kpf, H, d, seed=30 + R, wid=60)
    rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(nk), dev(nv), 1, 1)
    ref.reset_ref(REF_REPLACE, nk.values, nv.values, keep_recent=1)
    _check_step(kv, ref, kpf, H, d, C, 1, seed=40 + R)
    s = rtr.rtr_kv_get_state(kv).as_dict()
    assert s["ref_frames"] == 1 and s["frame_id"] == ref.frame_ids()
    kv.close()


@pytest.mark.parametrize("C,B,split", [(3, 3, False), (3, 2, False), (4, 1, False), (2, 7, False),
                                       (3, 3, True), (1, 1, True)])
def test_chunk_level_mask(C, B, split):
    kpf, H, d, W = 96, 2, 128, 2
    kv, ref = _setup(kpf, H, d, W, 1)
    rk, rv = _frames(1, kpf, H, d, seed=1, wid=62)
    rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(rk), dev(rv), 1, -1)
    ref.reset_ref(REF_REPLACE, rk.values, rv.values, keep_recent=-1)
    wk, wv = _frames(W, kpf, H, d, seed=2, wid=62)
    rtr.rtr_kv_append_evict(kv, dev(wk), dev(wv), W)
    ref.append(wk.values, wv.values)
    ws = rtr.new_workspace(d, rtr.RTR_BF16, "cuda") if split else None
    _check_step(kv, ref, kpf, H, d, C, B, seed=3 + 10 * C + B, ws=ws)
    kv.close()


def test_wan_shape_two_references_whole_chunk_block():
    """Wan-1.3B shape (12 heads, 1,560 tokens per frame, 6-frame window,
    3-frame chunk) with two anchored references and the whole chunk as one
    mask block, on sampled rows."""
    kpf, H, d, W, C = 1560, 12, 128, 6, 3
    kv, ref = _setup(kpf, H, d, W, 2)
    rk, rv = _frames(2, kpf, H, d, seed=5, wid=63)
    rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(rk), dev(rv), 2, -1)
    wk, wv = _frames(W, kpf, H, d, seed=6, wid=63)
    rtr.rtr_kv_append_evict(kv, dev(wk), dev(wv), W)
    x = gen.stream_inputs(kpf, H, d, C, 1, 1, "bf16", base_seed=7, wid=63)
    o, _ = rtr.rtr_attn_stream_step_blocked(kv, dev(x["q"]), dev(x["k"]), dev(x["v"]), C, C)
    pk = np.concatenate([rk.values.reshape(-1, H, d), wk.values.reshape(-1, H, d)])
    pv = np.concatenate([rv.values.reshape(-1, H, d), wv.values.reshape(-1, H, d)])
    rows = sorted(set(np.random.default_rng(8).choice(C * kpf, 24, replace=False).tolist()) | {0, C * kpf - 1})
    ro, _ = oracle.attn_stream_rows(pk, pv, x["q"].values, x["k"].values, x["v"].values, C * kpf, rows,
                                    [0, H - 1])
    torch.cuda.synchronize()
    assert_bf16_close(host(o[rows][:, [0, H - 1]]), ro, "wan blocked")
    kv.close()
