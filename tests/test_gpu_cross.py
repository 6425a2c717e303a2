"""GPU parity of the text cross-attention and its cache (RTR-DiT notes, Key
Designs 1: text injected through cross attention; Key Designs 4: the
cross-attention cache is re-initialised on a text switch), through the C ABI,
against the float64 oracle (attn_cross, TextKV)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import ListKV, TextKV, REF_KEEP, REF_REPLACE
from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from tests.gpu_util import assert_bf16_close, assert_f32_close, dev, host

pytestmark = pytest.mark.gpu


def _cache(cap, H, d, dtype=torch.bfloat16):
    kb = torch.zeros((cap, H, d), dtype=dtype, device="cuda")
    vb = torch.zeros_like(kb)
    code = rtr.RTR_BF16 if dtype == torch.bfloat16 else rtr.RTR_F32
    return rtr.rtr_text_cache_create(kb, vb, cap, H, d, code), kb, vb


@pytest.mark.parametrize("Tq,Lt,H,d", [
    (700, 77, 2, 128),     # ragged text (not a multiple of the 32-key tile) and ragged rows
    (300, 1, 1, 128),      # one text token
    (513, 512, 2, 128),    # the Wan text length
    (129, 300, 3, 64),     # head_dim 64 kernel
])
def test_cross_matches_oracle(Tq, Lt, H, d):
    q, k, v = gen.cross_inputs(Tq, Lt, H, d, "bf16", base_seed=Tq, wid=70)
    tc, kb, vb = _cache(max(Lt, 8), H, d)
    rtr.rtr_text_cache_reset(tc, dev(k), dev(v), Lt)
    o, lse = rtr.rtr_attn_cross(tc, dev(q), want_lse=True)
    ro, rl = oracle.attn_cross(q.values, k.values, v.values)
    torch.cuda.synchronize()
    print(f"Tq={Tq} Lt={Lt} H={H} d={d}", flush=True)
    assert_bf16_close(host(o), ro, "o")
    assert_bf16_close(host(lse), rl, "lse")
    # fp32 output of the same call
    o32, _ = rtr.rtr_attn_cross(tc, dev(q), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_bf16_close(host(o32), ro, "o f32 out")
    tc.close()


def test_cross_f32_inputs():
    Tq, Lt, H, d = 50, 19, 2, 64
    q, k, v = gen.cross_inputs(Tq, Lt, H, d, "f32", base_seed=1, wid=71)
    tc, kb, vb = _cache(32, H, d, torch.float32)
    rtr.rtr_text_cache_reset(tc, dev(k), dev(v), Lt)
    o, _ = rtr.rtr_attn_cross(tc, dev(q))
    ro, _ = oracle.attn_cross(q.values, k.values, v.values)
    torch.cuda.synchronize()
    assert_f32_close(host(o), ro, "f32 cross")
    tc.close()


def test_cross_full_size_with_workspace():
    """The Wan-1.3B chunk (3 frames of 1,560 tokens, 12 heads) against 512
    text tokens, plain and with a split-K workspace, on sampled rows."""
    w = gen.WORKLOADS["wan13b_cross_step"]
    Tq, Lt, H, d = w["C"] * w["k"], w["text_tokens"], w["H"], w["d"]
    q, k, v = gen.cross_inputs(Tq, Lt, H, d, "bf16", base_seed=0, wid=w["wid"])
    tc, kb, vb = _cache(Lt, H, d)
    rtr.rtr_text_cache_reset(tc, dev(k), dev(v), Lt)
    tq = dev(q)
    o, _ = rtr.rtr_attn_cross(tc, tq)
    ws = rtr.new_workspace(d, rtr.RTR_BF16, "cuda")
    o2, _ = rtr.rtr_attn_cross(tc, tq, workspace=ws)
    rows = sorted(set(np.random.default_rng(3).choice(Tq, 48, replace=False).tolist()) | {0, Tq - 1})
    ro, _ = oracle.attn_cross(q.values[rows], k.values, v.values)
    torch.cuda.synchronize()
    assert_bf16_close(host(o[rows]), ro, "plain")
    assert_bf16_close(host(o2[rows]), ro, "workspace")
    tc.close()


def test_text_switch_resets_only_the_text_cache():
    """A stream with a reference-only switch and a text switch: the text cache
    bytes and generation follow TextKV, the 3D cache follows ListKV, and every
    cross-attention call uses the current condition."""
    kpf, H, d, W = 64, 2, 128, 3
    tc, kb, vb = _cache(100, H, d)
    text = TextKV(100)
    kr = torch.zeros((W, kpf, H, d), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    kf = torch.zeros((1, kpf, H, d), dtype=torch.bfloat16, device="cuda")
    vf = torch.zeros_like(kf)
    kv = rtr.rtr_kv_create(kr, vr, kf, vf, W, 1, kpf, H, d)
    ref = ListKV(W)
    conds = [gen.cross_inputs(1, L, H, d, "bf16", base_seed=s, wid=72)[1:] for s, L in ((0, 77), (1, 40))]
    # start: text 0 and a reference
    rk, rv = gen.cross_inputs(kpf, kpf, H, d, "bf16", base_seed=9, wid=73)[1:]
    rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(rk)[None].contiguous(), dev(rv)[None].contiguous(), 1, -1)
    ref.reset_ref(REF_REPLACE, rk.values[None], rv.values[None], keep_recent=-1)
    rtr.rtr_text_cache_reset(tc, dev(conds[0][0]), dev(conds[0][1]), 77)
    text.set(conds[0][0].values, conds[0][1].values)
    for step in range(6):
        if step == 2:   # reference-only switch: the text cache is untouched
            rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(rv)[None].contiguous(), dev(rk)[None].contiguous(), 1, 1)
            ref.reset_ref(REF_REPLACE, rv.values[None], rk.values[None], keep_recent=1)
        if step == 4:   # text switch: new text cache, the 3D cache keeps its newest frame
            rtr.rtr_text_cache_reset(tc, dev(conds[1][0]), dev(conds[1][1]), 40)
            text.set(conds[1][0].values, conds[1][1].values)
            rtr.rtr_kv_reset_ref(kv, REF_KEEP, None, None, 1, 1)
            ref.reset_ref(REF_KEEP, keep_recent=1)
        q, ck, cv = gen.cross_inputs(kpf, kpf, H, d, "bf16", base_seed=100 + step, wid=74)
        o, _ = rtr.rtr_attn_cross(tc, dev(q))
        ro, _ = oracle.attn_cross(q.values, text.k, text.v)
        rtr.rtr_kv_append_evict(kv, dev(ck), dev(cv), 1)
        ref.append(ck.values[None], cv.values[None])
        torch.cuda.synchronize()
        assert_bf16_close(host(o), ro, f"cross step {step}")
        n, g = rtr.rtr_text_cache_state(tc)
        assert (n, g) == (text.tokens(), text.generation)
        n_ = text.tokens()
        assert np.array_equal(host(kb[:n_]), text.k) and np.array_equal(host(vb[:n_]), text.v)
        s = rtr.rtr_kv_get_state(kv).as_dict()
        assert s["frame_id"] == ref.frame_ids() and s["ref_generation"] == ref.ref_generation
    # clearing leaves no condition
    rtr.rtr_text_cache_reset(tc, None, None, 0)
    with pytest.raises(rtr.RtrError):
        rtr.rtr_attn_cross(tc, dev(q))
    kv.close()
    tc.close()
