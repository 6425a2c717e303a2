"""GPU parity of the position-aware reference (rtr_kv_set_ref_rope): with
rotary temporal encoding baked into cached K, each streaming call re-encodes
the anchored reference so that it sits in front of the oldest frame the call
sees (readings in oracle/rope.py), checked against the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from oracle import ListKV, REF_REPLACE
from oracle.rope import reference_shift, rope_rotate
from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from tests.gpu_util import assert_bf16_close, dev, host

pytestmark = pytest.mark.gpu

KPF, H, D, W, C, PAIRS, BASE = 64, 2, 128, 3, 2, 22, 10000.0


def _bf16(x):
    """float64 array -> bf16 HostTensor (round to nearest even)."""
    return gen.from_values(gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(np.asarray(x, np.float32))), "bf16")


def _raw(seed, n=1):
    return gen.normal((n * KPF, H, D), "bf16", seed, 80, 0, gen.TAG_K).values


@pytest.mark.parametrize("R", [1, 2])
def test_reference_follows_window(R):
    kr = torch.zeros((W, KPF, H, D), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    kf = torch.zeros((2, KPF, H, D), dtype=torch.bfloat16, device="cuda")
    vf = torch.zeros_like(kf)
    view = torch.zeros_like(kf)
    kv = rtr.rtr_kv_create(kr, vr, kf, vf, W, 2, KPF, H, D)
    rtr.rtr_kv_set_ref_rope(kv, view, PAIRS, BASE, R)
    ref = ListKV(W)

    def set_ref(seed):
        raw = _raw(seed, R)
        rot = np.concatenate([rope_rotate(raw[r * KPF:(r + 1) * KPF], np.full(KPF, r), PAIRS, BASE)
                              for r in range(R)])
        rk, rv = _bf16(rot), gen.normal((R * KPF, H, D), "bf16", seed, 81, 0, gen.TAG_V)
        rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(rk).view(R, KPF, H, D), dev(rv).view(R, KPF, H, D), R, 1)
        ref.reset_ref(REF_REPLACE, rk.values.reshape(R, KPF, H, D), rv.values.reshape(R, KPF, H, D), keep_recent=1)
        return rk

    rk = set_ref(1)
    fq, fk = _raw(2), _raw(3)
    fv = gen.normal((KPF, H, D), "bf16", 4, 80, 0, gen.TAG_V).values
    outs = []
    for step in range(9):
        if step == 6:
            rk = set_ref(7)     # a new reference: re-encoded for the new layout
        base_id = rtr.rtr_kv_get_state(kv).next_frame_id
        q = _bf16(np.concatenate([rope_rotate(fq, np.full(KPF, base_id + c + R), PAIRS, BASE) for c in range(C)]))
        k = _bf16(np.concatenate([rope_rotate(fk, np.full(KPF, base_id + c + R), PAIRS, BASE) for c in range(C)]))
        v = _bf16(np.concatenate([fv] * C))
        o, _ = rtr.rtr_attn_stream_step(kv, dev(q), dev(k), dev(v), C)
        ids = ref.frame_ids()
        shift = reference_shift((ids[0] if ids else base_id) + R, R)
        pk, pv = ref.prefix(KPF, H, D)
        pk = pk.copy()
        pk[:R * KPF] = rope_rotate(pk[:R * KPF], np.full(R * KPF, shift), PAIRS, BASE)
        ro, _ = oracle.attn_stream_step(pk, pv, q.values, k.values, v.values, KPF)
        torch.cuda.synchronize()
        assert_bf16_close(host(o), ro, f"step {step}")
        # the view holds the reference encoded at its current position (bf16 rounding)
        got = host(view[:R].reshape(-1, H, D))
        assert np.max(np.abs(got - pk[:R * KPF])) <= 2 ** -7 * np.max(np.abs(pk[:R * KPF]))
        outs.append(host(o))
        rtr.rtr_kv_append_evict(kv, dev(k), dev(v), C)
        ref.append(k.values.reshape(C, KPF, H, D), v.values.reshape(C, KPF, H, D))
    # periodic content: once the window is full the outputs no longer depend on time
    for o in outs[3:6]:
        assert_bf16_close(o, outs[2], "time invariance")
    # a restored snapshot rotates the reference again
    st = rtr.rtr_kv_get_state(kv)
    view.zero_()
    rtr.rtr_kv_set_state(kv, st)
    q = _bf16(np.concatenate([rope_rotate(fq, np.full(KPF, st.next_frame_id + c + R), PAIRS, BASE) for c in range(C)]))
    rtr.rtr_attn_stream_step(kv, dev(q), dev(k), dev(v), C)
    torch.cuda.synchronize()
    assert float(view[:R].abs().max()) > 0
    kv.close()
