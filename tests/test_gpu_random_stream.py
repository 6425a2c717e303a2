"""GPU parity of the streaming step and its backward on seeded random cache
states, through the C ABI, against the float64 oracle: random frame lengths
(token-level frames included), head counts, window sizes and fill levels (the
ring wrapped or not), reference counts, chunk lengths, in-chunk mask blocks,
cache gradients on or off and the position-aware reference on or off.  The
cases are drawn once from a fixed seed, so the set is the same on every run.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import ListKV, REF_REPLACE
from oracle.attention_bwd import attn_stream_step_bwd
from oracle.rope import reference_shift, rope_rotate
from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from tests.gpu_util import assert_bf16_close, assert_grad_close, dev, host

pytestmark = pytest.mark.gpu

D = 128


def _cases(n=48, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kpf = int(rng.choice([1, 3, 16, 33, 40, 64, 96, 130, 257]))
        H = int(rng.integers(1, 4))
        W = int(rng.integers(0, 6))
        R = int(rng.integers(0, 5))
        n_past = int(rng.integers(0, 2 * W + 2)) if W else 0
        C = int(rng.integers(1, 5))
        B = int(rng.integers(1, C + 2))
        cache_grads = bool(rng.integers(0, 2))
        rope = bool(R > 0 and rng.integers(0, 2))
        # keep the float64 oracle quick: at most ~1,500 keys and ~600 query rows
        while (R + min(n_past, W) + C) * kpf > 1500 or C * kpf > 600:
            kpf = max(1, kpf // 2)
        out.append((i, kpf, H, W, R, n_past, C, B, cache_grads, rope))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "k{1}h{2}w{3}r{4}p{5}c{6}b{7}{8}{9}".format(*c))
def test_random_stream_step_and_backward(case):
    i, kpf, H, W, R, n_past, C, B, cache_grads, rope = case
    print(f"case {case}", flush=True)
    kr = torch.zeros((max(W, 1), kpf, H, D), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    kf = torch.zeros((max(R, 1), kpf, H, D), dtype=torch.bfloat16, device="cuda")
    vf = torch.zeros_like(kf)
    kv = rtr.rtr_kv_create(kr, vr, kf, vf, W, max(R, 1), kpf, H, D)
    ref = ListKV(W)
    PAIRS, BASE = 22, 10000.0
    if rope:
        view = torch.zeros_like(kf)
        rtr.rtr_kv_set_ref_rope(kv, view, PAIRS, BASE, R)
    x = gen.stream_inputs(kpf, H, D, C, max(n_past, 1), max(R, 1), "bf16", base_seed=100 + i, wid=95)
    if R:
        rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(x["ref_k"]).view(R, kpf, H, D)[:R],
                             dev(x["ref_v"]).view(R, kpf, H, D)[:R], R, -1)
        ref.reset_ref(REF_REPLACE, x["ref_k"].values[:R], x["ref_v"].values[:R], keep_recent=-1)
    for f in range(n_past):
        fk, fv = x["ring_k"].values[f:f + 1], x["ring_v"].values[f:f + 1]
        rtr.rtr_kv_append_evict(kv, dev(gen.from_values(fk, "bf16")), dev(gen.from_values(fv, "bf16")), 1)
        ref.append(fk, fv)
    do = gen.normal((C * kpf, H, D), "bf16", 100 + i, 95, 0, gen.TAG_DO)
    q, k, v, tdo = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(do)
    o, lse = rtr.rtr_attn_stream_step_blocked(kv, q, k, v, C, B, want_lse=True)
    got = rtr.rtr_attn_stream_step_bwd(kv, q, k, v, o, lse, tdo, C, B, want_cache_grads=cache_grads)
    torch.cuda.synchronize()

    pk, pv = ref.prefix(kpf, H, D)
    shift = None
    if rope:
        ids = ref.frame_ids()
        st = rtr.rtr_kv_get_state(kv)
        shift = reference_shift((ids[0] if ids else st.next_frame_id) + R, R)
        pk = pk.copy()
        rot = rope_rotate(pk[:R * kpf], np.full(R * kpf, shift), PAIRS, BASE)
        pk[:R * kpf] = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rot.astype(np.float32)))
    unit = min(B, C) * kpf
    ro, rl = oracle.attn_stream_step(pk, pv, x["q"].values, x["k"].values, x["v"].values, unit)
    assert_bf16_close(host(o), ro, "o")
    assert_bf16_close(host(lse), rl, "lse")
    r = list(attn_stream_step_bwd(pk, pv, x["q"].values, x["k"].values, x["v"].values, do.values, unit))
    if rope:
        r[3] = r[3].copy()
        r[3][:R * kpf] = rope_rotate(r[3][:R * kpf], np.full(R * kpf, -shift), PAIRS, BASE)
    names = ("dq", "dk", "dv", "dk_cache", "dv_cache")
    for name, g_, r_ in list(zip(names, got, r))[:5 if cache_grads else 3]:
        if r_.shape[0] == 0 or not np.any(r_):
            continue
        assert_grad_close(host(g_), r_, name)
    if not cache_grads:
        assert got[3] is None
    kv.close()
