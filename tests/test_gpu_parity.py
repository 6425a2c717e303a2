"""GPU parity: the HIP library (through its C ABI) against the float64 oracle on
the same seeded inputs.

Bar: float32 inputs <= 1e-4 max abs error; bf16 inputs (fp32 accumulation)
<= 2e-2 max abs and <= 2e-3 mean abs error; KV ring state and bytes bit-exact
against the oracle's literal list window.  Full-size workloads are checked on
sampled rows that the oracle computes one by one, plus closed forms that hold
exactly at any size.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import ListKV, REF_CLEAR, REF_KEEP, REF_REPLACE
from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from tests.gpu_util import (assert_bf16_close, assert_f32_close, dev, guarded_empty, host, raw)

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
RTR_DT = {"bf16": rtr.RTR_BF16, "f32": rtr.RTR_F32}


def _workspace(d, dtype=rtr.RTR_BF16):
    """A split-K workspace inside guard bands (None when the configuration
    never splits), and the check that nothing was written outside it."""
    n = rtr.rtr_attn_workspace_size(d, dtype)
    if n == 0:
        return None, lambda: None
    return guarded_empty((n,), torch.uint8)


def _run_full(q, k, v, kpf, out_dtype, scale=0.0, split=False):
    T, H, d = q.shape
    o, chk_o = guarded_empty((T, H, d), out_dtype)
    lse, chk_l = guarded_empty((H, T), torch.float32)
    ws, chk_w = _workspace(d, RTR_DT["bf16"] if q.dtype == "bf16" else RTR_DT["f32"]) if split \
        else (None, lambda: None)
    rtr.rtr_attn_block_causal(dev(q), dev(k), dev(v), kpf, o=o, lse=lse, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    chk_o()
    chk_l()
    chk_w()
    return host(o), host(lse)


# ------------------------------------------------------------ tiny fp32 workload
@pytest.mark.parametrize("T", [144, 160])
def test_tiny_fp32_full_form(T):
    # 1 reference frame + 8 latent frames of 16 tokens (144), and the
    # 160-token reading (1 + 9 frames); 2 heads, head_dim 64.
    q, k, v = gen.full_sequence_inputs(T, 2, 64, "f32", base_seed=0, wid=1)
    o, lse = _run_full(q, k, v, 16, torch.float32)
    ro, rl = oracle.attn_block_causal(q.values, k.values, v.values, 16)
    assert_f32_close(o, ro, "o")
    assert_f32_close(lse, rl, "lse")


def _make_cache(W, R, kpf, H, d, dtype):
    tdt = TORCH_DT[dtype]
    kr = torch.zeros((max(W, 1), kpf, H, d), dtype=tdt, device="cuda")
    vr = torch.zeros_like(kr)
    kf = torch.zeros((max(R, 1), kpf, H, d), dtype=tdt, device="cuda")
    vf = torch.zeros_like(kf)
    kv = rtr.rtr_kv_create(kr if W else None, vr if W else None, kf if R else None,
                           vf if R else None, W, R, kpf, H, d, RTR_DT[dtype])
    return kv, kr, vr, kf, vf


def _ring_matches(kv, kr, vr, kf, vf, ref, dtype):
    """Ring state and bytes vs the ListKV oracle, bit-exact."""
    s = rtr.rtr_kv_get_state(kv).as_dict()
    assert s["frame_id"] == ref.frame_ids()
    assert s["ref_frames"] == ref.ref_frames()
    assert s["ref_generation"] == ref.ref_generation
    for p, (fid, k_bits, v_bits) in enumerate(ref.window):
        slot = s["slot"][p]
        assert np.array_equal(raw(kr[slot]), np.ascontiguousarray(k_bits).view(np.uint8)), (p, fid)
        assert np.array_equal(raw(vr[slot]), np.ascontiguousarray(v_bits).view(np.uint8)), (p, fid)
    if ref.ref is not None:
        R = len(ref.ref[1])
        assert np.array_equal(raw(kf[:R]), np.ascontiguousarray(ref.ref[1]).view(np.uint8))
        assert np.array_equal(raw(vf[:R]), np.ascontiguousarray(ref.ref[2]).view(np.uint8))


def _as_values(bits_or_vals, dtype):
    return gen.bf16_bits_to_f32(bits_or_vals) if dtype == "bf16" else bits_or_vals


def _stream_rollout(kpf, H, d, C, W, R, steps, dtype, switches=(), seed=0, out_dtype=None,
                    check_bytes=True, split=False):
    """Drive the library and the ListKV oracle in lockstep; returns worst errors."""
    kv, kr, vr, kf, vf = _make_cache(W, R, kpf, H, d, dtype)
    ws, chk_w = _workspace(d, RTR_DT[dtype]) if split else (None, lambda: None)
    ref = ListKV(W)
    out_dtype = out_dtype or TORCH_DT[dtype]
    worst = []
    for step in range(steps):
        sw = dict(switches).get(step)
        if sw is not None:
            mode, keep = sw
            if mode == REF_REPLACE:
                rk = gen.normal((R, kpf, H, d), dtype, seed, 7, step, gen.TAG_REFK)
                rv = gen.normal((R, kpf, H, d), dtype, seed, 7, step, gen.TAG_REFV)
                rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(rk), dev(rv), R, keep)
                ref.reset_ref(REF_REPLACE, rk.storage(), rv.storage(), keep_recent=keep)
            else:
                rtr.rtr_kv_reset_ref(kv, mode, None, None, R, keep)
                ref.reset_ref(mode, keep_recent=keep)
        q, k, v = (gen.normal((C * kpf, H, d), dtype, seed, 7, step, t)
                   for t in (gen.TAG_Q, gen.TAG_K, gen.TAG_V))
        o, chk = guarded_empty((C * kpf, H, d), out_dtype)
        lse, chk2 = guarded_empty((H, C * kpf), torch.float32)
        kd, vd = dev(k), dev(v)
        rtr.rtr_attn_stream_step(kv, dev(q), kd, vd, C, o=o, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        chk()
        chk2()
        chk_w()
        pk, pv = ref.prefix(kpf, H, d, dtype=k.storage().dtype)
        ro, rl = oracle.attn_stream_step(_as_values(pk, dtype), _as_values(pv, dtype), q.values,
                                         k.values, v.values, kpf)
        if dtype == "f32":
            worst.append((assert_f32_close(host(o), ro, f"step {step} o"),
                          assert_f32_close(host(lse), rl, f"step {step} lse")))
        else:
            worst.append(assert_bf16_close(host(o), ro, f"step {step} o"))
            assert_bf16_close(host(lse), rl, f"step {step} lse")
        rtr.rtr_kv_append_evict(kv, kd, vd, C)
        ref.append(k.storage().reshape(C, kpf, H, d), v.storage().reshape(C, kpf, H, d))
        torch.cuda.synchronize()
        if check_bytes:
            _ring_matches(kv, kr, vr, kf, vf, ref, dtype)
    return worst


def test_tiny_fp32_stream_form():
    # window 4 frames + anchored reference, chunk = 1 frame, 8 chunk steps
    _stream_rollout(kpf=16, H=2, d=64, C=1, W=4, R=1, steps=8, dtype="f32",
                    switches={0: (REF_REPLACE, -1)}.items())


# ------------------------------------------------------------ bf16, several tiles
FULL_CASES = [
    # T, k, H, d
    (737, 100, 3, 128),    # ragged query/key tails, frames straddle tiles
    (737, 100, 3, 64),
    (300, 1, 2, 128),      # k = 1: token-causal, every tile on the diagonal is partial
    (500, 1000, 2, 128),   # k >= T: bidirectional teacher, no mask
    (64, 64, 1, 128),      # exactly one tile
    (1, 1, 1, 128),        # a single token
    (129, 7, 2, 64),
    (2000, 160, 2, 128),
    # launches of one round that the forward planner serves with paired row
    # groups: frames of 160 and 96 rows (groups aligned to frames), an even
    # frame count (960 rows) and an odd one with a partial last frame
    (960, 160, 2, 128),
    (1000, 96, 2, 128),
]


@pytest.mark.parametrize("T,kpf,H,d", FULL_CASES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_bf16_full_form(T, kpf, H, d, out, split):
    q, k, v = gen.full_sequence_inputs(T, H, d, "bf16", base_seed=1, wid=30, step=T + kpf)
    o, lse = _run_full(q, k, v, kpf, TORCH_DT[out], split=split)
    ro, rl = oracle.attn_block_causal(q.values, k.values, v.values, kpf)
    assert_bf16_close(o, ro, "o")
    assert_bf16_close(lse, rl, "lse")


@pytest.mark.parametrize("T,kpf", [(300, 1), (737, 100)])
def test_fp32_full_form_several_tiles(T, kpf):
    q, k, v = gen.full_sequence_inputs(T, 2, 128, "f32", base_seed=2, wid=31, step=T)
    o, lse = _run_full(q, k, v, kpf, torch.float32, scale=0.05)
    ro, rl = oracle.attn_block_causal(q.values, k.values, v.values, kpf, scale=0.05)
    assert_f32_close(o, ro, "o")
    assert_f32_close(lse, rl, "lse")


@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_bf16_stream_with_switches(split):
    sw = {0: (REF_REPLACE, -1), 4: (REF_REPLACE, 1), 6: (REF_KEEP, 2), 8: (REF_CLEAR, 0),
          9: (REF_REPLACE, -1)}
    _stream_rollout(kpf=100, H=2, d=128, C=2, W=3, R=1, steps=11, dtype="bf16",
                    switches=sw.items(), split=split)


@pytest.mark.parametrize("kpf,H,d,C,W,R,steps", [
    (50, 2, 128, 1, 0, 0, 2),     # no window, no reference: the chunk alone
    (50, 1, 64, 3, 5, 1, 3),      # window filling up (count < W for two steps)
    (40, 2, 128, 4, 2, 1, 3),     # chunk longer than the window: only newest W kept
    (24, 1, 128, 16, 4, 1, 2),    # largest chunk
    (8, 1, 64, 1, 64, 1, 66),     # largest window, wraps around
])
@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_bf16_stream_edges(kpf, H, d, C, W, R, steps, split):
    sw = {0: (REF_REPLACE, -1)} if R else {}
    _stream_rollout(kpf=kpf, H=H, d=d, C=C, W=W, R=R, steps=steps, dtype="bf16",
                    switches=sw.items(), split=split)


def test_stream_f32_output_of_bf16_cache():
    _stream_rollout(kpf=100, H=2, d=128, C=2, W=2, R=1, steps=3, dtype="bf16",
                    switches={0: (REF_REPLACE, -1)}.items(), out_dtype=torch.float32)


# ------------------------------------------------------------ invariants on the GPU
@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_causality_bitwise_and_determinism(split):
    T, H, d, kpf = 1560 * 4, 2, 128, 1560
    q, k, v = gen.full_sequence_inputs(T, H, d, "bf16", base_seed=3, wid=32)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws = rtr.new_workspace(d) if split else None
    o1, l1 = rtr.rtr_attn_block_causal(qd, kd, vd, kpf, want_lse=True, workspace=ws)
    o2, l2 = rtr.rtr_attn_block_causal(qd, kd, vd, kpf, want_lse=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    cut = 2 * kpf
    kd2, vd2, qd2 = kd.clone(), vd.clone(), qd.clone()
    kd2[cut:] = -kd2[cut:] * 4
    vd2[cut:] = vd2[cut:] + 3
    qd2[cut:] = qd2[cut:] * 2
    o3, l3 = rtr.rtr_attn_block_causal(qd2, kd2, vd2, kpf, want_lse=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1[:cut].view(torch.int16), o3[:cut].view(torch.int16))
    assert torch.equal(l1[:, :cut], l3[:, :cut])
    assert not torch.equal(o1[cut:], o3[cut:])


@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_full_shape_closed_form_frame_mean(split):
    # Full block-causal workload shape (22 frames x 1560 tokens, 12 heads,
    # head_dim 128): Q = 0 makes all visible logits 0, and V_j = floor(j/k)
    # gives O_i = floor(i/k)/2 exactly and LSE_i = ln(k (floor(i/k) + 1)).
    kpf, F, H, d = 1560, 22, 12, 128
    T = kpf * F
    q = torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda")
    kk = torch.randn((T, H, d), device="cuda").to(torch.bfloat16) * 0
    fr = torch.arange(T, device="cuda") // kpf
    v = fr[:, None, None].expand(T, H, d).to(torch.bfloat16).contiguous()
    ws = rtr.new_workspace(d) if split else None
    o, lse = rtr.rtr_attn_block_causal(q, kk, v, kpf, want_lse=True, workspace=ws)
    torch.cuda.synchronize()
    expect = (fr.float() / 2)[:, None, None].expand(T, H, d)
    assert torch.equal(o.float(), expect)
    el = torch.log(kpf * (fr.double() + 1))[None, :].expand(H, T)
    assert float((lse.double() - el).abs().max()) < 2e-5


# ------------------------------------------------------------ full-size workloads, sampled
def _sample_rows(Tq, kpf, n_rand, seed):
    rows = {0, Tq - 1}
    for f in range(0, Tq, kpf):
        rows |= {f, min(f + kpf - 1, Tq - 1), min(f + kpf, Tq - 1)}
    for t in range(0, Tq, 128):
        rows |= {t, max(t - 1, 0), min(t + 64, Tq - 1)}
    rng = np.random.default_rng(seed)
    rows |= set(rng.integers(0, Tq, n_rand).tolist())
    return sorted(rows)


def _stream_workload(name, seed=0):
    """A streaming workload by name; a `_k<N>` suffix sets N tokens per frame."""
    base, _, k = name.partition("_k")
    w = dict(gen.WORKLOADS[base], **({"k": int(k)} if k else {}))
    kpf, H, d, C, W, R = w["k"], w["H"], w["d"], w["C"], w["W"], w["R"]
    x = gen.stream_inputs(kpf, H, d, C, W, R, "bf16", base_seed=seed, wid=w["wid"],
                          outlier_frac=w.get("outlier_frac", 0.0),
                          outlier_scale=w.get("outlier_scale", 1.0))
    kv, kr, vr, kf, vf = _make_cache(W, R, kpf, H, d, "bf16")
    rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(x["ref_k"]), dev(x["ref_v"]), R, -1)
    rtr.rtr_kv_append_evict(kv, dev(x["ring_k"]), dev(x["ring_v"]), W)
    return w, x, kv, (kr, vr, kf, vf)


_DENSE = {}


def _dense_stream_reference(name, x, w):
    """float64 oracle of the whole step (every head, every row), computed once
    per workload and shared by the plain and the split launch."""
    if name not in _DENSE:
        H, d, kpf = w["H"], w["d"], w["k"]
        pk = np.concatenate([x["ref_k"].values.reshape(-1, H, d), x["ring_k"].values.reshape(-1, H, d)])
        pv = np.concatenate([x["ref_v"].values.reshape(-1, H, d), x["ring_v"].values.reshape(-1, H, d)])
        _DENSE[name] = oracle.attn_stream_step(pk, pv, x["q"].values, x["k"].values, x["v"].values, kpf)
    return _DENSE[name]


@pytest.mark.parametrize("name", ["wan13b_stream_step", "wan14b_stream_step", "wan13b_stream_step_k2080"])
@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_full_size_stream_step_every_element(name, split):
    """The Wan-1.3B step and the Wan-14B step (1 % of key rows x8) at full
    size, every head and every row of O and LSE against the dense float64
    oracle over [reference | window | chunk]; also the Wan-1.3B step with
    2,080-token frames (40 x 52 patches of an 832 x 640 frame), whose 288
    workgroups take more than one round."""
    w, x, kv, bufs = _stream_workload(name)
    kpf, H, d, C = w["k"], w["H"], w["d"], w["C"]
    Tq = C * kpf
    o, chk = guarded_empty((Tq, H, d), torch.bfloat16)
    lse, chk2 = guarded_empty((H, Tq), torch.float32)
    ws, chk_w = _workspace(d) if split else (None, lambda: None)
    rtr.rtr_attn_stream_step(kv, dev(x["q"]), dev(x["k"]), dev(x["v"]), C, o=o, lse=lse,
                             workspace=ws)
    torch.cuda.synchronize()
    chk()
    chk2()
    chk_w()
    ro, rl = _dense_stream_reference(name, x, w)
    mx, mean = assert_bf16_close(host(o), ro, "o")
    lmx, lmean = assert_bf16_close(host(lse), rl, "lse")
    print(f"{name} {'split' if split else 'plain'}: o max {mx:.3g} mean {mean:.3g}; "
          f"lse max {lmx:.3g} mean {lmean:.3g}", flush=True)


@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_full_size_block_causal_sampled(split):
    w = gen.WORKLOADS["full_block_causal"]
    kpf, H, d, F = w["k"], w["H"], w["d"], w["frames"]
    T = kpf * F
    q, k, v = gen.full_sequence_inputs(T, H, d, "bf16", base_seed=0, wid=w["wid"])
    o, chk = guarded_empty((T, H, d), torch.bfloat16)
    lse, chk2 = guarded_empty((H, T), torch.float32)
    ws, chk_w = _workspace(d) if split else (None, lambda: None)
    rtr.rtr_attn_block_causal(dev(q), dev(k), dev(v), kpf, o=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    chk()
    chk2()
    chk_w()
    # every head; rows at every frame start and end and around every 128-row
    # tile boundary (every third of them) plus random rows
    rows = _sample_rows(T, kpf, 16, seed=6)[::3]
    if "full_block_causal" not in _DENSE:
        _DENSE["full_block_causal"] = oracle.attn_rows(q.values, k.values, v.values, kpf, rows)
    ro, rl = _DENSE["full_block_causal"]
    assert_bf16_close(host(o)[rows], ro, "o")
    assert_bf16_close(host(lse)[:, rows], rl, "lse")


def test_full_size_stream_closed_form_labels():
    # Streaming step at the Wan-1.3B shape with Q = K = 0 and V = a per-frame
    # integer label: chunk frame c must output the mean label of
    # [reference, window frames, chunk frames 0..c].  Pins which frames the
    # kernel reads from the ring after evictions and a reference swap.
    kpf, H, d, C, W = 1560, 12, 128, 3, 6
    kv, kr, vr, kf, vf = _make_cache(W, 1, kpf, H, d, "bf16")
    ref = ListKV(W)

    def lab(x, n=1):
        return torch.full((n, kpf, H, d), float(x), dtype=torch.bfloat16, device="cuda")

    zeros_chunk = torch.zeros((C * kpf, H, d), dtype=torch.bfloat16, device="cuda")
    ref_label = 250
    rtr.rtr_kv_reset_ref(kv, REF_REPLACE, lab(0), lab(ref_label), 1, -1)
    ref.reset_ref(REF_REPLACE, np.zeros(1), np.array([ref_label]), keep_recent=-1)
    fid = 0
    for step in range(6):
        if step == 4:
            ref_label = 249
            rtr.rtr_kv_reset_ref(kv, REF_REPLACE, lab(0), lab(ref_label), 1, 1)
            ref.reset_ref(REF_REPLACE, np.zeros(1), np.array([ref_label]), keep_recent=1)
        labels = [(fid + c) % 200 for c in range(C)]
        vch = torch.cat([lab(x)[0] for x in labels])
        o, _ = rtr.rtr_attn_stream_step(kv, zeros_chunk, zeros_chunk, vch, C,
                                        out_dtype=torch.float32)
        torch.cuda.synchronize()
        prefix = ([ref_label] if ref.ref is not None else []) + [i % 200 for i in ref.frame_ids()]
        for c in range(C):
            exp = np.mean(prefix + labels[:c + 1])
            blk = o[c * kpf:(c + 1) * kpf].double()
            assert float((blk - exp).abs().max()) <= 1e-5 * max(1.0, exp), (step, c)
        rtr.rtr_kv_append_evict(kv, torch.zeros((C, kpf, H, d), dtype=torch.bfloat16,
                                                device="cuda"), vch.view(C, kpf, H, d), C)
        ref.append(np.zeros((C, 1)), np.zeros((C, 1)))
        fid += C


def test_split_matches_plain_at_full_size():
    # The split schedule changes the order of the fp32 additions and, since
    # each piece rounds P to bf16 relative to its own exponent reference, the
    # bf16 rounding of individual weights (relative 2^-9, averaged over ~1.5e4
    # keys per row).  Against the one-workgroup-per-unit launch it must stay
    # an order of magnitude inside the bf16 bar on the max and mean.
    w, x, kv, bufs = _stream_workload("wan13b_stream_step", seed=3)
    C = w["C"]
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o1, l1 = rtr.rtr_attn_stream_step(kv, q, k, v, C, want_lse=True, out_dtype=torch.float32)
    o2, l2 = rtr.rtr_attn_stream_step(kv, q, k, v, C, want_lse=True, out_dtype=torch.float32,
                                      workspace=rtr.new_workspace(w["d"]))
    torch.cuda.synchronize()
    d = (o1 - o2).abs()
    assert float(d.max()) < 2e-3 and float(d.mean()) < 1e-4
    assert float((l1 - l2).abs().max()) < 1e-3   # row sums of bf16-rounded weights


def test_split_runs_and_matches_plain_one_frame_chunk():
    # A one-frame chunk on the Wan-1.3B layer (84 units of 256 rows for 256
    # compute units): the schedule splits, so the workspace must be written,
    # and the result must match the plain launch within the bars above.
    kpf, H, d, W, R = 1560, 12, 128, 6, 1
    x = gen.stream_inputs(kpf, H, d, 1, W, R, "bf16", base_seed=5, wid=2)
    kv, kr, vr, kf, vf = _make_cache(W, R, kpf, H, d, "bf16")
    rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(x["ref_k"]), dev(x["ref_v"]), R, -1)
    rtr.rtr_kv_append_evict(kv, dev(x["ring_k"]), dev(x["ring_v"]), W)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o1, l1 = rtr.rtr_attn_stream_step(kv, q, k, v, 1, want_lse=True, out_dtype=torch.float32)
    ws = rtr.new_workspace(d)
    ws.fill_(0xFF)
    o2, l2 = rtr.rtr_attn_stream_step(kv, q, k, v, 1, want_lse=True, out_dtype=torch.float32,
                                      workspace=ws)
    torch.cuda.synchronize()
    assert int((ws != 0xFF).sum()) > 0, "the split path did not run"
    d_o = (o1 - o2).abs()
    assert float(d_o.max()) < 2e-3 and float(d_o.mean()) < 1e-4
    assert float((l1 - l2).abs().max()) < 1e-3
    pk = np.concatenate([x["ref_k"].values.reshape(-1, H, d), x["ring_k"].values.reshape(-1, H, d)])
    pv = np.concatenate([x["ref_v"].values.reshape(-1, H, d), x["ring_v"].values.reshape(-1, H, d)])
    rows = _sample_rows(kpf, kpf, 16, seed=6)
    heads = [0, H - 1]
    ro, rl = oracle.attn_stream_rows(pk, pv, x["q"].values, x["k"].values, x["v"].values, kpf,
                                     rows, heads)
    assert_bf16_close(host(o2)[rows][:, heads], ro, "o")
    assert_bf16_close(host(l2)[heads][:, rows], rl, "lse")


@pytest.mark.parametrize("kpf,C,H", [(700, 3, 30), (1000, 2, 35)])
def test_overflow_split_runs_and_matches_oracle(kpf, C, H):
    # Units (heads x 256-row blocks: 270 and 280) just beyond one round of the
    # 256 compute units, behind a reference and a full 6-frame window: with a
    # workspace the launch runs the heavier query blocks whole and cuts the
    # first block of every head into pieces shared by all workgroups, so the
    # workspace must be written; every element of O and LSE against the dense
    # oracle, and against the plain launch within the split bars above.
    d, W, R = 128, 6, 1
    x = gen.stream_inputs(kpf, H, d, C, W, R, "bf16", base_seed=7, wid=3)
    kv, kr, vr, kf, vf = _make_cache(W, R, kpf, H, d, "bf16")
    rtr.rtr_kv_reset_ref(kv, REF_REPLACE, dev(x["ref_k"]), dev(x["ref_v"]), R, -1)
    rtr.rtr_kv_append_evict(kv, dev(x["ring_k"]), dev(x["ring_v"]), W)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    print(f"kpf={kpf} C={C} H={H}: units {(C * kpf + 255) // 256 * H}", flush=True)
    o1, l1 = rtr.rtr_attn_stream_step(kv, q, k, v, C, want_lse=True, out_dtype=torch.float32)
    ws, chk_w = _workspace(d)
    ws.fill_(0xFF)
    o2, chk_o = guarded_empty((C * kpf, H, d), torch.bfloat16)
    l2, chk_l = guarded_empty((H, C * kpf), torch.float32)
    rtr.rtr_attn_stream_step(kv, q, k, v, C, o=o2, lse=l2, workspace=ws)
    torch.cuda.synchronize()
    chk_w()
    chk_o()
    chk_l()
    assert int((ws != 0xFF).sum()) > 0, "the split path did not run"
    d_o = (o1 - o2.float()).abs()
    assert float(d_o.max()) < 2e-2 and float(d_o.mean()) < 1e-3
    assert float((l1 - l2).abs().max()) < 1e-3
    pk = np.concatenate([x["ref_k"].values.reshape(-1, H, d), x["ring_k"].values.reshape(-1, H, d)])
    pv = np.concatenate([x["ref_v"].values.reshape(-1, H, d), x["ring_v"].values.reshape(-1, H, d)])
    ro, rl = oracle.attn_stream_step(pk, pv, x["q"].values, x["k"].values, x["v"].values, kpf)
    assert_bf16_close(host(o2), ro, "o")
    assert_bf16_close(host(l2), rl, "lse")


def test_split_workspace_too_small_is_rejected():
    q = torch.zeros((512, 1, 128), dtype=torch.bfloat16, device="cuda")
    need = rtr.rtr_attn_workspace_size(128)
    assert need > 0
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(rtr.RtrError) as e:
        rtr.rtr_attn_block_causal(q, q, q, 64, workspace=small)
    assert e.value.code == rtr.RTR_EINVAL


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_softmax_reference_fallback_rows(out, split):
    # Rows whose scores grow far beyond their first key tile's maximum (here
    # by 512 / sqrt(128) natural units, i.e. a factor 2^65 in the softmax
    # numerator) take the exact-maximum second pass; rows of the same
    # workgroup with flat scores do not.  Both must match the oracle.
    T, H, d = 600, 2, 128
    rng = np.random.default_rng(7)
    q = np.zeros((T, H, d), dtype=np.float32)
    q[::2] = 1.0                                   # even rows: large growth, odd rows: flat
    k = np.zeros((T, H, d), dtype=np.float32)
    k[40:] = 4.0                                   # first 32-key tile scores 0, later 512
    k[300:310] = -4.0
    v = rng.standard_normal((T, H, d)).astype(np.float32)
    q, k, v = (gen.from_values(gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x)), "bf16")
               for x in (q, k, v))
    for kpf in (T, 100):
        o, lse = _run_full(q, k, v, kpf, TORCH_DT[out], split=split)
        ro, rl = oracle.attn_block_causal(q.values, k.values, v.values, kpf)
        assert_bf16_close(o, ro, f"o k={kpf}")
        assert_bf16_close(lse, rl, f"lse k={kpf}")
