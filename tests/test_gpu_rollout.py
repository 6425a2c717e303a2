"""Long streaming rollout at the Wan-1.3B layer shape (12 heads, head_dim 128,
1560 tokens per latent frame): 3-frame chunks through a 6-frame window with an
anchored reference that is swapped every 60 chunks (RTR-DiT notes, Key Designs
4).  Every step checks the ring metadata against the oracle's list window, the
ring and reference bytes bit-exactly, and every row of one head (the head
rotating with the chunk) of O and LSE against the dense float64 oracle.  A snapshot taken mid-rollout and restored into a fresh cache
must replay the rest bit-identically.

Input recipe for this long run: each frame's K/V (and each chunk's Q) is a
rotation, by an offset derived from the frame id, of one seeded N(0,1) bf16
pool per tensor kind.  The bytes of any frame can therefore be regenerated on
the host (numpy) and on the device (torch.roll) without storing 720 frames.
"""

import concurrent.futures
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ListKV, REF_REPLACE
from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from tests.gpu_util import assert_bf16_close, host

pytestmark = pytest.mark.gpu

KPF, H, D, C, W = 1560, 12, 128, 3, 6
N = KPF * H * D
REF_ID = 10_000_000


def _shift(ident, tag):
    return (ident * 104729 + tag * 7919 + 17) % N


class Frames:
    def __init__(self, seed):
        self.pool = {t: gen.normal((N,), "bf16", seed, 4, 0, t).bits
                     for t in (gen.TAG_Q, gen.TAG_K, gen.TAG_V)}
        self.pool_dev = {t: torch.from_numpy(p.view(np.int16)).cuda().view(torch.bfloat16)
                         for t, p in self.pool.items()}

    def host(self, ident, tag, h):
        x = np.roll(self.pool[tag], _shift(ident, tag)).reshape(KPF, H, D)[:, h, :]
        return gen.bf16_bits_to_f32(x)

    def dev(self, ident, tag):
        return torch.roll(self.pool_dev[tag], _shift(ident, tag)).view(KPF, H, D)


def _new_cache():
    kr = torch.zeros((W, KPF, H, D), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    kf = torch.zeros((1, KPF, H, D), dtype=torch.bfloat16, device="cuda")
    vf = torch.zeros_like(kf)
    kv = rtr.rtr_kv_create(kr, vr, kf, vf, W, 1, KPF, H, D, rtr.RTR_BF16)
    return kv, [kr, vr, kf, vf]


def _check_ring(kv, bufs, ref, fr):
    kr, vr, kf, vf = bufs
    s = rtr.rtr_kv_get_state(kv).as_dict()
    assert s["frame_id"] == ref.frame_ids()
    assert s["ref_frames"] == ref.ref_frames() and s["ref_generation"] == ref.ref_generation
    for p, fid in enumerate(ref.frame_ids()):
        slot = s["slot"][p]
        assert torch.equal(kr[slot].view(torch.int16), fr.dev(fid, gen.TAG_K).view(torch.int16))
        assert torch.equal(vr[slot].view(torch.int16), fr.dev(fid, gen.TAG_V).view(torch.int16))
    g = ref.ref[0]
    assert torch.equal(kf[0].view(torch.int16), fr.dev(REF_ID + g, gen.TAG_K).view(torch.int16))
    assert torch.equal(vf[0].view(torch.int16), fr.dev(REF_ID + g, gen.TAG_V).view(torch.int16))


def _chunk(fr, fid0, tag):
    return torch.cat([fr.dev(fid0 + c, tag) for c in range(C)]).contiguous()


def _step(kv, fr, i, ref, keep, check, rng):
    """One rollout chunk: optional reference swap, attention, commit."""
    if i % 60 == 0:
        g = ref.ref_generation + 1
        rk, rv = fr.dev(REF_ID + g, gen.TAG_K)[None], fr.dev(REF_ID + g, gen.TAG_V)[None]
        k_keep = -1 if i == 0 else keep
        rtr.rtr_kv_reset_ref(kv, REF_REPLACE, rk.contiguous(), rv.contiguous(), 1, k_keep)
        ref.reset_ref(REF_REPLACE, np.zeros((1, 1)), np.zeros((1, 1)), keep_recent=k_keep)
    fid0 = 3 * i
    q, k, v = (_chunk(fr, fid0, t) for t in (gen.TAG_Q, gen.TAG_K, gen.TAG_V))
    o, lse = rtr.rtr_attn_stream_step(kv, q, k, v, C, want_lse=check is not None)
    if check is not None:
        # every row of head i mod H against the dense float64 oracle, which
        # runs on a worker thread while the rollout goes on
        h = i % H
        ids = [REF_ID + ref.ref[0]] + ref.frame_ids()
        got_o, got_l = host(o[:, h:h + 1]), host(lse[h:h + 1])

        def job():
            pk = np.concatenate([fr.host(x, gen.TAG_K, h) for x in ids])[:, None, :]
            pv = np.concatenate([fr.host(x, gen.TAG_V, h) for x in ids])[:, None, :]
            cq, ck, cv = (np.concatenate([fr.host(fid0 + c, t, h) for c in range(C)])[:, None, :]
                          for t in (gen.TAG_Q, gen.TAG_K, gen.TAG_V))
            ro, rl = oracle.attn_stream_step(pk, pv, cq, ck, cv, KPF)
            assert_bf16_close(got_o, ro, f"chunk {i} head {h} o")
            assert_bf16_close(got_l, rl, f"chunk {i} head {h} lse")

        check.append(POOL.submit(job))
    rtr.rtr_kv_append_evict(kv, k, v, C)
    ref.append(np.zeros((C, 1)), np.zeros((C, 1)))
    return o


POOL = concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(8, (os.cpu_count() or 2) // 2)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("keep,chunks", [(1, 240), (-1, 125)])
def test_rollout_ring_bit_exact_each_step(keep, chunks):
    fr = Frames(seed=0)
    kv, bufs = _new_cache()
    ref = ListKV(W)
    rng = np.random.default_rng(11)
    snap = None
    outs_after = []
    checks = []
    for i in range(chunks):
        o = _step(kv, fr, i, ref, keep, checks, rng)
        torch.cuda.synchronize()
        _check_ring(kv, bufs, ref, fr)
        if i == 120:
            snap = (rtr.rtr_kv_get_state(kv), [b.clone() for b in bufs], ref.frame_ids(),
                    ref.ref_generation, ref.next_frame_id)
        elif snap is not None:
            outs_after.append(o)
    # resume from the snapshot in a fresh cache and replay the remaining chunks
    state, saved, ids, gen_, next_id = snap
    kv2, bufs2 = _new_cache()
    for dst, src in zip(bufs2, saved):
        dst.copy_(src)
    rtr.rtr_kv_set_state(kv2, state)
    ref2 = ListKV(W)
    ref2.window = [(x, None, None) for x in ids]
    ref2.ref = (gen_, np.zeros((1, 1)), np.zeros((1, 1)))
    ref2.ref_generation = gen_
    ref2.next_frame_id = next_id
    for j, i in enumerate(range(121, chunks)):
        o2 = _step(kv2, fr, i, ref2, keep, None, rng)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16), outs_after[j].view(torch.int16)), i
    _check_ring(kv2, bufs2, ref2, fr)
    assert rtr.rtr_kv_get_state(kv2).as_dict() == rtr.rtr_kv_get_state(kv).as_dict()
    for f in checks:
        f.result()
