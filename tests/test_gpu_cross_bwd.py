"""GPU parity of the text cross-attention's gradients (rtr_attn_cross_bwd,
through the C ABI) against the float64 oracle (attn_cross_bwd): the query
gradient and, optionally, the current text condition's key and value
gradients (RTR-DiT notes, Key Designs 1 and 3).  o and lse come from the
library's own cross-attention call."""

import numpy as np
import pytest
import torch

from oracle.attention_bwd import attn_cross_bwd
from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from tests.gpu_util import assert_grad_close, dev, guarded_empty, host

pytestmark = pytest.mark.gpu

D = 128


def _run(Tq, Lt, H, text_grads, seed, scale=0.0, cap=None):
    q, k, v = gen.cross_inputs(Tq, Lt, H, D, "bf16", base_seed=seed, wid=72)
    do = gen.normal((Tq, H, D), "bf16", seed, 72, 0, gen.TAG_DO)
    kb = torch.zeros((cap or Lt, H, D), dtype=torch.bfloat16, device="cuda")
    vb = torch.zeros_like(kb)
    tc = rtr.rtr_text_cache_create(kb, vb, cap or Lt, H, D, rtr.RTR_BF16)
    rtr.rtr_text_cache_reset(tc, dev(k), dev(v), Lt)
    tq = dev(q)
    o, lse = rtr.rtr_attn_cross(tc, tq, want_lse=True, scale=scale)
    outs, checks = {}, []
    for name, shape in (("dq", (Tq, H, D)), ("dk_text", (Lt, H, D)), ("dv_text", (Lt, H, D))):
        if name == "dq" or text_grads:
            outs[name], chk = guarded_empty(shape, torch.bfloat16)
            checks.append(chk)
    got = rtr.rtr_attn_cross_bwd(tc, tq, o, lse, dev(do), scale=scale, **outs)
    torch.cuda.synchronize()
    for chk in checks:
        chk()
    ref = attn_cross_bwd(q.values, k.values, v.values, do.values, scale=None if scale <= 0 else scale)
    tc.close()
    return got, ref


@pytest.mark.parametrize("Tq,Lt,H,text_grads", [
    (700, 77, 2, True),     # ragged rows and ragged text
    (300, 1, 1, True),      # one text token
    (513, 512, 2, False),   # the Wan text length, text held constant
    (33, 300, 3, True),     # fewer rows than one 256-row block
    (1, 20, 1, True),       # a single query row
])
def test_cross_bwd_matches_oracle(Tq, Lt, H, text_grads):
    print(f"Tq={Tq} Lt={Lt} H={H} text_grads={text_grads}", flush=True)
    got, ref = _run(Tq, Lt, H, text_grads, seed=Tq + Lt)
    n = 3 if text_grads else 1
    for name, g_, r_ in list(zip(("dq", "dk_text", "dv_text"), got, ref))[:n]:
        assert_grad_close(host(g_), r_, name)
    if not text_grads:
        assert got[1] is None and got[2] is None


def test_cross_bwd_scale_and_cache_larger_than_condition():
    got, ref = _run(200, 40, 2, True, seed=5, scale=0.05, cap=128)
    for name, g_, r_ in zip(("dq", "dk_text", "dv_text"), got, ref):
        assert_grad_close(host(g_), r_, name)


def test_cross_bwd_wan_chunk():
    """A 3-frame Wan-1.3B chunk (4,680 rows, 12 heads) against 512 text tokens,
    every gradient against the dense oracle."""
    got, ref = _run(4680, 512, 12, True, seed=9)
    for name, g_, r_ in zip(("dq", "dk_text", "dv_text"), got, ref):
        assert_grad_close(host(g_), r_, name)


@pytest.mark.parametrize("Tq,Lt,H,cap", [
    (4680, 77, 2, None),    # ragged text: the last key block holds 77 of 256 keys
    (1100, 300, 3, None),   # ragged rows and a second, partial text key block
    (1200, 100, 2, 256),    # a cache larger than the condition
])
def test_cross_bwd_split_pieces_with_ragged_text(Tq, Lt, H, cap):
    """The text key blocks split over the query rows (fp32 partials summed in
    fixed order) with text lengths that end inside a key block."""
    # the split is taken: its workspace carries the fp32 partial gradients
    assert rtr.rtr_attn_cross_bwd_workspace_size(Tq, Lt, H) > rtr.rtr_attn_bwd_workspace_size(Tq, H)
    print(f"Tq={Tq} Lt={Lt} H={H} cap={cap}", flush=True)
    got, ref = _run(Tq, Lt, H, True, seed=Tq + 3 * Lt, cap=cap)
    for name, g_, r_ in zip(("dq", "dk_text", "dv_text"), got, ref):
        assert_grad_close(host(g_), r_, name)
