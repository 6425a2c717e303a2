"""GPU parity of the attention gradients (rtr_attn_block_causal_bwd, through
the C ABI) against the float64 oracle's derivative of the Attn equation (RTR-DiT
notes, Key Designs 2).  The forward's o and lse come from the library's own
forward call, as the entry point requires; the oracle recomputes everything
from q, k, v and dO alone."""

import numpy as np
import pytest
import torch

from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from oracle.attention_bwd import attn_block_causal_bwd, attn_bwd_cols, attn_bwd_rows
from tests.gpu_util import assert_grad_close, dev, host

pytestmark = pytest.mark.gpu


def _run(T, H, kpf, seed, wid=40):
    q, k, v, do = gen.bwd_inputs(T, H, 128, "bf16", base_seed=seed, wid=wid)
    tq, tk, tv, tdo = (dev(x) for x in (q, k, v, do))
    o, lse = rtr.rtr_attn_block_causal(tq, tk, tv, kpf, want_lse=True)
    dq, dk, dv = rtr.rtr_attn_block_causal_bwd(tq, tk, tv, o, lse, tdo, kpf)
    torch.cuda.synchronize()
    return (q, k, v, do), (dq, dk, dv)


@pytest.mark.parametrize("T,H,kpf", [
    (700, 2, 96),     # frames straddle the 32-row and 256-row tiles, ragged tail
    (600, 1, 256),    # frame = one key block
    (513, 2, 1),      # token causality, one row past a block
    (300, 1, 4096),   # k >= T: unmasked
    (1560 * 2 + 77, 1, 1560),  # Wan frame length, two frames and a ragged third
    (1, 1, 1),
    (33, 3, 5),
])
def test_bwd_matches_oracle(T, H, kpf):
    (q, k, v, do), (dq, dk, dv) = _run(T, H, kpf, seed=T + kpf)
    rq, rk, rv = attn_block_causal_bwd(q.values, k.values, v.values, do.values, kpf)
    print(f"T={T} H={H} kpf={kpf}", flush=True)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert_grad_close(host(got), ref, f"{name} T={T} kpf={kpf}")


def test_bwd_is_deterministic_and_scale_argument():
    T, H, kpf = 900, 2, 200
    q, k, v, do = gen.bwd_inputs(T, H, 128, "bf16", base_seed=3, wid=41)
    tq, tk, tv, tdo = (dev(x) for x in (q, k, v, do))
    o, lse = rtr.rtr_attn_block_causal(tq, tk, tv, kpf, want_lse=True, scale=0.05)
    a = rtr.rtr_attn_block_causal_bwd(tq, tk, tv, o, lse, tdo, kpf, scale=0.05)
    b = rtr.rtr_attn_block_causal_bwd(tq, tk, tv, o, lse, tdo, kpf, scale=0.05)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    ref = attn_block_causal_bwd(q.values, k.values, v.values, do.values, kpf, scale=0.05)
    for name, got, r in zip(("dq", "dk", "dv"), a, ref):
        assert_grad_close(host(got), r, name)


def test_bwd_zero_tokens_is_noop():
    x = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, 0), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    dq, dk, dv = rtr.rtr_attn_block_causal_bwd(x, x, x, x, lse, x, 4, workspace=ws)
    assert dq.shape == (0, 2, 128)


def test_bwd_full_size_sampled():
    """The timed workload (22 frames of 1,560 tokens, 12 heads): dQ on sampled
    rows and dK/dV on sampled keys of two heads, each computed one by one by
    the oracle from the rows and keys it needs."""
    w = gen.WORKLOADS["full_block_causal_bwd"]
    kpf, H, F = w["k"], w["H"], w["frames"]
    T = kpf * F
    (q, k, v, do), (dq, dk, dv) = _run(T, H, kpf, seed=0, wid=w["wid"])
    rng = np.random.default_rng(5)
    heads = [0, H - 1]
    rows = sorted(set(rng.choice(T, 24, replace=False).tolist()) | {0, kpf - 1, kpf, T - 1})
    got = host(dq[rows][:, heads])
    ref = attn_bwd_rows(q.values, k.values, v.values, do.values, kpf, rows, heads)
    assert_grad_close(got, ref, "dq rows")
    # keys of the last three frames keep the oracle's row range short
    lo = (F - 3) * kpf
    cols = sorted(set(rng.choice(np.arange(lo, T), 24, replace=False).tolist()) | {lo, T - 1})
    rk, rv = attn_bwd_cols(q.values, k.values, v.values, do.values, kpf, cols, heads)
    assert_grad_close(host(dk[cols][:, heads]), rk, "dk cols")
    assert_grad_close(host(dv[cols][:, heads]), rv, "dv cols")


def test_bwd_many_heads_sampled():
    """40 heads (the Wan-14B layer's head count) over two frames and a ragged
    third: every head's blocks land on the right XCD ranges and rows."""
    kpf, H = 1560, 40
    T = 2 * kpf + 100
    (q, k, v, do), (dq, dk, dv) = _run(T, H, kpf, seed=9, wid=43)
    rng = np.random.default_rng(10)
    heads = [0, 17, 39]
    rows = sorted(set(rng.choice(T, 12, replace=False).tolist()) | {0, kpf, T - 1})
    assert_grad_close(host(dq[rows][:, heads]), attn_bwd_rows(q.values, k.values, v.values, do.values,
                                                             kpf, rows, heads), "dq rows")
    cols = sorted(set(rng.choice(T, 12, replace=False).tolist()) | {0, 2 * kpf, T - 1})
    rk, rv = attn_bwd_cols(q.values, k.values, v.values, do.values, kpf, cols, heads)
    assert_grad_close(host(dk[cols][:, heads]), rk, "dk cols")
    assert_grad_close(host(dv[cols][:, heads]), rv, "dv cols")
