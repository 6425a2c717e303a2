"""Where the gradient parity bar comes from (CPU).

The GPU backward takes bf16 q, k, v, o and dO, accumulates every product in
float32, rounds P to bf16 before dV = P^T dO and dS to bf16 before dK = scale
dS^T Q and dQ = scale dS K, and writes bf16 gradients.  This test emulates
exactly those roundings in numpy (float32 products of bf16-rounded operands) on
a 3-frame sequence of Wan-sized frames and one head, and measures the error of
the emulated gradients against the float64 gradient oracle, relative to the
RMS of each reference gradient.  The parity bar used by the GPU tests
(tests.gpu_util.GRAD_MAX_REL, GRAD_MEAN_REL) must hold these rounding errors
with margin, and must still reject a plausible mistake in a kernel (the
rowsum(dO * O) term dropped from dS).
"""

import numpy as np

import oracle
from causal_attention_frame_amd import inputs as gen
from tests.gpu_util import GRAD_MAX_REL, GRAD_MEAN_REL


def _bf16(x):
    """Round float32 values to bf16 (RNE), returned as float32."""
    return gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _emulate(q, k, v, do, kpf, drop_d=False):
    """One head: q, k, v, do [T, d] float32 holding bf16 values."""
    T, d = q.shape
    scale = np.float32(1.0 / np.sqrt(d))
    i = np.arange(T)
    vis = (i[None, :] // kpf) <= (i[:, None] // kpf)
    # forward as the kernel leaves it: bf16 O, float32 LSE
    s = (q @ k.T).astype(np.float32) * scale
    s = np.where(vis, s, -np.inf).astype(np.float32)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m).astype(np.float32)
    lsum = e.sum(axis=1, keepdims=True, dtype=np.float32)
    lse = (m + np.log(lsum)).astype(np.float32)
    o = _bf16((_bf16(e) @ v).astype(np.float32) / lsum)
    # backward
    p = np.exp(s - lse).astype(np.float32)
    dv = _bf16(_bf16(p).T @ do)
    dp = (do @ v.T).astype(np.float32)
    dd = np.zeros((T, 1), np.float32) if drop_d else (do * o).sum(axis=1, keepdims=True, dtype=np.float32)
    ds = _bf16(p * (dp - dd))
    dk = _bf16((ds.T @ q).astype(np.float32) * scale)
    dq = _bf16((ds @ k).astype(np.float32) * scale)
    return dq, dk, dv


def _rel_errors(got, ref):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    e = np.abs(got.astype(np.float64) - ref)
    return float(e.max()) / rms, float(e.mean()) / rms


def _case(drop_d=False):
    kpf, F, d = 512, 3, 128
    T = kpf * F
    q, k, v, do = gen.bwd_inputs(T, 1, d, "bf16", base_seed=0, wid=77)
    ref = oracle.attn_block_causal_bwd(q.values, k.values, v.values, do.values, kpf)
    em = _emulate(q.values[:, 0], k.values[:, 0], v.values[:, 0], do.values[:, 0], kpf, drop_d)
    return [_rel_errors(g, r[:, 0]) for g, r in zip(em, ref)]


def test_bar_holds_the_kernel_roundings_with_margin():
    errs = _case()
    for name, (mx, mean) in zip(("dq", "dk", "dv"), errs):
        print(f"{name}: max {mx:.4f} rms, mean {mean:.5f} rms")
        assert mx <= GRAD_MAX_REL / 2, (name, mx)
        assert mean <= GRAD_MEAN_REL / 2, (name, mean)


def test_bar_rejects_a_dropped_softmax_term():
    errs = _case(drop_d=True)
    # dS without the rowsum(dO * O) term is wrong in dq and dk
    assert any(mx > GRAD_MAX_REL or mean > GRAD_MEAN_REL for mx, mean in errs[:2])
