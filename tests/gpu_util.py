"""Helpers shared by the GPU tests: host<->device transfer of the seeded inputs
and the error metrics used by the parity bar."""

import numpy as np
import torch

from causal_attention_frame_amd import inputs as gen

# Parity bar: bf16 inputs with fp32 accumulation vs the float64 oracle; float32
# inputs (tiny workload).
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-4


def dev(t, device="cuda"):
    """HostTensor (or numpy float32) -> contiguous device tensor, same bits."""
    if isinstance(t, gen.HostTensor):
        if t.dtype == "bf16":
            return torch.from_numpy(t.bits.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(t.values).to(device)
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)


def host(x):
    """Device tensor -> float64 numpy (exact for bf16/f32)."""
    return x.detach().float().cpu().numpy().astype(np.float64)


def raw(x):
    """Device tensor -> its bytes as a numpy uint8 array."""
    return x.detach().contiguous().view(torch.uint8).cpu().numpy()


def errors(got, ref):
    e = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return float(e.max()), float(e.mean())


def assert_bf16_close(got, ref, what=""):
    mx, mean = errors(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, f"{what}: max {mx:.3g} mean {mean:.3g}"
    return mx, mean


def assert_f32_close(got, ref, what=""):
    mx, _ = errors(got, ref)
    assert mx <= F32_MAX_ABS, f"{what}: max {mx:.3g}"
    return mx


def guarded_empty(shape, dtype, pad=4096, fill=0x5A):
    """An output tensor with guard bands on both sides, filled with a byte
    pattern; `check()` asserts both bands are untouched."""
    n = int(np.prod(shape))
    esize = torch.empty((), dtype=dtype).element_size()
    padn = pad // esize
    buf = torch.empty(n + 2 * padn, dtype=dtype, device="cuda")
    buf.view(torch.uint8).fill_(fill)
    view = buf[padn:padn + n].view(*shape)

    def check():
        b = buf.view(torch.uint8)
        lo = b[:pad]
        hi = b[pad + n * esize:]
        assert bool((lo == fill).all()) and bool((hi == fill).all()), "guard band overwritten"

    return view, check


# Gradient bar (bf16 in and out, fp32 accumulation, P and dS rounded to bf16
# before their products).  Gradient magnitudes scale with the problem, so the
# bar is relative to the RMS of the float64 reference tensor: an emulation of
# exactly these roundings in numpy on a 3-frame Wan-1.3B head (4,680 tokens)
# gives max |err| = 0.046 rms and mean |err| = 0.0022 rms; the bar allows
# about 3.3x that.
GRAD_MAX_REL, GRAD_MEAN_REL = 0.15, 0.008


def assert_grad_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    mx, mean = errors(got, ref)
    if rms == 0.0:  # an exactly zero gradient (e.g. a row that sees only its own key)
        assert mx <= 1e-5, f"{what}: max {mx:.3g} where the reference is zero"
        return mx, mean
    assert mx <= GRAD_MAX_REL * rms and mean <= GRAD_MEAN_REL * rms, \
        f"{what}: max {mx:.3g} mean {mean:.3g} (rms {rms:.3g})"
    return mx / rms, mean / rms
