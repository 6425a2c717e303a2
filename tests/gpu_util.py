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
