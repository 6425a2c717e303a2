"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention or cache arithmetic: it only draws numbers and
rounds them to the storage dtype, so that the HIP library and the CPU oracle
receive bit-identical inputs.

Recipe: every tensor is drawn in float32 from
numpy.random.Generator(PCG64(SeedSequence([base_seed, workload_id, step, tag])))
as N(0, 1) and, for bf16 workloads, rounded once to bfloat16 with
round-to-nearest-even.  Tags: Q=0, K=1, V=2, reference K=3, reference V=4,
outlier row pick=5, upstream gradient dO=6, text K=7, text V=8.  The optional outlier treatment multiplies exactly
round(frac * rows) distinct (token, head) rows of a K tensor by a power of two
(exact in bfloat16, so it commutes with the rounding).
"""

import numpy as np

TAG_Q, TAG_K, TAG_V, TAG_REFK, TAG_REFV, TAG_OUTLIER, TAG_DO, TAG_TEXTK, TAG_TEXTV = range(9)

# Shapes of the synthetic workloads (Wan-DiT-shaped attention layers).
WORKLOADS = {
    "tiny_fp32": dict(wid=1, H=2, d=64, k=16, frames=9, dtype="f32",
                      stream=dict(C=1, W=4, R=1, chunks=8)),
    "wan13b_stream_step": dict(wid=2, H=12, d=128, k=1560, C=3, W=6, R=1, dtype="bf16"),
    "full_block_causal": dict(wid=3, H=12, d=128, k=1560, frames=22, dtype="bf16"),
    "rollout": dict(wid=4, H=12, d=128, k=1560, C=3, W=6, R=1, chunks=240,
                    swap_every=60, dtype="bf16"),
    "wan13b_cross_step": dict(wid=7, H=12, d=128, k=1560, C=3, text_tokens=512, dtype="bf16"),
    "wan13b_cross_step_bwd": dict(wid=9, H=12, d=128, k=1560, C=3, text_tokens=512, dtype="bf16"),
    "full_block_causal_bwd": dict(wid=6, H=12, d=128, k=1560, frames=22, dtype="bf16"),
    "wan13b_stream_step_bwd": dict(wid=8, H=12, d=128, k=1560, C=3, W=6, R=1, dtype="bf16"),
    "wan14b_stream_step": dict(wid=5, H=40, d=128, k=1560, C=3, W=9, R=1, dtype="bf16",
                               outlier_frac=0.01, outlier_scale=8.0),
}


def rng(base_seed, wid, step, tag):
    ss = np.random.SeedSequence([int(base_seed), int(wid), int(step), int(tag)])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.
    Inputs here are finite, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class HostTensor:
    """A host tensor in its storage dtype.  `values` is float32 holding the
    exact stored values; `bits` is the uint16 bf16 pattern (bf16 only)."""

    def __init__(self, values, dtype, bits=None):
        self.values = values
        self.dtype = dtype
        self.bits = bits

    @property
    def shape(self):
        return self.values.shape

    def storage(self):
        """The array whose bytes go to the device (uint16 for bf16)."""
        return self.bits if self.dtype == "bf16" else self.values


def normal(shape, dtype, base_seed, wid, step, tag, outlier_frac=0.0, outlier_scale=1.0):
    """N(0,1) tensor of `shape` = [..., rows..., d]; rows are all axes but the last.

    With outlier_frac > 0, exactly round(outlier_frac * rows) distinct rows are
    multiplied by outlier_scale (a power of two)."""
    g = rng(base_seed, wid, step, tag)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if outlier_frac > 0:
        d = shape[-1]
        flat = x.reshape(-1, d)
        n_out = int(round(outlier_frac * flat.shape[0]))
        pick = rng(base_seed, wid, step, TAG_OUTLIER).choice(flat.shape[0], size=n_out,
                                                             replace=False)
        flat[pick] *= np.float32(outlier_scale)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return HostTensor(bf16_bits_to_f32(bits), "bf16", bits)
    if dtype == "f32":
        return HostTensor(np.ascontiguousarray(x), "f32")
    raise ValueError(dtype)


def from_values(values, dtype):
    """Wrap values that are already exactly representable in `dtype`."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(v)
        if not np.array_equal(bf16_bits_to_f32(bits), v):
            raise ValueError("values are not exact in bfloat16")
        return HostTensor(v, "bf16", bits)
    return HostTensor(v, "f32")


def full_sequence_inputs(T, H, d, dtype, base_seed=0, wid=0, step=0):
    """Q, K, V of shape [T, H, d] for the full-sequence form."""
    return tuple(normal((T, H, d), dtype, base_seed, wid, step, t)
                 for t in (TAG_Q, TAG_K, TAG_V))


def bwd_inputs(T, H, d, dtype, base_seed=0, wid=0, step=0):
    """Q, K, V of a full sequence plus an upstream gradient dO, all [T, H, d]."""
    return (full_sequence_inputs(T, H, d, dtype, base_seed, wid, step)
            + (normal((T, H, d), dtype, base_seed, wid, step, TAG_DO),))


def cross_inputs(Tq, Lt, H, d, dtype, base_seed=0, wid=0, step=0):
    """Queries [Tq, H, d] and one text condition's K, V [Lt, H, d]."""
    return (normal((Tq, H, d), dtype, base_seed, wid, step, TAG_Q),
            normal((Lt, H, d), dtype, base_seed, wid, step, TAG_TEXTK),
            normal((Lt, H, d), dtype, base_seed, wid, step, TAG_TEXTV))


def stream_inputs(k, H, d, C, W, R, dtype, base_seed=0, wid=0, step=0, outlier_frac=0.0,
                  outlier_scale=1.0):
    """Inputs of one streaming step at steady state.

    Returns dict(ref_k, ref_v: [R, k, H, d]; ring_k, ring_v: [W, k, H, d] --
    the W past frames to commit, oldest first; q, k, v: [C*k, H, d])."""
    o = dict(outlier_frac=outlier_frac, outlier_scale=outlier_scale)
    out = {
        "ref_k": normal((R, k, H, d), dtype, base_seed, wid, step, TAG_REFK, **o),
        "ref_v": normal((R, k, H, d), dtype, base_seed, wid, step, TAG_REFV),
        "ring_k": normal((W, k, H, d), dtype, base_seed, wid, step + 1_000_000, TAG_K, **o),
        "ring_v": normal((W, k, H, d), dtype, base_seed, wid, step + 1_000_000, TAG_V),
        "q": normal((C * k, H, d), dtype, base_seed, wid, step, TAG_Q),
        "k": normal((C * k, H, d), dtype, base_seed, wid, step, TAG_K, **o),
        "v": normal((C * k, H, d), dtype, base_seed, wid, step, TAG_V),
    }
    return out
