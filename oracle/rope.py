"""Rotary position encoding along the temporal axis, and the position of an
anchored reference that follows a rolling window (test infrastructure only).

Context: the streaming VACE notes point out that rotary position encodings
are baked into cached K (so a reference concatenated into the causal history
cannot be removed without recomputing the cache); the RTR-DiT notes keep the
reference in a resident slot at the front (Key Designs 1 and 4).  Readings
(the pages give no formula): rotary encoding in the usual pairwise form --
element pairs (2i, 2i+1) of a head, for the first `pairs` pairs, rotated by
angle position * base^(-i / pairs); the temporal position of a latent frame is
its generation index plus a fixed offset, and the anchored reference frames
sit directly in front of the oldest frame an attention call sees, as the
reference frame sits in front of the first frame in the full sequence.
"""

import numpy as np


def rope_angles(positions, pairs, base):
    """[len(positions), pairs] rotation angles."""
    i = np.arange(pairs, dtype=np.float64)
    freq = np.power(float(base), -i / pairs)
    return np.asarray(positions, dtype=np.float64)[:, None] * freq[None, :]


def rope_rotate(x, positions, pairs, base=10000.0):
    """Rotate x [T, H, d] (float64 result): token t by positions[t]."""
    x = np.array(x, dtype=np.float64, copy=True)
    ang = rope_angles(positions, pairs, base)[:, None, :]   # [T, 1, pairs]
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[:, :, 0:2 * pairs:2].copy()
    x1 = x[:, :, 1:2 * pairs:2].copy()
    x[:, :, 0:2 * pairs:2] = x0 * c - x1 * s
    x[:, :, 1:2 * pairs:2] = x0 * s + x1 * c
    return x


def reference_shift(oldest_position, ref_frames):
    """Rotation to apply to reference frames encoded at positions 0..R-1 so
    that they sit at oldest_position - R .. oldest_position - 1."""
    return int(oldest_position) - int(ref_frames)
