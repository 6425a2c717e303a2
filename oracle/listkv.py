"""Literal list-based model of the reference-anchored rolling KV cache (test
infrastructure only).

Source: "DiT as Real-Time Rerenderer: Streaming Video Stylization with
Autoregressive Diffusion Transformer" (RTR-DiT notes):
  * Key Designs 4: the 3D-attention cache has a fixed length, newly generated
    frames are appended, and once it is full the oldest frames are evicted;
    the reference tokens are anchored at the front as a resident slot that is
    never evicted while the other positions keep rolling.  On a condition
    switch the 3D-attention cache keeps the most recent frame as a bridge, and
    a new reference image is anchored at the front as well.
  * Key Designs 1: the reference latent is prepended along the temporal axis,
    i.e. it counts as one latent frame placed before the first frame.

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * the window length W counts past latent frames only; the reference slot is
    extra and is never part of W;
  * eviction is whole latent frames, oldest first; appending n > W frames at
    once keeps only the newest W; W = 0 keeps none;
  * a condition switch first applies the reference mode (KEEP: unchanged,
    REPLACE: new reference anchored, CLEAR: no reference) and then keeps only
    the newest `keep_recent` window frames (-1 keeps all, 1 is the pages'
    "most recent frame as a bridge");
  * frames get consecutive ids in generation order; the reference gets a new
    generation number on every REPLACE.

The window is a plain Python list of (frame_id, K, V) tuples, oldest first.
"""

import numpy as np

REF_KEEP = 0
REF_REPLACE = 1
REF_CLEAR = 2


class ListKV:
    """One layer's 3D-attention cache: anchored reference + rolling window."""

    def __init__(self, window_frames):
        if window_frames < 0:
            raise ValueError("window_frames must be >= 0")
        self.W = int(window_frames)
        self.window = []          # [(frame_id, K[k,H,d], V[k,H,d])], oldest first
        self.ref = None           # None or (generation, K[R,k,H,d], V[R,k,H,d])
        self.ref_generation = 0
        self.next_frame_id = 0

    # -- Key Designs 4: append newly generated frames, evict the oldest ------
    def append(self, k_frames, v_frames):
        """k_frames, v_frames: [n, k, H, d]; frames are committed in order."""
        if len(k_frames) != len(v_frames):
            raise ValueError("k and v frame counts differ")
        for f in range(len(k_frames)):
            self.window.append((self.next_frame_id, np.array(k_frames[f], copy=True),
                                np.array(v_frames[f], copy=True)))
            self.next_frame_id += 1
            while len(self.window) > self.W:
                self.window.pop(0)

    # -- Key Designs 4: condition switch ------------------------------------
    def reset_ref(self, mode, k_ref=None, v_ref=None, keep_recent=1):
        if mode == REF_REPLACE:
            if k_ref is None or v_ref is None:
                raise ValueError("REPLACE needs the new reference K and V")
            self.ref_generation += 1
            self.ref = (self.ref_generation, np.array(k_ref, copy=True),
                        np.array(v_ref, copy=True))
        elif mode == REF_CLEAR:
            self.ref = None
        elif mode != REF_KEEP:
            raise ValueError("unknown reference mode")
        if keep_recent >= 0 and keep_recent < len(self.window):
            self.window = self.window[len(self.window) - keep_recent:]

    # -- views ---------------------------------------------------------------
    def frame_ids(self):
        return [fid for fid, _, _ in self.window]

    def ref_frames(self):
        return 0 if self.ref is None else len(self.ref[1])

    def prefix(self, tokens_per_frame, H, d, dtype=np.float64):
        """Cached keys/values in logical order: reference frame(s) first, then
        window frames oldest to newest.  Returns (K [P,H,d], V [P,H,d])."""
        ks, vs = [], []
        if self.ref is not None:
            ks.extend(list(self.ref[1]))
            vs.extend(list(self.ref[2]))
        for _, kf, vf in self.window:
            ks.append(kf)
            vs.append(vf)
        if not ks:
            z = np.zeros((0, H, d), dtype=dtype)
            return z, z.copy()
        return (np.concatenate([np.asarray(x).reshape(tokens_per_frame, H, d) for x in ks]),
                np.concatenate([np.asarray(x).reshape(tokens_per_frame, H, d) for x in vs]))


class TextKV:
    """One layer's cross-attention cache (RTR-DiT notes, Key Designs 4): a
    fixed-capacity cache initialised with the K/V of the current text
    condition, reused by every chunk, and re-initialised (the old condition
    discarded) when a new text prompt arrives.  Readings: the cache holds
    exactly the current condition's tokens (no rolling: text does not grow
    with the video); `set` replaces the whole content and counts a new
    generation; `clear` leaves no condition, after which cross-attention has
    nothing to attend to."""

    def __init__(self, capacity_tokens):
        if capacity_tokens < 1:
            raise ValueError("capacity_tokens must be >= 1")
        self.capacity = int(capacity_tokens)
        self.k = None
        self.v = None
        self.generation = 0

    def set(self, k_text, v_text):
        """k_text, v_text: [n, H, d] with 1 <= n <= capacity."""
        if len(k_text) != len(v_text) or not (1 <= len(k_text) <= self.capacity):
            raise ValueError("text K/V must have the same length in [1, capacity]")
        self.k = np.array(k_text, copy=True)
        self.v = np.array(v_text, copy=True)
        self.generation += 1

    def clear(self):
        self.k = self.v = None

    def tokens(self):
        return 0 if self.k is None else len(self.k)
