"""CPU oracle for frame-block-causal attention and the reference-anchored KV window.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
anything in this package; only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library: it takes
plain numpy arrays and computes in float64 with the most literal formulation of
the pages' definitions.

Sources (the pages are web notes on "DiT as Real-Time Rerenderer: Streaming
Video Stylization with Autoregressive Diffusion Transformer", RTR-DiT):
  * attention.py  -- Key Designs 2 ("Causal 3D attention for streaming
    autoregression"), the Attn(Q,K,V) equation with the frame mask M; and
    attn_cross, the text cross-attention of Key Designs 1 (text encoded by
    T5 and injected through cross attention), which has no mask.
  * rope.py       -- temporal rotary encoding and the position of the anchored
    reference in front of the rolling window (position-aware cache).
  * attention_bwd.py -- gradients (dQ, dK, dV) of the Key Designs 2 equation,
    the pass that Key Designs 3's post-training back-propagates through, for
    the full form, the streaming step and the text cross-attention.
  * listkv.py     -- Key Designs 4 ("Reference-preserving KV cache update and
    live style switching"), and Key Designs 1 for the reference as one extra
    latent frame placed before the first frame; its TextKV is the
    cross-attention cache of the same section.

Every function here is pinned by tests/test_oracle.py (which also holds the
ListKV pins), tests/test_oracle_bwd.py, tests/test_oracle_cross.py,
tests/test_oracle_blocks.py and tests/test_oracle_rope.py against things other
than itself (brute-force loops, textbook special cases, closed forms, hand
values and invariants); tests/test_oracle_mutants.py plants plausible slips and
checks that a pin fails for each.
"""

from .attention import (  # noqa: F401
    visible,
    attn_block_causal,
    attn_brute_force,
    attn_rows,
    attn_stream_step,
    attn_stream_rows,
    attn_cross,
)
from .attention_bwd import (  # noqa: F401
    attn_block_causal_bwd,
    attn_bwd_rows,
    attn_bwd_cols,
    attn_stream_step_bwd,
    attn_cross_bwd,
)
from .rope import rope_rotate, reference_shift  # noqa: F401
from .listkv import ListKV, TextKV, REF_KEEP, REF_REPLACE, REF_CLEAR  # noqa: F401
