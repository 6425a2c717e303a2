"""The backward under HIP graph capture (GPU, through the C ABI).

rtr_attn_block_causal_bwd enqueues its kernels on the caller's stream and
allocates nothing, so a caller can capture it into a graph.  Its kernels are
deterministic (no atomics), so every replay must give gradients bit-identical
to the eager call's.  The graph is replayed several times, with other backward
calls and synchronisations on the device between replays, and every replay is
checked against the eager result, and the eager result once against the
float64 oracle (the derivative of the Attn equation, RTR-DiT notes, Key
Designs 2)."""

import numpy as np
import pytest
import torch

from causal_attention_frame_amd import inputs as gen
from causal_attention_frame_amd import rtr
from oracle.attention_bwd import attn_block_causal_bwd
from tests.gpu_util import assert_grad_close, dev, host

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("T,H,kpf", [(700, 2, 96), (1560 + 300, 2, 1560)])
def test_bwd_graph_replays_match_eager(T, H, kpf):
    print(f"T={T} H={H} kpf={kpf}", flush=True)
    q, k, v, do = gen.bwd_inputs(T, H, 128, "bf16", base_seed=7, wid=93)
    tq, tk, tv, tdo = (dev(x) for x in (q, k, v, do))
    o, lse = rtr.rtr_attn_block_causal(tq, tk, tv, kpf, want_lse=True)
    eager = rtr.rtr_attn_block_causal_bwd(tq, tk, tv, o, lse, tdo, kpf)
    torch.cuda.synchronize()
    ref = attn_block_causal_bwd(q.values, k.values, v.values, do.values, kpf)
    for name, g_, r_ in zip(("dq", "dk", "dv"), eager, ref):
        assert_grad_close(host(g_), r_, f"eager {name}")
    want = [_bits(x) for x in eager]

    # other work between replays: a backward of different inputs, eager
    q2, k2, v2, do2 = (dev(x) for x in gen.bwd_inputs(T, H, 128, "bf16", base_seed=8, wid=93))
    o2, lse2 = rtr.rtr_attn_block_causal(q2, k2, v2, kpf, want_lse=True)

    ws = torch.empty(max(1, rtr.rtr_attn_bwd_workspace_size(T, H, 128)), dtype=torch.uint8, device=tq.device)
    outs = [torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rtr.rtr_attn_block_causal_bwd(tq, tk, tv, o, lse, tdo, kpf, dq=outs[0], dk=outs[1], dv=outs[2],
                                      workspace=ws)
    for rep in range(3):
        for x in outs:
            x.fill_(0)
        rtr.rtr_attn_block_causal_bwd(q2, k2, v2, o2, lse2, do2, kpf)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, exp in zip(("dq", "dk", "dv"), outs, want):
            assert np.array_equal(_bits(got), exp), f"replay {rep}: {name} differs from the eager call"
