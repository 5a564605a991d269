"""A decode step captured in a HIP graph (torch.cuda.graph) and replayed.

The library allocates nothing, never synchronises and launches only kernels
on the caller's stream, so a step (the K/V append, then attention, as two
calls or as one attn_forward_append) can be captured once and replayed. Every replay is checked against the same step run
eagerly, with eager work and synchronisations between replays, and after the
captured inputs are rewritten in place.
"""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import oracle
import workloads
from tests.parity import assert_close, dev, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["cache_write2 + attn_forward", "attn_forward_append"])
def test_decode_step_replays_from_a_graph(fused):
    t = torch()
    w = workloads.LLAMA_DECODE.replace(name="graph decode", S=4096, posOffset=4095)
    q, k, v, _ = w.tensors()
    pos = w.S - 1
    kc, vc = dev(k), dev(v)
    kc[pos:].zero_()
    vc[pos:].zero_()
    qd, new_k, new_v = dev(q), dev(k[pos:]), dev(v[pos:])
    out = t.empty((1, w.heads * w.Dv), dtype=t.float32, device="cuda")
    ws = t.empty(ga.attn_workspace_size(w.T, w.S, **w.params()), dtype=t.uint8, device="cuda")

    def step():
        if fused:
            ga.attn_forward_append(qd, kc, vc, new_k, new_v, pos, out=out, workspace=ws, **w.params())
        else:
            ga.attn_cache_write2(kc, new_k, vc, new_v, pos)
            ga.attn_forward(qd, kc, vc, out=out, workspace=ws, **w.params())

    step()
    t.cuda.synchronize()
    eager = out.clone()
    assert_close(eager.cpu().numpy(), oracle.attention(q, k, v, **w.params()), "eager step")

    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        for _ in range(3):
            step()
    t.cuda.current_stream().wait_stream(side)
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        step()

    for rep in range(4):
        out.fill_(float("nan"))
        kc[pos:].fill_(float("nan"))  # the replay writes the new row again
        vc[pos:].fill_(float("nan"))
        scratch = t.randn(1024, device="cuda") * 2.0  # eager work between replays
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), eager.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(kc[pos:].cpu().numpy().view(np.uint32), k[pos:].view(np.uint32))
        np.testing.assert_array_equal(vc[pos:].cpu().numpy().view(np.uint32), v[pos:].view(np.uint32))
        del scratch

    # New inputs written in place into the captured buffers.
    q2 = workloads.normal(q.shape, 77, 0)
    k2 = workloads.normal(new_k.shape, 77, 1)
    qd.copy_(dev(q2))
    new_k.copy_(dev(k2))
    graph.replay()
    t.cuda.synchronize()
    k_all = k.copy()
    k_all[pos:] = k2
    assert_close(out.cpu().numpy(), oracle.attention(q2, k_all, v, **w.params()), "replay with new q and K row")
