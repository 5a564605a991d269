"""attn_forward_noalloc (split state in the library's per-GPU scratch array,
no allocation) against attn_forward (caller's workspace) and the oracle, on
the GPU, through the C ABI.

Two calls in a row share the array: a large call, then a smaller one, each
checked to the parity bar (|err| <= 1e-4 + 1e-4 |ref|) against attn_forward
on the same inputs and against the oracle. The second call's state overlays
the first one's, so a merge that read stale state would show.
"""

import ctypes

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
from gqa_scaled_dot_amd import _lib
import oracle
import workloads
from tests.parity import assert_close, dev, torch

pytestmark = pytest.mark.gpu


def _noalloc_raw(q, k, v, bias, out, params):
    """The entry point called through ctypes on the C ABI directly."""
    T, S = q.shape[0], k.shape[0]
    kind = 0 if bias is None else (1 if bias.dim() == 2 else 2)
    p, keep = ga.make_params(T, S, bias_kind=kind, **params)
    rc = _lib.lib().attn_forward_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         bias.data_ptr() if bias is not None else None, out.data_ptr(),
                                         ctypes.c_void_p(torch().cuda.current_stream().cuda_stream))
    del keep
    return rc


def _case(w):
    t = torch()
    q, k, v, bias = w.tensors()
    qd, kd, vd, bd = dev(q), dev(k), dev(v), dev(bias)
    params = w.params()
    ref_lib = ga.attn_forward(qd, kd, vd, bd, **params)
    out = t.full_like(ref_lib, float("nan"))
    rc = _noalloc_raw(qd, kd, vd, bd, out, params)
    assert rc == 0, ga.attn_last_error()
    t.cuda.synchronize()
    got = out.cpu().numpy()
    assert_close(got, ref_lib.cpu().numpy().astype(np.float64), f"{w.name}: noalloc vs attn_forward")
    rows = None if w.T <= 64 else sorted(set([0, 1, w.T // 2, w.T - 2, w.T - 1]))
    ref = oracle.attention(q, k, v, bias, rows=rows, **params)
    assert_close(got if rows is None else got[rows], ref, f"{w.name}: noalloc vs oracle")
    return got


def test_noalloc_two_calls_second_smaller():
    big = workloads.LLAMA_DECODE.replace(name="noalloc decode S=32768 H=32 G=8", seed=11)
    small = workloads.Workload("noalloc decode S=3000 H=8 G=2", T=1, S=3000, heads=8, kvHeads=2,
                               headDim=128, posOffset=2999, alibi=True, softcap=30.0, seed=12)
    assert ga.attn_plan(big.T, big.S, **big.params())["splits"] > 1
    assert ga.attn_plan(small.T, small.S, **small.params())["splits"] > 1
    _case(big)
    _case(small)


def test_noalloc_prefill_key_splits_then_decode():
    # A prefill whose key range is split (state in the scratch array), then a
    # smaller decode call over the same array.
    pre = workloads.Workload("noalloc split prefill T=70 S=900", T=70, S=900, heads=8, kvHeads=2,
                             headDim=128, posOffset=830, bias="HTS", bias_mask_prob=0.1, seed=13)
    plan = ga.attn_plan(pre.T, pre.S, bias_kind=2, **pre.params())
    assert plan["path"] == "prefill" and plan["splits"] > 1, plan
    _case(pre)
    _case(workloads.Workload("noalloc decode S=700 H=4 G=1", T=1, S=700, heads=4, kvHeads=1, headDim=64,
                             posOffset=699, seed=14))


def test_noalloc_refuses_state_past_the_scratch():
    # The chunked prefill (512 query rows x 32 heads, key range in 4 parts)
    # needs ~34 MB of split state: refused on the host, before anything runs,
    # with the entry point's own message.
    t = torch()
    w = workloads.LLAMA_CHUNKED
    need = ga.attn_workspace_size(w.T, w.S, **w.params())
    if need <= _lib.ATTN_NOALLOC_SCRATCH_BYTES:
        pytest.skip("this plan fits the scratch array")
    q = t.zeros((w.T, w.heads * w.headDim), device="cuda")
    k = t.zeros((w.S, w.G * w.headDim), device="cuda")
    v = t.zeros_like(k)
    out = t.full((w.T, w.heads * w.Dv), 7.0, device="cuda")
    with pytest.raises(ga.AttnError, match="scratch"):
        ga.attn_forward_noalloc(q, k, v, out=out, **w.params())
    t.cuda.synchronize()
    assert bool((out == 7.0).all())
