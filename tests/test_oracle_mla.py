"""Pins for the latent (MLA) attention oracle (oracle/mla.py).

The pages give op_mla_attention's properties but no rule or example, so the
pins tie the oracle to things other than itself: the attention oracle's C
core (already pinned) fed the keys and values the reading defines, torch's
f64 scaled_dot_product_attention on the same, the special case with
identity up-projections (plain multi-query attention over the latent rows),
closed forms (one key, q = 0), the absorbed evaluation (q through k_b first,
v_b after the softmax) done independently, and invariants (linear in v_b,
heads permute, a shared k_pe offset cancels). Shapes are non-square so a
transposed weight cannot slip through.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla
import workloads


def _wl(**kw):
    base = dict(name="mla pin", T=5, S=11, heads=3, kv_rank=6, qk_nope=4, qk_rope=2, v_head_dim=5,
                seed=3)
    base.update(kw)
    return workloads.MlaWorkload(**base)


def _materialized_f64(w):
    q, state, k_b, v_b = w.tensors()
    R, N = w.kv_rank, w.qk_nope
    c = state[:, :R].astype(np.float64)
    keys = [np.concatenate([c @ k_b[h].astype(np.float64).T, state[:, R:].astype(np.float64)], axis=1)
            for h in range(w.heads)]
    vals = [c @ v_b[h].astype(np.float64).T for h in range(w.heads)]
    return q, np.concatenate(keys, axis=1), np.concatenate(vals, axis=1)


CASES = [
    dict(),
    dict(causal=False),
    dict(posOffset=6, S=11, T=5),
    dict(window=3, posOffset=4),
    dict(window=2, sinks=2, posOffset=5),
    dict(window=2, sinks=3, causal=False),
    dict(scale=0.7),
    dict(T=1, S=40, posOffset=39, heads=4),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_equals_attention_core_over_materialized_keys(case):
    # The attention oracle's C core (pinned on its own) over the keys and
    # values the reading defines, rounded to f32 on the way in.
    w = _wl(**CASES[case])
    q, K, V = _materialized_f64(w)
    N, P = w.qk_nope, w.qk_rope
    got = mla.mla_attention(*w.tensors(), **w.params())
    kw = dict(heads=w.heads, headDim=N + P, vHeadDim=w.v_head_dim)
    for key in ("causal", "posOffset", "window", "sinks"):
        if getattr(w, key) is not None:
            kw[key] = getattr(w, key)
    kw["scale"] = w.scale if w.scale is not None else 1.0 / math.sqrt(N + P)  # rounded to f32 by both
    want = oracle.attention(q, K.astype(np.float32), V.astype(np.float32), **kw)
    np.testing.assert_allclose(got, want, rtol=2e-6, atol=2e-6)


@pytest.mark.parametrize("case", [0, 1, 4, 5])
def test_matches_torch_sdpa_f64(case):
    w = _wl(**CASES[case])
    q, K, V = _materialized_f64(w)
    got = mla.mla_attention(*w.tensors(), **w.params())
    H, N, P, Dv, T, S = w.heads, w.qk_nope, w.qk_rope, w.v_head_dim, w.T, w.S
    p0 = w.posOffset or 0
    causal = True if w.causal is None else w.causal
    mask = np.zeros((T, S))
    for t in range(T):
        vis = mla.visible(causal, w.window or 0, w.sinks or 0, p0 + t, S)
        mask[t, ~vis] = -np.inf
    qt = torch.from_numpy(q.astype(np.float64).reshape(T, H, N + P).transpose(1, 0, 2).copy())
    kt = torch.from_numpy(K.reshape(S, H, N + P).transpose(1, 0, 2).copy())
    vt = torch.from_numpy(V.reshape(S, H, Dv).transpose(1, 0, 2).copy())
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=float(np.float32(1.0 / math.sqrt(N + P))))
    want = out.numpy().transpose(1, 0, 2).reshape(T, H * Dv)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window, sinks, causal", [(None, None, None), (3, 1, True), (2, 2, False)])
def test_identity_projections_are_multi_query_attention(window, sinks, causal):
    # k_b[h] = v_b[h] = identity (kv_rank = qk_nope = v_head_dim): every head
    # attends over the latent rows themselves, keys [c_s ; k_pe_s] and values
    # c_s, which is the attention op with one key/value head.
    R, P, H, T, S = 6, 2, 3, 4, 9
    q = workloads.normal((T, H * (R + P)), 1, 0)
    state = workloads.normal((S, R + P), 1, 1)
    eye = np.broadcast_to(np.eye(R, dtype=np.float32), (H, R, R)).copy()
    kw = dict(causal=causal, window=window, sinks=sinks, posOffset=3)
    got = mla.mla_attention(q, state, eye, eye, heads=H, kv_rank=R, qk_nope=R, qk_rope=P,
                            v_head_dim=R, **kw)
    want = oracle.attention(q, state, np.ascontiguousarray(state[:, :R]), heads=H, kvHeads=1,
                            headDim=R + P, vHeadDim=R, **kw)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_absorbed_evaluation_agrees():
    # q_lat = k_b[h]^T q_nope scores against c_s directly; v_b[h] is applied
    # to the softmax-weighted latent rows. Same numbers by associativity.
    w = _wl(T=3, S=13, heads=2, kv_rank=7, qk_nope=3, qk_rope=2, v_head_dim=4, posOffset=10)
    q, state, k_b, v_b = (x.astype(np.float64) for x in w.tensors())
    R, N, P, Dv, H = w.kv_rank, w.qk_nope, w.qk_rope, w.v_head_dim, w.heads
    scale = float(np.float32(1.0 / math.sqrt(N + P)))  # the op's numbers are f32
    want = np.zeros((w.T, H * Dv))
    for t in range(w.T):
        vis = np.arange(w.S) <= 10 + t
        for h in range(H):
            qh = q[t, h * (N + P):(h + 1) * (N + P)]
            q_lat = k_b[h].T @ qh[:N]
            x = scale * (state[vis, :R] @ q_lat + state[vis, R:] @ qh[N:])
            p = np.exp(x - x.max())
            o_lat = p @ state[vis, :R] / p.sum()
            want[t, h * Dv:(h + 1) * Dv] = v_b[h] @ o_lat
    got = mla.mla_attention(*w.tensors(), **w.params())
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_single_key_returns_projected_latent():
    w = _wl(T=1, S=1, posOffset=0)
    q, state, k_b, v_b = w.tensors()
    got = mla.mla_attention(q, state, k_b, v_b, **w.params())
    c = state[0, :w.kv_rank].astype(np.float64)
    want = np.concatenate([v_b[h].astype(np.float64) @ c for h in range(w.heads)])
    np.testing.assert_allclose(got[0], want, rtol=1e-13, atol=1e-14)


def test_zero_query_is_projected_mean_of_visible_latents():
    w = _wl(T=2, S=10, posOffset=6, window=4)
    q, state, k_b, v_b = w.tensors()
    q = np.zeros_like(q)
    got = mla.mla_attention(q, state, k_b, v_b, **w.params())
    for t, (lo, hi) in enumerate([(3, 7), (4, 8)]):
        c = state[lo:hi, :w.kv_rank].astype(np.float64).mean(axis=0)
        want = np.concatenate([v_b[h].astype(np.float64) @ c for h in range(w.heads)])
        np.testing.assert_allclose(got[t], want, rtol=1e-12, atol=1e-13)


def test_linear_in_value_projection():
    w = _wl()
    q, state, k_b, v_b = w.tensors()
    v2 = workloads.normal(v_b.shape, 9, 6)
    a = mla.mla_attention(q, state, k_b, v_b, **w.params())
    b = mla.mla_attention(q, state, k_b, v2, **w.params())
    ab = mla.mla_attention(q, state, k_b, v_b + v2, **w.params())
    np.testing.assert_allclose(ab, a + b, rtol=1e-6, atol=1e-6)


def test_heads_permute_with_their_weights():
    w = _wl(heads=4)
    q, state, k_b, v_b = w.tensors()
    perm = [2, 0, 3, 1]
    N, P, Dv = w.qk_nope, w.qk_rope, w.v_head_dim
    qp = np.concatenate([q[:, h * (N + P):(h + 1) * (N + P)] for h in perm], axis=1)
    got = mla.mla_attention(qp, state, k_b[perm], v_b[perm], **w.params())
    ref = mla.mla_attention(q, state, k_b, v_b, **w.params())
    want = np.concatenate([ref[:, h * Dv:(h + 1) * Dv] for h in perm], axis=1)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-15)


def test_shared_rope_offset_cancels_but_per_key_rope_counts():
    # Adding one vector u to every k_pe shifts each row's scores by q_pe.u, a
    # constant the softmax removes; changing one key's k_pe changes the output.
    w = _wl(causal=False)
    q, state, k_b, v_b = w.tensors()
    R = w.kv_rank
    ref = mla.mla_attention(q, state, k_b, v_b, **w.params())
    shifted = state.copy()
    shifted[:, R:] += np.float32(0.75)
    np.testing.assert_allclose(mla.mla_attention(q, shifted, k_b, v_b, **w.params()), ref,
                               rtol=1e-6, atol=1e-6)
    one = state.copy()
    one[4, R:] += np.float32(3.0)
    assert np.abs(mla.mla_attention(q, one, k_b, v_b, **w.params()) - ref).max() > 1e-3


def test_default_scale_is_the_materialized_head_width():
    r = mla.resolve(1, 1, heads=1, kv_rank=8, qk_nope=12, qk_rope=4, v_head_dim=3)
    assert r["scale"] == float(np.float32(0.25))


def test_rows_subset_equals_full():
    w = _wl(T=6, posOffset=5)
    full = mla.mla_attention(*w.tensors(), **w.params())
    sub = mla.mla_attention(*w.tensors(), rows=[5, 0, 3], **w.params())
    np.testing.assert_array_equal(sub, full[[5, 0, 3]])


@pytest.mark.parametrize("bad", [dict(heads=0), dict(kv_rank=0), dict(window=-1), dict(sinks=-1),
                                 dict(posOffset=-2)])
def test_invalid_params_refused(bad):
    kw = dict(heads=2, kv_rank=4, qk_nope=2, qk_rope=2, v_head_dim=2)
    kw.update(bad)
    with pytest.raises(ValueError):
        mla.resolve(1, 4, **kw)
