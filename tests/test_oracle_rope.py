"""Pins of the oracle's rotary position embedding (op `rope`), on the CPU.

Each pin ties the oracle to something other than itself: the closed form of
one rotated pair, invariants every rotation obeys (pair norms, the dot
product depending only on the position difference, pass-through channels),
the equivalence of the two pairings under a channel permutation, and the
transformers library's own rope routines (rotation and inverse-frequency
tables), computed independently.
"""

import math
import warnings

import numpy as np
import pytest

import oracle


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


# ---- closed forms --------------------------------------------------------------

@pytest.mark.parametrize("p", [0, 1, 2, 7, 100, 12345, 2**20 + 3])
@pytest.mark.parametrize("interleaved", [False, True])
def test_single_pair_turns_by_its_position(p, interleaved):
    # headDim 2: one pair with invFreq = base^0 = 1, so the angle is the position.
    x = np.array([[1.0, 0.0], [0.0, 1.0], [3.0, -2.0]], dtype=np.float32)
    got = oracle.rope(x, headDim=2, offset=p, interleaved=interleaved)
    c0, s0 = math.cos(p), math.sin(p)
    c1, s1 = math.cos(p + 1), math.sin(p + 1)
    c2, s2 = math.cos(p + 2), math.sin(p + 2)
    want = np.array([[c0, s0], [-s1, c1], [3 * c2 + 2 * s2, 3 * s2 - 2 * c2]])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_attention_factor_scales_cos_and_sin():
    x = np.array([[1.0, 0.0, 5.0]], dtype=np.float32)
    got = oracle.rope(x, headDim=3, rotaryDim=2, offset=3, attentionFactor=0.5)
    np.testing.assert_allclose(got, [[0.5 * math.cos(3), 0.5 * math.sin(3), 5.0]], atol=1e-12)


def test_position_zero_is_the_identity():
    x = rnd((1, 4 * 64), 1)
    for inter in (False, True):
        got = oracle.rope(x, headDim=64, interleaved=inter, base=500000.0)
        np.testing.assert_array_equal(got, x.astype(np.float64))


# ---- invariants ----------------------------------------------------------------

def pairs(D, rd, interleaved):
    h = rd // 2
    if interleaved:
        return [(2 * i, 2 * i + 1) for i in range(h)]
    return [(i, i + h) for i in range(h)]


@pytest.mark.parametrize("D, rd, inter", [(64, 64, False), (64, 64, True), (96, 32, False),
                                          (10, 6, True), (10, 6, False)])
def test_pair_norms_kept_and_passthrough_untouched(D, rd, inter):
    x = rnd((7, 3 * D), 2)
    got = oracle.rope(x, headDim=D, rotaryDim=rd, interleaved=inter, offset=1000,
                      attentionFactor=1.25).reshape(7, 3, D)
    xs = x.astype(np.float64).reshape(7, 3, D)
    for a, b in pairs(D, rd, inter):
        np.testing.assert_allclose(np.hypot(got[..., a], got[..., b]),
                                   1.25 * np.hypot(xs[..., a], xs[..., b]), rtol=1e-12)
    np.testing.assert_array_equal(got[..., rd:], xs[..., rd:])


SCALINGS = [None, {"rope_type": "linear", "factor": 4.0},
            {"rope_type": "llama3", "factor": 8.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
             "original_max_position_embeddings": 8192},
            {"rope_type": "yarn", "factor": 4.0, "original_max_position_embeddings": 4096}]


@pytest.mark.parametrize("scaling", SCALINGS)
@pytest.mark.parametrize("inter", [False, True])
def test_scores_depend_only_on_the_position_difference(scaling, inter):
    # The defining property of rotary embeddings: <R(m) q, R(n) k> = <q, R(n - m) k>.
    D = 32
    q, k = rnd((1, D), 3), rnd((1, D), 4)
    kw = dict(headDim=D, interleaved=inter, scaling=scaling, base=10000.0)

    def score(m, n):
        return float(oracle.rope(q, offset=m, **kw)[0] @ oracle.rope(k, offset=n, **kw)[0])

    for m, n in [(5, 2), (300, 17), (40000, 39990)]:
        ref = score(m, n)
        for shift in (1, 123, 5000):
            assert score(m + shift, n + shift) == pytest.approx(ref, rel=1e-9, abs=1e-9)
    assert score(0, 5) != pytest.approx(score(0, 6), rel=1e-6)


@pytest.mark.parametrize("rd", [64, 48, 2])
def test_interleaved_is_a_permuted_half_split(rd):
    D = 64
    x = rnd((5, 2 * D), 5)
    # Half-split channel i (i < rd/2) plays interleaved channel 2i; i + rd/2 plays 2i + 1.
    perm = np.arange(D)
    perm[:rd // 2] = 2 * np.arange(rd // 2)
    perm[rd // 2:rd] = 2 * np.arange(rd // 2) + 1
    xh = x.reshape(5, 2, D)[..., perm].reshape(5, 2 * D)
    half = oracle.rope(xh, headDim=D, rotaryDim=rd, offset=77).reshape(5, 2, D)
    inter = oracle.rope(x, headDim=D, rotaryDim=rd, offset=77, interleaved=True).reshape(5, 2, D)
    back = np.empty_like(half)
    back[..., perm] = half
    np.testing.assert_array_equal(inter, back)


def test_rows_take_consecutive_positions():
    x = rnd((9, 128), 6)
    whole = oracle.rope(x, headDim=64, offset=500)
    for t in range(9):
        np.testing.assert_array_equal(whole[t], oracle.rope(x[t:t + 1], headDim=64, offset=500 + t)[0])


def test_explicit_table_wins_over_base_and_scaling():
    inv = np.linspace(1.0, 0.01, 16)
    t, af = oracle.rope_table(32, base=123.0, scaling={"rope_type": "linear", "factor": 2.0},
                              invFreq=inv, attentionFactor=0.75)
    np.testing.assert_array_equal(t, inv.astype(np.float32))
    assert af == 0.75
    _, af2 = oracle.rope_table(32, scaling={"rope_type": "yarn", "factor": 4.0,
                                            "original_max_position_embeddings": 4096,
                                            "attention_factor": 1.5})
    assert af2 == 1.5


def test_table_is_f32_and_default_base_is_10000():
    t, af = oracle.rope_table(8)
    assert t.dtype == np.float32 and af == 1.0
    np.testing.assert_array_equal(t, np.float32([1.0, 0.1, 0.01, 0.001]))


@pytest.mark.parametrize("kw", [dict(rotaryDim=3), dict(rotaryDim=80), dict(offset=-1),
                                dict(scaling={"rope_type": "ntk-by-magic", "factor": 2.0}),
                                dict(invFreq=[1.0, 2.0]), dict(base=-5.0)])
def test_invalid_params_are_refused(kw):
    with pytest.raises(ValueError):
        oracle.rope(rnd((2, 64), 7), headDim=64, **kw)


def test_width_must_be_whole_heads():
    with pytest.raises(ValueError):
        oracle.rope(rnd((2, 100), 7), headDim=64)


# ---- the transformers library's rope routines -----------------------------------

transformers = pytest.importorskip("transformers")
torch = pytest.importorskip("torch")


def hf_table(rp, D, max_pos=16384, seq_len=None):
    from transformers import LlamaConfig
    from transformers import modeling_rope_utils as mru
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding
    transformers.logging.set_verbosity_error()
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        cfg = LlamaConfig(hidden_size=8 * D, num_attention_heads=8, head_dim=D,
                          max_position_embeddings=max_pos, rope_parameters=dict(rp))
        if rp["rope_type"] == "default":
            inv, af = LlamaRotaryEmbedding.compute_default_rope_parameters(cfg)
        elif seq_len is not None:
            inv, af = mru.ROPE_INIT_FUNCTIONS[rp["rope_type"]](cfg, None, seq_len=seq_len)
        else:
            inv, af = mru.ROPE_INIT_FUNCTIONS[rp["rope_type"]](cfg, None)
    return inv.double().numpy(), float(af)


LONG = list(np.linspace(1.0, 8.0, 32))
SHORT = list(np.linspace(1.0, 2.0, 32))
HF_CASES = [
    ("default", dict(rope_type="default", rope_theta=10000.0), None),
    ("default-500k", dict(rope_type="default", rope_theta=500000.0), None),
    ("linear", dict(rope_type="linear", rope_theta=10000.0, factor=4.0), None),
    ("llama3", dict(rope_type="llama3", rope_theta=500000.0, factor=8.0, low_freq_factor=1.0,
                    high_freq_factor=4.0, original_max_position_embeddings=8192), None),
    ("yarn", dict(rope_type="yarn", rope_theta=10000.0, factor=4.0,
                  original_max_position_embeddings=4096), None),
    ("yarn-mscale", dict(rope_type="yarn", rope_theta=10000.0, factor=4.0,
                         original_max_position_embeddings=4096, beta_fast=16, beta_slow=2,
                         mscale=0.707, mscale_all_dim=0.707), None),
    ("yarn-untruncated", dict(rope_type="yarn", rope_theta=1e6, factor=4.0,
                              original_max_position_embeddings=4096, truncate=False), None),
    ("dynamic-long", dict(rope_type="dynamic", rope_theta=10000.0, factor=2.0), 32768),
    ("dynamic-short", dict(rope_type="dynamic", rope_theta=10000.0, factor=2.0), 8000),
    ("longrope-short", dict(rope_type="longrope", rope_theta=10000.0, short_factor=SHORT,
                            long_factor=LONG, original_max_position_embeddings=4096), None),
    ("longrope-long", dict(rope_type="longrope", rope_theta=10000.0, short_factor=SHORT,
                           long_factor=LONG, original_max_position_embeddings=4096), 9000),
]


@pytest.mark.parametrize("name, rp, seq_len", HF_CASES, ids=[c[0] for c in HF_CASES])
def test_tables_match_transformers(name, rp, seq_len):
    # transformers computes its tables in f32 arithmetic; the oracle rounds an
    # f64 computation once. They agree to a few f32 ulps.
    want, af_want = hf_table(rp, 64, seq_len=seq_len)
    sc = dict(rp)
    base = sc.pop("rope_theta")
    sc["max_position_embeddings"] = 16384
    got, af = oracle.rope_table(64, base=base, scaling=sc, seq_len=seq_len or 1)
    np.testing.assert_allclose(got.astype(np.float64), want, rtol=5e-7, atol=0)
    assert af == pytest.approx(af_want, rel=1e-6)


@pytest.mark.parametrize("rd", [64, 32])
def test_half_split_rotation_matches_llama(rd):
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    D, H, T, p0 = 64, 3, 6, 40
    inv, _ = hf_table(dict(rope_type="default", rope_theta=10000.0), rd)
    x = rnd((T, H * D), 8)
    pos = np.arange(p0, p0 + T, dtype=np.float64)
    ang = np.concatenate([pos[:, None] * inv[None, :]] * 2, axis=1)      # [T, rd]
    cos, sin = torch.from_numpy(np.cos(ang))[None], torch.from_numpy(np.sin(ang))[None]
    xt = torch.from_numpy(x.astype(np.float64)).reshape(1, T, H, D).transpose(1, 2)
    rot, _ = apply_rotary_pos_emb(xt[..., :rd], xt[..., :rd], cos, sin)
    want = torch.cat([rot, xt[..., rd:]], dim=-1).transpose(1, 2).reshape(T, H * D).numpy()
    got = oracle.rope(x, headDim=D, rotaryDim=rd, offset=p0, invFreq=inv.astype(np.float32))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_interleaved_rotation_matches_gptj():
    from transformers.models.gptj.modeling_gptj import apply_rotary_pos_emb
    D, rd, H, T, p0 = 64, 32, 2, 5, 9
    inv, _ = oracle.rope_table(rd)
    x = rnd((T, H * D), 9)
    pos = np.arange(p0, p0 + T, dtype=np.float64)
    ang = pos[:, None] * inv.astype(np.float64)[None, :]                 # [T, rd/2]
    sin, cos = torch.from_numpy(np.sin(ang))[None], torch.from_numpy(np.cos(ang))[None]  # [1, T, rd/2]
    xt = torch.from_numpy(x.astype(np.float64)).reshape(1, T, H, D)
    rot = apply_rotary_pos_emb(xt[..., :rd], sin, cos)
    want = torch.cat([rot, xt[..., rd:]], dim=-1).reshape(T, H * D).numpy()
    got = oracle.rope(x, headDim=D, rotaryDim=rd, offset=p0, interleaved=True, invFreq=inv)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ---- every table entry against a 50-digit evaluation ------------------------------
#
# The oracle computes each table entry in f64 (the C library's pow, log and
# exp) and rounds it to f32 once. Here the same definitions are evaluated in
# 50-digit decimal arithmetic, with pi from Machin's formula and powers as
# exp(e ln b), and every f32 entry must be exactly the f32 nearest to that
# value: the last bit of the oracle's table is then fixed by the mathematics,
# not by the library's pow.

from decimal import Decimal as Dec, localcontext

DIGITS = 50


def _dpi() -> Dec:
    """pi = 16 atan(1/5) - 4 atan(1/239) (Machin), atan by its Taylor series."""
    def atan_inv(n):
        x = Dec(1) / n
        x2, term, total, k = x * x, x, x, 1
        while True:
            term *= -x2
            k += 2
            nxt = total + term / k
            if nxt == total:
                return total
            total = nxt
    return 16 * atan_inv(5) - 4 * atan_inv(239)


def _dpow(b: Dec, e: Dec) -> Dec:
    return (e * b.ln()).exp()


def exact_table(rd, base, scaling=None, seq_len=1):
    """(invFreq entries, attention factor) as 50-digit decimals, following the
    definitions the oracle's docstrings state (RoFormer's base^(-2i/rd); the
    linear, llama3, yarn, dynamic and longrope scalings)."""
    with localcontext() as ctx:
        ctx.prec = DIGITS
        pi = _dpi()
        b = Dec(base)
        s = dict(scaling or {})
        kind = s.get("rope_type", "default")
        if kind == "dynamic":
            orig = Dec(s.get("original_max_position_embeddings") or s["max_position_embeddings"])
            f = Dec(s["factor"])
            if seq_len > orig:
                b = b * _dpow(f * seq_len / orig - (f - 1), Dec(rd) / (rd - 2))
        theta = [_dpow(b, Dec(-2 * i) / rd) for i in range(rd // 2)]
        af = Dec(1)
        if kind == "linear":
            inv = [t / Dec(s["factor"]) for t in theta]
        elif kind == "llama3":
            f, lo_f, hi_f = Dec(s["factor"]), Dec(s["low_freq_factor"]), Dec(s["high_freq_factor"])
            orig = Dec(s["original_max_position_embeddings"])
            inv = []
            for t in theta:
                wl = 2 * pi / t
                if wl < orig / hi_f:
                    inv.append(t)
                elif wl > orig / lo_f:
                    inv.append(t / f)
                else:
                    sm = (orig / wl - lo_f) / (hi_f - lo_f)
                    inv.append((1 - sm) * t / f + sm * t)
        elif kind == "yarn":
            f, orig = Dec(s["factor"]), Dec(s["original_max_position_embeddings"])
            b_fast, b_slow = Dec(s.get("beta_fast") or 32), Dec(s.get("beta_slow") or 1)

            def index_for(turns):
                return rd * (orig / (turns * 2 * pi)).ln() / (2 * b.ln())

            lo, hi = index_for(b_fast), index_for(b_slow)
            if s.get("truncate", True):
                lo, hi = Dec(math.floor(lo)), Dec(math.ceil(hi))
            lo, hi = max(lo, Dec(0)), min(hi, Dec(rd - 1))
            if lo == hi:
                hi += Dec("0.001")
            inv = []
            for i, t in enumerate(theta):
                ramp = min(max((i - lo) / (hi - lo), Dec(0)), Dec(1))
                inv.append(t * (1 - ramp) + t / f * ramp)

            def mscale(k):
                return Dec("0.1") * k * f.ln() + 1 if f > 1 else Dec(1)
            m, m_all = s.get("mscale"), s.get("mscale_all_dim")
            af = mscale(Dec(m)) / mscale(Dec(m_all)) if m and m_all else mscale(Dec(1))
        elif kind == "longrope":
            orig = Dec(s["original_max_position_embeddings"])
            ext = s["long_factor"] if seq_len > orig else s["short_factor"]
            inv = [t / Dec(float(e)) for t, e in zip(theta, ext)]
            f = Dec(s["factor"]) if s.get("factor") is not None else Dec(s["max_position_embeddings"]) / orig
            af = (1 + f.ln() / orig.ln()).sqrt() if f > 1 else Dec(1)
        else:
            inv = theta
        return inv, af


def nearest_f32(x: Dec) -> np.float32:
    """The f32 nearest to x, checked against both neighbours in decimal."""
    f = np.float32(float(x))
    with localcontext() as ctx:
        ctx.prec = DIGITS
        d = abs(x - Dec(float(f)))
        for nb in (np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))):
            assert d <= abs(x - Dec(float(nb))), f"{x} rounds nearer to {nb!r} than {f!r}"
    return f


EXACT_CASES = [
    ("default-128", 128, 10000.0, None, 1),
    ("default-64-500k", 64, 500000.0, None, 1),
    ("default-96-1e6", 96, 1e6, None, 1),
    ("linear", 128, 10000.0, dict(rope_type="linear", factor=4.0), 1),
    ("llama3.1", 128, 500000.0, dict(rope_type="llama3", factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                                      original_max_position_embeddings=8192), 1),
    ("yarn", 64, 10000.0, dict(rope_type="yarn", factor=4.0, original_max_position_embeddings=4096), 1),
    ("yarn-mscale", 64, 10000.0, dict(rope_type="yarn", factor=4.0, original_max_position_embeddings=4096,
                                      beta_fast=16, beta_slow=2, mscale=0.707, mscale_all_dim=1.0), 1),
    ("yarn-untruncated", 128, 1e6, dict(rope_type="yarn", factor=4.0, original_max_position_embeddings=4096,
                                        truncate=False), 1),
    ("dynamic-long", 64, 10000.0, dict(rope_type="dynamic", factor=2.0, max_position_embeddings=16384), 32768),
    ("dynamic-short", 64, 10000.0, dict(rope_type="dynamic", factor=2.0, max_position_embeddings=16384), 8000),
    ("longrope-short", 64, 10000.0, dict(rope_type="longrope", short_factor=SHORT, long_factor=LONG,
                                         original_max_position_embeddings=4096, max_position_embeddings=131072),
     4096),
    ("longrope-long", 64, 10000.0, dict(rope_type="longrope", short_factor=SHORT, long_factor=LONG,
                                        original_max_position_embeddings=4096, max_position_embeddings=131072),
     9000),
]


@pytest.mark.parametrize("name, rd, base, scaling, seq_len", EXACT_CASES, ids=[c[0] for c in EXACT_CASES])
def test_table_entries_are_the_nearest_f32(name, rd, base, scaling, seq_len):
    want, af_want = exact_table(rd, base, scaling, seq_len)
    got, af = oracle.rope_table(rd, base=base, scaling=scaling, seq_len=seq_len)
    want32 = np.array([nearest_f32(x) for x in want], dtype=np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), want32.view(np.uint32), err_msg=name)
    assert np.float32(af) == nearest_f32(af_want), name
