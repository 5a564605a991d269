"""The oracle's pins must catch plausible slips.

Each case plants one mistake in a temporary copy of the oracle's C core (a
flipped sign, a wrong index or stride, an off-by-one in the window rule, a
dropped term) and runs the pin suite against that copy in a subprocess. A
mutant that passes every pin would mean the pins cannot tell it from the
definition. Everything here runs on the CPU; the real oracle is untouched.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "alibi_sign": ("xs -= a->slopes[h] * dist;", "xs += a->slopes[h] * dist;"),
    "gqa_mapping": ("const int64_t g = (h * a->G) / a->H;", "const int64_t g = h % a->G;"),
    "bias_index": ("j->bias[(h * a->T + t) * a->S + s]", "j->bias[(t * a->H + h) * a->S + s]"),
    "causal_window_edge": ("!(pos - a->window < s)", "!(pos - a->window <= s)"),
    "noncausal_window_edge": ("if (dist > a->window) return 0;", "if (dist >= a->window) return 0;"),
    "scale_dropped": ("double xs = a->scale * dot;", "double xs = dot;"),
    "k_stride": ("j->k + s * (a->G * D) + g * D", "j->k + s * D + g * D"),
    "v_stride": ("j->v + s * (a->G * Dv) + g * Dv", "j->v + s * Dv + g * Dv"),
    "causal_diagonal": ("if (s > pos) return 0;", "if (s >= pos) return 0;"),
    "pos_offset_dropped": ("const int64_t pos = a->pos_offset + t;", "const int64_t pos = t;"),
    "softcap_after_bias": (
        "if (a->softcap > 0.0) xs = a->softcap * tanh(xs / a->softcap);\n"
        "        if (a->slopes) {",
        "if (a->slopes) {"),
    "max_not_subtracted": ("double p = exp(x[s] - M);", "double p = exp(x[s]);"),
    "sink_edge": ("const int sink = a->window > 0 && s < a->sinks;",
                  "const int sink = a->window > 0 && s <= a->sinks;"),
    "sink_ignores_causal": ("        if (s > pos) return 0;\n        if (sink) return 1;",
                            "        if (sink) return 1;\n        if (s > pos) return 0;"),
    "sink_noncausal_dropped": ("if (a->window > 0 && !sink) {", "if (a->window > 0) {"),
    # ALiBi distance signed (BLOOM's one-sided form carried over to
    # non-causal rows), and a penalty of |pos - s| + 1: equal to the reading
    # on causal rows up to a row constant, so only the non-causal pins see them.
    "alibi_signed_distance": ("double dist = (double)(pos > s ? pos - s : s - pos);",
                              "double dist = (double)(pos - s);"),
    "alibi_distance_plus_one": ("double dist = (double)(pos > s ? pos - s : s - pos);",
                                "double dist = (double)(pos > s ? pos - s : s - pos) + 1.0;"),
}

# Slips in the rotary embedding (oracle/rope.py), caught by tests/test_oracle_rope.py.
ROPE_MUTANTS = {
    "rope_turn_sense": ("out[:, :, ia] = a * c - b * s", "out[:, :, ia] = a * c + b * s"),
    "rope_half_partner": ("np.arange(half) + half", "np.arange(half) + half - 1"),
    "rope_freq_exponent": ("float(base) ** (-2.0 * i / rd)", "float(base) ** (-1.0 * i / rd)"),
    "rope_factor_dropped": ("c = (np.cos(ang) * af)[:, None, :]", "c = np.cos(ang)[:, None, :]"),
    "rope_position_shift": ("pos = (p0 + np.arange(T, dtype=np.int64))",
                            "pos = (p0 + 1 + np.arange(T, dtype=np.int64))"),
    "rope_passthrough_scaled": ("out = y.copy()", "out = y.copy() * af"),
    "rope_yarn_ramp_reversed": ("return theta * (1.0 - ramp) + (theta / factor) * ramp",
                                "return theta * ramp + (theta / factor) * (1.0 - ramp)"),
    "rope_llama3_blend_reversed": ("out[i] = (1.0 - smooth) * f / factor + smooth * f",
                                   "out[i] = smooth * f / factor + (1.0 - smooth) * f"),
    "rope_linear_multiplies": ("return theta / float(s[\"factor\"])", "return theta * float(s[\"factor\"])"),
    "rope_dynamic_exponent": ("** (rd / (rd - 2.0))", "** (rd / (rd - 1.0))"),
    "rope_longrope_sets_swapped": ('ext = s["long_factor"] if seq_len > orig else s["short_factor"]',
                                   'ext = s["short_factor"] if seq_len > orig else s["long_factor"]'),
    "rope_yarn_temperature": ("return 0.1 * k * math.log(scale) + 1.0", "return 0.1 * k * math.log(scale)"),
    # One table entry one f32 ulp off, and the frequencies computed in f32:
    # both within the transformers pin's 5e-7, caught by the exact-table pin.
    "rope_table_one_ulp": ("    return _f32(inv), float(np.float32(af))",
                           "    inv = _f32(inv)\n"
                           "    inv[len(inv) // 3] = np.nextafter(inv[len(inv) // 3], np.float32(1))\n"
                           "    return inv, float(np.float32(af))"),
    "rope_table_f32_power": ("[float(base) ** (-2.0 * i / rd) for i in range(rd // 2)]",
                             "[float(np.float32(base) ** np.float32(-2.0 * i / rd)) for i in range(rd // 2)]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    tree = tmp_path / "tree"
    tree.mkdir()
    shutil.copytree(os.path.join(ROOT, "oracle"), tree / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tree / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py"))
    shutil.copy(os.path.join(ROOT, "workloads.py"), tree / "workloads.py")
    src = (tree / "oracle" / "oracle.c").read_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    if name == "softcap_after_bias":
        # Move the cap below the bias term instead of dropping it.
        src = src.replace(old, new)
        cap = "        if (a->softcap > 0.0) xs = a->softcap * tanh(xs / a->softcap);\n"
        anchor = "        x[s] = xs;\n"
        src = src.replace(anchor, cap + anchor, 1)
    else:
        src = src.replace(old, new)
    (tree / "oracle" / "oracle.c").write_text(src)
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "tests/test_oracle.py", "-x", "-q",
         "-p", "no:cacheprovider"],
        cwd=tree, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, f"mutant {name} passed every pin:\n{proc.stdout[-2000:]}"
    assert "failed" in proc.stdout, proc.stdout[-2000:] + proc.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_rope_pins_kill_mutant(name, tmp_path):
    old, new = ROPE_MUTANTS[name]
    tree = tmp_path / "tree"
    tree.mkdir()
    shutil.copytree(os.path.join(ROOT, "oracle"), tree / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tree / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py"))
    shutil.copy(os.path.join(ROOT, "workloads.py"), tree / "workloads.py")
    path = tree / "oracle" / "rope.py"
    src = path.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path.write_text(src.replace(old, new))
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "tests/test_oracle_rope.py", "-x", "-q",
         "-p", "no:cacheprovider"],
        cwd=tree, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, f"mutant {name} passed every pin:\n{proc.stdout[-2000:]}"
    assert "failed" in proc.stdout, proc.stdout[-2000:] + proc.stderr[-2000:]


# Slips in the latent attention oracle (oracle/mla.py), caught by tests/test_oracle_mla.py.
MLA_MUTANTS = {
    # k_b read as if stored [kv_rank, qk_nope] per head
    "mla_k_b_layout": ("keys[h, :, :N] = c @ k_b[h].astype(np.float64).T",
                       "keys[h, :, :N] = c @ k_b[h].astype(np.float64).reshape(R, N)"),
    "mla_rope_part_dropped": ("keys[h, :, N:] = kpe", "keys[h, :, N:] = 0.0"),
    "mla_head_weights": ("vals[h] = c @ v_b[h].astype(np.float64).T",
                         "vals[h] = c @ v_b[0].astype(np.float64).T"),
    "mla_rope_from_latent": ("kpe = state[:, R:R + P].astype(np.float64)",
                             "kpe = state[:, :P].astype(np.float64)"),
    "mla_default_scale": ("np.float32(1.0 / math.sqrt(N + P))", "np.float32(1.0 / math.sqrt(N))"),
    "mla_sink_edge": ("seen = in_window | (s < sinks)", "seen = in_window | (s <= sinks)"),
    "mla_causal_diagonal": ("seen &= s <= pos", "seen &= s < pos"),
    "mla_pos_offset_dropped": ('r["P0"] + t, S)', "t, S)"),
    "mla_q_head_stride": ("qh = q[t, h * (N + P):(h + 1) * (N + P)]", "qh = q[t, h * N:h * N + N + P]"),
}


@pytest.mark.parametrize("name", sorted(MLA_MUTANTS))
def test_mla_pins_kill_mutant(name, tmp_path):
    old, new = MLA_MUTANTS[name]
    tree = tmp_path / "tree"
    tree.mkdir()
    shutil.copytree(os.path.join(ROOT, "oracle"), tree / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tree / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py"))
    shutil.copy(os.path.join(ROOT, "workloads.py"), tree / "workloads.py")
    path = tree / "oracle" / "mla.py"
    src = path.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path.write_text(src.replace(old, new))
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "tests/test_oracle_mla.py", "-x", "-q",
         "-p", "no:cacheprovider"],
        cwd=tree, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, f"mutant {name} passed every pin:\n{proc.stdout[-2000:]}"
    assert "failed" in proc.stdout, proc.stdout[-2000:] + proc.stderr[-2000:]


# Slips in the relative-position terms of the C core, caught by tests/test_oracle_relpos.py.
RELPOS_MUTANTS = {
    "pb_threshold_edge": ("if (a->pb_bounds[i] <= dist) b = i;", "if (a->pb_bounds[i] < dist) b = i;"),
    "pb_bidirectional_side": ("if (a->pb_bidirectional && s > pos) b += a->pb_n;",
                              "if (a->pb_bidirectional && s < pos) b += a->pb_n;"),
    "pb_head_stride": ("a->pb_weight[pb_row(a, pos, s) * a->H + h]", "a->pb_weight[pb_row(a, pos, s) + h]"),
    "rel_sign": ("int64_t r = s - pos;", "int64_t r = pos - s;"),
    "rel_clip_edge": ("if (r < -a->rel_max) r = -a->rel_max;", "if (r < -a->rel_max) r = -a->rel_max + 1;"),
    "rel_v_unweighted": ("for (int64_t e = 0; e < Dv; ++e) orow[e] += p * (double)rv[e];",
                         "for (int64_t e = 0; e < Dv; ++e) orow[e] += (double)rv[e];"),
    "rel_k_unscaled": ("        double xs = a->scale * dot;\n",
                       "        double xs = a->scale * dot;\n        if (a->rel_k) xs += dot * (1.0 - a->scale);\n"),
}


@pytest.mark.parametrize("name", sorted(RELPOS_MUTANTS))
def test_relpos_pins_kill_mutant(name, tmp_path):
    old, new = RELPOS_MUTANTS[name]
    tree = tmp_path / "tree"
    tree.mkdir()
    shutil.copytree(os.path.join(ROOT, "oracle"), tree / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tree / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py"))
    shutil.copy(os.path.join(ROOT, "workloads.py"), tree / "workloads.py")
    path = tree / "oracle" / "oracle.c"
    src = path.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path.write_text(src.replace(old, new))
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "tests/test_oracle_relpos.py", "-x", "-q",
         "-p", "no:cacheprovider"],
        cwd=tree, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, f"mutant {name} passed every pin:\n{proc.stdout[-2000:]}"
    assert "failed" in proc.stdout, proc.stdout[-2000:] + proc.stderr[-2000:]
