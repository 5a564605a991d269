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
