"""The oracle pins catch plausible mistakes: each case plants one mistake in a
temporary copy of the oracle (on the CPU) and requires the pin suite to fail
against it; the unmodified copy must pass."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "lrm_oracle.py")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

MUTATIONS = {
    "score_drops_weight_square": ("return (w * w) * g_sumsq * x_sumsq",
                                  "return w * g_sumsq * x_sumsq"),
    "tie_break_reversed": ("order = np.lexsort((cand, -score[cand]))",
                           "order = np.lexsort((-cand, -score[cand]))"),
    "keeps_smallest": ("order = np.lexsort((cand, -score[cand]))",
                       "order = np.lexsort((cand, score[cand]))"),
    "dW_drops_weight": ("return g.T @ (w[:, None] * x)", "return g.T @ x"),
    "dx_weight_twice": ("return w[:, None] * (g @ We)",
                        "return w[:, None] * (g @ We) * w[:, None]"),
    "dsilu_sign": ("return s * (1.0 + a * (1.0 - s))", "return s * (1.0 - a * (1.0 - s))"),
    "gb_uses_a": ("return u * b * dsilu(a), u * silu(a)", "return u * b * dsilu(a), u * a"),
    "up_path_uses_gate_weight": ('dx[iu] += wu[:, None] * (gb[iu] @ f64(p["W_up"][e]))',
                                 'dx[iu] += wu[:, None] * (gb[iu] @ f64(p["W_gate"][e]))'),
    "hidden_grad_scaled": ('u = g @ f64(p["W_down"][e])',
                           'u = g @ f64(p["W_down"][e]) * 1.0001'),
    "pack_offsets_shifted": ("np.cumsum(sizes, out=offsets[1:])",
                             "np.cumsum(sizes, out=offsets[1:]); offsets[1:] += 1"),
    # the threshold is the smallest kept score, not the largest
    "threshold_max_not_min": ("return float(np.min(np.asarray(score, np.float64)[kept_e]))",
                              "return float(np.max(np.asarray(score, np.float64)[kept_e]))"),
    # off by one in the kept count: the (M_e - 1)-th largest score, and None
    # for one kept pair instead of for all kept
    "threshold_count_off_by_one": ("    m = kept_e.shape[0]\n    if m == 0 or m == n_e:",
                                   "    m = kept_e.shape[0] - 1\n    if m == 0 or m == n_e:"),
    # the (M_e + 1)-th largest: the best dropped score instead of the worst kept
    "threshold_next_below": ("return float(np.min(np.asarray(score, np.float64)[kept_e]))",
                             "return float(np.sort(np.asarray(score, np.float64))[::-1][m])"),
}


def _run_pins(tmp_path, source: str) -> int:
    pkg = tmp_path / "oracle"
    pkg.mkdir(exist_ok=True)
    (pkg / "__init__.py").write_text("")
    (pkg / "lrm_oracle.py").write_text(source)
    # run from the temporary directory: it comes first on sys.path, so the
    # planted copy shadows the real oracle
    env = dict(os.environ, PYTHONPATH=str(tmp_path) + os.pathsep + ROOT)
    probe = subprocess.run([sys.executable, "-c", "import oracle, sys; print(oracle.__file__)"],
                           cwd=str(tmp_path), env=env, capture_output=True, text=True)
    assert probe.stdout.strip().startswith(str(tmp_path)), probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        PINS], cwd=str(tmp_path), env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode


def test_unmodified_copy_passes(tmp_path):
    assert _run_pins(tmp_path, open(ORACLE).read()) == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(ORACLE).read()
    assert src.count(old) >= 1, f"mutation site not found: {old}"
    assert _run_pins(tmp_path, src.replace(old, new, 1)) != 0, f"pins missed: {name}"
