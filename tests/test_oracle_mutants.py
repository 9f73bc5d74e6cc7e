"""Planted mistakes in the oracle must fail its pins.

Each case below copies the oracle package to a temporary folder with one plausible slip
written into ``kda_oracle.c`` (a reversed tap order, an off-by-one window, a dropped scale,
bias or exponential, a wrong sign, a q/k/v or head index mixed up, ...) or into the pooled
and accept-step functions of ``__init__.py`` (a pool row taken from the wrong index array,
the wrong snapshot committed, padding not skipped), builds that copy,
and runs ``tests/test_oracle_pins.py`` against it in a child process: at least one pin must
fail. Two tests of that file do not count here, since they cannot tell a slip from the
truth on their own: the stored tiny fixture (written by the oracle itself) and the torch
composition (the same formulas typed a second time). An unmodified copy must pass every
pin, so that a failing mutant means a pin caught it and not a broken harness.

CPU only: the mistakes go into copies of the oracle, never into GPU code.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC_PATH = os.path.join(ROOT, "oracle", "kda_oracle.c")
PY_PATH = os.path.join(ROOT, "oracle", "__init__.py")

# (name, text in kda_oracle.c, text that replaces it)
MUTANTS = [
    ("silu-is-sigmoid", "double oracle_silu(double y) { return y / (1.0 + exp(-y)); }",
     "double oracle_silu(double y) { return 1.0 / (1.0 + exp(-y)); }"),
    ("sigmoid-sign", "double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }",
     "double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(x)); }"),
    ("conv-taps-reversed", "y += conv_weight[(size_t)c * ORACLE_W + j] *",
     "y += conv_weight[(size_t)c * ORACLE_W + (ORACLE_W - 1 - j)] *"),
    ("conv-window-off-by-one", "ext_raw(mixed_qkv, conv_state, T, C, n, c, t + 1 + j);",
     "ext_raw(mixed_qkv, conv_state, T, C, n, c, t + j);"),
    ("rolled-cache-off-by-one", "ext_raw(mixed_qkv, conv_state, T, C, n, c, T + j);",
     "ext_raw(mixed_qkv, conv_state, T, C, n, c, T - 1 + j);"),
    ("l2norm-no-sqrt", "double r = 1.0 / sqrt(s + eps);", "double r = 1.0 / (s + eps);"),
    ("l2norm-eps-outside", "double r = 1.0 / sqrt(s + eps);", "double r = 1.0 / (sqrt(s) + eps);"),
    ("q-not-scaled", "oracle_l2norm(K, a + (size_t)h * K, eps, scale, qn);",
     "oracle_l2norm(K, a + (size_t)h * K, eps, 1.0, qn);"),
    ("k-reads-q-channels", "oracle_l2norm(K, a + (size_t)H * K + (size_t)h * K, eps, 1.0, kn);",
     "oracle_l2norm(K, a + (size_t)h * K, eps, 1.0, kn);"),
    ("softplus-no-beta-divide", "if (b * x <= threshold) return log1p(exp(b * x)) / b;",
     "if (b * x <= threshold) return log1p(exp(b * x));"),
    ("softplus-branch-flipped", "if (b * x <= threshold) return log1p(exp(b * x)) / b;",
     "if (b * x >= threshold) return log1p(exp(b * x)) / b;"),
    ("gate-no-exp-A", "if (mode == 0) return -exp(A_log) * oracle_softplus(",
     "if (mode == 0) return -A_log * oracle_softplus("),
    ("gate-sign", "if (mode == 0) return -exp(A_log) * oracle_softplus(",
     "if (mode == 0) return exp(A_log) * oracle_softplus("),
    ("gate-no-dt-bias", "double gamma = g + dt_bias;", "double gamma = g;"),
    ("safe-gate-no-exp-A", "return lower_bound * oracle_sigmoid(exp(A_log) * gamma);",
     "return lower_bound * oracle_sigmoid(gamma);"),
    ("decay-row-index", "for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= alpha[i];",
     "for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= alpha[(i + 1) % K];"),
    ("decay-not-exponentiated", "alpha[i] = exp(oracle_log_decay(", "alpha[i] = (oracle_log_decay("),
    ("u-uses-q", "for (int i = 0; i < K; ++i) u += k[i] * S[(size_t)i * V + j];",
     "for (int i = 0; i < K; ++i) u += q[i] * S[(size_t)i * V + j];"),
    ("correction-sign", "double d = beta * (v[j] - u);", "double d = beta * (u - v[j]);"),
    ("correction-no-beta", "double d = beta * (v[j] - u);", "double d = (v[j] - u);"),
    ("output-reads-k", "for (int i = 0; i < K; ++i) acc += q[i] * S[(size_t)i * V + j];",
     "for (int i = 0; i < K; ++i) acc += k[i] * S[(size_t)i * V + j];"),
    ("gva-head-modulo", "const int h = hv / g;", "const int h = hv % H;"),
    ("v-from-qk-head", "const double* vv = a + 2 * (size_t)H * K + (size_t)hv * V;",
     "const double* vv = a + 2 * (size_t)H * K + (size_t)h * V;"),
    ("dt-bias-by-qk-head", "dt_bias[(size_t)hv * K + i]", "dt_bias[(size_t)h * K + i]"),
    ("A-log-by-qk-head", "A_log[hv], lower_bound", "A_log[h], lower_bound"),
    ("beta-not-squashed", "const double b = oracle_sigmoid(beta[nth]);", "const double b = beta[nth];"),
    ("gate-index-by-qk-head", "gate[nth * K + i]", "gate[(((size_t)n * T + t) * HV + h) * K + i]"),
]

# the same, in the pooled and accept-step functions of oracle/__init__.py
PY_MUTANTS = [
    ("pooled-conv-row-by-sequence", '"conv_state": cs_pool[c:c + 1]', '"conv_state": cs_pool[n:n + 1]'),
    ("pooled-state-row-by-sequence", '"state": st_pool[s_:s_ + 1]', '"state": st_pool[n:n + 1]'),
    ("pooled-snapshot-row-by-cache-index", 'out_is[i] = r["inter_ssm"][0]', 'out_is[s_] = r["inter_ssm"][0]'),
    ("pooled-window-row-by-conv-index", 'out_cw[i] = r["conv_window"][0]', 'out_cw[c] = r["conv_window"][0]'),
    ("pooled-cache-not-written", 'cs_pool[c] = r["conv_state"][0]', 'pass'),
    ("commit-wrong-token", "st[s_] = isp[i, a - 1]", "st[s_] = isp[i, a - 2]"),
    ("commit-last-window", "cs[c] = cwp[i, a - 1]", "cs[c] = cwp[i, T - 1]"),
    ("commit-accepts-zero", "if not (1 <= a <= T and", "if not (0 <= a <= T and"),
]

# Child process: load the copy as the module `oracle` before pytest imports anything, build
# it, then run the pins. Exit 7 if the copy does not build.
_DRIVER = r"""
import importlib.util, sys
tmp = sys.argv[1]
spec = importlib.util.spec_from_file_location("oracle", tmp + "/oracle/__init__.py",
                                              submodule_search_locations=[tmp + "/oracle"])
mod = importlib.util.module_from_spec(spec)
sys.modules["oracle"] = mod
spec.loader.exec_module(mod)
try:
    mod.build()
except Exception as e:
    print("BUILD FAILED", e)
    sys.exit(7)
import pytest
sys.exit(pytest.main(["tests/test_oracle_pins.py", "-x", "-q", "-p", "no:cacheprovider",
                      "--deselect", "tests/test_oracle_pins.py::test_tiny_regression_fixture",
                      "-k", "not independent_torch_composition"]))
"""


def _run_copy(sources):
    d = tempfile.mkdtemp(prefix="kda_oracle_mutant_")
    try:
        os.makedirs(os.path.join(d, "oracle"))
        c_src, py_src = sources
        with open(os.path.join(d, "oracle", "kda_oracle.c"), "w") as f:
            f.write(c_src)
        with open(os.path.join(d, "oracle", "__init__.py"), "w") as f:
            f.write(py_src)
        r = subprocess.run([sys.executable, "-c", _DRIVER, d], cwd=ROOT, capture_output=True, text=True,
                           timeout=600)
        caught = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
        return r.returncode, (caught[0] if caught else r.stdout[-400:])
    finally:
        shutil.rmtree(d, ignore_errors=True)


@pytest.fixture(scope="module")
def results():
    src, py = open(SRC_PATH).read(), open(PY_PATH).read()
    jobs = {"control": (src, py)}
    # each planted text must name exactly one place, so the lists follow the sources
    for name, old, new in MUTANTS:
        jobs[name] = (src.replace(old, new), py) if src.count(old) == 1 else None
    for name, old, new in PY_MUTANTS:
        jobs[name] = (src, py.replace(old, new)) if py.count(old) == 1 else None
    todo = {k: v for k, v in jobs.items() if v is not None}
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        done = dict(zip(todo, ex.map(_run_copy, todo.values())))
    return {k: done.get(k) for k in jobs}


def test_unmodified_copy_passes_every_pin(results):
    rc, info = results["control"]
    assert rc == 0, info


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS + PY_MUTANTS])
def test_planted_mistake_fails_a_pin(results, name):
    got = results[name]
    assert got is not None, f"{name}: its text is not found exactly once in the oracle source"
    rc, info = got
    assert rc != 7, f"{name}: the mutant copy did not build: {info}"
    assert rc == 1, f"{name}: no pin failed (exit {rc}): {info}"
