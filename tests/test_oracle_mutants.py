"""Each plausible mistake, planted in a private copy of the oracle, must be
caught by at least one pin.  The copies are compiled into a temporary
directory; the oracle itself is never modified."""
import os
import shutil
import subprocess
import tempfile

import pytest

from oracle import svo
import oracle_pins as P

HERE = os.path.dirname(os.path.abspath(svo.__file__))

# (name, original text, replacement)
MUTANTS = [
    ("residual_sign", "double d = pa[v] - qa[v];", "double d = qa[v] - pa[v];"),
    ("accept_ratio_inverted", "int accept = (double)u[i] * qi < pi;",
     "int accept = (double)u[i] * pi < qi;"),
    ("accept_non_strict_wrong_side", "int accept = (double)u[i] * qi < pi;",
     "int accept = (double)u[i] < pi;"),
    ("bonus_from_previous_row",
     "softmax_row(target, dtype, t_row(b, k, a, stride), V, tau, p);\n    if (a < k)",
     "softmax_row(target, dtype, t_row(b, k, a < k ? a : k - 1, stride), V, tau, p);\n    if (a < k)"),
    ("draft_without_temperature",
     "softmax_row(draft, dtype, d_row(b, k, i, stride), V, tau, q);",
     "softmax_row(draft, dtype, d_row(b, k, i, stride), V, 1.0, q);"),
    ("temperature_multiplies", "prob[v] = exp((logit(base, dtype, row_off + v) - M) / tau);",
     "prob[v] = exp((logit(base, dtype, row_off + v) - M) * tau);"),
    ("cdf_non_strict", "if (w[v] > 0.0 && C > r) {", "if (w[v] > 0.0 && C >= r) {"),
    ("cdf_unnormalised", "C += w[v] / S;\n        if", "C += w[v];\n        if"),
    ("residual_from_target_only", "double d = pa[v] - qa[v];", "double d = pa[v];"),
    ("argmax_last_tie", "if (x > bv) {", "if (x >= bv) {"),
    ("candidate_last_tie", "if (a > best_a) {", "if (a >= best_a) {"),
    ("greedy_emits_draft", "out[i] = argmax_row(target, dtype, (base + i) * row_stride, V);",
     "out[i] = i < best_a ? draft_tokens[((int64_t)b * G + best_c) * k + i] : 0;"),
    ("token_row_offset", "return ((int64_t)b * (k + 1) + i) * stride;",
     "return ((int64_t)b * k + i) * stride;"),
    ("softmax_no_max_shift", "prob[v] = exp((logit(base, dtype, row_off + v) - M) / tau);",
     "prob[v] = exp(logit(base, dtype, row_off + v) / tau) + 0.0 * M;"),
]


def _fails_some_pin(lib):
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError):
            return pin.__name__
    return None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    src = open(os.path.join(HERE, "svo.c")).read()
    assert old in src, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as tmp:
        shutil.copy(os.path.join(HERE, "svo.h"), tmp)
        with open(os.path.join(tmp, "svo.c"), "w") as f:
            f.write(src.replace(old, new, 1))
        so = os.path.join(tmp, f"libsvo_{name}.so")
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC",
                        os.path.join(tmp, "svo.c"), "-o", so, "-lm"], check=True)
        lib = svo.load(so)
        caught_by = _fails_some_pin(lib)
    assert caught_by is not None, f"mutant {name} passed every pin"
