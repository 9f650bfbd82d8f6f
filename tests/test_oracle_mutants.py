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
    ("greedy_emits_draft", "for (int i = 0; i <= best_a; ++i) out[i] = argmax_row(target, dtype, row0 + i * stride, V);",
     "for (int i = 0; i <= best_a; ++i) out[i] = i < best_a ? x[best_c * k + i] : 0;"),
    ("ragged_target_offset", "const int64_t t0 = (int64_t)cu[b] + b, d0 = cu[b];",
     "const int64_t t0 = (int64_t)cu[b], d0 = cu[b];"),
    ("ragged_greedy_offset", "((int64_t)cu[b] + b) * row_stride, accept_len + b, out, NULL, NULL);",
     "((int64_t)cu[b]) * row_stride, accept_len + b, out, NULL, NULL);"),
    ("sample_last_tie_argmax", "tokens[b] = argmax_row(logits, dtype, (int64_t)b * row_stride, V);",
     "tokens[b] = V - 1 - argmax_row(logits, dtype, (int64_t)b * row_stride, V);"),
    ("sample_no_temperature", "softmax_row(logits, dtype, (int64_t)b * row_stride, V, temperature, p);",
     "softmax_row(logits, dtype, (int64_t)b * row_stride, V, 1.0, p);"),
    ("token_row_offset", "return ((int64_t)b * (k + 1) + i) * stride;",
     "return ((int64_t)b * k + i) * stride;"),
    ("softmax_no_max_shift", "prob[v] = exp((logit(base, dtype, row_off + v) - M) / tau);",
     "prob[v] = exp(logit(base, dtype, row_off + v) / tau) + 0.0 * M;"),
    ("tree_ignores_parent_acceptance", "            if (acc[pj]) {", "            if (1) {"),
    ("tree_argmax_of_own_row",
     "const int g = argmax_row(target, dtype, ((int64_t)b * N + pj) * row_stride, V);",
     "const int g = argmax_row(target, dtype, ((int64_t)b * N + j) * row_stride, V);"),
    ("tree_last_tie", "if (acc[j] && depth[j] > depth[best]) best = j;",
     "if (acc[j] && depth[j] >= depth[best]) best = j;"),
    ("tree_bonus_from_parent",
     "out_t[d] = argmax_row(target, dtype, ((int64_t)b * N + best) * row_stride, V);",
     "out_t[d] = argmax_row(target, dtype, ((int64_t)b * N + (best ? par[best] : 0)) * row_stride, V);"),
    ("commit_drops_extra_token", "for (int j = 0; j <= a && L < capacity; ++j) h[L++] = t[j];",
     "for (int j = 0; j < a && L < capacity; ++j) h[L++] = t[j];"),
    ("commit_next_is_last_draft", "next_token[(int64_t)b * next_stride] = t[a];",
     "next_token[(int64_t)b * next_stride] = t[a > 0 ? a - 1 : 0];"),
    ("commit_ignores_capacity", "for (int j = 0; j <= a && L < capacity; ++j) h[L++] = t[j];",
     "for (int j = 0; j <= a && L < history_stride; ++j) h[L++] = t[j];"),
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
