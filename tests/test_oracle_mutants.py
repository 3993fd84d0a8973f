"""Plants one plausible mistake at a time in a copy of the oracle's C source
(CPU only), builds it, and runs the oracle pins against it: each mutant must
fail at least one pin, so a mistake of that kind in the oracle itself would not
go unnoticed.  The mutated copies live in a temporary folder; the oracle
package loads one through MOE_ORACLE_LIB."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

# (name, text in moe_oracle.c, replacement, pin tests expected to catch it)
MUTANTS = [
    ("gate_up_swapped",
     "g += elem(w13, (size_t)f * d + i, dtype) * x[i];\n            u += elem(w13, (size_t)(d_ff + f) * d + i, dtype) * x[i];",
     "u += elem(w13, (size_t)f * d + i, dtype) * x[i];\n            g += elem(w13, (size_t)(d_ff + f) * d + i, dtype) * x[i];",
     "test_oracle_pins.py::test_expert_ffn_matches_dense"),
    ("w2_transposed",
     "acc += elem(w2, (size_t)o * d_ff + f, dtype) * h[f];",
     "acc += elem(w2, (size_t)f * d + o, dtype) * h[f];",
     "test_oracle_pins.py::test_expert_ffn_matches_dense"),
    ("ties_to_higher_index",
     "if (ok[i] && (b < 0 || key[i] > key[b]))",
     "if (ok[i] && (b < 0 || key[i] >= key[b]))",
     "test_oracle_pins.py::test_tie_break_lower_index_and_zero_denominator"),
    ("bias_dropped",
     "key[i] = bias ? s[i] + bias[i] : s[i];",
     "key[i] = s[i];",
     "test_oracle_pins.py::test_group_limited_routing_worked_example"),
    ("group_score_largest_key_only",
     "for (int r = 0; r < group_topk; ++r) {",
     "for (int r = 0; r < 1; ++r) {",
     "test_oracle_pins.py::test_group_limited_routing_worked_example"),
    ("gates_not_renormalised",
     "gates[j] = (sum > 0.0) ? (float)(g[j] / sum) : (float)(1.0 / k);",
     "gates[j] = (float)g[j];",
     "test_oracle_pins.py::test_router_worked_example"),
    ("tokens_descending_in_expert",
     "for (int t = 0; t < T; ++t)\n            for (int j = 0; j < k; ++j)\n                if (ids[(size_t)t * k + j] == e) {",
     "for (int t = T - 1; t >= 0; --t)\n            for (int j = 0; j < k; ++j)\n                if (ids[(size_t)t * k + j] == e) {",
     "test_oracle_pins.py::test_dispatch_combine_toy"),
]


@pytest.mark.parametrize("name, old, new, pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_its_pin(tmp_path, name, old, new, pin):
    src = open(SRC).read()
    assert src.count(old) == 1, "the text to mutate must occur exactly once"
    mutant = tmp_path / "moe_oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-o", str(lib),
                    str(mutant), "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    # the pin (which passes on the oracle as it is, in the rest of this suite)
    # fails on the mutant
    bad = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", pin)], cwd=ROOT, capture_output=True,
                         text=True, env=env)
    assert bad.returncode == 1, "mutant %s passed %s:\n%s" % (name, pin, bad.stdout[-2000:])
