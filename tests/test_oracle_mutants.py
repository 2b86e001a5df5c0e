"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of ``oracle/oracle.c`` (a temperature applied the wrong
way, noise with the wrong sign or the wrong key, a reversed inverse CDF, a dropped term, a transposed
operand, a wrong tie rule, ...), builds the copy in a temporary directory and runs the oracle's pins
(``tests/test_oracle.py``) against it in a child process.  The pins must fail for every mutant: a mutant that
survives names a part of the oracle that nothing pins.  The mistakes live only in the temporary copies.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, mutated text): the first occurrence is replaced
MUTANTS = [
    ("sample-mass-l-times-T", "S += exp(l[ord[i1++]] / T - M)", "S += exp(l[ord[i1++]] * T - M)"),
    ("sample-noise-sign", "log(S) + oracle_gumbel(", "log(S) - oracle_gumbel("),
    ("sample-race-noise-id", "(uint32_t)(2 * q));", "(uint32_t)(q));"),
    ("sample-target-noise-id", "(uint32_t)(2 * J + 1));", "(uint32_t)(2 * J));"),
    ("sample-reversed-cdf", "const double target = u * SJ;", "const double target = (1.0 - u) * SJ;"),
    ("sample-block-of-8", "static int block_of(int32_t id) { return id / 16; }",
     "static int block_of(int32_t id) { return id / 8; }"),
    ("sample-mass-ignores-max", "double pv = exp(l[ord[i]] / T - M);", "double pv = exp(l[ord[i]] / T);"),
    ("sample-logprob-no-T", "out->logprob = l[tok] / T - out->lse;", "out->logprob = l[tok] - out->lse;"),
    ("sample-lse-drops-a-block", "        total += S;\n        if (S > 0.0) {", "        if (S > 0.0) {"),
    ("greedy-ties-to-higher-id", "if (best < 0 || l[s] > k1) {", "if (best < 0 || l[s] >= k1) {"),
    ("greedy-lse-no-max", "total += exp(l[s] - M);", "total += exp(l[s]);"),
    ("reach-race-too-tight", "kf >= kf_other - 2.0 * eps", "kf >= kf_other - 0.2 * eps"),
    ("reach-greedy-too-tight", "(l[fslot] >= k1 - 2.0 * eps)", "(l[fslot] >= k1 - 0.2 * eps)"),
    ("bias-transposed-w2", "bias += x[j] * w2_at(W2, dtype, layout, V, r, j, v);",
     "bias += x[j] * w2_at(W2, dtype, 1 - layout, V, r, j, v);"),
    ("bias-drops-last-term", "for (int j = 0; j < r; ++j) bias +=", "for (int j = 0; j + 1 < r; ++j) bias +="),
    ("gate-dropped", "x[j] = Hk ? w * Hk[j] : w;", "x[j] = w;"),
    ("chain-ignores-anchor", "        int prev = anchor[b];\n        for (int k = 0; k < K; ++k) {\n            const float* Uk",
     "        int prev = 0;\n        for (int k = 0; k < K; ++k) {\n            const float* Uk"),
    ("topk-ties-to-higher-id", "return ia < ib;", "return ia > ib;"),
    ("selector-table-predecessor", "int a = (t == 0) ? anchor[b] : cand[(size_t)(t - 1) * topk + i];",
     "int a = (t == 0) ? anchor[b] : cand[(size_t)t * topk + i];"),
    ("gate-sigmoid-sign", "H[(size_t)i * r + j] = 1.0 / (1.0 + exp(-z));", "H[(size_t)i * r + j] = 1.0 / (1.0 + exp(z));"),
    ("noise-uniform-offset", "return (2.0 * (double)(h >> 9) + 1.0) / 16777216.0;", "return (2.0 * (double)(h >> 9) + 0.5) / 16777216.0;"),
    ("confidence-predecessor", "const int prev = (k == 0) ? anchor[b] : tokens[(size_t)b * K + k - 1];",
     "const int prev = (k == 0) ? anchor[b] : tokens[(size_t)b * K + k];"),
    ("schedule-non-strict", "if (!(t2 > theta)) break;", "if (!(t2 >= theta)) break;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert old in text, f"mutation site of {name} not found in oracle.c"
    so = str(tmp_path / "liboracle_mutant.so")
    c = tmp_path / "oracle_mutant.c"
    c.write_text(text.replace(old, new, 1))
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                    str(c), "-o", so, "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_PATH=so, OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"), "-x", "-q",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"mutant {name} survived every pin:\n{res.stdout[-2000:]}"
