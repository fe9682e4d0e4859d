"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutant is a textual edit of a copy of oracle/sol_oracle.c, compiled to a temporary library.
The edit must apply (the test fails loudly if the oracle's text changes under it), and the pins
of tests/oracle_pins.py must then catch it.  The real oracle is never modified.
"""
import os
import subprocess
import tempfile

import pytest

from oracle import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sol_oracle.c")

MUTANTS = {
    "pooled_logit_uses_ln_block": ("s[j] + log((double)(hi - lo))", "s[j] + log((double)block)"),
    "sample_std": ("sqrt(m2 / (double)M);\n\n", "sqrt(m2 / (double)(M - 1));\n\n"),
    "strict_threshold": ("else sel[j] = s[j] >= t;", "else sel[j] = s[j] > t;"),
    "select_strict_threshold": ("if (s[j] >= t) mask[i * W + j / 32]", "if (s[j] > t) mask[i * W + j / 32]"),
    "pool_divides_by_block": ("xbar[j * d + c] = sum / n;", "xbar[j * d + c] = sum / (double)block;"),
    "proxy_without_scale": ("s[j] = dot(qi, kbar + j * d, d) * inv_sqrt_d;\n\n        /* Step 2",
                            "s[j] = dot(qi, kbar + j * d, d);\n\n        /* Step 2"),
    "threshold_sign": ("else t = m1 + beta * sd;", "else t = m1 - beta * sd;"),
    "pooled_value_is_kbar": ("acc[c] += w * vbar[j * d + c];", "acc[c] += w * kbar[j * d + c];"),
    "pooled_tokens_dropped": ("} else if (!drop) {\n            double w", "} else if (0) {\n            double w"),
    "exact_logit_unscaled": ("double w = exp(dotf(qi, k + kk * d, d) * inv_sqrt_d - mx);",
                             "double w = exp(dotf(qi, k + kk * d, d) - mx);"),
    "exact_value_transposed": ("acc[c] += w * (double)v[kk * d + c];", "acc[c] += w * (double)k[kk * d + c];"),
    "mean_off_by_one": ("m1 /= (double)M;\n        double m2 = 0.0;\n        for (int64_t j = 0; j < M; ++j) m2 += (s[j] - m1) * (s[j] - m1);\n        double sd = sqrt(m2 / (double)M);\n\n",
                        "m1 /= (double)(M + 1);\n        double m2 = 0.0;\n        for (int64_t j = 0; j < M; ++j) m2 += (s[j] - m1) * (s[j] - m1);\n        double sd = sqrt(m2 / (double)M);\n\n"),
    "last_block_short": ("return hi < N ? hi : N;", "return hi < N ? hi : N - 1;"),
    "route_ties_high_index_first": ("return (x->j > y->j) - (x->j < y->j);",
                                    "return (x->j < y->j) - (x->j > y->j);"),
    "topp_without_block_size": ("if (mode == 1) sj += log(", "if (mode == 2) sj += log("),
    "topp_counts_blocks_not_mass": ("w[r] = exp(it[r].key - it[0].key);", "w[r] = 1.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found in the oracle source"
    mutated = src.replace(old, new)
    path = tmp_path / "mut.c"
    path.write_text(mutated)
    lib_path = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", *oracle.CFLAGS, str(path), "-o", lib_path, "-lm"], check=True)
    lib = oracle.load(lib_path)
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
