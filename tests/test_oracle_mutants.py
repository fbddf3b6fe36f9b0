"""Plants plausible mistakes in a copy of the oracle's C source and checks
that the pins catch every one (no GPU; the oracle source itself is untouched).
"""
import os
import shutil

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("router_drops_bias", "z[e] = acc + (bias ? (double)bias[e] : 0.0);", "z[e] = acc;"),
    ("router_reversed_index", "acc += bf(xt[h]) * bf(w[h]);", "acc += bf(xt[h]) * bf(w[H - 1 - h]);"),
    ("select_smallest", "return z[a] > z[b] || (z[a] == z[b] && a < b);",
     "return z[a] < z[b] || (z[a] == z[b] && a < b);"),
    ("tie_to_higher_index", "return z[a] > z[b] || (z[a] == z[b] && a < b);",
     "return z[a] > z[b] || (z[a] == z[b] && a > b);"),
    ("silu_wrong_sign", "static double silu(double v) { return v / (1.0 + exp(-v)); }",
     "static double silu(double v) { return v / (1.0 + exp(v)); }"),
    ("gate_used_as_up", "const uint16_t* u = w13 + (size_t)(n + i) * H;",
     "const uint16_t* u = w13 + (size_t)i * H;"),
    ("down_reversed_index", "acc += bf(row[i]) * hbuf[i];", "acc += bf(row[n - 1 - i]) * hbuf[i];"),
    ("no_residual", "o[r] = c->add_residual ? bf(xt[r]) : 0.0;", "o[r] = 0.0;"),
    ("no_shared_expert", "if (Is > 0) {\n            swiglu_ffn", "if (0) {\n            swiglu_ffn"),
    ("sigmoid_not_renormalised", "c->renormalize ? sigm(z[idx[j]]) / den : sigm(z[idx[j]]);",
     "sigm(z[idx[j]]);"),
    ("no_routed_scale", "for (int j = 0; j < k; ++j) w[j] *= c->routed_scale;", ""),
    ("softmax_over_all_experts_when_renormalised",
     "for (int j = 0; j < k; ++j) den += exp(z[idx[j]] - m);",
     "for (int e = 0; e < E; ++e) den += exp(z[e] - m);"),
    ("weights_unsorted_to_experts", "o[r] += wt[j] * y[r];", "o[r] += wt[k - 1 - j] * y[r];"),
]


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, orig, mut):
    src = open(SRC).read()
    assert src.count(orig) == 1, "mutation anchor not found once: %s" % name
    msrc = tmp_path / "moe_oracle_mut.c"
    msrc.write_text(src.replace(orig, mut))
    lib = oracle.build(force=True, src=str(msrc), dst=str(tmp_path / "libmut.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, KeyError, RuntimeError) as e:
            caught.append(check.__name__)
    assert caught, "no pin caught the planted mistake %s" % name
