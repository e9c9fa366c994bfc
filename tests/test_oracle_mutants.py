"""Plant plausible mistakes in a copy of the oracle's C source and check that
the pin battery catches every one.

This shows the pins are strong enough: a dropped term, a wrong sign or index,
a transposed operand, each makes some pin fail.  The mutants are built in a
temporary directory on the CPU; the real oracle is never modified.
"""
import os
import tempfile

import pytest

import oracle
from oracle_pins import ALL_PINS

# (name, anchor text in fff_oracle.c, replacement)
MUTANTS = [
    ("direction_swapped", "go_right = !(a < 0.0);", "go_right = (a < 0.0);"),
    ("zero_goes_left", "go_right = !(a < 0.0);", "go_right = (a > 0.0);"),
    ("bias_dropped", "double a = dot(xt, w, d) + bp[n];", "double a = dot(xt, w, d);"),
    ("leaf_not_evaluated",
     "for (int level = 0; level <= D; ++level) {\n        const double *w = Wp + n * (int64_t)d;",
     "for (int level = 0; level < D; ++level) {\n        const double *w = Wp + n * (int64_t)d;"),
    ("gelu_cubic_term_dropped", "k0 * (a + k1 * a * a * a)", "k0 * (a + k1 * a * a)"),
    ("gelu_half_dropped", "return 0.5 * a * (1.0 + tanh(", "return a * (1.0 + tanh("),
    ("child_index_off_by_one", "n = 2 * n + 1 + go_right;", "n = 2 * n + go_right;"),
    ("v_row_by_level", "const double *v = Vp + n * (int64_t)h;",
     "const double *v = Vp + level * (int64_t)h;"),
    ("outputs_not_summed", "acc[j] += g * v[j];", "acc[j] = g * v[j];"),
    ("concat_order_reversed", "alive ? alive + p * N : NULL, Ht + (int64_t)p * h,",
     "alive ? alive + p * N : NULL, Ht + (int64_t)(P - 1 - p) * h,"),
    ("projection_transposed", "yt[c] += hk * wk[c];", "yt[c] += hk * Wout[(int64_t)c * K + k];"),
    ("path_is_node_id", "return (int32_t)(n - (((int64_t)1 << D) - 1));", "return (int32_t)n;"),
    ("forced_bits_reversed", "go_right = (forced_leaf >> (D - 1 - level)) & 1;",
     "go_right = (forced_leaf >> level) & 1;"),
    ("threshold_without_x_norm", "rec_thr[level] = 1e-4 * xnorm * sqrt(dot(w, w, d));",
     "rec_thr[level] = 1e-4 * sqrt(dot(w, w, d));"),
    ("post_gelu_on_each_node", "double g = variant == 1 ? a : gelu_tanh(a);",
     "double g = gelu_tanh(a);"),
    ("post_final_gelu_dropped", "acc[j] = gelu_tanh(acc[j]);", "acc[j] = acc[j];"),
    ("prune_mask_ignored", "if (alive && !alive[2 * n + 1 + go_right])",
     "if (0 && alive && !alive[2 * n + 1 + go_right])"),
    ("prune_alive_is_and", "alive[n] = alive[2 * n + 1] | alive[2 * n + 2];",
     "alive[n] = alive[2 * n + 1] & alive[2 * n + 2];"),
    ("prune_forced_step_always_right", "                    go_right = !go_right;",
     "                    go_right = 1;"),
    ("prune_leaves_reversed", "alive[first_leaf + i] = leaf_alive[i] != 0;",
     "alive[first_leaf + i] = leaf_alive[first_leaf - i] != 0;"),
    ("bwd_gelu_grad_cubic_dropped", "(1.0 + 3.0 * k1 * a * a)", "(1.0)"),
    ("bwd_dv_weight_is_logit", ": gelu_tanh(a) * dHp[j];", ": a * dHp[j];"),
    ("bwd_dx_without_da", "dxt[c] += dal * w[c];", "dxt[c] += w[c];"),
    ("bwd_dwout_columns_reversed", "row[c] += hk * dyt[c];", "row[c] += hk * dyt[d - 1 - c];"),
    ("bwd_post_ds_without_gelu_grad",
     "const double dj = variant == 1 ? gelu_tanh_grad(Sp[j]) * dHp[j] : dHp[j];",
     "const double dj = dHp[j];"),
    ("post_variant_ignored", "if (variant == 1)\n", "if (0)\n"),
]


def _caught(lib):
    failures = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except Exception:  # a wrong value, a rejected valid input, or unusable output
            failures.append(pin.__name__)
    return failures


@pytest.mark.parametrize("name,anchor,replacement", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, anchor, replacement):
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(anchor) == 1, f"anchor for {name} must occur exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, f"mutant_{name}.c")
        with open(path, "w") as f:
            f.write(src.replace(anchor, replacement))
        so = oracle.compile_oracle(path, os.path.join(tmp, f"libmutant_{name}.so"))
        lib = oracle.load(so)
        failures = _caught(lib)
    assert failures, f"no pin caught mutant {name}"
