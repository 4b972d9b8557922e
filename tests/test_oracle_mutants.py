"""Plant plausible mistakes in a copy of the oracle and check that a pin fails.

Each mutant is a textual edit of oracle/ce_oracle.c compiled into a temporary
library on the CPU; the real oracle is never modified.  A mutant that every pin
lets through would mean the pins cannot tell that mistake from the truth.
"""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ce_oracle.c")

# (name, text in ce_oracle.c, replacement, expected number of occurrences)
MUTANTS = [
    ("loss_drops_smoothing_mass",
     "double q = or_q(smooth, alpha, V, j == tgt);\n        if (q != 0.0) loss -= q",
     "double q = (j == tgt ? 1.0 - alpha : 0.0);\n        if (q != 0.0) loss -= q", 1),
    ("loss_zero_weights_not_skipped", "if (q != 0.0) loss -= q * (or_elem(x, off + j) - lse);",
     "loss -= q * (or_elem(x, off + j) - lse);", 1),
    ("grad_sign_flipped", "gout[j] = s * (p - or_q(smooth, alpha, V, j == tgt));",
     "gout[j] = s * (or_q(smooth, alpha, V, j == tgt) - p);", 1),
    ("grad_target_off_by_one", "gout[j] = s * (p - or_q(smooth, alpha, V, j == tgt));",
     "gout[j] = s * (p - or_q(smooth, alpha, V, j == tgt + 1));", 1),
    ("grad_smoothing_conventions_confused", "gout[j] = s * (p - or_q(smooth, alpha, V, j == tgt));",
     "gout[j] = s * (p - or_q(OR_SMOOTH_OTHERS, alpha, V, j == tgt));", 1),
    ("smoothing_conventions_swapped", "if (smooth == OR_SMOOTH_OTHERS) return is_target",
     "if (smooth == OR_SMOOTH_ALL) return is_target", 1),
    ("uniform_share_over_v_minus_1", "return alpha / (double)V + (is_target",
     "return alpha / (double)(V - 1) + (is_target", 1),
    ("others_share_over_v", "alpha / (double)(V - 1) : 0.0);", "alpha / (double)V : 0.0);", 1),
    ("others_target_keeps_uniform_share", "return is_target ? 1.0 - alpha :",
     "return is_target ? 1.0 - alpha + alpha / (double)V :", 1),
    ("others_loss_over_v", "loss += alpha * other / (double)(V - 1);", "loss += alpha * other / (double)V;", 1),
    ("others_loss_counts_target", "if (j != tgt) other +=", "other +=", 1),
    ("row_strides_swapped", "return i0 * x->s0 + i1 * x->s1;", "return i0 * x->s1 + i1 * x->s0;", 1),
    ("target_strides_swapped", "return t->data[i0 * t->s0 + i1 * t->s1];", "return t->data[i0 * t->s1 + i1 * t->s0];", 1),
    ("no_max_shift", "s += exp(or_elem(x, off + j) - m);\n  return m + log(s);",
     "s += exp(or_elem(x, off + j));\n  return log(s);", 1),
    ("mean_divides_by_rows", "return s / (double)n_valid;", "return s / (double)nrows;", 1),
    ("mean_grad_ignores_n", "if (reduce == OR_REDUCE_MEAN) return g_scalar / (double)n_valid;",
     "if (reduce == OR_REDUCE_MEAN) return g_scalar;", 1),
    ("sum_grad_divides_by_n", "if (reduce == OR_REDUCE_SUM) return g_scalar;",
     "if (reduce == OR_REDUCE_SUM) return g_scalar / (double)n_valid;", 1),
    ("sum_loss_is_mean_over_rows", "  return s;\n}", "  return s / (double)nrows;\n}", 1),
    ("bf16_widened_wrong", "((const uint16_t*)x->data)[off] << 16;", "((const uint16_t*)x->data)[off] << 15;", 1),
    ("linear_bf16_widened_wrong", "((const uint16_t*)p)[off] << 16;", "((const uint16_t*)p)[off] << 15;", 1),
    ("combine_no_rescale", "D += st[1] * exp(st[0] - M);", "D += st[1];", 1),
    ("combine_drops_target_gather", "xt += st[2];", "xt = st[2];", 1),
    ("combine_forgets_target_term", "D += exp(xt - M); /* the target's term", "D += 0.0; /* the target's term", 1),
    ("shard_stats_keep_target_term", "if (o + j != tgt) d += exp(v - m);", "d += exp(v - m);", 1),
    ("combine_others_sign", "(R - xt)) / (double)(vocab_total - 1)", "(R + xt)) / (double)(vocab_total - 1)", 1),
    ("combine_ignores_convention", "if (smooth == OR_SMOOTH_OTHERS) {\n      double loss",
     "if (0) {\n      double loss", 1),
    ("shard_grad_uses_local_v", "or_q(smooth, alpha, Vt, o + j == tgt)", "or_q(smooth, alpha, V, o + j == tgt)", 1),
    ("shard_target_column_unshifted", "or_elem(x, off + (tgt - o))", "or_elem(x, off + tgt % V)", 1),
    ("ignored_row_not_zeroed", "loss_out[k] = 0.0;\n      if (lse_out) lse_out[k] = NAN;\n      continue;\n    }\n    if (tgt < 0 || tgt >= V)",
     "if (lse_out) lse_out[k] = NAN;\n    }\n    if (tgt < 0 || tgt >= V)", 1),
    ("count_counts_ignored", "if (or_target(t, d1, r) != ignore_idx) ++n;", "++n;", 1),
    ("linear_logits_unrounded", "if (round_mode == 1) {", "if (0) {", 1),
    ("linear_f32_rounded_to_bf16", "acc = dtype == OR_BF16 ? (double)or_round_bf16(f) : (double)f;",
     "acc = (double)or_round_bf16(f);", 1),
    ("linear_bf16_truncated", "u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;", "u = u & 0xffff0000u;", 1),
    ("linear_grad_unscaled", "x[j] = s * (exp(x[j] - lse) - or_q(smooth, alpha, V, j == tgt));",
     "x[j] = (exp(x[j] - lse) - or_q(smooth, alpha, V, j == tgt));", 1),
    ("linear_dh_sign", "dh_out[r * D + d] = acc;", "dh_out[r * D + d] = -acc;", 1),
    ("linear_dw_keeps_last_row", "acc += G[r * V + j] * or_load(h, dtype, r * h_ld + d);",
     "acc = G[r * V + j] * or_load(h, dtype, r * h_ld + d);", 1),
]


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_some_pin_catches(tmp_path, name, old, new, count):
    src = open(SRC).read()
    assert src.count(old) == count, f"mutation anchor for {name} not found {count}x"
    mutated = src.replace(old, new)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-I", os.path.dirname(SRC),
                    "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    orc = oracle.Oracle(oracle.load(str(so_path)))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, oracle.OracleError) as e:  # a pin failed: the mistake is seen
            caught.append((pin.__name__, str(e)[:80]))
            break
    assert caught, f"no pin catches mutant {name}"
