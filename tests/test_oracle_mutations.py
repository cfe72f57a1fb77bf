"""Planted mistakes in the oracle, on the CPU: each edit below is a plausible
slip (a dropped term, a wrong sign or index, a transposed operand, a wrong
constant, a wrong tie rule).  Every edited build must fail at least one of the
oracle's pins, which shows the pins are strong enough to trust the oracle.

Every edit keeps all memory accesses in bounds, so a broken build fails a
check instead of crashing the test process.
"""
import os
import subprocess

import pytest

from oracle import oracle as O
from tests import oracle_pins as P

MUTANTS = {
    "swap_gate_up": ("double g = gu[i], u = gu[I + i];", "double g = gu[I + i], u = gu[i];"),
    "silu_sign": ("return z / (1.0 + exp(-a * z));", "return z / (1.0 + exp(a * z));"),
    "alpha_ignored": ("return z / (1.0 + exp(-a * z));", "return z / (1.0 + exp(-z));"),
    "clamp_up_one_side": ("u = u < -L_ ? -L_ : (u > L_ ? L_ : u);", "u = u > L_ ? L_ : u;"),
    "clamp_gate_both_sides": ("g = g < L_ ? g : L_;", "g = g < -L_ ? -L_ : (g > L_ ? L_ : g);"),
    "clamp_swapped": ("g = g < L_ ? g : L_;\n            u = u < -L_ ? -L_ : (u > L_ ? L_ : u);",
                      "u = u < L_ ? u : L_;\n            g = g < -L_ ? -L_ : (g > L_ ? L_ : g);"),
    "nongated_times_self": ("act[i] = or_silu_a(gu[i], L->act_alpha);",
                            "act[i] = or_silu_a(gu[i], L->act_alpha) * gu[i];"),
    "weight_on_input_and_output": ("out[h] += (L->weight_on_input ? 1.0 : w[k]) * s->y[h];",
                                   "out[h] += w[k] * s->y[h];"),
    "weight_on_input_ignored": ("s->xw[h] = w[k] * s->x[h];", "s->xw[h] = s->x[h];"),
    "router_gate_transposed": ("(double)((const float *)gate)[e * H + h]",
                               "(double)((const float *)gate)[h * E + e]"),
    "router_dropped_term": ("for (int64_t h = 0; h < H; h++) {\n                double x = x_dtype",
                            "for (int64_t h = 1; h < H; h++) {\n                double x = x_dtype"),
    "sigmoid_sign": ("score[e] = 1.0 / (1.0 + exp(-(double)l[e]));",
                     "score[e] = 1.0 / (1.0 + exp((double)l[e]));"),
    "no_renormalize": ("w[k] /= denom;", "w[k] /= 1.0;"),
    "no_rsf": ("w[k] *= rsf;", "w[k] *= 1.0;"),
    "bias_in_weight": ("w[k] = score[be];", "w[k] = key[be];"),
    "group_score_max_only": ("gscore[j] = (bias && per >= 2) ? best1 + best2 : best1;",
                             "gscore[j] = best1;"),
    "tie_to_higher": ("if (eligible[e] && !taken[e] && (be < 0 || key[e] > key[be]))",
                      "if (eligible[e] && !taken[e] && (be < 0 || key[e] >= key[be]))"),
    # a total order that ranks -0 below +0 (as an integer key of the raw
    # bits would), for experts and for groups
    "neg_zero_below_pos_zero": (
        "if (eligible[e] && !taken[e] && (be < 0 || key[e] > key[be]))",
        "if (eligible[e] && !taken[e] && (be < 0 || key[e] > key[be] ||"
        " (key[e] == key[be] && signbit(key[be]) && !signbit(key[e]))))"),
    "neg_zero_group_below_pos_zero": (
        "if (!gkeep[j] && (bj < 0 || gscore[j] > gscore[bj]))",
        "if (!gkeep[j] && (bj < 0 || gscore[j] > gscore[bj] ||"
        " (gscore[j] == gscore[bj] && signbit(gscore[bj]) && !signbit(gscore[j]))))"),
    "strided_groups":("eligible[e] = gkeep[e / per];", "eligible[e] = gkeep[e % G];"),
    "unstable_permutation": ("int64_t r = cursor[ids[i]]++;",
                             "int64_t r = offsets[ids[i]] + offsets[ids[i] + 1] - 1 - cursor[ids[i]]++;"),
    "shared_scaled_by_rsf": ("            out[h] += s->y[h];",
                             "            out[h] += L->routed_scaling_factor * s->y[h];"),
    "shared_uses_routed_I": ("or_expert_mlp(L, or_shared_I(L), L->shared_w13",
                             "or_expert_mlp(L, L->I, L->shared_w13"),
    "combine_wrong_weight": ("(L->weight_on_input ? 1.0 : w[k]) * s->y[h];",
                             "(L->weight_on_input ? 1.0 : w[0]) * s->y[h];"),
    "w13_transposed": ("acc += x[h] * or_weight(w13, s13, L->w_dtype, H, n, h);",
                       "acc += x[h] * or_weight(w13, s13, L->w_dtype, N1, h, n);"),
    "w2_transposed": ("acc += act[i] * or_weight(w2, s2, L->w_dtype, I, h, i);",
                      "acc += act[i] * or_weight(w2, s2, L->w_dtype, H, i, h);"),
    "e4m3_exponent_bias": ("mag = ldexp(1.0 + m / 8.0, e - 7);", "mag = ldexp(1.0 + m / 8.0, e - 8);"),
    "e4m3_subnormal_scale": ("mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    "e4m3_ties_down": ("best = ((c - 1) & 1) ? c : c - 1; /* tie: even code */", "best = c - 1;"),
    "fnuz_max": ("scale = fmaxf(amax, 1e-10f) / 448.0f;", "scale = fmaxf(amax, 1e-10f) / 240.0f;"),
    "no_act_quant": ("    if (L->act_fp8) {\n        for (int64_t i = 0; i < I; i++)",
                     "    if (0) {\n        for (int64_t i = 0; i < I; i++)"),
    "no_input_quant": ("    if (L->act_fp8) {\n        or_quant_fp8_groups(1, H, 128",
                       "    if (0) {\n        or_quant_fp8_groups(1, H, 128"),
    "bf16_shift": ("uint32_t u = (uint32_t)v << 16;", "uint32_t u = (uint32_t)v << 15;"),
    "block_scale_index": ("return q * (double)scale[(n / 128) * kb + (k / 128)];",
                          "return q * (double)scale[(k / 128) * kb + (n / 128)];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(O.SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %s" % name
    mutated = tmp_path / "moe_oracle.c"
    mutated.write_text(src.replace(old, new))
    hdr = os.path.join(os.path.dirname(O.SRC), "moe_oracle.h")
    (tmp_path / "moe_oracle.h").write_text(open(hdr).read())
    so = tmp_path / ("libmut_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                           str(mutated), "-o", str(so), "-lm"])
    lib_ = O.load_variant(str(so))
    for check in P.ALL_CHECKS:
        try:
            check(lib_=lib_)
        except (AssertionError, ValueError):
            return  # caught
    pytest.fail("planted mistake %r passed every pin" % name)
