"""Planted mistakes in the oracle must fail at least one pin.

Each mutant is a one-line edit of a copy of oracle/moe_oracle.c (a dropped
term, a wrong sign, index or operand), compiled on the CPU into a temporary
library; the pins of tests/pins.py then run against it and at least one must
fail.  This shows that the pins would catch such a mistake in the oracle.
"""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

MUTANTS = {
    "tie_break_flipped": ("  return a < b;\n}", "  return a > b;\n}"),
    "router_bias_dropped": ("if (router_bias) acc = acc + router_bias[e];", "(void)router_bias;"),
    "router_chunk_dropped": ("        acc = acc + p;", "        acc = p;"),
    "renormalise_skipped": ("if (d->renormalize)\n", "if (0)\n"),
    "softmax_wrong_index": ("w[j] = expf(l[idx[j]] - m) / z;", "w[j] = expf(l[j] - m) / z;"),
    "nibble_order_reversed": ("(bits * (k % per))", "(bits * (per - 1 - k % per))"),
    "code_width_fixed_4": ("const int32_t per = 32 / bits;", "const int32_t per = 8;"),
    "group_size_fixed_64": ("const int32_t G = d->group_size;", "const int32_t G = 64;"),
    "gelu_cubic_dropped": ("(g + 0.044715f * g * g * g)", "(g)"),
    "geglu_runs_silu": ("    if (d->activation == 1) {\n      if (d->glu_round) {",
                        "    if (0) {\n      if (d->glu_round) {"),
    "geglu_grad_runs_silu": ("  if (d->activation == 1) {\n    const float a = 0.7978845608028654f",
                             "  if (0) {\n    const float a = 0.7978845608028654f"),
    "geglu_rounding_skipped": ("h[n] = round_act(d, round_act(d, gelu_tanh(g)) * u);", "h[n] = gelu_tanh(g) * u;"),
    "scale_bias_swapped": ("out[k] = s * (float)q + b;", "out[k] = b * (float)q + s;"),
    "group_index_wrong": ("float s = half_at(d, sc[(int64_t)(k / G) * N]);", "float s = half_at(d, sc[0]);"),
    "f16_exponent_bias": ("(int)e - 25", "(int)e - 24"),
    "swiglu_grad_dropped_term": ("*dg = dh * u * (s * (1.0f + g * (1.0f - s)));", "*dg = dh * u * s;"),
    "gelu_grad_cubic_coeff": ("a * (1.0f + 3.0f * b * g * g)", "a * (1.0f + b * g * g)"),
    "router_grad_dropped": ("dxr[k] = dxr[k] + a;", "dxr[k] = dxr[k] + 0.0f * a;"),
    "renorm_grad_mean_dropped": ("dl[idx[j]] = wt[j] * (dw[j] - dot);", "dl[idx[j]] = wt[j] * dw[j];"),
    "expert_grad_unweighted": ("glu_grad(d, g[n], u[n], c * dh[n], &dg, &du);", "glu_grad(d, g[n], u[n], dh[n], &dg, &du);"),
    "f16_subnormal_scale": ("ldexpf((float)m, -24)", "ldexpf((float)m, -25)"),
    "f16_scales_read_as_bf16": ("return d->act_f16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);",
                                "return d->act_f16 && 0 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);"),
    "fused_up_reads_gate": ("oracle_dequant_row(d, &w->gate_up, e, F + n, 2 * F, D, row);",
                            "oracle_dequant_row(d, &w->gate_up, e, n, 2 * F, D, row);"),
    "separate_gate_reads_up": ("oracle_dequant_row(d, &w->gate, e, n, F, D, row);",
                               "oracle_dequant_row(d, &w->up, e, n, F, D, row);"),
    "backward_up_reads_gate": ("    up_row(d, w, e, n, row);\n    for (int32_t k = 0; k < D; ++k) dxr[k]",
                               "    gate_row(d, w, e, n, row);\n    for (int32_t k = 0; k < D; ++k) dxr[k]"),
    "silu_sign": ("static float silu(float g) { return g / (1.0f + expf(-g)); }",
                  "static float silu(float g) { return g / (1.0f + expf(g)); }"),
    "sigmoid_not_rounded": ("float s = round_act(d, sigmoid(g));", "float s = sigmoid(g);"),
    "f16_layers_round_to_bf16": ("return d->act_f16 ? round_f16(f) : round_bf16(f);", "return round_bf16(f);"),
    "f16_ties_away": ("if (rem > half || (rem == half && (q & 1u))) q += 1u;", "if (rem >= half) q += 1u;"),
    "f16_subnormals_flushed": ("if (e < -14) return (uint16_t)(sign | q);", "if (e < -14) return sign;"),
    "dispatch_unstable": ("return i < j ? -1 : (i > j);", "return i < j ? 1 : -(i > j);"),
    "row_map_modulo": ("row_map[p] = order[p] / top_k;", "row_map[p] = order[p] % top_k;"),
    "tile_off_floor": ("(cnt + tile_rows - 1) / tile_rows", "cnt / tile_rows"),
    "shared_dropped": ("for (int32_t s = 0; s < d->n_shared; ++s) {", "for (int32_t s = 0; s < 0; ++s) {"),
    "slot_weight_wrong": ("yr[m] = yr[m] + wt[j] * o[m];", "yr[m] = yr[m] + wt[0] * o[m];"),
    "bf16_ties_away": ("u += 0x7fffu + lsb;", "u += 0x7fffu + 1u;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mpath = tmp_path / "moe_oracle.c"
    mpath.write_text(src.replace(old, new))
    (tmp_path / "moe_oracle.h").write_text(open(SRC[:-2] + ".h").read())
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", str(lib), str(mpath), "-lm"], check=True)
    failed = []
    with oracle.use_library(str(lib)):
        for pname, fn, args in pins.ALL_PINS:
            try:
                fn(*args)
            except AssertionError:
                failed.append(pname)
                break
    assert failed, f"mutant {name} passed every pin"
