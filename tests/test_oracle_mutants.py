"""Every planted mistake in the oracle must be caught by at least one pin.

A mutant is a copy of oracle/oracle.c with one piece of its text replaced by a
plausible mistake; the copy is compiled and every pin of tests/pins.py runs on
it, and at least one must fail.  The oracle's own source carries no hooks for
this: each mutant names the exact text it replaces, which must occur exactly
once."""
import os

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "nibble_order": ("            int code = (c & 1) ? (byte >> 4) : (byte & 0xF);",
                     "            int code = (c & 1) ? (byte & 0xF) : (byte >> 4);"),
    "silu_on_w3": ("\n            double a = G / (1.0 + exp(-G)) * U;",
                   "\n            double a = U / (1.0 + exp(-U)) * G;"),
    "scale_bias_126": ("return ldexp(1.0, e - 127);", "return ldexp(1.0, e - 126);"),
    "one_scale_per_row": ("oracle_ue8m0(s[(size_t)r * (cols / 32) + g]);",
                          "oracle_ue8m0(s[(size_t)r * (cols / 32) + 0]);"),
    "ties_to_higher_index": ("return (x->e < y->e) ? -1 : (x->e > y->e);",
                             "return (x->e > y->e) ? -1 : (x->e < y->e);"),
    "softmax_over_all_experts": (
        "        for (int j = 0; j < k; ++j) gates[(size_t)t * k + j] = (float)(ex[j] / den);",
        "        for (int j = k; j < E; ++j) den += exp((double)keys[j].v - l0);\n"
        "        for (int j = 0; j < k; ++j) gates[(size_t)t * k + j] = (float)(ex[j] / den);"),
    "no_gate": ("double gj = (double)g[p];", "double gj = 1.0;"),
    "w2_transposed": (
        "            decode_row(w2, s2, I, m, r2);\n"
        "            for (int n = 0; n < I; ++n) acc += hv[n] * r2[n];",
        "            for (int n = 0; n < I; ++n) {\n"
        "                uint8_t b_ = w2[(size_t)n * (H / 2) + (m >> 1)];\n"
        "                int c_ = (m & 1) ? (b_ >> 4) : (b_ & 0xF);\n"
        "                acc += hv[n] * oracle_e2m1(c_) * oracle_ue8m0(s2[(size_t)n * (H / 32) + (m >> 5)]);\n"
        "            }"),
    "h_not_rounded": ("hv[n] = oracle_bf16_to_double(h[n]);", "hv[n] = a;"),
    "last_column_dropped": ("    for (int c = 0; c < K; ++c) {\n        if (B > 0",
                            "    for (int c = 0; c < K - 1; ++c) {\n        if (B > 0"),
    "subnormal_1": ("(E == 0) ? 0.5 * m", "(E == 0) ? 1.0 * m"),
    "sign_ignored": ("    return s ? -mag : mag;", "    return mag;"),
    "mx8_scale_exponent": ("se = (e - 1) - 8 + 127;", "se = (e - 1) - 8 + 128;"),
    "fp8_not_saturated": ("    if (q > 448.0) q = 448.0;\n", ""),
    "fp8_sign_dropped": ("int s = signbit(r) ? 1 : 0;", "int s = 0;"),
    "fp8_ties_away": ("q = nearbyint(a / quantum) * quantum;", "q = round(a / quantum) * quantum;"),
    "router_last_input_dropped": (
        "            for (int c = 0; c < H; ++c) {\n"
        "                const double xv = oracle_bf16_to_double(x[(size_t)t * H + c]);\n"
        "                const double wv",
        "            for (int c = 0; c < H - 1; ++c) {\n"
        "                const double xv = oracle_bf16_to_double(x[(size_t)t * H + c]);\n"
        "                const double wv"),
    "router_weight_transposed": ("oracle_bf16_to_double(wr[(size_t)e * H + c]);",
                                 "oracle_bf16_to_double(wr[((size_t)c * E + e) % ((size_t)E * H)]);"),
    "saliency_norm_misses_a_row": ("for (int m = 0; m < H; ++m) ss += Y[m] * Y[m];",
                                   "for (int m = 0; m < H - 1; ++m) ss += Y[m] * Y[m];"),
    "saliency_without_gate": ("sal[i] += (double)g[p] * sqrt(ss);", "sal[i] += sqrt(ss);"),
    "shared_block_scale_transposed": ("const int si = (r / 32) * (cols / 32) + c / 32;",
                                      "const int si = (c / 32) * (cols / 32) + r / 32;"),
    "shared_w2_transposed": ("acc += hv[n] * fp8w(w2, s2, I, m, n);",
                             "acc += hv[n] * fp8w(w2, s2, I, n % H, m % I);"),
    "hbound_without_U_term": (
        "const double e = M * dG * (fabs(U) + dU) + fabs(silu) * dU;",
        "const double e = M * dG * (fabs(U) + dU);"),
    "hbound_without_G_term": (
        "const double e = M * dG * (fabs(U) + dU) + fabs(silu) * dU;",
        "const double e = fabs(silu) * dU;"),
    "hbound_gamma_of_I": ("hbound[n] = h_bound(G, U, acc_bound(am, H, Ga, Gp), acc_bound(am, H, Ua, Up));",
                          "hbound[n] = h_bound(G, U, acc_bound(am, I, Ga, Gp), acc_bound(am, I, Ua, Up));"),
    "hbound_prefix_mass_dropped": ("        if (B > 0 && c > 0 && c % B == 0) pm += fabs(s);\n", ""),
    "stack_without_residual": ("x[i] = (float)((double)x[i] + (double)y[i]);", "x[i] = y[i];"),
    "stack_adds_normed_input": ("x[i] = (float)((double)x[i] + (double)y[i]);",
                                "x[i] = (float)(oracle_bf16_to_double(u[i]) + (double)y[i]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutant {name}: the text it replaces occurs {text.count(old)} times"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(text.replace(old, new))
    o = oracle.Oracle(oracle.build(str(tmp_path / f"liboracle_{name}.so"), src=str(src)))
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            return  # caught
    pytest.fail(f"mutant {name} passes every pin")
