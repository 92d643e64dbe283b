"""Planted mistakes in the oracle, on the CPU: each mutant is a copy of oracle.c with one
plausible slip (a dropped term, a wrong sign, index or comparison, a transposed operand).
The pins must reject every one of them; a mutant that passes every pin would mean the pins
cannot tell that mistake from the correct oracle."""
import os
import subprocess

import pytest

import oracle
import oracle.oracle as orc
import pins

SRC = os.path.join(os.path.dirname(orc.__file__), "oracle.c")

# (name, text to replace, replacement, which occurrence: 0 = first)
MUTANTS = [
    ("forward_drops_b_a", "      a += b_a ? (double)b_a[i] : 0.0;\n      double h", "      double h", 0),
    ("forward_relu_on_product", "        h = h * u;", "        h = (a * u > 0.0) ? a * u : 0.0;", 0),
    ("forward_transposed_w_o", "y[j] += h * elem(Wo, w_dtype, (size_t)i * d + j)",
     "y[j] += h * elem(Wo, w_dtype, (size_t)j * n + i)", 0),
    ("forward_drops_b_o", "    if (b_o)\n", "    if (0 && b_o)\n", 0),
    ("forward_gate_for_up", "u += elem(Wu, w_dtype,", "u += elem(Wa, w_dtype,", 0),
    ("forward_tokmask_inverted", "if (tokmask && !((tokmask[k] >> b) & 1)) continue;",
     "if (tokmask && ((tokmask[k] >> b) & 1)) continue;", 0),
    ("forward_relu_ge", "      double h = (a > 0.0) ? a : 0.0;", "      double h = (a >= -1e-3) ? a : 0.0;", 0),
    ("dense_drops_last_neuron", "    for (int32_t i = 0; i < n; ++i) {\n      double a = 0.0;",
     "    for (int32_t i = 0; i < n - 1; ++i) {\n      double a = 0.0;", 0),
    ("threshold_not_strict", "M[k] = (S[k] > tau) ? 1 : 0;", "M[k] = (S[k] >= tau) ? 1 : 0;", 0),
    ("threshold_nan_active", "M[k] = (S[k] > tau) ? 1 : 0;", "M[k] = !(S[k] <= tau) ? 1 : 0;", 0),
    ("compact_skips_first", "  for (int32_t i = 0; i < n; ++i) {\n    uint64_t bits",
     "  for (int32_t i = 1; i < n; ++i) {\n    uint64_t bits", 0),
    ("compact_bit_order", "bits |= (uint64_t)1 << b;", "bits |= (uint64_t)1 << (B - 1 - b);", 0),
    ("predict_transposed_p2", "elem(P2, p_dtype, (size_t)i * r + j)", "elem(P2, p_dtype, (size_t)j * n + i)", 0),
    ("predict_drops_c", "S[(size_t)b * n + i] = acc + (c ? (double)c[i] : 0.0);", "S[(size_t)b * n + i] = acc;", 0),
    ("predict_wrong_x_index", "acc += elem(P1, p_dtype, (size_t)j * d + t) * (double)x[t];",
     "acc += elem(P1, p_dtype, (size_t)j * d + t) * (double)x[d - 1 - t];", 0),
    ("half_bias_off_by_one", "v = ldexp((double)(1024 + frac), expo - 25);",
     "v = ldexp((double)(1024 + frac), expo - 24);", 0),
    ("half_subnormal_wrong", "v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);", 0),
    ("perm_tiebreak_reversed", "return a < b ? -1 : (a > b ? 1 : 0);", "return a < b ? 1 : (a > b ? -1 : 0);", 0),
    ("perm_cold_sorted_by_count", "  for (int32_t i = 0; i < n; ++i)\n    if (!is_hot[i]) perm[k++] = i;",
     "  for (; k < n; ++k) perm[k] = order[k];", 0),
    ("pack_inverse", "memcpy((char*)dst + (size_t)i * row_bytes, (const char*)src + (size_t)perm[i] * row_bytes,",
     "memcpy((char*)dst + (size_t)perm[i] * row_bytes, (const char*)src + (size_t)i * row_bytes,", 0),
    ("profile_counts_ge", "if (a > 0.0) ++cnt;", "if (a >= 0.0) ++cnt;", 0),
    ("round_half_ties_away", "return copysign(nearbyint(a / q) * q, v);",
     "return copysign(round(a / q) * q, v);", 0),
    ("round_half_no_subnormal_spacing", "  if (e < -14) e = -14;", "  if (e < -24) e = -24;", 0),
    ("round_half_overflow_early", "if (a >= 65520.0)", "if (a > 65504.0)", 0),
    ("f16act_h_unrounded", "      h = oracle_round_half(h);\n", "", 0),
    ("f16act_x_unrounded", "xr[t] = oracle_round_half((double)x[t]);", "xr[t] = (double)x[t];", 0),
]


def _apply(src, old, new, occ):
    pos = -1
    for _ in range(occ + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation site not found: {old!r}"
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, occ):
    src = open(SRC, encoding="utf-8").read()
    mut = _apply(src, old, new, occ)
    assert mut != src
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"lib{name}.so"
    c_path.write_text(mut, encoding="utf-8")
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-o",
                    str(so_path), str(c_path), "-lm"], check=True)
    oracle.load()
    prev = orc.set_library(orc.open_library(str(so_path)))
    caught = []
    try:
        for pin in pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
                break
    finally:
        orc.set_library(prev)
    assert caught, f"mutant {name} passed every pin"
