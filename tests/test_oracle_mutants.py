"""Plant plausible mistakes in copies of the oracle source (on the CPU) and check
that each one trips at least one pin.  The planted copies live in a temporary
directory; the oracle itself is never modified."""

import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "nibble_order_reversed": ("(4 * (unsigned)(k % 8))", "(4 * (unsigned)(7 - k % 8))"),
    "pack_order_reversed": ("<< (4 * j)", "<< (4 * (7 - j))"),
    "zero_point_7": ("(float)(q - 8)", "(float)(q - 7)"),
    "group_of_packed_row": ("return g == -1 ? 0 : k / g;", "return g == -1 ? 0 : (k / 8) / g;"),
    "per_channel_as_k_groups": ("return g == -1 ? 0 : k / g;", "return g == -1 ? k / 16 : k / g;"),
    "dropped_last_k": ("for (int64_t k = 0; k < K; ++k) {\n                double xk",
                       "for (int64_t k = 0; k < K - 1; ++k) {\n                double xk"),
    "fp32_accumulator": ("double acc[256];", "float acc[256];"),
    "x_transposed": ("act_to_double(x[m * K + k], act);", "act_to_double(x[k * M + m], act);"),
    "bf16_exponent_bias": ("exp - 134", "exp - 133"),
    "bf16_subnormal_scale": ("ldexp((double)man, -133)", "ldexp((double)man, -132)"),
    "bf16_fraction_width": ("int man = h & 0x7F;", "int man = h & 0xFF;"),
    "bf16_read_as_half": ("return act ? bf16_to_double(h) : half_to_double(h);",
                          "return half_to_double(h);"),
    "abs_sign_kept": ("return absval ? fabs(xk) * fabs(w) : xk * w;",
                      "return absval ? fabs(xk) * w : xk * w;"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "gate_up_swapped": ("silu(y[m * N + 2 * j]) * y[m * N + 2 * j + 1]",
                        "silu(y[m * N + 2 * j + 1]) * y[m * N + 2 * j]"),
    "half_exponent_bias": ("exp - 25", "exp - 24"),
    "half_subnormal_scale": ("ldexp((double)man, -24)", "ldexp((double)man, -23)"),
    "half_sign_dropped": ("return sign ? -v : v;", "return v;"),
    "scale_column_offset": ("scales[group_of(k, g) * N + n]", "scales[group_of(k, g) * N + (n ^ 1)]"),
    "bf16_scale_read_as_half": ("return stype == 1 ? bf16_to_double(h) : half_to_double(h);",
                                "return half_to_double(h);"),
    "zp_v1_ignored": ("return (int)zero_at(qzeros, N, gi, n) + (zv1 ? 1 : 0);",
                      "return (int)zero_at(qzeros, N, gi, n);"),
    "zp_v1_subtracts": ("return (int)zero_at(qzeros, N, gi, n) + (zv1 ? 1 : 0);",
                        "return (int)zero_at(qzeros, N, gi, n) - (zv1 ? 1 : 0);"),
    "zp_scales_read_as_half": ("(float)scale_to_double(scales[gi * N + n], stype);\n            acc",
                               "(float)half_to_double(scales[gi * N + n]);\n            acc"),
    "lora_a_transposed": ("act_to_double(A[j * K + k], act)", "act_to_double(A[k * r + j], act)"),
    "lora_b_row_offset": ("act_to_double(B[n * r + j], act)", "act_to_double(B[(n ^ 1) * r + j], act)"),
    "lora_scale_dropped": ("return (absval ? fabs(scale) : scale) * acc;", "return acc;"),
    "lora_delta_subtracted": ("out[i] += d[i];", "out[i] -= d[i];"),
    "lora_a_read_as_half": ("act_to_double(A[j * K + k], act)", "act_to_double(A[j * K + k], 0)"),
    "zp_nibble_order_reversed": ("(4 * (unsigned)(n % 8))) & 0xFu;", "(4 * (unsigned)(7 - n % 8))) & 0xFu;"),
    "zp_v1_offset": ("return (word >> (4 * (unsigned)(n % 8))) & 0xFu;",
                     "return ((word >> (4 * (unsigned)(n % 8))) & 0xFu) + 1u;"),
    "zp_added": ("(float)(q - z)", "(float)(q + z - 16)"),
    "zp_row_of_k": ("zero_point(qzeros, zv1, N, gi, n)",
                    "zero_point(qzeros, zv1, N, k / 8 % (gi + 1), n)"),
    "decode_act_as_half": ("out[i] = act_to_double(x[i], act);", "out[i] = act_to_double(x[i], 0);"),
    "lora_last_rank_dropped": ("for (int64_t j = 0; j < r; ++j)\n        acc +=",
                               "for (int64_t j = 0; j + 1 < r; ++j)\n        acc +="),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SRC_PATH) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src_m = src.replace(old, new)
    path = os.path.join(tmp_path, f"{name}.c")
    with open(path, "w") as f:
        f.write(src_m)
    lib = oracle.compile_source(path, os.path.join(tmp_path, f"lib{name}.so"))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
