"""Each plausible mistake planted in a copy of the oracle (on the CPU) must fail at least one pin.

The copies are built from oracle/oracle.cpp by a one-line textual change, compiled with g++ into a
temporary directory, and run through every pin in tests/pins.py. A mutant that passes every pin
would mean the pins cannot tell that mistake from the method.
"""
import os
import shutil
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")

# (name, exact text in oracle.cpp, replacement, occurrence to replace: 0 = all)
MUTANTS = [
    ("nibble_order", "(k % 2 == 0) ? (byte & 0xF) : (byte >> 4)", "(k % 2 == 0) ? (byte >> 4) : (byte & 0xF)", 0),
    ("scale_index", "scales[r * (K / 16) + k / 16]", "scales[r * (K / 16) + k / 32]", 0),
    ("e4m3_bias_8", "std::ldexp(1.0 + m / 8.0, e - 7)", "std::ldexp(1.0 + m / 8.0, e - 8)", 0),
    ("e4m3_subnormal", "std::ldexp(m / 8.0, -6)", "std::ldexp(m / 8.0, -7)", 0),
    ("e2m1_subnormal", "0.5 * m : std::ldexp", "1.0 * m : std::ldexp", 0),
    ("e2m1_sign_dropped", "return s ? -mag : mag;\n}\n\n// E4M3", "return mag;\n}\n\n// E4M3", 0),
    ("e2m1_ties_up", "return (lo & 1) ? hi : lo;  // tie", "return hi;  // tie", 0),
    ("e4m3_ties_up", "  return (lo & 1) ? hi : lo;\n}", "  return hi;\n}", 0),
    ("e2m1_no_saturation", "if (a >= 6.0) return 7;", "if (a >= 6.0) return 6;", 0),
    ("e4m3_saturation", "if (v >= 448.0) return 0x7E;", "if (v >= 448.0) return 0x7D;", 0),
    ("neg_zero_code", "if (mag == 0) return 0;", "if (mag == 0) return (q < 0.0) ? 8 : 0;", 0),
    ("tensor_scale_constant", "amax / 2688.0", "amax / 2048.0", 0),
    ("block_scale_six", "const double six_ts = 6.0 *", "const double six_ts = 4.0 *", 0),
    ("ts_not_applied", "orc_dequant(codes, scales, static_cast<double>(ts), N, K, Wd.data());",
     "orc_dequant(codes, scales, 1.0, N, K, Wd.data());", 0),
    ("pqs_dropped", "bf16_to_double(x[m * K + k]) * (pqs ? static_cast<double>(pqs[k]) : 1.0)",
     "bf16_to_double(x[m * K + k])", 0),
    ("lora_sees_prescaled_x", "s += bf16_to_double(x[m * K + k]) * bf16_to_double(A[j * K + k]);",
     "s += act[m * K + k] * bf16_to_double(A[j * K + k]);", 1),
    ("alpha_over_rank_dropped", "strength * alpha / static_cast<double>(rank)", "strength", 0),
    ("rank_over_alpha", "strength * alpha / static_cast<double>(rank)", "strength * static_cast<double>(rank) / alpha", 0),
    ("B_transposed", "bf16_to_double(B[n * rank + j])", "bf16_to_double(B[j * N + n])", 0),
    ("A_transposed", "bf16_to_double(A[j * K + k])", "bf16_to_double(A[k * rank + j])", 0),
    ("delta_sign", "y[m * N + n] = base + c * delta;", "y[m * N + n] = base - c * delta;", 0),
    ("w4a4_ts_a_dropped", "static_cast<double>(ts_a), M, K, act.data()", "1.0, M, K, act.data()", 0),
    ("silu_sign", "g / (1.0 + std::exp(-g)) * u", "g / (1.0 + std::exp(g)) * u", 0),
    ("gate_up_swapped", "g = y[m * 2 * F + j], u = y[m * 2 * F + F + j]", "u = y[m * 2 * F + j], g = y[m * 2 * F + F + j]", 0),
    ("prescale_f32_no_pqs", "const double p = pqs ? static_cast<double>(pqs[k]) : 1.0;", "const double p = 1.0;", 0),
    ("rope_sign", "orow[c0 + o + i] = u[o + i] * c - u[o + i + half] * s;",
     "orow[c0 + o + i] = u[o + i] * c + u[o + i + half] * s;", 0),
    ("rope_cos_sin_swapped", "const double c = cos_t[m * tab + o / 2 + i], s = sin_t[m * tab + o / 2 + i];",
     "const double c = sin_t[m * tab + o / 2 + i], s = cos_t[m * tab + o / 2 + i];", 0),
    ("rope_adjacent_pairs", "orow[c0 + o + i + half] = u[o + i + half] * c + u[o + i] * s;",
     "orow[c0 + o + i + half] = u[o + i + half] * c + u[o + (i + 1) % half] * s;", 0),
    # sections: every section reads the table from its first column; the section offset advances by
    # half a width (dims and table columns confused); the sections are ignored (one split over rot)
    ("rope_section_table_offset", "const double c = cos_t[m * tab + o / 2 + i], s = sin_t[m * tab + o / 2 + i];",
     "const double c = cos_t[m * tab + i], s = sin_t[m * tab + i];", 0),
    ("rope_section_offset_half", "        o += sec[j];\n", "        o += sec[j] / 2;\n", 0),
    ("rope_sections_ignored", "  if (!sec) {\n    sec = one;", "  if (true) {\n    sec = one;", 0),
    ("rmsnorm_whole_width", "for (int64_t i = 0; i < hd; ++i) ss += yr[c0 + i] * yr[c0 + i];",
     "for (int64_t i = 0; i < qw; ++i) ss += yr[(c0 / qw) * qw + i] * yr[(c0 / qw) * qw + i];", 0),
    ("rmsnorm_eps_outside", "1.0 / std::sqrt(ss / static_cast<double>(hd) + eps)",
     "1.0 / (std::sqrt(ss / static_cast<double>(hd)) + eps)", 0),
    ("rmsnorm_gamma_swapped", "c0 < qw ? gamma_q + c0 : gamma_k + (c0 - qw)", "c0 < qw ? gamma_k + c0 : gamma_q + (c0 - qw)", 0),
    ("merge_pqs_multiplied", "m[n * K + k] = static_cast<float>(Wd[n * K + k] + c * s / p);",
     "m[n * K + k] = static_cast<float>(Wd[n * K + k] + c * s * p);", 0),
    ("merge_c_dropped", "m[n * K + k] = static_cast<float>(Wd[n * K + k] + c * s / p);",
     "m[n * K + k] = static_cast<float>(Wd[n * K + k] + s / p);", 0),
    ("merge_A_transposed", "s += bf16_to_double(B[n * rank + j]) * bf16_to_double(A[j * K + k]);",
     "s += bf16_to_double(B[n * rank + j]) * bf16_to_double(A[k * rank + j]);", 0),
    ("merge_base_dropped", "m[n * K + k] = static_cast<float>(Wd[n * K + k] + c * s / p);",
     "m[n * K + k] = static_cast<float>(c * s / p);", 0),
    ("adaln_table_order", "for (int64_t q = 0; q < rb; ++q) row[q] = static_cast<double>(u[i * rb + q]);",
     "for (int64_t q = 0; q < rb; ++q) row[rl + q] = static_cast<double>(u[i * rb + q]);", 0),
    ("adaln_silu_dropped", "s += bf16_to_double(A[(b * rl + j) * E + k]) * (z / (1.0 + std::exp(-z)));",
     "s += bf16_to_double(A[(b * rl + j) * E + k]) * z;", 0),
    ("adaln_c_dropped", "row[rb + j] = c * s;", "row[rb + j] = s;", 0),
    ("adaln_interp_swapped", "v[q] = (1.0 - th) * t0[q] + th * t1[q];", "v[q] = th * t0[q] + (1.0 - th) * t1[q];", 0),
    ("adaln_grid_S", "const double p = tt * static_cast<double>(S - 1);", "const double p = tt * static_cast<double>(S);", 0),
    ("adaln_bias_dropped", "double acc = bias ? static_cast<double>(bias[b * rows + r]) : 0.0;", "double acc = 0.0;", 0),
    ("bf16_truncates", "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0u;", 0),
    ("bf16_ties_up", "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;", 0),
    ("mirror_ts_dropped", "y_bits[m * N + n] = orc_f32_to_bf16(ts * static_cast<float>(acc));",
     "y_bits[m * N + n] = orc_f32_to_bf16(static_cast<float>(acc));", 0),
    ("mirror_f_keeps_ts", "strength * alpha / (static_cast<double>(rank) * static_cast<double>(ts))",
     "strength * alpha / static_cast<double>(rank)", 0),
    ("mirror_lora_sees_xs", "s += bf16_to_double(x[m * K + k]) * bf16_to_double(A[j * K + k]);\n      tq[j]",
     "s += xs[k] * bf16_to_double(A[j * K + k]);\n      tq[j]", 0),
    ("rmsnorm_touches_v", "for (int64_t c0 = 0; c0 < 2 * qw; c0 += hd) {", "for (int64_t c0 = 0; c0 < N; c0 += hd) {", 0),
]


@pytest.fixture(scope="module")
def mutant_libs():
    src = open(SRC).read()
    tmp = tempfile.mkdtemp(prefix="oracle_mutants_")

    def make(m):
        name, old, new, which = m
        assert src.count(old) >= max(1, which), f"mutant {name}: pattern not found"
        if which == 0:
            text = src.replace(old, new)
        else:  # only the which-th occurrence
            at = -1
            for _ in range(which):
                at = src.index(old, at + 1)
            text = src[:at] + new + src[at + len(old):]
        path = os.path.join(tmp, f"{name}.cpp")
        with open(path, "w") as f:
            f.write(text)
        return name, oracle.build(os.path.join(tmp, f"lib{name}.so"), src=path)

    with ThreadPoolExecutor(max_workers=4) as ex:
        built = dict(ex.map(make, MUTANTS))
    yield built
    shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_mutant_is_caught(name, mutant_libs):
    lib = oracle.load(mutant_libs[name])
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake '{name}'"
