"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutant is a textual change to a copy of ``oracle/q4_oracle.c`` -- a
dropped term, a wrong sign, a swapped index or operand -- compiled into a
temporary library.  Every pin in ``test_oracle_pins.ALL_CHECKS`` runs against
it, and at least one must fail.  The mistakes live only in these temporary
copies; the real oracle is untouched.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import ALL_CHECKS

MUTANTS = {
    "nibble_order_swapped": (
        "(k % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4)",
        "(k % 2 == 0) ? (byte >> 4) : (byte & 0x0Fu)"),
    "bias_dropped": ("w[k] = sq + b;", "w[k] = sq;"),
    "bias_sign": ("w[k] = sq + b;", "w[k] = sq - b;"),
    "zero_point_code": ("s * (float)q;", "s * ((float)q - 8.0f);"),
    "scale_plane_transposed": (
        "(uint64_t)n * (uint64_t)groups + (uint64_t)g",
        "(uint64_t)g * (uint64_t)N + (uint64_t)n"),
    "scale_bias_planes_swapped": (
        "memcpy(&s_bits, W + scale_off + 2 * idx, 2);\n"
        "        memcpy(&b_bits, W + bias_off + 2 * idx, 2);",
        "memcpy(&s_bits, W + bias_off + 2 * idx, 2);\n"
        "        memcpy(&b_bits, W + scale_off + 2 * idx, 2);"),
    "group_width_32": (
        ("const int64_t groups = K / Q4O_GROUP;",
         "const int64_t groups = K / 32;"),
        ("for (int64_t k = g * Q4O_GROUP; k < (g + 1) * Q4O_GROUP; ++k) {",
         "for (int64_t k = g * 32; k < (g + 1) * 32; ++k) {")),
    "output_transposed": (
        "const uint64_t o = (uint64_t)m * (uint64_t)N + (uint64_t)n;",
        "const uint64_t o = (uint64_t)n * (uint64_t)M + (uint64_t)m;"),
    "row_stride_halved": (
        "W + nib_off + (uint64_t)n * (uint64_t)(K / 2);",
        "W + nib_off + (uint64_t)(n / 2) * (uint64_t)(K / 2);"),
    "fp32_accumulator": ("double acc = 0.0, acc_abs = 0.0;",
                         "float acc = 0.0f; double acc_abs = 0.0;"),
    "abs_sum_signed": ("acc_abs += fabs(p);", "acc_abs += p;"),
    "last_input_skipped": ("for (int64_t k = 0; k < K; ++k) {\n"
                           "                const double p",
                           "for (int64_t k = 0; k < K - 1; ++k) {\n"
                           "                const double p"),
    "activation_row_offset": (
        "job->x + (uint64_t)m * (uint64_t)K;",
        "job->x + (uint64_t)(m > 0 ? m - 1 : 0) * (uint64_t)K;"),
    "size_factor_8": ("elements / 16u, (uint64_t)9u", "elements / 16u, (uint64_t)8u"),
}


def _mutant_source(edits) -> str:
    """Apply one (find, replace) pair or a tuple of them to the source."""
    with open(oracle.SOURCE) as fh:
        src = fh.read()
    if isinstance(edits[0], str):
        edits = (edits,)
    for find, repl in edits:
        assert src.count(find) == 1, f"mutation anchor not unique: {find!r}"
        src = src.replace(find, repl)
    return src


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = tmp_path / f"{name}.c"
    src.write_text(_mutant_source(MUTANTS[name]))
    lib = oracle.compile_source(str(src), str(tmp_path / f"{name}.so"),
                                extra=("-Wno-error",))
    orc = oracle.Oracle(lib)
    caught = []
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):  # a mutant may overflow a cast
                check(orc)
        except (AssertionError, oracle.OracleError, ValueError):
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
