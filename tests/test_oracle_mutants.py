"""Planted mistakes in the oracle must each be caught by at least one pin.

Each mutant is the oracle's C source with one plausible slip (a dropped
term, a wrong sign or index, a transposed operand, an off-by-one mask),
compiled on the CPU into a throwaway library. The pins in ``pins.py`` run
against it and at least one must fail; this shows the pins can tell a wrong
oracle from a right one.
"""
import os

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle_fp64.c")

MUTANTS = {
    "drop_scale": ("row[j] = dot * scale;", "row[j] = dot;"),
    "no_max_subtraction": ("row[j] = exp(row[j] - m);", "row[j] = exp(row[j]);"),
    "no_normalisation": ("row[j] /= sum;", "row[j] /= 1.0;"),
    "sign_error_in_dot": ("dot += qi[d] * kj[d];", "dot -= qi[d] * kj[d];"),
    "causal_excludes_diagonal": ("return j <= i;", "return j < i + (i == 0);"),
    "window_one_too_wide": ("j > i - window;", "j >= i - window;"),
    "window_not_causal": ("return j <= i && j > i - window;", "return j > i - window;"),
    "grouped_heads_modulo": ("return h / (H / Hkv);", "return h % Hkv;"),
    "bhsd_query_layout": ("return ((b * S + i) * H + h) * D;", "return ((b * H + h) * S + i) * D;"),
    "kv_head_ignored": ("return ((b * S + j) * Hkv + g) * D;", "return ((b * S + j) * Hkv) * D;"),
    "keys_used_as_values": ("reproject_row(att + (size_t)i * S, v,", "reproject_row(att + (size_t)i * S, k,"),
    "rows_keys_as_values": ("reproject_row(row, v,", "reproject_row(row, k,"),
    "last_key_dropped": ("for (int j = 0; j < S; ++j) {\n        if (!visible",
                         "for (int j = 0; j < S; ++j) {\n        if (j == S - 1 && S > 1) { row[j] = -INFINITY; continue; }\n        if (!visible"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    find, repl = MUTANTS[name]
    assert source.count(find) == 1, f"mutation site for {name} not unique/present"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(find, repl))
    lib = oracle.compile_library(str(src), str(tmp_path / f"{name}.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"mutant {name} passed every pin"
