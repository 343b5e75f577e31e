"""Mutation check of the pins: each plausible mistake, planted in a copy of the
oracle's C source and compiled on the CPU, must make at least one pin fail.

The copies live in a temporary directory; the real oracle is untouched."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "rattn_oracle.c")

# (name, exact text in the oracle source, replacement)
MUTANTS = [
    ("distance_off_by_one", "int dist = p - j;", "int dist = p - j + 1;"),
    ("table_reversed", "r[dist < R - 1 ? dist : R - 1]", "r[R - 1 - (dist < R - 1 ? dist : R - 1)]"),
    ("clamp_to_zero", "r[dist < R - 1 ? dist : R - 1]", "r[dist < R - 1 ? dist : 0]"),
    ("scale_one_over_d", "1.0 / sqrt((double)head_dim)", "1.0 / (double)head_dim"),
    ("bias_also_scaled", "s[j - lo] = dot * scale + r[", "s[j - lo] = (dot + 0.0) * scale + scale * r["),
    ("window_one_too_wide", "p - W + 1 > 0) ? p - W + 1 : 0", "p - W > 0) ? p - W : 0"),
    ("kv_heads_interleaved", "const int kvh = h / group;", "const int kvh = h % Hkv;"),
    ("queries_top_left", "const int p = ctx - n_q + t;", "const int p = t + (ctx - n_q) * 0 + (ctx - ctx);"),
    ("lse_missing_max", "lse[row] = m + log(Z);", "lse[row] = log(Z);"),
    ("queries_not_causal", "const int hi = p;", "const int hi = ctx - 1;"),
    ("values_from_keys", "widen(v, kv_offset(", "widen(k, kv_offset("),
    ("paged_slot_reversed", "(((size_t)phys * block_size + j % block_size)",
     "(((size_t)phys * block_size + (block_size - 1 - j % block_size))"),
    ("bf16_widened_wrong", "uint32_t u = (uint32_t)s[e] << 16;", "uint32_t u = (uint32_t)s[e] << 15;"),
    # token-dependent bias: the row's own table
    ("tokbias_head_table", "bias + (size_t)(bias_per_row ? row : h) * R", "bias + (size_t)(bias_per_row ? h : h) * R"),
    ("tokbias_neighbour_row", "bias + (size_t)(bias_per_row ? row : h) * R",
     "bias + (size_t)(bias_per_row ? (row + Hq) % rows : h) * R"),
    ("tokbias_heads_reversed", "bias + (size_t)(bias_per_row ? row : h) * R",
     "bias + (size_t)(bias_per_row ? row - h + (Hq - 1 - h) : h) * R"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    hdr = os.path.join(os.path.dirname(os.path.dirname(SRC)), "include", "rattn_oracle.h")
    (tmp_path / "rattn_oracle.h").write_text(open(hdr).read())
    so = tmp_path / f"libmut_{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-o", str(so), str(mut), "-lm"],
                   check=True)
    lib = oracle.load_library(str(so))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
