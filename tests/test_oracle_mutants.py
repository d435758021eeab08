"""The oracle's pins must reject plausible mistakes.

Each case plants one mistake into a temporary copy of the oracle's C source
(a dropped term, a wrong index or sign, a transposed operand), builds it on
the CPU and runs the pin suite against it: at least one pin has to fail.
The unmodified source must pass the same suite.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "photon_oracle.c")

MUTANTS = {
    "gqa_head_modulo": ("const int64_t g = h / group;", "const int64_t g = h % num_kv_heads;"),
    "no_max_subtraction": ("exp(s[t] - m)", "exp(s[t])"),
    "scale_dropped": ("s[t] = scale * dot;", "s[t] = dot;"),
    "scale_squared": ("s[t] = scale * dot;", "s[t] = scale * scale * dot;"),
    "table_index_mod": ("block_tables[b * max_blocks + t / block_size]",
                        "block_tables[b * max_blocks + t % block_size]"),
    "offset_div": ("+ t % block_size) * head_dim", "+ t / block_size) * head_dim"),
    "pool_head_block_transposed": ("((blk * num_kv_heads + g) * block_size",
                                   "((g * num_blocks + blk) * block_size"),
    "context_one_short": ("for (int64_t t = 0; t < ctx; ++t) {\n            const int64_t blk = block_tables[b * max_blocks + t / block_size];\n            const int64_t row = ((blk * num_kv_heads + g) * block_size + t % block_size) * head_dim;\n            const double e",
                          "for (int64_t t = 0; t < ctx - 1; ++t) {\n            const int64_t blk = block_tables[b * max_blocks + t / block_size];\n            const int64_t row = ((blk * num_kv_heads + g) * block_size + t % block_size) * head_dim;\n            const double e"),
    "no_normalisation": ("o[j] /= l;", "o[j] /= 1.0;"),
    "v_from_k_pool": ("widen(v_cache, row + j, dtype)", "widen(k_cache, row + j, dtype)"),
    "q_batch_index_dropped": ("widen(q, pair * head_dim + j, dtype)", "widen(q, h * head_dim + j, dtype)"),
    "half_bias_off_by_one": ("expo - 25", "expo - 24"),
    "half_subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -23)"),
    "half_sign_dropped": ("mag = ldexp((double)(frac | 0x400), expo - 25);\n    return sign ? -mag : mag;",
                          "mag = ldexp((double)(frac | 0x400), expo - 25);\n    return mag;"),
    "bf16_bias_off_by_one": ("expo - 134", "expo - 133"),
    "bf16_fraction_bits": ("const int frac = bits & 0x7f;", "const int frac = bits & 0x3f;"),
    "bf16_subnormal_scale": ("ldexp((double)frac, -133)", "ldexp((double)frac, -126)"),
    "bf16_read_as_half": ("return oracle_bfloat16_to_double(((const uint16_t *)base)[idx]);",
                          "return oracle_half_to_double(((const uint16_t *)base)[idx]);"),
    "write_head_block_transposed": ("((blk * num_kv_heads + h) * block_size + off)",
                                    "((h * num_blocks + blk) * block_size + off)"),
    "write_offset_swapped": ("const int64_t off = s % block_size;", "const int64_t off = s / block_size % block_size;"),
    "write_v_from_k": ("(const char *)v + src", "(const char *)k + src"),
    "no_duplicate_check": ("if (seen[s]) {", "if (0) {"),
    "empty_ctx_not_zeroed": ("memset(o, 0, sizeof(double) * (size_t)head_dim);\n            continue;",
                             "continue;"),
}


def _pin_suite():
    failures = []
    checks = [
        ("golden_attn", pins.test_golden_two_blocks_gqa, ()),
        ("golden_write", pins.test_golden_cache_write, ()),
        ("tiny_sdpa", pins.test_tiny_config_matches_sdpa, ()),
        ("one_token_f16", pins.test_one_token_returns_its_value_row, (np.float16,)),
        ("dominant_key", pins.test_dominant_key_selects_its_value, (1000.0,)),
        ("empty_ctx", pins.test_empty_context_gives_zero_row, ()),
        ("half_all", pins.test_half_decoder_matches_numpy_on_all_bit_patterns, ()),
        ("bf16_all", pins.test_bfloat16_decoder_matches_torch_on_all_bit_patterns, ()),
        ("write_brute_f16", pins.test_cache_write_brute_force, (np.float16,)),
        ("preconditions", pins.test_precondition_errors, ()),
    ] + [(f"sdpa_{s}", pins.test_matches_torch_sdpa_float64, (np.float32, s)) for s in range(3)]
    for name, fn, args in checks:
        try:
            fn(*args)
        except Exception as e:  # noqa: BLE001 - any failure counts as a rejection
            failures.append(f"{name}: {type(e).__name__}")
    return failures


def _build_variant(tmp_path, text, tag):
    src = tmp_path / f"oracle_{tag}.c"
    lib = tmp_path / f"liboracle_{tag}.so"
    src.write_text(text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w",
                           "-o", str(lib), str(src), "-lm"])
    return str(lib)


def _run_suite_in_child(lib):
    """Run the pin suite against ``lib`` in a child process.

    A mutant may index outside its arrays and crash; a crash counts as a
    rejection, so the child keeps that from taking the test run down.
    Returns (exit status, printed failures).
    """
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys, oracle, tests.test_oracle_mutants as m\n"
            f"with oracle.use_library({lib!r}):\n"
            "    f = m._pin_suite()\n"
            "print('FAILURES', len(f), f)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=300, env={**os.environ, "OMP_NUM_THREADS": "2"})
    return r.returncode, r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""


def test_unmodified_source_passes(tmp_path):
    lib = _build_variant(tmp_path, open(SRC).read(), "clean")
    rc, line = _run_suite_in_child(lib)
    assert rc == 0 and line == "FAILURES 0 []", line


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert old in text, f"mutation anchor for {name} not found"
    lib = _build_variant(tmp_path, text.replace(old, new), name)
    rc, line = _run_suite_in_child(lib)
    assert rc != 0 or not line.startswith("FAILURES 0"), f"no pin rejects the '{name}' mutant"
