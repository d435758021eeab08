"""The oracle's pins must reject plausible mistakes.

Each case plants one mistake into a temporary copy of the oracle's C source
(a dropped term, a wrong index or sign, a transposed operand), builds it on
the CPU and runs the pin suite against it: at least one pin has to fail (or
the build must crash on them).  The unmodified source must pass the same
suite.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import tests.test_oracle_pins as pins
import tests.test_oracle_multi_query as mq
import tests.test_oracle_rope as rp

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
    "rope_sign": ("out[row + ia] = xa * c - xb * s;", "out[row + ia] = xa * c + xb * s;"),
    "rope_frequency_exponent": ("pow(base, -2.0 * (double)j / (double)head_dim)",
                                "pow(base, -1.0 * (double)j / (double)head_dim)"),
    "rope_pairing": ("const int64_t ib = interleaved ? 2 * j + 1 : j + half;",
                     "const int64_t ib = interleaved ? 2 * j + 1 : head_dim - 1 - j;"),
    "rope_position_off_by_one": ("const double angle = (double)positions[i] *",
                                 "const double angle = (double)(positions[i] + 1) *"),
    "rope_sin_cos_swapped": ("const double c = cos(angle), s = sin(angle);",
                             "const double c = sin(angle), s = cos(angle);"),
    "mq_causal_limit_exclusive": ("const int64_t len = p + 1;", "const int64_t len = p;"),
    "mq_causal_limit_open": ("const int64_t len = p + 1;", "const int64_t len = context_lens[b];"),
    "mq_positions_from_zero": ("const int64_t p = (int64_t)context_lens[b] - n + j;",
                               "const int64_t p = j;"),
    "mq_sequence_lookup": ("while (query_start[b + 1] <= tok)", "while (query_start[b + 1] < tok)"),
    "mq_query_row_uses_kv_head": ("widen(q, row * head_dim + d, dtype)",
                                  "widen(q, (tok * num_q_heads + g) * head_dim + d, dtype)"),
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
        ("rope_gptj", rp.test_adjacent_pairs_match_transformers_gptj, (np.float32,)),
        ("mq_sdpa_0", mq.test_matches_torch_sdpa_with_causal_mask, (np.float32, 0)),
        ("mq_sdpa_1", mq.test_matches_torch_sdpa_with_causal_mask, (np.float16, 1)),
        ("mq_prefix", mq.test_whole_prompt_rows_are_prefix_decodes, ()),
        ("mq_decode", mq.test_one_new_token_per_sequence_is_the_decode_step, ()),
        ("rope_llama", rp.test_rotate_half_matches_transformers_llama, (64,)),
        ("rope_identities", rp.test_rotation_identities, (False,)),
    ] + [(f"sdpa_{s}", pins.test_matches_torch_sdpa_float64, (np.float32, s)) for s in range(3)]
    for name, fn, args in checks:
        try:
            fn(*args)
        except Exception as e:  # noqa: BLE001 - any failure counts as a rejection
            failures.append(f"{name}: {type(e).__name__}")
    return failures


def _build_variant(dirpath, text, tag):
    src = os.path.join(dirpath, f"oracle_{tag}.c")
    lib = os.path.join(dirpath, f"liboracle_{tag}.so")
    with open(src, "w") as f:
        f.write(text)
    return src, lib, subprocess.Popen(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w",
                                       "-o", lib, src, "-lm"])


_CHILD = """
import sys, oracle, tests.test_oracle_mutants as m
for tag, lib in zip(sys.argv[1::2], sys.argv[2::2]):
    print('START', tag, flush=True)
    with oracle.use_library(lib):
        f = m._pin_suite()
    print('RESULT', tag, len(f), flush=True)
"""


def _run_suites(items):
    """Run the pin suite against each (tag, lib) in child processes.

    One child runs them in turn (importing the pins once).  A mutant may
    index outside its arrays and crash its child: a crash counts as a
    rejection of that mutant, and a new child goes on with the rest.
    Returns {tag: number of failing pins, or -1 for a crash}.
    """
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    results, todo = {}, list(items)
    while todo:
        args = [x for item in todo for x in item]
        r = subprocess.run([sys.executable, "-c", _CHILD, *args], cwd=root, capture_output=True,
                           text=True, timeout=900, env={**os.environ, "OMP_NUM_THREADS": "2"})
        started = None
        for line in r.stdout.splitlines():
            parts = line.split()
            if parts[:1] == ["START"]:
                started = parts[1]
            elif parts[:1] == ["RESULT"]:
                results[parts[1]] = int(parts[2])
                started = None
        if r.returncode != 0:
            if started is None:
                raise RuntimeError(f"mutation child failed outside a suite: {r.stderr[-2000:]}")
            results[started] = -1
        todo = [item for item in todo if item[0] not in results]
    return results


@pytest.fixture(scope="module")
def suite_results(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("mutants"))
    text = open(SRC).read()
    builds = {"clean": _build_variant(d, text, "clean")}
    for name, (old, new) in MUTANTS.items():
        assert old in text, f"mutation anchor for {name} not found"
        builds[name] = _build_variant(d, text.replace(old, new), name)
    for tag, (_, _, proc) in builds.items():
        assert proc.wait() == 0, f"build of {tag} failed"
    return _run_suites([(tag, lib) for tag, (_, lib, _) in builds.items()])


def test_unmodified_source_passes(suite_results):
    assert suite_results["clean"] == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(suite_results, name):
    assert suite_results[name] != 0, f"no pin rejects the '{name}' mutant"
