"""Plants plausible mistakes in copies of the C oracle (never in the GPU path)
and checks that each one fails at least one pin.  The real oracle source is
only read; each mutant is compiled into a temporary directory and exercised in
a subprocess of its own, so a mutant that corrupts memory cannot disturb the
test process."""
import json
import os
import subprocess
import sys

import pytest

import oracle

MUTANTS = {
    # head -> group map off by one (uses i instead of i-1 in the 1-based form)
    "group_map_off_by_one": ("int64_t g1 = (i1 - 1) / R + 1;", "int64_t g1 = (i1) / R + 1;"),
    # strided grouping i mod H_kv instead of contiguous i / R
    "group_map_strided": ("int64_t g = oracle_group_of(i, R);", "int64_t g = i % H_kv;"),
    # the last valid token is dropped from the weighted sum
    "drop_last_token": ("for (int64_t t = 0; t < n; ++t) {\n    double wt", "for (int64_t t = 0; t + 1 < n; ++t) {\n    double wt"),
    # the first token is left out of the normaliser
    "normaliser_skips_first": ("for (int64_t t = 0; t < n; ++t) z += exp", "for (int64_t t = 1; t < n; ++t) z += exp"),
    # scale not applied to the scores
    "scale_dropped": ("s[t] = scale * acc;", "s[t] = acc;"),
    # sign error in the exponent
    "exponent_sign": ("exp(s[t] - m)", "exp(m - s[t])"),
    # no normalisation
    "no_normalisation": ("double wt = exp(s[t] - m) / z;", "double wt = exp(s[t] - m);"),
    # values read from the key cache
    "values_from_keys": ("kv_elem(V, row + c)", "kv_elem(K, row + c)"),
    # transposed key operand
    "keys_transposed": ("kv_elem(K, row + c)", "kv_elem(K, cache_row(L, b, g, 0) * d + c * n + t)"),
    # query row of the group's first head used for every head
    "query_of_group": ("(b * H_q + i) * d, dtype, K, V, d, L, b, g,", "(b * H_q + g * R) * d, dtype, K, V, d, L, b, g,"),
    # KV heads interleaved per token instead of stored one after another
    "kv_layout_interleaved": ("return kv_offsets[b] * H_kv + h * cap + t;", "return kv_offsets[b] * H_kv + h + t * H_kv;"),
    # bf16 widened with the wrong shift
    "bf16_widening": ("[idx]) << 16;", "[idx]) << 15;"),
    # every sequence uses the first sequence's length
    "seq_len_of_first": ("(int64_t)seq_lens[b], scale, s, NULL", "(int64_t)seq_lens[0], scale, s, NULL"),
    # one token too many (reads a padding position)
    "extra_token": ("if (n < 0 || n > cap) return -1;\n  for", "n = n < cap ? n + 1 : n;\n  if (n < 0 || n > cap) return -1;\n  for"),
    # paged cache: token offset and page index swapped
    "paged_row_swapped": ("return (p * L->H_kv + h) * L->page + t % L->page;", "return (p * L->H_kv + h) * L->page + t / L->page;"),
    # paged cache: pages stored token-major instead of head-major
    "paged_head_major": ("return (p * L->H_kv + h) * L->page + t % L->page;", "return (p * L->page + t % L->page) * L->H_kv + h;"),
    # E4M3: exponent bias 8 instead of 7
    "e4m3_bias": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    # E4M3: subnormals decoded with the implicit leading one
    "e4m3_subnormal_as_normal": ("e == 0 ? ldexp((double)m / 8.0, 1 - 7)", "e == 0 ? ldexp(1.0 + (double)m / 8.0, 1 - 7)"),
    # E4M3: the NaN code read as a finite value (480)
    "e4m3_nan_code": ("if (e == 0xF && m == 0x7) return NAN;", ""),
    # E4M3 cache: the key and value scales swapped
    "fp8_scales_swapped": ("const kv_array K = {k8, ORACLE_E4M3, k_scale}, V = {v8, ORACLE_E4M3, v_scale};",
                           "const kv_array K = {k8, ORACLE_E4M3, v_scale}, V = {v8, ORACLE_E4M3, k_scale};"),
    # E4M3 encoder: ties away from zero instead of to even
    "e4m3_encode_ties_away": ("int m = (int)nearbyint((ldexp(a, -e) - 1.0) * 8.0);",
                              "int m = (int)round((ldexp(a, -e) - 1.0) * 8.0);"),
    # E4M3 encoder: overflow to NaN instead of saturating
    "e4m3_encode_no_saturation": ("if (a >= 448.0) return sign | 0x7E;", "if (a > 464.0) return 0x7F;"),
    # E4M3 encoder: subnormal grid of 2^-8 instead of 2^-9
    "e4m3_encode_subnormal_grid": ("(uint8_t)nearbyint(ldexp(a, 9))", "(uint8_t)nearbyint(ldexp(a, 8))"),
    # rotary embedding: turning the other way
    "rope_orientation": ("out[v * d + 2 * j] = x0 * c - x1 * s;", "out[v * d + 2 * j] = x0 * c + x1 * s;"),
    # rotary embedding: pairs (j, j + d/2) instead of consecutive elements
    "rope_half_split_pairs": ("load_elem(x, v * d + 2 * j, dtype), x1 = load_elem(x, v * d + 2 * j + 1, dtype);",
                              "load_elem(x, v * d + j, dtype), x1 = load_elem(x, v * d + j + d / 2, dtype);"),
    # rotary embedding: frequencies base^(-j/d) instead of base^(-2j/d)
    "rope_frequency": ("pow(base, -2.0 * (double)j / (double)d)", "pow(base, -1.0 * (double)j / (double)d)"),
    # rotary embedding: position off by one
    "rope_position_off_by_one": ("const double a = (double)pos[v] * theta;", "const double a = (double)(pos[v] + 1) * theta;"),
}

_RUNNER = r"""
import json, sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import oracle
from oracle_pins import ORACLE_PINS
orc = oracle.Oracle(sys.argv[1])
failed = []
for pin in ORACLE_PINS:
    try:
        pin(orc)
    except Exception:
        failed.append(pin.__name__)
print("FAILED_PINS " + json.dumps(failed), flush=True)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, "mutation site not found: %s" % name
    path = os.path.join(tmp_path, "gqa_oracle_%s.c" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(path, os.path.join(tmp_path, "lib_%s.so" % name))
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(tests_dir)
    r = subprocess.run([sys.executable, "-c", _RUNNER, lib, root, tests_dir], capture_output=True, text=True,
                       timeout=300, env=dict(os.environ, OMP_NUM_THREADS="2"))
    lines = [l for l in r.stdout.splitlines() if l.startswith("FAILED_PINS ")]
    if r.returncode != 0 and not lines:
        return  # the mutant crashed the process: caught
    assert lines, r.stdout + r.stderr
    failed = json.loads(lines[-1][len("FAILED_PINS "):])
    print(name, "caught by", failed)
    assert failed, "mutant %s passed every pin" % name
