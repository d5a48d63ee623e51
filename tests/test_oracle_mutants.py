"""The oracle's pins must catch plausible mistakes in the oracle.

Each case copies oracle/oracle.c, plants one mistake by text substitution
(a dropped term, a wrong index or sign, a reversed order, a wrong rounding of
the shard size ...), builds the copy on the CPU with the oracle's own flags
and runs every pin in test_oracle_pins.py against it.  At least one pin has
to fail for every planted mistake.  The real oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle
from oracle import build_oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "drop_last_rank": ("for (int32_t r = 1; r < N; r++)\n                    acc",
                       "for (int32_t r = 1; r < N - 1; r++)\n                    acc"),
    "sum_from_plus_zero": ("float acc = load_elem(first[(int64_t)0 * P + i], k, dtype);\n"
                           "                for (int32_t r = 1;",
                           "float acc = 0.0f;\n                for (int32_t r = 0;"),
    "reverse_rank_order": ("float acc = load_elem(first[(int64_t)0 * P + i], k, dtype);\n"
                           "                for (int32_t r = 1; r < N; r++)\n"
                           "                    acc = acc + load_elem(first[(int64_t)r * P + i], k, dtype);",
                           "float acc = load_elem(first[(int64_t)(N - 1) * P + i], k, dtype);\n"
                           "                for (int32_t r = 1; r < N; r++)\n"
                           "                    acc = acc + load_elem(first[(int64_t)(N - 1 - r) * P + i], k, dtype);"),
    "floor_rows": ("c[i] = (d0[i] + N - 1) / N;", "c[i] = d0[i] / N + (d0[i] % N > 1);"),
    "ignore_align": ("off[i] = round_up(pos, align);", "off[i] = pos;"),
    "src_without_inner": ("*src = (int64_t)r * c * inner;", "*src = (int64_t)r * c;"),
    "no_row_clamp": ("    if (rows > c) rows = c;\n", ""),
    "ag_reads_wrong_index": ("for (int64_t k = 0; k < L; k++) to[src + k] = from[off[i] + k];\n            } else",
                             "for (int64_t k = 0; k < L; k++) to[src + k] = from[src + k];\n            } else"),
    "negative_zero_padding": ("for (int64_t j = 0; j < S; j++) out[j] = 0.0f;",
                              "for (int64_t j = 0; j < S; j++) out[j] = -0.0f;"),
    "traffic_counts_self": ("*real = (int64_t)(N - 1) * sum;", "*real = (int64_t)N * sum;"),
    "widen_wrong_shift": ("uint32_t bits = (uint32_t)b << 16;", "uint32_t bits = (uint32_t)b << 15;"),
    "widen_round_trip_loses_sign": ("uint32_t bits = (uint32_t)b << 16;",
                                    "uint32_t bits = ((uint32_t)b & 0x7fffu) << 16;"),
    "shard_owner_off_by_one": ("int64_t rows = d0 - (int64_t)r * c;",
                               "int64_t rows = d0 - (int64_t)(r + (r > 1)) * c;"),
    "skip_last_tail_round": ("*S = round_up(pos, align);", "*S = pos;"),
    "mean_not_divided": ("if (avg) acc = acc / (float)N;", "(void)avg;"),
    "mean_divides_by_n_minus_1": ("if (avg) acc = acc / (float)N;",
                                  "if (avg) acc = acc / (float)(N > 1 ? N - 1 : 1);"),
    "mean_by_reciprocal": ("if (avg) acc = acc / (float)N;",
                           "if (avg) acc = acc * (1.0f / (float)N);"),
    "f16_wrong_bias": ("bits = (sign << 31) | ((e - 15u + 127u) << 23) | (frac << 13);",
                       "bits = (sign << 31) | ((e - 16u + 127u) << 23) | (frac << 13);"),
    "f16_subnormal_scale": ("f = (float)frac * 0x1p-24f;", "f = (float)frac * 0x1p-25f;"),
    "f16_nan_drops_payload": ("bits = (sign << 31) | 0x7f800000u | (frac << 13);",
                              "bits = (sign << 31) | 0x7f800000u | (frac ? 0x400000u : 0u);"),
    "round_ties_away_from_zero": ("return (t & 1u) ? up : t;", "return up;"),
    "round_toward_zero": ("    if (d_up < d_t) return up;\n", ""),
    "round_nan_payload_cut": ("if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);",
                              "if (isnan(x)) return (uint16_t)(u >> 16);"),
    "round_overflow_saturates": ("double aup = ((up & 0x7fffu) == 0x7f80u) ? ldexp(1.0, 128)",
                                 "if ((up & 0x7fffu) == 0x7f80u) return t;\n    double aup = 0 ? 0"),
    "pack_pads_with_ones": ("memset(slot, 0, (size_t)N * (size_t)S * (size_t)elem_bytes);",
                            "memset(slot, 1, (size_t)N * (size_t)S * (size_t)elem_bytes);"),
    "pack_previous_offset": ("char *to = (char *)slot + ((int64_t)q * S + off[i]) * elem_bytes;",
                             "char *to = (char *)slot + ((int64_t)q * S + (i ? off[i - 1] : 0)) * elem_bytes;"),
    "pack_ignores_owner": ("const char *from = (const char *)tensors[i] + src * elem_bytes;",
                           "const char *from = (const char *)tensors[i];"),
    "f32_read_as_half_width": ("memcpy(&f, (const char *)run + 4 * k, sizeof f);",
                               "memcpy(&f, (const char *)run + 2 * k, sizeof f);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    lib = build_oracle.build(src=str(src), out=str(tmp_path / f"lib{name}.so"))
    proc = subprocess.run([sys.executable, "-c", RUNNER, lib], cwd=ROOT,
                          capture_output=True, text=True, timeout=600)
    if proc.returncode < 0:
        return                       # crashed: the mistake is visible
    assert proc.returncode == 0, proc.stderr[-2000:]
    caught = [x for x in proc.stdout.split() if x.startswith("pin_")]
    assert caught, f"planted mistake {name} passed every pin"


RUNNER = """
import sys
sys.path[:0] = ['.', 'tests']
import oracle
import test_oracle_pins as pins
m = oracle.Oracle(sys.argv[1])
for pin in pins.PINS:
    try:
        pin(m)
    except Exception:
        print(pin.__name__, flush=True)
"""
