"""The pins catch plausible mistakes: each mutant is a copy of the oracle
source with one planted error, compiled in a temporary directory; the pin
suite, run on it in a child process, must fail (an assertion or a crash)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "szref.c")

MUTANTS = {
    "exponent_field_shift": ("return (w >> 7) & 0xFFu;", "return (w >> 8) & 0xFFu;"),
    "mantissa_mask": ("return w & 0x7Fu;", "return w & 0x3Fu;"),
    "sign_bit_slot": ("(bf16_sign(w) << 7)", "(bf16_sign(w) << 6)"),
    "recombine_exponent_shift": ("(exponent << 7)", "(exponent << 8)"),
    "encode_nibble_order": ("if (i % 2 == 0)\n            nibbles[i / 2] = (uint8_t)code;",
                            "if (i % 2 == 1)\n            nibbles[i / 2] = (uint8_t)code;"),
    "decode_nibble_order": ("(i % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4)",
                            "(i % 2 == 1) ? (byte & 0x0Fu) : (byte >> 4)"),
    "tie_toward_larger": ("return a < b;", "return a > b;"),
    "least_frequent_first": ("return hist[a] > hist[b];", "return hist[a] < hist[b];"),
    "codebook_reversed": ("codebook[c] = (uint8_t)order[c];", "codebook[c] = (uint8_t)order[15 - c];"),
    "escape_code_nonzero": (": 0u;", ": 15u;"),
    "nibble_bytes_floor": ("uint64_t nibble_bytes = (n + 1) / 2;", "uint64_t nibble_bytes = n / 2;"),
    "escape_record_4_bytes": ("uint64_t escape_bytes = 5 * e;", "uint64_t escape_bytes = 4 * e;"),
    "header_stores_kept_count": ("put_u64(dst + 16, e);", "put_u64(dst + 16, n - e);"),
    "segment_off_by_one": ("if (seg_end[s] <= k) segment += 1;", "if (seg_end[s] < k) segment += 1;"),
    "segment_width": ("per_segment[positions[k] >> 32]", "per_segment[(positions[k] >> 32) / 2]"),
    "decode_code_lookup": ("codebook[code]", "codebook[15 - code]"),
    "duplicates_accepted": ("if (k > 0 && p <= previous)", "if (k > 0 && p < previous)"),
    "histogram_skips_odd": ("for (uint64_t i = 0; i < n; i++) hist[bf16_exponent(words[i])] += 1;",
                            "for (uint64_t i = 0; i < n; i++) hist[bf16_exponent(words[i & ~1ull])] += 1;"),
}

RUNNER = r"""
import sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import oracle, oracle_pins
O = oracle.OracleLib(sys.argv[1])
for check in oracle_pins.ALL_CHECKS:
    try:
        check(O)
    except AssertionError as e:
        print("caught by", check.__name__)
        sys.exit(1)
    except Exception as e:
        print("caught by", check.__name__, type(e).__name__)
        sys.exit(1)
print("NOT CAUGHT")
sys.exit(0)
"""


def test_mutation_list_applies():
    src = open(SRC).read()
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) >= 1, name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src
    mutated = tmp_path / "szref.c"
    mutated.write_text(src.replace(old, new))
    (tmp_path / "szref.h").write_text(open(os.path.join(ROOT, "oracle", "szref.h")).read())
    lib = tmp_path / "libszref_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(lib), str(mutated)],
                   check=True)
    r = subprocess.run([sys.executable, "-c", RUNNER, str(lib), ROOT,
                        os.path.join(ROOT, "tests")],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout}\n{r.stderr}"
