"""Pins for the CPU oracle: checks against facts that do not come from the
oracle itself -- closed forms, exhaustive enumeration, brute-force optimality,
hand-derived containers and the one worked example the SplitZip pages give.

Each ``check_*`` takes an ``oracle.OracleLib`` and raises ``AssertionError``
on a violation, so the same checks run against the real oracle
(test_oracle_pins.py) and against copies with planted mistakes
(test_oracle_mutants.py).
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

import szformat

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CORRUPT = 4


def _golden_hex(name: str) -> np.ndarray:
    """Read a golden byte file: hex pairs, '#' starts a comment."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            out.extend(int(tok, 16) for tok in line.split())
    return np.array(out, dtype=np.uint8)


def _roundtrip(O, words: np.ndarray) -> np.ndarray:
    c = O.encode(words)
    back = O.decode(c, words.size)
    assert np.array_equal(back, words), "round trip is not bit-exact"
    return c


# -- hand-derived containers (layout, nibble order, sm byte, escape record) --

def check_hand_vector_two_words(O) -> None:
    words = np.array([0x3F80, 0xC000], dtype=np.uint16)
    want = _golden_hex("two_words.hex")
    got = _roundtrip(O, words)
    assert np.array_equal(got, want), (got.tolist(), want.tolist())


def check_hand_vector_seventeen_exponents(O) -> None:
    i = np.arange(17, dtype=np.uint16)
    words = ((i & 1) << 15) | ((116 - i) << 7) | i
    want = _golden_hex("seventeen_exponents.hex")
    got = _roundtrip(O, words.astype(np.uint16))
    assert np.array_equal(got, want), (got.tolist(), want.tolist())


def check_empty_input(O) -> None:
    words = np.zeros(0, dtype=np.uint16)
    c = _roundtrip(O, words)
    assert c.size == 176
    r = szformat.read(c)
    assert r.n == 0 and r.e == 0 and r.total == 176
    assert np.array_equal(r.codebook, np.arange(16, dtype=np.uint8))
    assert not r.seg_end.any()


# -- the worked example of the pages -----------------------------------------

def check_worked_example(O) -> None:
    with open(os.path.join(GOLDEN, "worked_example_escape.json")) as f:
        g = json.load(f)
    words = np.array(g["words"], dtype=np.uint16)
    c = _roundtrip(O, words)
    r = szformat.read(c)
    got = [[int(p), int(x)] for p, x in zip(r.positions, r.exps)]
    assert got == g["expected_escapes"], got


# -- exhaustive: every BF16 bit pattern ----------------------------------------

def check_every_pattern_in_one_tensor(O) -> None:
    words = np.arange(65536, dtype=np.uint16)
    c = _roundtrip(O, words)
    r = szformat.read(c)
    # every exponent occurs 256 times: all tied, so the 16 smallest win
    assert np.array_equal(r.codebook, np.arange(16, dtype=np.uint8))
    assert r.e == 65536 - 16 * 256
    szformat.check_against_input(r, words)


def check_every_pattern_alone(O) -> None:
    """N = 1 for each of the 65536 words, compared with containers built by
    hand from the layout: the word's exponent is code 0 and the 15 smallest
    other exponents fill codes 1..15 in ascending order."""
    w = np.arange(65536, dtype=np.uint32)
    ex = (w >> 7) & 0xFF
    want = np.zeros((65536, 178), dtype=np.uint8)
    want[:, 0:4] = [0x53, 0x5A, 0x4B, 0x56]
    want[:, 4] = 1
    want[:, 6] = 1
    want[:, 8] = 1        # N = 1
    want[:, 24] = 178     # total bytes
    others = np.arange(16)[None, :15] + (np.arange(16)[None, :15] >= ex[:, None])
    want[:, 160] = ex
    want[:, 161:176] = others
    want[:, 176] = 0      # code 0, pad nibble 0
    want[:, 177] = ((w >> 15) << 7) | (w & 0x7F)
    dst = np.empty(O.max_compressed_size(1), dtype=np.uint8)
    out = np.empty(1, dtype=np.uint16)
    for v in range(65536):
        one = np.array([v], dtype=np.uint16)
        size = O.encode_into(one, dst)
        assert size == 178
        assert np.array_equal(dst[:178], want[v]), (hex(v), dst[:178].tolist())
        st, back = O.decode_status(dst[:178], 1, out)
        assert st == 0 and back[0] == v, hex(v)


# -- closed forms --------------------------------------------------------------

def check_size_closed_form(O) -> None:
    rng = np.random.default_rng(11)
    for n in list(range(0, 301)) + [1 << 16, (1 << 16) + 1]:
        words = rng.integers(0, 65536, n, dtype=np.uint16)
        c = _roundtrip(O, words)
        r = szformat.read(c)
        assert c.size == r.total == 176 + (n + 1) // 2 + n + 5 * r.e
        assert r.e <= (15 * n) // 16
        assert O.max_compressed_size(n) == 176 + (n + 1) // 2 + n + 5 * ((15 * n) // 16)
    assert O.max_compressed_size(1 << 36) > 0
    assert O.max_compressed_size((1 << 36) + 1) == 0


def check_worst_case_is_reached(O) -> None:
    """All 256 exponents equally often: exactly floor(15N/16) escapes."""
    for k in (1, 3):
        n = 256 * k
        words = (np.arange(n, dtype=np.uint32) % 256 << 7).astype(np.uint16)
        c = _roundtrip(O, words)
        assert c.size == O.max_compressed_size(n)


def check_histogram(O) -> None:
    rng = np.random.default_rng(12)
    for n in (0, 1, 7, 1000, 12345):
        words = rng.integers(0, 65536, n, dtype=np.uint16)
        h = O.exponent_histogram(words)
        want = np.bincount((words >> 7) & 0xFF, minlength=256)
        assert np.array_equal(h, want)
        assert int(h.sum()) == n


def check_codebook_rank_closed_form(O) -> None:
    rng = np.random.default_rng(13)
    cases = [np.zeros(256, dtype=np.uint64), np.full(256, 7, dtype=np.uint64)]
    for _ in range(300):
        h = rng.integers(0, 6, 256).astype(np.uint64)          # many ties
        h[rng.integers(0, 256, 20)] += rng.integers(0, 1 << 40, 20).astype(np.uint64)
        cases.append(h)
    for h in cases:
        rank = szformat.rank_of_each_exponent(h)
        want = np.zeros(16, dtype=np.uint8)
        for x in range(256):
            if rank[x] < 16:
                want[rank[x]] = x
        assert np.array_equal(O.select_codebook(h), want), (h, want)


def check_codebook_boundary_tie(O) -> None:
    """Exponents 40 and 200 tie for the 16th place: the smaller one enters."""
    h = np.zeros(256, dtype=np.uint64)
    h[100:115] = 1000 + np.arange(15)  # 15 clear winners
    h[200] = 5
    h[40] = 5
    cb = O.select_codebook(h)
    assert cb[15] == 40 and 200 not in cb.tolist()
    assert cb.tolist()[:15] == list(range(114, 99, -1))


def check_codebook_is_optimal(O) -> None:
    """Brute force over every 16-subset of an 18-exponent alphabet: no other
    codebook leaves fewer escapes than the one chosen."""
    rng = np.random.default_rng(14)
    for trial in range(25):
        alphabet = rng.choice(256, 18, replace=False)
        counts = rng.integers(1, 9, 18)
        ex = np.repeat(alphabet, counts)
        rng.shuffle(ex)
        words = ((rng.integers(0, 2, ex.size) << 15) | (ex << 7) |
                 rng.integers(0, 128, ex.size)).astype(np.uint16)
        c = _roundtrip(O, words)
        r = szformat.read(c)
        best = min(int(counts.sum() - counts[list(s)].sum())
                   for s in itertools.combinations(range(18), 16))
        assert r.e == best, (trial, r.e, best)


# -- all fields against their definitions ---------------------------------------

def check_fields_small_sweep(O) -> None:
    rng = np.random.default_rng(15)
    for n in range(0, 200):
        width = int(rng.integers(1, 48))
        lo = int(rng.integers(0, 256 - width + 1))
        ex = rng.integers(lo, lo + width, n)
        words = ((rng.integers(0, 2, n) << 15) | (ex << 7) |
                 rng.integers(0, 128, n)).astype(np.uint16)
        c = _roundtrip(O, words)
        szformat.check_against_input(szformat.read(c), words)


def check_tiny_exhaustive(O) -> None:
    """Every input of length <= 3 over 12 words that include +-0, a subnormal,
    the smallest normal, the largest finite value, +-Inf-like and NaN."""
    alphabet = [0x0000, 0x8000, 0x0001, 0x0080, 0x7F7F, 0x7F80, 0xFFC1, 0x3F80,
                0xBF80, 0x4000, 0x3F7F, 0xC2F6]
    for n in range(0, 4):
        for combo in itertools.product(alphabet, repeat=n):
            words = np.array(combo, dtype=np.uint16)
            c = _roundtrip(O, words)
            szformat.check_against_input(szformat.read(c), words)


# -- escapes beyond 2^32 -----------------------------------------------------------

def check_segment_table(O) -> None:
    T = 1 << 32
    pos = np.array([5, T - 1, T, T + 7, 3 * T + 2, 15 * T + 9], dtype=np.uint64)
    seg = O.segment_table(pos)
    want = np.array([2, 4, 4, 5] + [5] * 11 + [6], dtype=np.uint64)
    assert np.array_equal(seg, want), seg
    for k, p in enumerate(pos.tolist()):
        assert O.escape_position(seg, k, p & 0xFFFFFFFF) == p
    assert not O.segment_table(np.zeros(0, dtype=np.uint64)).any()


# -- the decoder rejects broken containers ------------------------------------------

def _escape_heavy_container(O):
    rng = np.random.default_rng(16)
    n = 333
    words = ((rng.integers(0, 2, n) << 15) | (rng.integers(90, 130, n) << 7) |
             rng.integers(0, 128, n)).astype(np.uint16)
    return words, O.encode(words)


def check_corruption_rejected(O) -> None:
    words, good = _escape_heavy_container(O)
    n = words.size
    r = szformat.read(good)
    assert r.e >= 2
    st, _ = O.decode_status(good, n)
    assert st == 0

    def bad(mutate, src_bytes=None, nn=n):
        c = good.copy()
        mutate(c)
        if src_bytes is not None:
            c = c[:src_bytes]
        st, _ = O.decode_status(c, nn)
        return st

    esc = 176 + (n + 1) // 2 + n
    assert bad(lambda c: c.__setitem__(0, c[0] ^ 1)) == CORRUPT          # magic
    assert bad(lambda c: c.__setitem__(4, 2)) == CORRUPT                 # version
    assert bad(lambda c: c.__setitem__(6, 2)) == CORRUPT                 # element type
    assert bad(lambda c: None, nn=n - 1) == CORRUPT                      # N mismatch
    assert bad(lambda c: c.__setitem__(8, c[8] ^ 1)) == CORRUPT          # N field
    assert bad(lambda c: c.__setitem__(16, c[16] ^ 1)) == CORRUPT        # E field
    assert bad(lambda c: c.__setitem__(24, c[24] ^ 1)) == CORRUPT        # total field
    assert bad(lambda c: None, src_bytes=good.size - 1) == CORRUPT       # truncated
    assert bad(lambda c: c.__setitem__(32, 0)) == CORRUPT                # seg_end[0] != E
    assert bad(lambda c: c.__setitem__(40, c[40] + 1)) == CORRUPT        # seg_end[1] != E
    big = np.frombuffer(np.uint32(n).tobytes(), dtype=np.uint8)
    assert bad(lambda c: c.__setitem__(slice(esc, esc + 4), big)) == CORRUPT  # pos >= N
    p0 = good[esc:esc + 4].copy()
    p1 = good[esc + 4:esc + 8].copy()

    def swap(c):
        c[esc:esc + 4] = p1
        c[esc + 4:esc + 8] = p0
    assert bad(swap) == CORRUPT                                            # not ascending

    def dup(c):
        c[esc + 4:esc + 8] = p0
    assert bad(dup) == CORRUPT                                             # repeated
    assert bad(lambda c: None, src_bytes=100) == CORRUPT                   # shorter than header


ALL_CHECKS = [
    check_hand_vector_two_words,
    check_hand_vector_seventeen_exponents,
    check_empty_input,
    check_worked_example,
    check_segment_table,
    check_codebook_boundary_tie,
    check_histogram,
    check_corruption_rejected,
    check_every_pattern_in_one_tensor,
    check_worst_case_is_reached,
    check_codebook_rank_closed_form,
    check_codebook_is_optimal,
    check_size_closed_form,
    check_fields_small_sweep,
    check_tiny_exhaustive,
    check_every_pattern_alone,
]
