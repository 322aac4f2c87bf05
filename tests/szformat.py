"""Independent reader of the SplitZip BF16 container, for the tests.

Written from the container definition alone (not from either encoder), with
NumPy: it splits a container into its fields so that tests can check each one
against a definition computed another way.  It is a second, separate reading
of the layout; neither the oracle nor the GPU library uses it.

Layout (little-endian):
  0 magic u32 = 0x564B5A53 | 4 version u16 = 1 | 6 element type u16 = 1
  8 N u64 | 16 E u64 | 24 total bytes u64 | 32 seg_end u64[16]
  160 codebook u8[16] | 176 nibbles u8[ceil(N/2)] (element 2j low nibble)
  then sign|mantissa u8[N] | escape pos_lo u32[E] | escape exponent u8[E]
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MAGIC = 0x564B5A53
PREFIX = 176


@dataclass
class Container:
    magic: int
    version: int
    elem_type: int
    n: int
    e: int
    total: int
    seg_end: np.ndarray     # uint64[16]
    codebook: np.ndarray    # uint8[16]
    codes: np.ndarray       # uint8[N], one 4-bit code per element
    pad_nibble: int         # high nibble of the last byte when N is odd, else 0
    sm: np.ndarray          # uint8[N]
    positions: np.ndarray   # uint64[E], full positions (segment table applied)
    pos_lo: np.ndarray      # uint32[E]
    exps: np.ndarray        # uint8[E]


def _u(buf: np.ndarray, off: int, width: int) -> int:
    return int.from_bytes(buf[off:off + width].tobytes(), "little")


def read_header(container) -> dict:
    """The fixed 176-byte prefix only: header fields and codebook."""
    b = np.ascontiguousarray(container, dtype=np.uint8).reshape(-1)
    assert b.size >= PREFIX
    return {
        "magic": _u(b, 0, 4), "version": _u(b, 4, 2), "elem_type": _u(b, 6, 2),
        "n": _u(b, 8, 8), "e": _u(b, 16, 8), "total": _u(b, 24, 8),
        "seg_end": [_u(b, 32 + 8 * s, 8) for s in range(16)],
        "codebook": [int(v) for v in b[160:176]],
    }


def read(container) -> Container:
    b = np.ascontiguousarray(container, dtype=np.uint8).reshape(-1)
    n = _u(b, 8, 8)
    e = _u(b, 16, 8)
    seg_end = np.array([_u(b, 32 + 8 * s, 8) for s in range(16)], dtype=np.uint64)
    nib_bytes = (n + 1) // 2
    nib = b[PREFIX:PREFIX + nib_bytes]
    codes = np.empty(n, dtype=np.uint8)
    codes[0::2] = nib[: (n + 1) // 2] & 0x0F
    codes[1::2] = nib[: n // 2] >> 4
    pad = int(nib[-1] >> 4) if n % 2 == 1 else 0
    sm_off = PREFIX + nib_bytes
    sm = b[sm_off:sm_off + n].copy()
    esc_off = sm_off + n
    pos_lo = b[esc_off:esc_off + 4 * e].copy().view("<u4").astype(np.uint32)
    exps = b[esc_off + 4 * e:esc_off + 5 * e].copy()
    # escape k lies in segment s where seg_end[s-1] <= k < seg_end[s]
    k = np.arange(e, dtype=np.uint64)
    seg = np.searchsorted(seg_end, k, side="right").astype(np.uint64)
    positions = (seg << np.uint64(32)) | pos_lo.astype(np.uint64)
    return Container(
        magic=_u(b, 0, 4), version=_u(b, 4, 2), elem_type=_u(b, 6, 2), n=n, e=e,
        total=_u(b, 24, 8), seg_end=seg_end, codebook=b[160:176].copy(), codes=codes,
        pad_nibble=pad, sm=sm, positions=positions, pos_lo=pos_lo, exps=exps)


# ---- definitions computed directly from the input words ---------------------

def exponents(words: np.ndarray) -> np.ndarray:
    return ((words.astype(np.uint32) >> 7) & 0xFF).astype(np.uint8)


def sign_mantissa(words: np.ndarray) -> np.ndarray:
    w = words.astype(np.uint32)
    return (((w >> 15) & 1) << 7 | (w & 0x7F)).astype(np.uint8)


def rank_of_each_exponent(hist: np.ndarray) -> np.ndarray:
    """rank(x) = #{y : h[y] > h[x] or (h[y] == h[x] and y < x)} -- the closed
    form of "most frequent first, ties toward the smaller exponent"; no sort."""
    h = hist.astype(np.uint64)
    y = np.arange(256)
    more = h[None, :] > h[:, None]
    tie_smaller = (h[None, :] == h[:, None]) & (y[None, :] < y[:, None])
    return (more | tie_smaller).sum(axis=1)


def expected_codebook(words: np.ndarray) -> np.ndarray:
    hist = np.bincount(exponents(words), minlength=256)
    rank = rank_of_each_exponent(hist)
    cb = np.zeros(16, dtype=np.uint8)
    for x in range(256):
        if rank[x] < 16:
            cb[rank[x]] = x
    return cb


def check_against_input(c: Container, words: np.ndarray) -> None:
    """Assert every field of a container follows from the input by definition."""
    words = np.ascontiguousarray(words, dtype=np.uint16).reshape(-1)
    n = words.size
    assert c.magic == MAGIC and c.version == 1 and c.elem_type == 1
    assert c.n == n
    ex = exponents(words)
    cb = expected_codebook(words)
    assert np.array_equal(c.codebook, cb), (c.codebook, cb)
    in_cb = np.zeros(256, dtype=bool)
    in_cb[cb] = True
    esc = ~in_cb[ex]
    escaped_at = np.nonzero(esc)[0].astype(np.uint64)
    assert c.e == escaped_at.size
    assert c.total == PREFIX + (n + 1) // 2 + n + 5 * c.e
    code_of = np.zeros(256, dtype=np.uint8)
    code_of[cb] = np.arange(16, dtype=np.uint8)
    want_codes = np.where(esc, 0, code_of[ex]).astype(np.uint8)
    assert np.array_equal(c.codes, want_codes)
    assert c.pad_nibble == 0
    assert np.array_equal(c.sm, sign_mantissa(words))
    assert np.array_equal(c.positions, escaped_at)
    assert np.array_equal(c.exps, ex[esc])
    seg_want = np.array([(escaped_at < (np.uint64(s + 1) << np.uint64(32))).sum()
                         for s in range(16)], dtype=np.uint64)
    assert np.array_equal(c.seg_end, seg_want)
