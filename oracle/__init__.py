"""CPU oracle for the SplitZip BF16 container -- TEST INFRASTRUCTURE ONLY.

This package wraps ``libszref.so`` (plain single-threaded C99, built from
``szref.c`` by ``make -C oracle``) for the test suite, the smoke check and the
benchmark's CPU-baseline leg.  Nothing in the product package imports it; it
shares no code, header, table or constant with the HIP library.

What it computes (SplitZip explainers, gist.science, arXiv 2605.01708):
split each BF16 word into sign, exponent and mantissa (section "1. La
structure de la Note"); give the 16 most frequent exponents fixed 4-bit
codes packed two per byte and write every other exponent as a
(position, exponent) escape (section "3. La strategie SplitZip"); decode by
code lookup, recombination and escape overwrite (section "4. Pourquoi est-ce
rapide ?"), bit-exactly (section "Les Resultats").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libszref.so")

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_CAPACITY = 2
ERR_TOO_LARGE = 3
ERR_CORRUPT = 4

HEADER_BYTES = 160
CODEBOOK_BYTES = 16
PREFIX_BYTES = HEADER_BYTES + CODEBOOK_BYTES


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


def build() -> str:
    """Compile libszref.so with the oracle's own Makefile (gcc)."""
    subprocess.run(["make", "-s", "-C", _HERE], check=True)
    return _LIB_PATH


class OracleLib:
    """ctypes view of one build of the oracle library (the default build, or
    a copy compiled elsewhere, e.g. by the tests that plant mistakes)."""

    def __init__(self, path: str = _LIB_PATH):
        if path == _LIB_PATH and not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        L.szref_max_compressed_size.argtypes = [u64]
        L.szref_max_compressed_size.restype = u64
        L.szref_container_size.argtypes = [u64, u64]
        L.szref_container_size.restype = u64
        L.szref_exponent_histogram.argtypes = [p, u64, p]
        L.szref_exponent_histogram.restype = None
        L.szref_select_codebook.argtypes = [p, p]
        L.szref_select_codebook.restype = None
        L.szref_segment_table.argtypes = [p, u64, p]
        L.szref_segment_table.restype = None
        L.szref_escape_position.argtypes = [p, u64, ctypes.c_uint32]
        L.szref_escape_position.restype = u64
        L.szref_encode.argtypes = [p, u64, p, u64, ctypes.POINTER(u64)]
        L.szref_encode.restype = ctypes.c_int
        L.szref_decode.argtypes = [p, u64, p, u64]
        L.szref_decode.restype = ctypes.c_int
        self.L = L

    def max_compressed_size(self, n: int) -> int:
        return int(self.L.szref_max_compressed_size(n))

    def container_size(self, n: int, e: int) -> int:
        return int(self.L.szref_container_size(n, e))

    def exponent_histogram(self, words) -> np.ndarray:
        w = _words(words)
        hist = np.zeros(256, dtype=np.uint64)
        self.L.szref_exponent_histogram(_ptr(w), w.size, hist.ctypes.data)
        return hist

    def select_codebook(self, hist) -> np.ndarray:
        h = np.ascontiguousarray(hist, dtype=np.uint64)
        assert h.shape == (256,)
        cb = np.zeros(16, dtype=np.uint8)
        self.L.szref_select_codebook(h.ctypes.data, cb.ctypes.data)
        return cb

    def segment_table(self, positions) -> np.ndarray:
        pos = np.ascontiguousarray(positions, dtype=np.uint64)
        seg = np.zeros(16, dtype=np.uint64)
        self.L.szref_segment_table(_ptr(pos), pos.size, seg.ctypes.data)
        return seg

    def escape_position(self, seg_end, k: int, pos_lo: int) -> int:
        s = np.ascontiguousarray(seg_end, dtype=np.uint64)
        return int(self.L.szref_escape_position(s.ctypes.data, k, pos_lo))

    def encode_into(self, words, dst: np.ndarray) -> int:
        """Encode into a caller buffer; returns the container size in bytes."""
        w = _words(words)
        out = ctypes.c_uint64(0)
        st = self.L.szref_encode(_ptr(w), w.size, _ptr(dst), dst.size, ctypes.byref(out))
        if st != OK:
            raise OracleError(st, "szref_encode")
        return int(out.value)

    def encode(self, words) -> np.ndarray:
        """Encode a flat BF16 (uint16 bit pattern) array; returns the container."""
        w = _words(words)
        dst = np.empty(max(self.max_compressed_size(w.size), PREFIX_BYTES), dtype=np.uint8)
        size = self.encode_into(w, dst)
        return dst[:size]

    def decode_status(self, container, n: int, out: np.ndarray | None = None):
        """Decode; returns (status, words) without raising."""
        c = np.ascontiguousarray(container, dtype=np.uint8).reshape(-1)
        if out is None:
            out = np.empty(n, dtype=np.uint16)
        st = self.L.szref_decode(_ptr(c), c.size, _ptr(out), n)
        return int(st), out

    def decode(self, container, n: int, out: np.ndarray | None = None) -> np.ndarray:
        st, words = self.decode_status(container, n, out)
        if st != OK:
            raise OracleError(st, "szref_decode")
        return words


_default: OracleLib | None = None


def default() -> OracleLib:
    global _default
    if _default is None:
        _default = OracleLib()
    return _default


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data if a.size else 0


def _words(x) -> np.ndarray:
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint16:
        a = a.view(np.uint16) if a.dtype.itemsize == 2 else a.astype(np.uint16)
    return a.reshape(-1)


def max_compressed_size(n: int) -> int:
    return default().max_compressed_size(n)


def container_size(n: int, e: int) -> int:
    return default().container_size(n, e)


def exponent_histogram(words) -> np.ndarray:
    return default().exponent_histogram(words)


def select_codebook(hist) -> np.ndarray:
    return default().select_codebook(hist)


def segment_table(positions) -> np.ndarray:
    return default().segment_table(positions)


def escape_position(seg_end, k: int, pos_lo: int) -> int:
    return default().escape_position(seg_end, k, pos_lo)


def encode_into(words, dst: np.ndarray) -> int:
    return default().encode_into(words, dst)


def encode(words) -> np.ndarray:
    return default().encode(words)


def decode_status(container, n: int, out: np.ndarray | None = None):
    return default().decode_status(container, n, out)


def decode(container, n: int, out: np.ndarray | None = None) -> np.ndarray:
    return default().decode(container, n, out)
