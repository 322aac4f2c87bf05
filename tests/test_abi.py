"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/splitzip.h declares, and its host-only logic (size bounds,
argument checks that return before anything touches a device) behaves as
the header states.  No kernel is launched here."""
import os
import re
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "splitzip.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sz_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def sz():
    import lossless_bf16_kv_split_amd as m
    return m


def test_header_declares_the_codec_calls():
    names = declared_functions()
    for must in ("sz_max_compressed_size", "sz_encode", "sz_decode"):
        assert must in names


def test_every_declared_symbol_is_exported(sz):
    out = subprocess.run(["nm", "-D", "--defined-only", sz.lib_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sz_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(sz._lib, n)


def test_no_oracle_in_product_library(sz):
    out = subprocess.run(["nm", "-D", sz.lib_path], capture_output=True, text=True,
                         check=True).stdout
    assert "szref" not in out
    deps = subprocess.run(["ldd", sz.lib_path], capture_output=True, text=True).stdout
    assert "szref" not in deps


def test_max_compressed_size_matches_closed_form(sz):
    for n in list(range(0, 100)) + [1 << 20, (1 << 29) + 1, 1 << 36]:
        assert sz.sz_max_compressed_size(n) == 176 + (n + 1) // 2 + n + 5 * ((15 * n) // 16)
        assert sz.sz_max_compressed_size(n) == oracle.max_compressed_size(n)
    assert sz.sz_max_compressed_size((1 << 36) + 1) == 0


def test_workspace_is_small(sz):
    assert sz.sz_workspace_size(0) > 0
    for n in (1, 4096, 1 << 21, 1 << 29, 5 << 30, 58720255, 134217727, 1 << 36):
        ws = sz.sz_workspace_size(n)
        assert 0 < ws <= 4_300_000, (n, ws)
    assert sz.sz_workspace_size((1 << 36) + 1) == 0


def test_status_strings(sz):
    for s in range(6):
        assert sz.sz_status_string(s)
    assert sz.sz_status_string(99) == "unknown status"


# Fake device addresses: the calls below must reject them on the host, before
# any HIP call, so they are never dereferenced.
A = 0x7F0000000000
MIS = A + 2


def status_of(fn, *args):
    try:
        fn(*args)
    except Exception as e:  # SplitZipError
        return e.status
    return 0


def test_encode_host_checks(sz):
    cap = sz.sz_max_compressed_size(1000)
    assert status_of(sz.sz_encode, A, (1 << 36) + 1, A + (1 << 40), 1 << 62, None, 0) == 3
    assert status_of(sz.sz_encode, A, 1000, None, cap, None, 0) == 1
    assert status_of(sz.sz_encode, None, 1000, A + (1 << 30), cap, None, 0) == 1
    assert status_of(sz.sz_encode, MIS, 1000, A + (1 << 30), cap, None, 0) == 1
    assert status_of(sz.sz_encode, A, 1000, A + (1 << 30) + 8, cap, None, 0) == 1
    assert status_of(sz.sz_encode, A, 1000, A + (1 << 30), cap - 1, None, 0) == 2
    assert status_of(sz.sz_encode, A, 1000, A + 1024, cap, None, 0) == 1      # overlap


def test_noalloc_encode_host_checks(sz):
    """The allocation-free encode makes the same host checks as sz_encode,
    and its fixed workspace holds the workspace of every size."""
    cap = sz.sz_max_compressed_size(1000)
    f = sz.sz_encode_noalloc
    assert status_of(f, A, (1 << 36) + 1, A + (1 << 40), 1 << 62, None, 0) == 3
    assert status_of(f, A, 1000, None, cap, None, 0) == 1
    assert status_of(f, MIS, 1000, A + (1 << 30), cap, None, 0) == 1
    assert status_of(f, A, 1000, A + (1 << 30), cap - 1, None, 0) == 2
    assert status_of(f, A, 1000, A + 1024, cap, None, 0) == 1                 # overlap
    for k in range(37):
        for n in ((1 << k) - 1, 1 << k, (1 << k) + 1, 3 << max(k - 2, 0)):
            if n <= 1 << 36:
                assert sz.sz_workspace_size(n) <= sz.NOALLOC_WORKSPACE_BYTES, n


def test_decode_host_checks(sz):
    n = 1000
    fixed = 176 + (n + 1) // 2 + n
    B = A + (1 << 30)
    assert status_of(sz.sz_decode, A, fixed, B, (1 << 36) + 1, None, 0) == 3
    assert status_of(sz.sz_decode, None, fixed, B, n, None, 0) == 1
    assert status_of(sz.sz_decode, A, fixed, None, n, None, 0) == 1
    assert status_of(sz.sz_decode, MIS, fixed, B, n, None, 0) == 1
    assert status_of(sz.sz_decode, A, fixed - 1, B, n, None, 0) == 4          # too short
    assert status_of(sz.sz_decode, A, fixed + 3, B, n, None, 0) == 4          # not 5E
    too_many = fixed + 5 * ((15 * n) // 16 + 1)
    assert status_of(sz.sz_decode, A, too_many, B, n, None, 0) == 4
    assert status_of(sz.sz_decode, A, fixed, A + 64, n, None, 0) == 1         # overlap
    for fn in (sz.sz_decode_unpack, sz.sz_decode_scatter):
        assert status_of(fn, A, fixed - 1, B, n, None, 0) == 4


def test_staged_host_checks(sz):
    n = 1 << 20
    ws = sz.sz_workspace_size(n)
    cap = sz.sz_max_compressed_size(n)
    W, D = A + (1 << 32), A + (1 << 33)
    assert status_of(sz.sz_encode_histogram, A, n, W, ws - 1, 0) == 1        # small workspace
    assert status_of(sz.sz_encode_histogram, A, n, W + 16, ws, 0) == 1       # misaligned
    assert status_of(sz.sz_encode_histogram, A, n, None, ws, 0) == 1
    assert status_of(sz.sz_encode_codebook, n, W, ws, D, cap - 1, None, 0) == 2
    assert status_of(sz.sz_encode_codebook, n, W, ws - 256, D, cap, None, 0) == 1
    assert status_of(sz.sz_encode_pack, A, n, W, ws, D, cap - 1, 0) == 2
    assert status_of(sz.sz_encode_pack, A, n, None, ws, D, cap, 0) == 1
    # the one-launch codebook and pack: 1 to 2^21 words only
    assert status_of(sz.sz_encode_pack_ranked, A, n, W, ws, D, cap - 1, None, 0) == 2
    assert status_of(sz.sz_encode_pack_ranked, A, n, None, ws, D, cap, None, 0) == 1
    big = (1 << 21) + 1
    assert status_of(sz.sz_encode_pack_ranked, A, big, W, sz.sz_workspace_size(big), D,
                     sz.sz_max_compressed_size(big), None, 0) == 1
    assert status_of(sz.sz_encode_pack_ranked, A, 0, W, sz.sz_workspace_size(0), D,
                     sz.sz_max_compressed_size(0), None, 0) == 1


def test_single_read_host_checks(sz):
    assert not sz.sz_encode_single_read((1 << 26) - 1)
    assert sz.sz_encode_single_read(1 << 26)
    assert sz.sz_encode_single_read(1 << 36)
    assert not sz.sz_encode_single_read((1 << 36) + 1)
    W, D = A + (1 << 32), A + (1 << 36)
    for fn, tail in ((sz.sz_encode_first_pass, (0,)), (sz.sz_encode_finish, (None, 0))):
        small = (1 << 20) - 8                                             # below the sample size
        assert status_of(fn, A, small, W, sz.sz_workspace_size(small), D,
                         sz.sz_max_compressed_size(small), *tail) == 1
        n = 1 << 20
        ws, cap = sz.sz_workspace_size(n), sz.sz_max_compressed_size(n)
        assert status_of(fn, A, n, W, ws - 1, D, cap, *tail) == 1         # small workspace
        assert status_of(fn, A, n, W, ws, D, cap - 1, *tail) == 2         # small destination
        assert status_of(fn, A, n, W, ws, D + 8, cap, *tail) == 1         # misaligned
        assert status_of(fn, A, (1 << 36) + 1, W, ws, D, cap, *tail) == 3
    small = (1 << 20) - 8
    assert status_of(sz.sz_encode_sample, A, small, W, sz.sz_workspace_size(small), 0) == 1
    n = 1 << 20
    assert status_of(sz.sz_encode_sample, A, n, W, sz.sz_workspace_size(n) - 1, 0) == 1
    assert status_of(sz.sz_encode_sample, MIS, n, W, sz.sz_workspace_size(n), 0) == 1


def test_tile_decode_host_checks(sz):
    def align(x):
        return -(-x // 256) * 256
    for n in (0, 1, 2048, 2049, 8193, 1 << 29, 5 << 30, 1 << 36):
        # u64 first record per 2048-word tile (+ end entry); a u32 fault flag
        # per index wave of 64 items for the largest E (at most 2^20
        # launched); a 64-byte record slot per tile
        tiles = -(-n // 2048)
        flags = min(-(-((15 * n) // 16 + 1) // 64), 1 << 20)
        want = align(align(align(8 * (tiles + 1)) + 4 * flags) + 64 * tiles)
        assert sz.sz_decode_workspace_size(n) == want, n
    assert sz.sz_decode_workspace_size((1 << 36) + 1) == 0
    n = 1000
    fixed = 176 + (n + 1) // 2 + n
    W, D = A + (1 << 32), A + (1 << 33)
    ws = sz.sz_decode_workspace_size(n)
    assert status_of(sz.sz_decode_index, A, fixed, n, W, ws - 1, 0) == 1          # small
    assert status_of(sz.sz_decode_index, A, fixed, n, W + 16, ws, 0) == 1         # misaligned
    assert status_of(sz.sz_decode_index, A, fixed, n, None, ws, 0) == 1
    assert status_of(sz.sz_decode_index, MIS, fixed, n, W, ws, 0) == 1
    assert status_of(sz.sz_decode_index, A, fixed + 3, n, W, ws, 0) == 4          # not 5E
    assert status_of(sz.sz_decode_index, A, fixed, n, A + 256, ws, 0) == 1        # overlap
    assert status_of(sz.sz_decode_tiles, A, fixed, W, ws - 1, D, n, None, 0) == 1
    assert status_of(sz.sz_decode_tiles, A, fixed - 1, W, ws, D, n, None, 0) == 4
    assert status_of(sz.sz_decode_tiles, A, fixed, W, ws, W + 256, n, None, 0) == 1  # overlap
    assert status_of(sz.sz_decode_tiles, A, fixed, A + 256, ws, D, n, None, 0) == 1  # with src
    assert status_of(sz.sz_decode_tiles, A, fixed, W, ws, D, (1 << 36) + 1, None, 0) == 3


def test_ship_host_checks(sz):
    import numpy as np
    n = 1000
    offs = np.zeros(n // 8 + 2, dtype=np.uint64)
    H = A + (1 << 34)  # stands in for a host buffer: never touched
    to_host, from_host = sz.sz_ship_to_host, sz.sz_ship_from_host
    assert status_of(to_host, A, (1 << 36) + 1, 64, H, 1 << 40, offs, 0) == 3
    for bad_chunk in (0, 7, 12):
        assert status_of(to_host, A, n, bad_chunk, H, 1 << 40, offs, 0) == 1
        assert status_of(from_host, H, offs, n, bad_chunk, A, None, 0) == 1
    assert status_of(to_host, A, n, 64, H, 1 << 40, None, 0) == 1
    assert status_of(to_host, A, n, 64, None, 1 << 40, offs, 0) == 1
    assert status_of(to_host, MIS, n, 64, H, 1 << 40, offs, 0) == 1
    assert status_of(from_host, H, offs, n, 64, MIS, None, 0) == 1
    # nothing to ship: the one offset is written, nothing else happens
    offs[:] = 7
    assert status_of(to_host, A, 0, 64, H, 0, offs, 0) == 0 and offs[0] == 0
    assert status_of(from_host, H, offs, 0, 64, A, None, 0) == 0
    # offsets that cannot describe containers are rejected before any copy
    chunk = 512
    sizes = [176 + chunk // 2 + chunk, 176 + (n - chunk + 1) // 2 + (n - chunk)]
    good = np.array([0, sizes[0], sizes[0] + sizes[1]], dtype=np.uint64)
    for bad in ([0, sizes[0] - 1, sizes[0] + sizes[1]],          # first too small
                [0, sizes[0] + 3, sizes[0] + 3 + sizes[1]],      # not 176 + ... + 5E
                [0, sizes[0] + sizes[1], sizes[0]]):             # out of order
        assert status_of(from_host, H, np.array(bad, dtype=np.uint64), n, chunk, A, None, 0) == 4
    assert good[-1] == sizes[0] + sizes[1]


def test_pages_host_checks(sz):
    n = 100000
    P = 1 << 14
    used = -(-n // P)
    T = A + (1 << 35)   # stands in for a device page table: never read on the host
    cap = sz.sz_max_compressed_size(n)
    D = A + (1 << 33)
    enc, dec = sz.sz_encode_pages, sz.sz_decode_pages
    assert status_of(enc, T, used, P, (1 << 36) + 1, D, 1 << 62, None, None, 0) == 3
    for bad_page in (0, 1000, 1 << 13, (1 << 14) + 8, 3 << 14):
        assert status_of(enc, T, used, bad_page, n, D, cap, None, None, 0) == 1
        assert status_of(dec, D, 1 << 20, T, used, bad_page, n, None, 0) == 1
    assert status_of(enc, T, used - 1, P, n, D, cap, None, None, 0) == 1      # too few pages
    assert status_of(enc, None, used, P, n, D, cap, None, None, 0) == 1
    assert status_of(enc, T + 4, used, P, n, D, cap, None, None, 0) == 1       # misaligned table
    assert status_of(enc, T, used, P, n, None, cap, None, None, 0) == 1
    assert status_of(enc, T, used, P, n, D + 8, cap, None, None, 0) == 1
    assert status_of(enc, T, used, P, n, D, cap - 1, None, None, 0) == 2
    fixed = 176 + (n + 1) // 2 + n
    assert status_of(dec, D, fixed - 1, T, used, P, n, None, 0) == 4
    assert status_of(dec, D, fixed + 3, T, used, P, n, None, 0) == 4
    assert status_of(dec, None, fixed, T, used, P, n, None, 0) == 1
    assert status_of(dec, D, fixed, T, used - 1, P, n, None, 0) == 1


def planned_workspace(g: int) -> int:
    """The encode workspace of g chunks before the sample area: counts
    u32[256][g], hist u64[256], bases u64[g], totals u64[4][256], escapes
    u32[g], each region 256-byte aligned."""
    align = lambda x: (x + 255) // 256 * 256
    return align(align(align(align(align(g * 1024) + 2048) + g * 8) + 8192) + g * 4)


def test_blocks_host_checks(sz):
    """The per-block calls refuse bad counts, pointers, pitches and
    workspaces on the host, and size their workspace as one encode
    workspace per block plus a flag word each."""
    import bench
    n, nb = 1 << 21, 32
    r256 = lambda x: (x + 255) // 256 * 256
    sample_area = sz.sz_workspace_size(1) - planned_workspace(1)

    def block_ws(m, count):
        # chunks planned for all the blocks' words, clamped to [2^14, a block]
        fit = 14
        while fit < 32 and (1 << fit) < m:
            fit += 1
        c = min(bench.chunk_log2(m * count), fit)
        g = -(-m >> c)
        return count * r256(planned_workspace(g) + sample_area) + r256(4 * count)

    for m, count in ((n, nb), (5000, 300), (1 << 24, 32), (1 << 24, 1), ((1 << 20) + 3, 7),
                     (0, 4), (1 << 33, 2)):
        assert sz.sz_blocks_workspace_size(m, count) == block_ws(m, count), (m, count)
    # 32 blocks of 2^24 words are counted in chunks of 2^17 words, as one
    # tensor of 2^29 words is
    assert block_ws(1 << 24, 32) < 32 * sz.sz_workspace_size(1 << 24)
    for bad in ((n, 0), (n, 65536), ((1 << 36) + 1, 1)):
        assert sz.sz_blocks_workspace_size(*bad) == 0
    T = A + (1 << 35)    # stands in for a device block table: never read on the host
    D = A + (1 << 33)
    S = A + (1 << 34)
    W = A + (1 << 36)
    cap = sz.sz_max_compressed_size(n)
    pitch = (cap + 15) // 16 * 16
    wb = sz.sz_blocks_workspace_size(n, nb)
    enc, dec = sz.sz_encode_blocks, sz.sz_decode_blocks
    assert status_of(enc, T, nb, (1 << 36) + 1, D, 1 << 60, S, W, 1 << 40, None, 0) == 3
    for args in ((T, 0, n, D, pitch, S, W, wb), (T, 65536, n, D, pitch, S, W, wb),
                 (None, nb, n, D, pitch, S, W, wb), (T + 4, nb, n, D, pitch, S, W, wb),
                 (T, nb, n, None, pitch, S, W, wb), (T, nb, n, D + 8, pitch, S, W, wb),
                 (T, nb, n, D, pitch + 8, S, W, wb), (T, nb, n, D, pitch, None, W, wb),
                 (T, nb, n, D, pitch, S + 4, W, wb), (T, nb, n, D, pitch, S, None, wb),
                 (T, nb, n, D, pitch, S, W + 128, wb), (T, nb, n, D, pitch, S, W, wb - 1)):
        assert status_of(enc, *args, None, 0) == 1, args
    assert status_of(enc, T, nb, n, D, pitch, S, W, wb, MIS, 0) == 1
    assert status_of(enc, T, nb, n, D, pitch - 16, S, W, wb, None, 0) == 2
    fixed = 176 + n // 2 + n
    assert status_of(dec, D, pitch, S, nb, n, T, None, None, 0, 0) == 1                 # status required
    assert status_of(dec, D, pitch, S, nb, n, T, MIS, None, 0, 0) == 1
    assert status_of(dec, D, (fixed - 1) // 16 * 16, S, nb, n, T, A, None, 0, 0) == 1    # no room
    assert status_of(dec, D, pitch, None, nb, n, T, A, None, 0, 0) == 1
    assert status_of(dec, D, pitch, S, 0, n, T, A, None, 0, 0) == 1
    assert status_of(dec, D, pitch, S, nb, n, None, A, None, 0, 0) == 1
    assert status_of(dec, D + 8, pitch, S, nb, n, T, A, None, 0, 0) == 1
    assert status_of(dec, D, pitch, S, nb, (1 << 36) + 1, T, A, None, 0, 0) == 3
    # the tile form's workspace: a tile index, a fault flag per 16384 words
    # (64 to 4096) and the record slots per block, at 256-byte strides
    def dws(m, count):
        tiles = -(-m // 2048)
        waves = min(max(m // 16384, 64), 4096)
        return count * r256(r256(r256(8 * (tiles + 1)) + 4 * waves) + 64 * tiles)
    for m, count in ((n, nb), (5000, 3), (1 << 24, 32), (1 << 30, 2)):
        assert sz.sz_blocks_decode_workspace_size(m, count) == dws(m, count), (m, count)
    dwb = sz.sz_blocks_decode_workspace_size(n, nb)
    for bad in ((n, 0), (n, 65536), ((1 << 36) + 1, 1)):
        assert sz.sz_blocks_decode_workspace_size(*bad) == 0
    assert status_of(dec, D, pitch, S, nb, n, T, A, W + 128, dwb, 0) == 1    # misaligned
    assert status_of(dec, D, pitch, S, nb, n, T, A, W, dwb - 1, 0) == 1      # too small


def test_bench_chunk_plan_matches_library(sz):
    """bench.py predicts the single-read finish case from its own copy of the
    encode's chunk plan; the library's workspace size (per-chunk counts and
    bases, the whole input's counts, per-chunk escape counts, then a fixed
    sample area) fixes the chunk count it planned."""
    import bench
    planned = planned_workspace
    sample_area = sz.sz_workspace_size(1) - planned(1)
    sizes = [1, 4096, 1 << 21, (1 << 25) + 123, 3 * (1 << 24) + 5, (1 << 26) - 5,
             (1 << 27) + 77, 3 << 26, 1 << 28, 1280 * (1 << 18) - 3, 1537 * (1 << 18) - 1,
             1 << 29, 5368709120, 1 << 36]
    for n in sizes:
        g = -(-n >> bench.chunk_log2(n))
        assert sz.sz_workspace_size(n) == planned(g) + sample_area, (n, g)


def test_ship_context_host_checks(sz):
    """A transfer context is refused for a chunk size the calls cannot take,
    before anything touches a device."""
    for bad in (0, 12, (1 << 36) + 8):
        with pytest.raises(sz.SplitZipError) as e:
            sz.ShipContext(bad)
        assert e.value.status == 1
    import ctypes
    assert sz._lib.sz_ship_context_create(65536, None) == 1
    sz._lib.sz_ship_context_destroy(None)   # NULL is ignored
