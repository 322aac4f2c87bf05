"""GPU parity: the HIP codec against the CPU oracle, through the C ABI.

Bit-exact everywhere (the codec is integer-only): the compressed container
must equal the oracle's byte for byte, and decoding must give back every
input bit.  Both directions of cross-decoding are checked (GPU decode of the
oracle's container, oracle decode of the GPU's container).  Full-size
workloads are compared in full; the 10.7 GB one against the oracle's stored
SHA-256 (tests/golden/workload_digests.json, written by
tests/golden/make_workload_digests.py from the oracle alone)."""
import hashlib
import json
import os
import sys

import numpy as np
import pytest

import kvgen
import oracle
import szformat

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a ROCm device"
    t.cuda.set_device(0)
    return t


@pytest.fixture(scope="module")
def sz(torch):
    import lossless_bf16_kv_split_amd as m
    return m


def to_dev(torch, words: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).cuda()


def gpu_encode(torch, sz, x, n):
    cap = sz.sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    sz.sz_encode(x, n, dst, cap, size)
    total = int(size.item())
    return dst[:total]


GUARD = 64
SENTINEL = 0x5A5A


DECODE_FORMS = ("auto", "fused", "dense", "tiles", "staged")


def gpu_decode(torch, sz, container_dev, n, form="auto"):
    """Decode into a buffer with GUARD sentinel words after element n; returns
    (words tensor of n, device status, guard intact).  form: "auto" is
    sz_decode, "fused" the single pass with staged record batches, "dense" the
    single pass with a per-word exponent map, "tiles" the single pass over
    grid-stride tiles after a tile index (caller workspace), "staged" unpack
    then escape scatter."""
    out = torch.full((n + GUARD,), SENTINEL, dtype=torch.int16, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    if form == "staged":
        sz.sz_decode_unpack(container_dev, container_dev.numel(), out, n, status)
        sz.sz_decode_scatter(container_dev, container_dev.numel(), out, n, status)
    elif form == "fused":
        sz.sz_decode_fused(container_dev, container_dev.numel(), out, n, status)
    elif form == "dense":
        sz.sz_decode_dense(container_dev, container_dev.numel(), out, n, status)
    elif form == "tiles":
        ws_bytes = sz.sz_decode_workspace_size(n)
        ws = torch.full((ws_bytes,), 0x5A, dtype=torch.uint8, device="cuda")  # stale content
        sz.sz_decode_index(container_dev, container_dev.numel(), n, ws, ws_bytes)
        sz.sz_decode_tiles(container_dev, container_dev.numel(), ws, ws_bytes, out, n, status)
    else:
        sz.sz_decode(container_dev, container_dev.numel(), out, n, status)
    torch.cuda.synchronize()
    guard_ok = bool((out[n:] == SENTINEL).all().item())
    return out[:n], int(status.item()), guard_ok


# ---- inputs -------------------------------------------------------------------

def make_words(kind: str, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, n, len(kind)])
    if kind == "kv":
        return kvgen.small_kv(n, seed)
    if kind == "random":          # every exponent: escape heavy
        return rng.integers(0, 65536, n, dtype=np.uint16)
    if kind == "narrow":          # fewer than 16 distinct exponents
        e = rng.choice(np.array([3, 77, 126, 127, 200], dtype=np.uint16), n)
        return ((rng.integers(0, 2, n, dtype=np.uint16) << 15) | (e << 7) |
                rng.integers(0, 128, n, dtype=np.uint16)).astype(np.uint16)
    if kind == "wide40":          # exponents uniform over 40 values
        e = rng.integers(100, 140, n, dtype=np.uint16)
        return ((rng.integers(0, 2, n, dtype=np.uint16) << 15) | (e << 7) |
                rng.integers(0, 128, n, dtype=np.uint16)).astype(np.uint16)
    if kind == "gapped":          # 240 exponents, none = 1 (mod 16): most keys are candidates
        e = rng.integers(0, 240, n, dtype=np.uint16)
        e = (e + e // 15 + 2) % 256  # skips 1, 17, 33, ..., 241
        return ((rng.integers(0, 2, n, dtype=np.uint16) << 15) | (e << 7) |
                rng.integers(0, 128, n, dtype=np.uint16)).astype(np.uint16)
    if kind == "ties":            # 20 exponents, equal counts: tie-break decides
        e = (np.arange(n) % 20 + 110).astype(np.uint16)
        rng.shuffle(e)
        return ((e << 7) | rng.integers(0, 128, n, dtype=np.uint16)).astype(np.uint16)
    if kind == "special":         # zeros, subnormals, Inf, NaN mixed into KV
        w = kvgen.small_kv(n, seed)
        pick = rng.integers(0, 8, n)
        pay = rng.integers(1, 128, n, dtype=np.uint16)
        sign = (rng.integers(0, 2, n, dtype=np.uint16) << 15).astype(np.uint16)
        w = np.where(pick == 0, sign, w)
        w = np.where(pick == 1, sign | pay, w)
        w = np.where(pick == 2, sign | 0x7F80, w)
        w = np.where(pick == 3, sign | 0x7F80 | pay, w)
        return w.astype(np.uint16)
    raise KeyError(kind)


SIZES = [0, 1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257,
         1000, 2047, 2048, 2049, 4095, 4096, 4097, 8191, 8192, 8193, 12345, 65535, 65536,
         65537, (1 << 20) - 1, (1 << 20) + 1, 3 * (1 << 20) + 17]
KINDS = ["kv", "random", "narrow", "wide40", "ties", "special", "gapped"]


def check_case(torch, sz, words: np.ndarray, label: str):
    n = words.size
    say(label, "n =", n)
    want = oracle.encode(words)
    x = to_dev(torch, words) if n else torch.empty(0, dtype=torch.int16, device="cuda")
    got_dev = gpu_encode(torch, sz, x, n)
    got = got_dev.cpu().numpy()
    assert got.size == want.size, (label, got.size, want.size)
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError(f"{label}: {bad.size} container bytes differ, first at {bad[:8]}")
    # GPU decode (every form) of the GPU container, GPU decode of the oracle
    # container
    for form in DECODE_FORMS:
        y, st, guard = gpu_decode(torch, sz, got_dev, n, form)
        assert st == 0 and guard, (label, form, st, guard)
        assert torch.equal(y, x), (label, form)
    y2, st2, guard2 = gpu_decode(torch, sz, torch.from_numpy(want).cuda(), n)
    assert st2 == 0 and guard2 and torch.equal(y2, x), label
    # oracle decode of the GPU container
    assert np.array_equal(oracle.decode(got, n), words), label


@pytest.mark.parametrize("kind", KINDS)
def test_small_sizes(torch, sz, kind):
    for i, n in enumerate(SIZES):
        check_case(torch, sz, make_words(kind, n, 1000 + i), f"{kind}")


def test_every_pattern(torch, sz):
    words = np.arange(65536, dtype=np.uint16)
    check_case(torch, sz, words, "all 65536 patterns")
    rng = np.random.default_rng(5)
    check_case(torch, sz, rng.permutation(np.tile(words, 7)), "all patterns x7 shuffled")


def test_worked_example(torch, sz):
    with open(os.path.join(GOLDEN, "worked_example_escape.json")) as f:
        g = json.load(f)
    words = np.array(g["words"], dtype=np.uint16)
    check_case(torch, sz, words, "worked example")
    got = gpu_encode(torch, sz, to_dev(torch, words), words.size).cpu().numpy()
    r = szformat.read(got)
    assert [[int(p), int(e)] for p, e in zip(r.positions, r.exps)] == g["expected_escapes"]


def test_many_chunks_ragged(torch, sz):
    # more than 2048 minimum-size chunks: larger chunks, a ragged last chunk;
    # from 2^26 words the single-read encode
    for n in (2048 * 16384 + 123, 3 * (1 << 24) + 5, (1 << 26) - 5, (1 << 26) + 3 * 16384,
              8192 * 16384 + 77):
        check_case(torch, sz, make_words("kv", n, 7), "many chunks kv")


@pytest.mark.parametrize("n", [(1 << 22) + 16385, (1 << 26) + 3 * 16384 + 1])
def test_gapped_exponents(torch, sz, n):
    """Exponents of 240 values, none of them 1 modulo 16, in a 256-workgroup
    codebook pass (257 chunks) and in the single-read encode (sample, first
    pass, finish): the ranking's shortcut (about 16 keys near the top) does
    not apply and every key is ranked against all 256."""
    check_case(torch, sz, make_words("gapped", n, 11), "gapped")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("n", [1280 * (1 << 18) - 3, 1537 * (1 << 18) - 1, (1 << 29) - 3])
def test_halved_chunk_plans(torch, sz, n):
    """Plans that halve 2^18-word chunks: 2560 and 3074 chunks of 2^17 words
    (a fuller last wave of pack workgroups), whose counts the select reads
    three and four chunks per thread in two rounds, and 4096 (more than 3072,
    a multiple of 4), read four chunks per 16-byte load; each with a ragged
    last chunk."""
    words = make_words("kv", n, 9)
    want = oracle.encode(words)
    x = to_dev(torch, words)
    got = gpu_encode(torch, sz, x, n).cpu().numpy()
    assert got.size == want.size and np.array_equal(got, want), n
    y, status, guard_ok = gpu_decode(torch, sz, torch.from_numpy(want).cuda(), n)
    assert status == 0 and guard_ok and torch.equal(y, x), n
    check_case(torch, sz, make_words("wide40", 2048 * 16384 + 5, 8), "many chunks wide40")


def sha256(a: np.ndarray) -> str:
    h = hashlib.sha256()
    mv = memoryview(np.ascontiguousarray(a).reshape(-1).view(np.uint8))
    for i in range(0, len(mv), 1 << 28):
        h.update(mv[i:i + (1 << 28)])
    return h.hexdigest()


def digests():
    with open(os.path.join(GOLDEN, "workload_digests.json")) as f:
        return json.load(f)


def two_read_encode(torch, sz, x, n):
    """The staged two-read encode (histogram, codebook, pack) over a caller
    workspace; returns the container on the device."""
    ws_bytes = sz.sz_workspace_size(n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    cap = sz.sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    sz.sz_encode_histogram(x, n, ws, ws_bytes)
    sz.sz_encode_codebook(n, ws, ws_bytes, dst, cap, size)
    sz.sz_encode_pack(x, n, ws, ws_bytes, dst, cap)
    return dst[:int(size.item())]


@pytest.mark.parametrize("kind", ["kv", "random", "ties", "gapped", "narrow"])
def test_staged_ranked_pack(torch, sz, kind):
    """sz_encode_histogram then sz_encode_pack_ranked (the two-launch encode
    sz_encode takes for 1 to 2^21 words) over a workspace that comes in
    filled with other bytes, twice in a row on it: the oracle's container
    and size each time, and the same as the three staged passes."""
    for i, n in enumerate([1, 17, 16384, 16385, 3 * 16384 + 7, (1 << 20) + 5, 1 << 21]):
        words = make_words(kind, n, 300 + i)
        want = oracle.encode(words)
        x = to_dev(torch, words)
        ws_bytes = sz.sz_workspace_size(n)
        ws = torch.full((ws_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
        cap = sz.sz_max_compressed_size(n)
        for rep in range(2):
            dst = torch.full((cap,), 0x3C, dtype=torch.uint8, device="cuda")
            size = torch.zeros(1, dtype=torch.int64, device="cuda")
            sz.sz_encode_histogram(x, n, ws, ws_bytes)
            sz.sz_encode_pack_ranked(x, n, ws, ws_bytes, dst, cap, size)
            total = int(size.item())
            assert total == want.size, (kind, n, rep, total, want.size)
            assert np.array_equal(dst[:total].cpu().numpy(), want), (kind, n, rep)
        three = two_read_encode(torch, sz, x, n).cpu().numpy()
        assert np.array_equal(three, want), (kind, n)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["single_layer_kv", "llama3_8b_kv_8k", "escape_heavy",
                                  "special_values"])
def test_workload_full(torch, sz, name):
    say("workload", name)
    words = kvgen.generate(name)
    d = digests()[name]
    assert sha256(words) == d["input_sha256"], "input generator drifted"
    x = to_dev(torch, words)
    got_dev = gpu_encode(torch, sz, x, words.size)
    got = got_dev.cpu().numpy()
    want = oracle.encode(words)
    assert got.size == want.size == d["container_bytes"]
    assert np.array_equal(got, want), f"{name}: container differs from the oracle"
    assert sha256(got) == d["container_sha256"]
    # the two-read form too (for the 1 GiB tensor, on its 4096-chunk plan)
    two = two_read_encode(torch, sz, x, words.size).cpu().numpy()
    assert np.array_equal(two, want), f"{name}: two-read container differs from the oracle"
    del two
    for form in DECODE_FORMS:
        y, st, guard = gpu_decode(torch, sz, got_dev, words.size, form)
        assert st == 0 and guard and torch.equal(y, x), (name, form)
        del y
    assert np.array_equal(oracle.decode(got, words.size), words)


@pytest.mark.slow
@pytest.mark.timeout(1100)
def test_workload_70b_32k(torch, sz):
    """10.7 GB, more than 2^32 elements: two position segments."""
    name = "llama3_70b_kv_32k"
    d = digests()[name]
    say("workload", name, "generate")
    words = kvgen.generate(name)
    assert words.size > (1 << 32)
    assert sha256(words) == d["input_sha256"], "input generator drifted"
    say("upload")
    x = to_dev(torch, words)
    del words
    say("encode")
    got_dev = gpu_encode(torch, sz, x, x.numel())
    assert got_dev.numel() == d["container_bytes"]
    say("header")
    h = szformat.read_header(got_dev[:176].cpu().numpy())
    assert h["magic"] == szformat.MAGIC and h["n"] == d["n"]
    assert h["e"] == d["escapes"] and h["total"] == d["container_bytes"]
    assert h["codebook"] == d["codebook"]
    assert h["seg_end"] == d["seg_end"]
    assert h["seg_end"][0] < h["e"], "escapes on both sides of 2^32 expected"
    say("digest")
    assert sha256(got_dev.cpu().numpy()) == d["container_sha256"]
    say("two-read encode")
    two = two_read_encode(torch, sz, x, x.numel())
    assert two.numel() == d["container_bytes"]
    assert sha256(two.cpu().numpy()) == d["container_sha256"], "two-read container differs"
    del two
    for form in DECODE_FORMS:
        say("decode", form)
        y, st, guard = gpu_decode(torch, sz, got_dev, x.numel(), form)
        assert st == 0 and guard, (form, st, guard)
        assert torch.equal(y, x), form
        del y


def test_staged_calls_match_encode(torch, sz):
    words = kvgen.generate("single_layer_kv")
    n = words.size
    x = to_dev(torch, words)
    ws_bytes = sz.sz_workspace_size(n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    cap = sz.sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    sz.sz_encode_histogram(x, n, ws, ws_bytes)
    sz.sz_encode_codebook(n, ws, ws_bytes, dst, cap, size)
    sz.sz_encode_pack(x, n, ws, ws_bytes, dst, cap)
    staged = dst[: int(size.item())].cpu().numpy()
    assert np.array_equal(staged, oracle.encode(words))
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    c = dst[: int(size.item())]
    sz.sz_decode_unpack(c, c.numel(), out, n, status)
    sz.sz_decode_scatter(c, c.numel(), out, n, status)
    assert int(status.item()) == 0 and torch.equal(out, x)


def test_deterministic_and_streams(torch, sz):
    words = kvgen.generate("escape_heavy")[: 1 << 24]
    n = words.size
    x = to_dev(torch, words)
    first = gpu_encode(torch, sz, x, n).clone()
    for _ in range(5):
        assert torch.equal(gpu_encode(torch, sz, x, n), first)
    # two encodes at once on two streams
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    cap = sz.sz_max_compressed_size(n)
    d1 = torch.empty(cap, dtype=torch.uint8, device="cuda")
    d2 = torch.empty(cap, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        sz.sz_encode(x, n, d1, cap, None, s1)
        sz.sz_encode(x, n, d2, cap, None, s2)
    torch.cuda.synchronize()
    m = first.numel()
    assert torch.equal(d1[:m], first) and torch.equal(d2[:m], first)


def test_corrupt_containers_flagged_on_device(torch, sz):
    rng = np.random.default_rng(16)
    n = 5000
    words = ((rng.integers(0, 2, n) << 15) | (rng.integers(90, 130, n) << 7) |
             rng.integers(0, 128, n)).astype(np.uint16)
    good = oracle.encode(words)
    r = szformat.read(good)
    assert r.e > 10
    esc = 176 + (n + 1) // 2 + n

    def status(c):
        sts = []
        for form in DECODE_FORMS:
            _, st, guard = gpu_decode(torch, sz, torch.from_numpy(c).cuda(), n, form)
            assert guard, "decode wrote past element n"
            sts.append(st)
        assert len(set(sts)) == 1, sts
        return sts[0]

    assert status(good) == 0
    cases = {
        "magic": (0, good[0] ^ 1), "version": (4, 2), "type": (6, 2), "n": (8, good[8] ^ 1),
        "e": (16, good[16] ^ 1), "total": (24, good[24] ^ 1), "seg_end0": (32, 0),
        "seg_end1": (40, good[40] + 1),
    }
    for what, (off, val) in cases.items():
        c = good.copy()
        c[off] = val
        assert status(c) == 4, what
    for what, pos in {"pos >= n": n, "pos = 2^32 - 1": 0xFFFFFFFF}.items():
        c = good.copy()
        c[esc + 4 * 3:esc + 4 * 4] = np.frombuffer(np.uint32(pos).tobytes(), np.uint8)
        assert status(c) == 4, what
    c = good.copy()
    c[esc:esc + 4], c[esc + 4:esc + 8] = good[esc + 4:esc + 8].copy(), good[esc:esc + 4].copy()
    assert status(c) == 4, "not ascending"
    c = good.copy()
    last = esc + 4 * (r.e - 1)
    c[last:last + 4] = c[last - 4:last]
    assert status(c) == 4, "last repeats"


def test_corrupt_escapes_many_ranges(torch, sz):
    """Escape-dense input over many decode ranges and record batches: an
    out-of-order record deep inside is flagged by both decode forms, and
    neither writes past the output."""
    n = 3 * 8192 * 7 + 5
    words = make_words("wide40", n, 21)
    good = oracle.encode(words)
    r = szformat.read(good)
    assert r.e > 4096 * 3
    esc = 176 + (n + 1) // 2 + n
    for k in (1, 4095, 4096, 4097, r.e // 2, r.e - 1):
        c = good.copy()
        a, b = esc + 4 * (k - 1), esc + 4 * k
        c[a:a + 4], c[b:b + 4] = good[b:b + 4].copy(), good[a:a + 4].copy()
        for form in DECODE_FORMS:
            _, st, guard = gpu_decode(torch, sz, torch.from_numpy(c).cuda(), n, form)
            assert guard and st == 4, (k, form, st)


@pytest.mark.parametrize("kind", ["wide40", "kv"])
def test_corrupt_escapes_dense_slices(torch, sz, kind):
    """The dense decode with a 16-byte aligned escape stream (n a multiple of
    32) and two sub-ranges per range: escape-dense input (sub-range bounds
    searched, records spread over the waves' slices) and sparse KV input
    (the range's records read whole for each sub-range).  Records swapped
    with their successor right at a sub-range's first record, at lane,
    step and wave-slice boundaries of its slices, and deep inside are each
    flagged, and the intact container decodes exactly."""
    n = (1 << 27) + (1 << 15)
    say("dense slices", kind, n)
    words = make_words(kind, n, 22)
    good = oracle.encode(words)
    r = szformat.read(good)
    esc = 176 + n // 2 + n
    assert esc % 16 == 0
    pos = np.frombuffer(good[esc:esc + 4 * r.e].tobytes(), dtype=np.uint32).astype(np.int64)
    dev = torch.from_numpy(good).cuda()
    out, st, guard = gpu_decode(torch, sz, dev, n, "dense")
    assert st == 0 and guard and np.array_equal(out.cpu().numpy().view(np.uint16), words)
    # the second sub-range (16384 words) of range 100 (32768 words)
    sub = 100 * 32768 + 16384
    k0 = int(np.searchsorted(pos, sub))
    k1 = int(np.searchsorted(pos, sub + 16384))
    s0 = k0 & ~3
    per_wave = max(256, -(-(k1 - s0) // 32) * 4)
    picks = {k0, k0 + 1, k0 + 3, k0 + 4, s0 + 255, s0 + 256, s0 + 257, s0 + per_wave - 1,
             s0 + per_wave, s0 + per_wave + 1, k1 - 1, r.e // 2, r.e - 1}
    for k in sorted(x for x in picks if 1 <= x < r.e):
        c = good.copy()
        a, b = esc + 4 * (k - 1), esc + 4 * k
        c[a:a + 4], c[b:b + 4] = good[b:b + 4].copy(), good[a:a + 4].copy()
        dev.copy_(torch.from_numpy(c))
        _, st, guard = gpu_decode(torch, sz, dev, n, "dense")
        assert guard and st == 4, (kind, k, st)


def test_host_errors_with_real_buffers(torch, sz):
    n = 4096
    x = torch.zeros(n, dtype=torch.int16, device="cuda")
    cap = sz.sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    with pytest.raises(sz.SplitZipError) as e:
        sz.sz_encode(x, n, dst, cap - 1)
    assert e.value.status == 2
    with pytest.raises(sz.SplitZipError) as e:
        sz.sz_encode(x[1:], n - 1, dst, cap)
    assert e.value.status == 1
    c = sz.encode(x)
    with pytest.raises(sz.SplitZipError) as e:
        sz.sz_decode(c, c.numel() - 1, x, n)
    assert e.value.status == 4
