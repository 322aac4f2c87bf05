"""Compressed transfer to and from pinned host memory (sz_ship_to_host /
sz_ship_from_host) against the oracle: every chunk's container must equal
the oracle's container of that chunk byte for byte, and the words must come
back bit-exactly; capacity and corruption are reported as the header says."""
import sys

import numpy as np
import pytest

import oracle
from test_gpu_parity import make_words

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-ship]", *a, flush=True)
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


def ship_round_trip(torch, sz, words: np.ndarray, chunk: int, label: str):
    n = words.size
    say(label, "n", n, "chunk", chunk)
    x = torch.from_numpy(words.view(np.int16)).cuda()
    chunks = -(-n // chunk)
    cap = sum(sz.sz_max_compressed_size(min(chunk, n - c * chunk)) for c in range(chunks))
    host = torch.empty(max(cap, 1), dtype=torch.uint8, pin_memory=True)
    offs = np.zeros(chunks + 1, dtype=np.uint64)
    sz.sz_ship_to_host(x, n, chunk, host, cap, offs)
    hb = host.numpy()
    for c in range(chunks):
        want = oracle.encode(words[c * chunk:(c + 1) * chunk])
        got = hb[int(offs[c]):int(offs[c + 1])]
        assert got.size == want.size and np.array_equal(got, want), (label, c)
    out = torch.full((n + 64,), 0x5A5A, dtype=torch.int16, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    sz.sz_ship_from_host(host, offs, n, chunk, out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, label
    assert torch.equal(out[:n], x), label
    assert bool((out[n:] == 0x5A5A).all()), label
    return host, offs


@pytest.mark.parametrize("kind,n,chunk", [
    ("kv", 3 * 65536 + 1000, 65536),     # ragged last chunk
    ("kv", 4 * 65536, 65536),            # whole chunks
    ("kv", 5000, 65536),                 # one short chunk
    ("wide40", 2 * 40000 + 8, 40000),    # escape-heavy, chunk not a power of two
    ("kv", 1 << 22, 1 << 20),            # several sizeable chunks
    ("kv", (1 << 26) + 4104, 1 << 26),   # a chunk encoded in the single-read form
])
def test_ship_round_trip(torch, sz, kind, n, chunk):
    ship_round_trip(torch, sz, make_words(kind, n, 31), chunk, f"{kind} {n}/{chunk}")


def test_ship_capacity(torch, sz):
    n, chunk = 3 * 65536, 65536
    words = make_words("kv", n, 32)
    x = torch.from_numpy(words.view(np.int16)).cuda()
    first = oracle.encode(words[:chunk]).size
    host = torch.empty(first + 100, dtype=torch.uint8, pin_memory=True)
    offs = np.zeros(4, dtype=np.uint64)
    with pytest.raises(sz.SplitZipError) as e:
        sz.sz_ship_to_host(x, n, chunk, host, first + 100, offs)
    assert e.value.status == 2
    # the chunk that fitted was shipped and its offset written
    assert int(offs[1]) == first
    assert np.array_equal(host.numpy()[:first], oracle.encode(words[:chunk]))


def test_ship_corrupt_chunk_flagged(torch, sz):
    n, chunk = 3 * 65536, 65536
    words = make_words("wide40", n, 33)
    host, offs = ship_round_trip(torch, sz, words, chunk, "before corruption")
    # swap two escape records of the middle chunk: positions out of order
    hb = host.numpy()
    base = int(offs[1])
    esc = base + 176 + chunk // 2 + chunk
    a, b = esc + 4 * 10, esc + 4 * 11
    hb[a:a + 4], hb[b:b + 4] = hb[b:b + 4].copy(), hb[a:a + 4].copy()
    out = torch.empty(n + 64, dtype=torch.int16, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(sz.SplitZipError) as e:
        sz.sz_ship_from_host(host, offs, n, chunk, out, status)
    assert e.value.status == 4
    assert int(status.item()) == 4


def test_ship_context_reused(torch, sz):
    """One transfer context serves several transfers of different sizes, both
    ways, each container the oracle's; a later decode with more chunks than
    any before it still reports a corrupt chunk."""
    chunk = 65536
    ctx = sz.ShipContext(chunk)
    try:
        for i, (kind, n) in enumerate([("kv", 3 * chunk + 1000), ("wide40", chunk - 8),
                                       ("kv", 9 * chunk + 24)]):
            label = f"context {kind} {n}"
            say(label)
            words = make_words(kind, n, 40 + i)
            x = torch.from_numpy(words.view(np.int16)).cuda()
            chunks = -(-n // chunk)
            cap = sum(sz.sz_max_compressed_size(min(chunk, n - c * chunk)) for c in range(chunks))
            host = torch.empty(cap, dtype=torch.uint8, pin_memory=True)
            offs = np.zeros(chunks + 1, dtype=np.uint64)
            ctx.to_host(x, n, host, cap, offs)
            hb = host.numpy()
            for c in range(chunks):
                want = oracle.encode(words[c * chunk:(c + 1) * chunk])
                assert np.array_equal(hb[int(offs[c]):int(offs[c + 1])], want), (label, c)
            out = torch.full((n + 64,), 0x5A5A, dtype=torch.int16, device="cuda")
            status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            ctx.from_host(host, offs, n, out, status)
            torch.cuda.synchronize()
            assert int(status.item()) == 0 and torch.equal(out[:n], x), label
            assert bool((out[n:] == 0x5A5A).all()), label
        # the last tensor again, its fifth chunk's escape records swapped
        base = int(offs[4])
        esc = base + 176 + chunk // 2 + chunk
        e = (int(offs[5]) - esc) // 5
        assert e >= 2
        hb[esc:esc + 4], hb[esc + 4:esc + 8] = hb[esc + 4:esc + 8].copy(), hb[esc:esc + 4].copy()
        status.fill_(-1)
        with pytest.raises(sz.SplitZipError) as err:
            ctx.from_host(host, offs, n, out, status)
        assert err.value.status == 4 and int(status.item()) == 4
    finally:
        ctx.close()
