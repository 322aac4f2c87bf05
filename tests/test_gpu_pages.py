"""Paged tensors (sz_encode_pages / sz_decode_pages) against the oracle: the
container of a tensor spread over pages must equal the oracle's container
of the pages' concatenation byte for byte, decoding into pages must give
every page back bit-exactly (through each decode form, picked by escape
density), and a bad page table must touch no page."""
import sys

import numpy as np
import pytest

import oracle
from test_gpu_parity import make_words

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A


def say(*a):
    print("[gpu-pages]", *a, flush=True)
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


def paged(torch, n: int, page: int, seed: int, spare: int = 2):
    """A pool of page slots in one allocation, handed out in a shuffled
    order (as a page allocator would), filled with the sentinel; returns
    the pool, the device page table and the slot of each page."""
    used = -(-n // page)
    slots = used + spare
    pool = torch.full((slots * page,), SENTINEL, dtype=torch.int16, device="cuda")
    order = np.random.default_rng(seed).permutation(slots)[:used]
    base = pool.data_ptr()
    table = torch.tensor([base + 2 * page * int(s) for s in order], dtype=torch.int64,
                         device="cuda")
    return pool, table, order


def scatter_to_pages(torch, pool, order, words: np.ndarray, page: int):
    for i, s in enumerate(order):
        chunk = words[i * page:(i + 1) * page]
        pool[int(s) * page:int(s) * page + chunk.size] = torch.from_numpy(chunk.view(np.int16))


def gather_pages(pool, order, n: int, page: int) -> np.ndarray:
    host = pool.cpu().numpy().view(np.uint16)
    out = np.concatenate([host[int(s) * page:(int(s) + 1) * page] for s in order])
    return out[:n]


@pytest.mark.parametrize("kind,n,page", [
    ("kv", 5 * (1 << 14) + 1234, 1 << 14),       # fused decode, partial last page
    ("kv", 8 * (1 << 16), 1 << 16),              # whole pages
    ("wide40", 3 * (1 << 14) + 8, 1 << 14),      # dense decode
    ("narrow", 4 * (1 << 14) + 5, 1 << 14),      # no escapes: unpack (+ scatter)
    ("kv", (1 << 22) + 77, 1 << 14),             # 257 pages, chunks spanning pages
])
def test_pages_round_trip(torch, sz, kind, n, page):
    label = f"{kind} n={n} page={page}"
    say(label)
    words = make_words(kind, n, 41)
    pool, table, order = paged(torch, n, page, 7)
    scatter_to_pages(torch, pool, order, words, page)
    cap = sz.sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    sz.sz_encode_pages(table, table.numel(), page, n, dst, cap, size, status)
    total = int(size.item())
    assert int(status.item()) == 0, label
    want = oracle.encode(words)
    got = dst[:total].cpu().numpy()
    assert got.size == want.size and np.array_equal(got, want), label
    # decode into a fresh set of pages, in another order
    out_pool, out_table, out_order = paged(torch, n, page, 8)
    status.fill_(-1)
    sz.sz_decode_pages(dst[:total], total, out_table, out_table.numel(), page, n, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, label
    assert np.array_equal(gather_pages(out_pool, out_order, n, page), words), label
    # nothing outside the used words of the used pages was written
    host = out_pool.cpu().numpy().view(np.uint16)
    used = set(int(s) for s in out_order)
    for s in range(host.size // page):
        if s not in used:
            assert (host[s * page:(s + 1) * page] == SENTINEL).all(), (label, s)
    last = int(out_order[-1])
    tail = n - (len(out_order) - 1) * page
    assert (host[last * page + tail:(last + 1) * page] == SENTINEL).all(), label


def test_pages_flat_equivalence(torch, sz):
    """The paged container decodes with sz_decode, and a flat container
    decodes into pages."""
    n, page = 6 * (1 << 14), 1 << 14
    words = make_words("kv", n, 42)
    x = torch.from_numpy(words.view(np.int16)).cuda()
    cap = sz.sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    sz.sz_encode(x, n, dst, cap, size)
    total = int(size.item())
    pool, table, order = paged(torch, n, page, 9)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    sz.sz_decode_pages(dst[:total], total, table, table.numel(), page, n, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(gather_pages(pool, order, n, page), words)


def test_pages_bad_table_touches_nothing(torch, sz):
    n, page = 4 * (1 << 14), 1 << 14
    words = make_words("kv", n, 43)
    pool, table, order = paged(torch, n, page, 10)
    scatter_to_pages(torch, pool, order, words, page)
    cap = sz.sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for bad in (0, int(table[2].item()) + 2):     # NULL, then misaligned
        t2 = table.clone()
        t2[2] = bad
        status.fill_(-1)
        sz.sz_encode_pages(t2, t2.numel(), page, n, dst, cap, None, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 1
        # decode: a good container, a bad output table: no page is written
        good = torch.from_numpy(oracle.encode(words)).cuda()
        out_pool, out_table, out_order = paged(torch, n, page, 11)
        t3 = out_table.clone()
        t3[1] = bad
        status.fill_(-1)
        sz.sz_decode_pages(good, good.numel(), t3, t3.numel(), page, n, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 1
        assert bool((out_pool == SENTINEL).all())
