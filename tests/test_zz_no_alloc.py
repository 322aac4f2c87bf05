"""The allocation-free encode (sz_encode_noalloc, workspace in a fixed device
array of the library) against sz_encode, through the C ABI: two calls in a
row on the same GPU, the second with a smaller input, each container equal
to sz_encode's and to the oracle's byte for byte.  The first call takes the
single-read passes (2^26 words and more), the second the two-read passes,
so the second reuses an array the first left full of another plan's data.
Then the same call captured into a graph and replayed over changing input."""
import sys

import numpy as np
import pytest

import oracle
from test_gpu_parity import make_words

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-noalloc]", *a, flush=True)
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


def encode_with(torch, sz, fn, x, n):
    """Container of fn (sz_encode or sz_encode_noalloc) into a buffer whose
    bytes start at 0xA5, so nothing depends on a zeroed destination."""
    cap = sz.sz_max_compressed_size(n)
    dst = torch.full((cap,), 0xA5, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    fn(x, n, dst, cap, size)
    torch.cuda.synchronize()
    return dst[:int(size.item())].cpu().numpy()


@pytest.mark.parametrize("kinds", [("kv", "kv"), ("wide40", "special")])
def test_noalloc_matches_sz_encode(torch, sz, kinds):
    sizes = ((1 << 26) + 4096 + 40, (1 << 21) + 7)   # single-read form, then two-read
    assert sz.sz_encode_single_read(sizes[0]) and not sz.sz_encode_single_read(sizes[1])
    for call, (kind, n) in enumerate(zip(kinds, sizes)):
        words = make_words(kind, n, 90 + call)
        x = torch.from_numpy(words.view(np.int16)).cuda()
        say("call", call, kind, "n", n)
        got = encode_with(torch, sz, sz.sz_encode_noalloc, x, n)
        ref = encode_with(torch, sz, sz.sz_encode, x, n)
        want = oracle.encode(words)
        assert got.size == want.size, (call, got.size, want.size)
        assert np.array_equal(got, ref), call
        assert np.array_equal(got, want), call
        del x


def test_noalloc_graph_replays(torch, sz):
    n = (1 << 20) + 4096
    words = make_words("kv", n, 93)
    x = torch.from_numpy(words.view(np.int16)).cuda()
    total = oracle.encode(words).size            # the same for every permutation
    cap = sz.sz_max_compressed_size(n)
    dst = torch.zeros(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sz.sz_encode_noalloc(x, n, dst, cap, size)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sz.sz_encode_noalloc(x, n, dst, cap, size)
    rng = np.random.default_rng(94)
    for replay in range(3):
        perm = torch.from_numpy(rng.permutation(n)).cuda()
        x.copy_(x[perm])                         # eager work between replays
        size.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        now = x.cpu().numpy().view(np.uint16)
        want = oracle.encode(now)
        say("replay", replay, "size", int(size.item()))
        assert want.size == total == int(size.item())
        assert np.array_equal(dst[:total].cpu().numpy(), want), replay
