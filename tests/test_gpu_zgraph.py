"""The staged encode calls (both forms) and the single-pass decode captured in a HIP graph
(torch.cuda.CUDAGraph on ROCm) and replayed: every replay must give the
oracle's container of the input as it is at that replay, and decode it
bit-exactly.  Between replays the input is permuted in place (eager work on
the device): a permutation keeps the exponent histogram, hence the
container size the captured decode call was given, while changing every
byte of the nibble, sign|mantissa and escape streams."""
import sys

import numpy as np
import pytest

import oracle
from test_gpu_parity import make_words

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-graph]", *a, flush=True)
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


@pytest.mark.parametrize("kind,form,single", [("kv", "fused", False), ("wide40", "dense", False),
                                              ("kv", "auto", False), ("narrow", "auto", False),
                                              ("kv", "auto", True), ("wide40", "auto", True),
                                              ("kv", "tiles", True)])
def test_graph_replays(torch, sz, kind, form, single):
    n = (1 << 20) + 4096
    words = make_words(kind, n, 51)
    x = torch.from_numpy(words.view(np.int16)).cuda()
    total = oracle.encode(words).size          # the same for every permutation
    ws_bytes = sz.sz_workspace_size(n)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    cap = sz.sz_max_compressed_size(n)
    dst = torch.zeros(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    dws_bytes = sz.sz_decode_workspace_size(n)
    dws = torch.zeros(dws_bytes, dtype=torch.uint8, device="cuda")

    def tiles(c, total_, out_, n_, status_):
        sz.sz_decode_index(c, total_, n_, dws, dws_bytes)
        sz.sz_decode_tiles(c, total_, dws, dws_bytes, out_, n_, status_)

    decode = {"fused": sz.sz_decode_fused, "dense": sz.sz_decode_dense, "auto": sz.sz_decode,
              "tiles": tiles}[form]

    def codec():
        if single:                                # the single-read passes
            sz.sz_encode_sample(x, n, ws, ws_bytes)
            sz.sz_encode_first_pass(x, n, ws, ws_bytes, dst, cap)
            sz.sz_encode_finish(x, n, ws, ws_bytes, dst, cap, size)
        else:
            sz.sz_encode_histogram(x, n, ws, ws_bytes)
            sz.sz_encode_codebook(n, ws, ws_bytes, dst, cap, size)
            sz.sz_encode_pack(x, n, ws, ws_bytes, dst, cap)
        decode(dst[:total], total, out, n, status)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        codec()                                   # one eager run on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        codec()
    rng = np.random.default_rng(52)
    for replay in range(4):
        perm = torch.from_numpy(rng.permutation(n)).cuda()
        x.copy_(x[perm])                          # eager work between replays
        out.zero_()
        status.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        now = x.cpu().numpy().view(np.uint16)
        want = oracle.encode(now)
        say(kind, form, "single" if single else "two-read", "replay", replay, "size",
            int(size.item()))
        assert want.size == total
        assert int(size.item()) == total
        assert np.array_equal(dst[:total].cpu().numpy(), want), (kind, form, replay)
        assert int(status.item()) == 0, (kind, form, replay)
        assert torch.equal(out, x), (kind, form, replay)


def test_pool_calls_refused_under_capture(torch, sz):
    """sz_encode, sz_encode_pages and sz_decode_pages take memory from the
    library pool, so under capture they return SZ_ERR_INVALID_ARGUMENT and
    launch nothing; sz_decode captures its workspace-free dense form, which
    replays to the oracle's words."""
    n = (1 << 20) + 4096
    page = 1 << 16
    words = make_words("kv", n, 55)
    want = oracle.encode(words)
    x = torch.from_numpy(words.view(np.int16)).cuda()
    cap = sz.sz_max_compressed_size(n)
    dst = torch.full((cap,), 0x3C, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    pages = -(-n // page)
    pool = torch.zeros(pages * page, dtype=torch.int16, device="cuda")
    table = torch.tensor([pool.data_ptr() + 2 * page * i for i in range(pages)],
                         dtype=torch.int64, device="cuda")
    container = torch.from_numpy(want).cuda()
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    refused = []
    with torch.cuda.graph(graph):
        for name, call in (
                ("sz_encode", lambda: sz.sz_encode(x, n, dst, cap, size)),
                ("sz_encode_pages", lambda: sz.sz_encode_pages(table, pages, page, n, dst, cap,
                                                               size, status)),
                ("sz_decode_pages", lambda: sz.sz_decode_pages(container, want.size, table,
                                                               pages, page, n, status))):
            try:
                call()
            except sz.SplitZipError as e:
                refused.append((name, e.status))
        sz.sz_decode(container, want.size, out, n, status)
    say("refused under capture:", refused)
    assert refused == [("sz_encode", 1), ("sz_encode_pages", 1), ("sz_decode_pages", 1)]
    for replay in range(2):
        out.zero_()
        status.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, replay
        assert torch.equal(out, x), replay
        assert int(size.item()) == 0                       # no encode ran
        assert bool((dst == 0x3C).all().item())
        assert bool((pool == 0).all().item())              # no page written
