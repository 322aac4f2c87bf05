"""Per-layer blocks (sz_encode_blocks / sz_decode_blocks) against the oracle:
every block's container must equal the oracle's container of that block
alone, byte for byte, with its size in the size array; decoding must give
every block back bit-exactly; a bad block address or a corrupt container
must be reported for that block only, with no write outside the blocks'
own memory."""
import sys

import numpy as np
import pytest

import oracle
from test_gpu_parity import make_words

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A
FILL = 0xA5


def say(*a):
    print("[gpu-blocks]", *a, flush=True)
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


class Blocks:
    """n_blocks blocks of n words in a pool of slots (16-byte aligned, a
    guard of sentinel words after each), handed out in a shuffled order as
    a serving stack's allocator would; the device table holds each block's
    address."""

    def __init__(self, torch, n: int, n_blocks: int, seed: int):
        self.n, self.count = n, n_blocks
        self.stride = (n + 7) // 8 * 8 + 64
        self.pool = torch.full((n_blocks * self.stride + 64,), SENTINEL, dtype=torch.int16,
                               device="cuda")
        self.slot = np.random.default_rng(seed).permutation(n_blocks)
        base = self.pool.data_ptr()
        self.addr = [base + 2 * self.stride * int(s) for s in self.slot]
        self.table = torch.tensor(self.addr, dtype=torch.int64, device="cuda")

    def fill(self, torch, blocks):
        for b, w in enumerate(blocks):
            s = int(self.slot[b]) * self.stride
            if w.size:
                self.pool[s:s + w.size] = torch.from_numpy(w.view(np.int16)).cuda()

    def fill_bulk(self, torch, blocks):
        """All blocks in one copy (for many short blocks)."""
        host = np.full(self.pool.numel(), SENTINEL, dtype=np.uint16)
        for b, w in enumerate(blocks):
            s = int(self.slot[b]) * self.stride
            host[s:s + w.size] = w
        self.pool.copy_(torch.from_numpy(host.view(np.int16)))

    def read(self, b: int) -> np.ndarray:
        s = int(self.slot[b]) * self.stride
        return self.host[s:s + self.n]

    def snapshot(self):
        self.host = self.pool.cpu().numpy().view(np.uint16)
        return self.host

    def guards_intact(self) -> bool:
        h = self.host
        for s in range(self.count):
            if not (h[s * self.stride + self.n:(s + 1) * self.stride] == SENTINEL).all():
                return False
        return bool((h[self.count * self.stride:] == SENTINEL).all())


def encode_blocks(torch, sz, blk: Blocks, ws_fill: int = 0xFF, status=None):
    n, nb = blk.n, blk.count
    pitch = (sz.sz_max_compressed_size(n) + 15) // 16 * 16
    dst = torch.full((nb * pitch,), FILL, dtype=torch.uint8, device="cuda")
    sizes = torch.full((nb,), -1, dtype=torch.int64, device="cuda")
    wb = sz.sz_blocks_workspace_size(n, nb)
    ws = torch.full((wb,), ws_fill, dtype=torch.uint8, device="cuda")
    sz.sz_encode_blocks(blk.table, nb, n, dst, pitch, sizes, ws, wb, status)
    return dst, pitch, sizes


def single_read(n: int, nb: int) -> bool:
    """Whether sz_encode_blocks takes the single-read passes: 2^26 words in
    all, blocks of at least 2^20 words."""
    return n >= 1 << 20 and n * nb >= 1 << 26


FORMS = ("dense", "tiles")


def decode_blocks(torch, sz, src, pitch, sizes, nb, n, table, status, form, stream=None):
    """sz_decode_blocks in one of its forms: "dense" without a workspace,
    "tiles" with one (holding stale bytes)."""
    if form == "tiles":
        wb = sz.sz_blocks_decode_workspace_size(n, nb)
        ws = torch.full((wb,), 0x5A, dtype=torch.uint8, device="cuda")
        sz.sz_decode_blocks(src, pitch, sizes, nb, n, table, status, ws, wb, stream=stream)
        return ws
    sz.sz_decode_blocks(src, pitch, sizes, nb, n, table, status, stream=stream)
    return None


def check_containers(dst, pitch, sizes, blocks, skip=()):
    host = dst.cpu().numpy()
    sz_host = sizes.cpu().numpy().astype(np.uint64)
    n, nb = blocks[0].size, len(blocks)
    for b, w in enumerate(blocks):
        if b in skip:
            continue
        want = oracle.encode(w)
        got = host[b * pitch:b * pitch + want.size]
        assert int(sz_host[b]) == want.size, (b, int(sz_host[b]), want.size)
        assert np.array_equal(got, want), b
        # nothing past the container within the block's pitch, or, for the
        # single-read passes, past their scratch area
        tail = oracle.max_compressed_size(n) if single_read(n, nb) else want.size
        assert (host[b * pitch + tail:(b + 1) * pitch] == FILL).all(), b
    return host, sz_host


KIND_MIX = ["kv", "narrow", "random", "ties", "special", "wide40"]


@pytest.mark.parametrize("kind,n,nb", [
    ("kv", 5000, 3),               # one short chunk per block
    ("wide40", 40008, 4),          # escape heavy
    ("kv", 3 * 65536 + 1000, 5),   # several chunks, ragged last chunk
    ("mix", 70001, 6),             # a different distribution per block, odd n
    ("kv", 0, 2),                  # empty blocks: header-only containers
    ("kv", 1 << 21, 32),           # a 4 MiB layer block for each of 32 layers: single read
    ("mix", (1 << 20) + 24, 64),   # single read, every finish case among the blocks
])
def test_blocks_round_trip(torch, sz, kind, n, nb):
    label = f"{kind} n={n} blocks={nb}"
    say(label)
    kinds = [KIND_MIX[b % len(KIND_MIX)] if kind == "mix" else kind for b in range(nb)]
    words = [make_words(k, n, 50 + b) for b, k in enumerate(kinds)]
    blk = Blocks(torch, n, nb, 9)
    blk.fill(torch, words)
    status = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    dst, pitch, sizes = encode_blocks(torch, sz, blk, status=status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all(), label
    check_containers(dst, pitch, sizes, words)
    # the input is untouched
    blk.snapshot()
    for b in range(nb):
        assert np.array_equal(blk.read(b), words[b]), (label, b)

    # decode into a fresh pool in another order, in both forms
    for form in FORMS:
        out = Blocks(torch, n, nb, 10)
        dstatus = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        decode_blocks(torch, sz, dst, pitch, sizes, nb, n, out.table, dstatus, form)
        torch.cuda.synchronize()
        assert (dstatus.cpu().numpy() == 0).all(), (label, form)
        out.snapshot()
        for b in range(nb):
            assert np.array_equal(out.read(b), words[b]), (label, form, b)
        assert out.guards_intact(), (label, form)


@pytest.mark.parametrize("fill", [0x00, 0xA5, 0xFF])
@pytest.mark.parametrize("n,nb", [(3 * 65536 + 8, 4), (1 << 20, 64)])
def test_blocks_any_workspace_bytes(torch, sz, fill, n, nb):
    """The workspace may hold anything when the call starts, including the
    state a previous call on other data left (both encode forms)."""
    say("workspace fill", fill, "n", n, "blocks", nb)
    words = [make_words("kv", n, 60 + b) for b in range(nb)]
    blk = Blocks(torch, n, nb, 11)
    blk.fill(torch, words)
    pitch = (sz.sz_max_compressed_size(n) + 15) // 16 * 16
    wb = sz.sz_blocks_workspace_size(n, nb)
    ws = torch.full((wb,), fill, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        dst = torch.full((nb * pitch,), FILL, dtype=torch.uint8, device="cuda")
        sizes = torch.zeros(nb, dtype=torch.int64, device="cuda")
        sz.sz_encode_blocks(blk.table, nb, n, dst, pitch, sizes, ws, wb)
        torch.cuda.synchronize()
        check_containers(dst, pitch, sizes, words)


def test_blocks_decode_by_single_tensor_call(torch, sz):
    """A block's container is an ordinary one: sz_decode reads it, and a
    container from sz_encode decodes through sz_decode_blocks."""
    n, nb = 100000, 3
    words = [make_words("kv", n, 70 + b) for b in range(nb)]
    blk = Blocks(torch, n, nb, 12)
    blk.fill(torch, words)
    dst, pitch, sizes = encode_blocks(torch, sz, blk)
    torch.cuda.synchronize()
    s = sizes.cpu().numpy()
    for b in range(nb):
        out = torch.empty(n, dtype=torch.int16, device="cuda")
        sz.sz_decode(dst[b * pitch:], int(s[b]), out, n)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), words[b]), b
    # containers of sz_encode placed at a pitch
    flat = torch.full((nb * pitch,), 0, dtype=torch.uint8, device="cuda")
    fsizes = torch.zeros(nb, dtype=torch.int64, device="cuda")
    for b in range(nb):
        x = torch.from_numpy(words[b].view(np.int16)).cuda()
        sz.sz_encode(x, n, flat[b * pitch:], pitch, fsizes[b:])
    for form in FORMS:
        out = Blocks(torch, n, nb, 13)
        st = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        decode_blocks(torch, sz, flat, pitch, fsizes, nb, n, out.table, st, form)
        torch.cuda.synchronize()
        assert (st.cpu().numpy() == 0).all(), form
        out.snapshot()
        for b in range(nb):
            assert np.array_equal(out.read(b), words[b]), (form, b)


@pytest.mark.parametrize("n,nb", [(65536 + 40, 5), ((1 << 20) + 8, 70)])
def test_blocks_bad_address(torch, sz, n, nb):
    """A NULL or misaligned block address flags that block alone: its
    status is SZ_ERR_INVALID_ARGUMENT, its size 0, and neither call touches
    its memory; the other blocks round-trip (both encode forms)."""
    say("bad addresses, n", n, "blocks", nb)
    words = [make_words("kv", n, 80 + b) for b in range(nb)]
    blk = Blocks(torch, n, nb, 14)
    blk.fill(torch, words)
    bad = {1: 0, 3: blk.addr[3] + 2}
    for b, a in bad.items():
        blk.table[b] = a
    status = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    dst, pitch, sizes = encode_blocks(torch, sz, blk, status=status)
    torch.cuda.synchronize()
    st = status.cpu().numpy()
    want_st = [1 if b in bad else 0 for b in range(nb)]
    assert list(st) == want_st, st
    host, s = check_containers(dst, pitch, sizes, words, skip=bad.keys())
    for b in bad:
        assert int(s[b]) == 0
        assert (host[b * pitch:(b + 1) * pitch] == FILL).all(), b

    # decode the good containers into a pool whose table has the same holes;
    # the misaligned block's slot must keep its sentinels
    out = Blocks(torch, n, nb, 15)
    for b, a in bad.items():
        out.table[b] = 0 if a == 0 else out.addr[b] + 2
    dsizes = sizes.clone()
    dst2 = dst.clone()
    # the flagged blocks get valid containers, so only the address stops them
    for b in bad:
        x = torch.from_numpy(words[b].view(np.int16)).cuda()
        sz.sz_encode(x, n, dst2[b * pitch:], pitch, dsizes[b:])
    for form in FORMS:
        out.pool.fill_(SENTINEL)
        dstatus = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        decode_blocks(torch, sz, dst2, pitch, dsizes, nb, n, out.table, dstatus, form)
        torch.cuda.synchronize()
        assert list(dstatus.cpu().numpy()) == want_st, form
        out.snapshot()
        for b in range(nb):
            if b in bad:
                s0 = int(out.slot[b]) * out.stride
                assert (out.host[s0:s0 + out.stride] == SENTINEL).all(), (form, b)
            else:
                assert np.array_equal(out.read(b), words[b]), (form, b)
        assert out.guards_intact(), form


def test_blocks_corrupt_flagged(torch, sz):
    """Corrupt containers are reported for their block only: a size that is
    no container size, a size past the pitch, a header that disagrees, and
    escape records out of order."""
    n, nb = 2 * 65536 + 24, 6
    words = [make_words("wide40", n, 90 + b) for b in range(nb)]
    blk = Blocks(torch, n, nb, 16)
    blk.fill(torch, words)
    dst, pitch, sizes = encode_blocks(torch, sz, blk)
    torch.cuda.synchronize()
    s = sizes.cpu().numpy().astype(np.int64)
    host = dst.cpu().numpy()
    # the containers again at the tightest pitch, so that a size can run
    # past the pitch while still meaning a possible escape count
    tight = int(s.max() + 15) // 16 * 16
    fixed = 176 + n // 2 + n
    packed = np.zeros(nb * tight, dtype=np.uint8)
    for b in range(nb):
        packed[b * tight:b * tight + s[b]] = host[b * pitch:b * pitch + s[b]]
    s[1] -= 1                                   # not 176 + ceil(n/2) + n + 5E
    s[2] += 5 * ((tight - s[2]) // 5 + 1)       # past the pitch, E still possible
    assert s[2] > tight and (s[2] - fixed) % 5 == 0 and (s[2] - fixed) // 5 <= 15 * n // 16
    packed[4 * tight + 16] ^= 1                 # header E
    esc = 5 * tight + fixed                     # first two escape records swapped
    packed[esc:esc + 4], packed[esc + 4:esc + 8] = (packed[esc + 4:esc + 8].copy(),
                                                    packed[esc:esc + 4].copy())
    dst2 = torch.from_numpy(packed).cuda()
    sizes2 = torch.from_numpy(s).cuda()
    for form in FORMS:
        out = Blocks(torch, n, nb, 17)
        dstatus = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        decode_blocks(torch, sz, dst2, tight, sizes2, nb, n, out.table, dstatus, form)
        torch.cuda.synchronize()
        assert list(dstatus.cpu().numpy()) == [0, 4, 4, 0, 4, 4], form
        out.snapshot()
        for b in (0, 3):
            assert np.array_equal(out.read(b), words[b]), (form, b)
        assert out.guards_intact(), form


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("n,nb", [(65536 * 2 + 16, 4), (1 << 20, 64)])
def test_blocks_graph_replay(torch, sz, n, nb, form):
    """Both calls allocate nothing, so a graph can hold them: every replay,
    with other work between, gives the eager containers and words (both
    encode forms)."""
    say("graph, n", n, "blocks", nb, form)
    words = [make_words("kv", n, 100 + b) for b in range(nb)]
    blk = Blocks(torch, n, nb, 18)
    blk.fill(torch, words)
    pitch = (sz.sz_max_compressed_size(n) + 15) // 16 * 16
    wb = sz.sz_blocks_workspace_size(n, nb)
    ws = torch.full((wb,), 0xFF, dtype=torch.uint8, device="cuda")
    dst = torch.full((nb * pitch,), FILL, dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(nb, dtype=torch.int64, device="cuda")
    out = Blocks(torch, n, nb, 19)
    st = torch.zeros(nb, dtype=torch.int32, device="cuda")
    dwb = sz.sz_blocks_decode_workspace_size(n, nb)
    dws = torch.full((dwb,), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        cs = torch.cuda.current_stream()
        sz.sz_encode_blocks(blk.table, nb, n, dst, pitch, sizes, ws, wb, None, cs)
        if form == "tiles":
            sz.sz_decode_blocks(dst, pitch, sizes, nb, n, out.table, st, dws, dwb, stream=cs)
        else:
            sz.sz_decode_blocks(dst, pitch, sizes, nb, n, out.table, st, stream=cs)
    for rep in range(3):
        out.pool.fill_(SENTINEL)
        st.fill_(-1)
        sizes.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_containers(dst, pitch, sizes, words)
        assert (st.cpu().numpy() == 0).all(), rep
        out.snapshot()
        for b in range(nb):
            assert np.array_equal(out.read(b), words[b]), (rep, b)
        _ = (torch.arange(1 << 20, device="cuda") * 3).sum()   # eager work between replays


def test_blocks_full_size(torch, sz):
    """The 1 GiB Llama-3-8B-shaped KV tensor as 32 layer blocks of 2^24
    words, in the launch configuration the bench times: two sampled blocks'
    containers against the oracle, every block's container against
    sz_encode's of that block, and every block back bit-exactly."""
    import kvgen
    words = kvgen.generate("llama3_8b_kv_8k")
    nb = 32
    n = words.size // nb
    say("full size: 32 blocks of", n)
    blocks = [words[b * n:(b + 1) * n] for b in range(nb)]
    blk = Blocks(torch, n, nb, 21)
    blk.fill(torch, blocks)
    status = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    dst, pitch, sizes = encode_blocks(torch, sz, blk, status=status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    s = sizes.cpu().numpy()
    for b in (3, 30):
        want = oracle.encode(blocks[b])
        assert int(s[b]) == want.size, b
        assert np.array_equal(dst[b * pitch:b * pitch + want.size].cpu().numpy(), want), b
    one = torch.empty(pitch, dtype=torch.uint8, device="cuda")
    one_size = torch.zeros(1, dtype=torch.int64, device="cuda")
    for b in range(nb):
        x = torch.from_numpy(blocks[b].view(np.int16)).cuda()
        sz.sz_encode(x, n, one, pitch, one_size)
        torch.cuda.synchronize()
        assert int(one_size.item()) == int(s[b]), b
        assert torch.equal(one[:int(s[b])], dst[b * pitch:b * pitch + int(s[b])]), b
    del one
    for form in FORMS:
        out = Blocks(torch, n, nb, 22)
        dstatus = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        ws = decode_blocks(torch, sz, dst, pitch, sizes, nb, n, out.table, dstatus, form)
        torch.cuda.synchronize()
        assert (dstatus.cpu().numpy() == 0).all(), form
        out.snapshot()
        for b in range(nb):
            assert np.array_equal(out.read(b), blocks[b]), (form, b)
        assert out.guards_intact(), form
        del out, ws


def test_blocks_helpers(torch, sz):
    """encode_blocks / decode_blocks on a list of layer tensors: each
    container is the oracle's, the words come back, a corrupt container
    raises naming its block."""
    n, nb = 3 * 65536 + 40, 5
    words = [make_words(KIND_MIX[b % len(KIND_MIX)], n, 110 + b) for b in range(nb)]
    layers = [torch.from_numpy(w.view(np.int16)).cuda() for w in words]
    bc = sz.encode_blocks(layers)
    assert len(bc) == nb
    for b in range(nb):
        assert np.array_equal(bc.container(b).cpu().numpy(), oracle.encode(words[b])), b
    outs = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(nb)]
    sz.decode_blocks(bc, outs)
    for b in range(nb):
        assert torch.equal(outs[b], layers[b]), b
    bc.data[3 * bc.pitch + 16] ^= 1  # block 3's header E
    with pytest.raises(sz.SplitZipError) as e:
        sz.decode_blocks(bc, outs)
    assert e.value.status == 4 and "block 3" in str(e.value)


def test_blocks_maximum_count(torch, sz):
    """The largest block count a launch takes (65535, the grid's height), of
    short blocks with every distribution: every container is the oracle's
    and both decode forms give every block back."""
    n, nb = 40, 65535
    say("maximum block count", nb)
    rng = np.random.default_rng(120)
    kinds = rng.integers(0, len(KIND_MIX), nb)
    words = [make_words(KIND_MIX[int(k)], n, 121 + b) for b, k in enumerate(kinds)]
    blk = Blocks(torch, n, nb, 23)
    blk.fill_bulk(torch, words)
    status = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    dst, pitch, sizes = encode_blocks(torch, sz, blk, status=status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    check_containers(dst, pitch, sizes, words)
    for form in FORMS:
        out = Blocks(torch, n, nb, 24)
        dstatus = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        decode_blocks(torch, sz, dst, pitch, sizes, nb, n, out.table, dstatus, form)
        torch.cuda.synchronize()
        assert (dstatus.cpu().numpy() == 0).all(), form
        out.snapshot()
        got = out.host[:nb * out.stride].reshape(nb, out.stride)
        for b in range(nb):
            assert np.array_equal(got[out.slot[b], :n], words[b]), (form, b)
        assert out.guards_intact(), form


@pytest.mark.parametrize("seed", range(6))
def test_blocks_random(torch, sz, seed):
    """Random block counts, lengths (ragged, aligned or not), distributions
    and decode forms, each block against the oracle."""
    rng = np.random.default_rng([130, seed])
    nb = int(rng.integers(1, 40))
    n = int(rng.choice([int(rng.integers(1, 5000)), int(rng.integers(5000, 300000)),
                        32 * int(rng.integers(1, 9000))]))
    kinds = [KIND_MIX[int(k)] for k in rng.integers(0, len(KIND_MIX), nb)]
    say("random blocks", seed, "n", n, "blocks", nb)
    words = [make_words(k, n, 140 + 97 * seed + b) for b, k in enumerate(kinds)]
    blk = Blocks(torch, n, nb, 30 + seed)
    blk.fill(torch, words)
    dst, pitch, sizes = encode_blocks(torch, sz, blk, ws_fill=int(rng.integers(0, 256)))
    torch.cuda.synchronize()
    check_containers(dst, pitch, sizes, words)
    form = FORMS[seed % 2]
    out = Blocks(torch, n, nb, 40 + seed)
    dstatus = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    decode_blocks(torch, sz, dst, pitch, sizes, nb, n, out.table, dstatus, form)
    torch.cuda.synchronize()
    assert (dstatus.cpu().numpy() == 0).all(), form
    out.snapshot()
    for b in range(nb):
        assert np.array_equal(out.read(b), words[b]), (form, b)
    assert out.guards_intact()
