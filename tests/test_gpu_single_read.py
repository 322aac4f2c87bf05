"""The single-read encode, case by case.

sz_encode_sample; sz_encode_first_pass; sz_encode_finish (what sz_encode
runs from 2^26 words on) read the input once when they can: the first pass
packs every chunk with a provisional codebook ranked from a fixed sample of
the input (512 blocks of 2048 words, block j at the 2048-word boundary at or
below j * n / 512) while it counts the exact exponents; the finish pass
ranks the exact codebook and keeps what the first one wrote (same codes), remaps the 4-bit codes (same
16 exponents in another order), or packs again (another set, a chunk with
more escapes than its scratch slots, or a sample that predicted too many
escapes).  Whatever the case, the container must be the oracle's, byte for
byte.

Each input below is built to land in one case; the test works the case out
on the host from the same sample rule and the oracle's codebook rule, and
checks that the input does land there, so that every branch of the finish
pass is exercised."""
import sys

import numpy as np
import pytest

import bench
import kvgen
import oracle
from test_gpu_parity import make_words
from test_gpu_pages import gather_pages, paged, scatter_to_pages

pytestmark = pytest.mark.gpu

SAMPLE_BLOCKS = 512
SAMPLE_BLOCK_WORDS = 2048


def say(*a):
    print("[gpu-single-read]", *a, flush=True)
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


def exponents(words: np.ndarray) -> np.ndarray:
    return ((words >> 7) & 0xFF).astype(np.int64)


def sample_starts(n: int) -> np.ndarray:
    j = np.arange(SAMPLE_BLOCKS, dtype=np.int64)
    return (j * (n // SAMPLE_BLOCKS)) // SAMPLE_BLOCK_WORDS * SAMPLE_BLOCK_WORDS


def expected_case(words: np.ndarray) -> str:
    """Which branch the last pass takes for these words."""
    n = words.size
    idx = (sample_starts(n)[:, None] + np.arange(SAMPLE_BLOCK_WORDS)[None, :]).ravel()
    sample_hist = np.bincount(exponents(words[idx]), minlength=256).astype(np.uint64)
    prov = oracle.select_codebook(sample_hist)
    total = int(sample_hist.sum())
    top = int(sample_hist[prov.astype(np.int64)].sum())
    if (total - top) * 32 > total:
        return "full:sample"
    c = bench.chunk_log2(n)                  # the library's chunk plan
    esc = ~np.isin(exponents(words), prov.astype(np.int64))
    per_chunk = np.add.reduceat(esc.astype(np.int64), np.arange(0, n, 1 << c))
    if per_chunk.max() > (1 << c) // 16:
        return "full:overflow"
    exact = oracle.select_codebook(np.bincount(exponents(words), minlength=256).astype(np.uint64))
    if set(prov.tolist()) != set(exact.tolist()):
        return "full:set"
    return "copy" if np.array_equal(prov, exact) else "remap"


def pattern(n: int, seed: int, frequent: list, rare_rate: float) -> np.ndarray:
    """Random signs and mantissas; exponents drawn uniformly from `frequent`,
    except a `rare_rate` share drawn from 60 rare values."""
    rng = np.random.default_rng([seed, n])
    e = rng.choice(np.array(frequent, dtype=np.uint16), n)
    rare = rng.random(n) < rare_rate
    e[rare] = rng.integers(10, 70, int(rare.sum()), dtype=np.uint16)
    return ((rng.integers(0, 2, n, dtype=np.uint16) << 15) | (e << 7) |
            rng.integers(0, 128, n, dtype=np.uint16)).astype(np.uint16)


def words_for(case: str, n: int) -> np.ndarray:
    if case == "copy":
        return make_words("kv", n, 62)
    if case == "remap":
        # 16 exponents of equal probability: the sample ranks them in another order
        return pattern(n, 62, list(range(110, 126)), 0.005)
    if case == "full:set":
        # the sampled blocks favour exponent 200, the rest of the input 201
        w = pattern(n, 63, list(range(110, 125)), 0.0)
        rng = np.random.default_rng([64, n])
        in_sample = np.zeros(n, dtype=bool)
        for s in sample_starts(n):
            in_sample[s:s + SAMPLE_BLOCK_WORDS] = True
        pick = rng.random(n)
        mant = w & np.uint16(0x807F)
        w = np.where(in_sample & (pick < 0.10), mant | np.uint16(200 << 7), w)
        w = np.where(~in_sample & (pick < 0.05), mant | np.uint16(201 << 7), w)
        return w.astype(np.uint16)
    if case == "full:overflow":
        # one chunk of exponents spread over all 256 values
        w = make_words("kv", n, 65)
        rng = np.random.default_rng([66, n])
        w[1 << 15:(1 << 15) + (1 << 14)] = rng.integers(0, 65536, 1 << 14, dtype=np.uint16)
        return w
    if case == "full:sample":
        return make_words("wide40", n, 67)
    raise KeyError(case)


CASES = [
    ("copy", (1 << 22) + 77),
    ("copy", 1 << 20),                    # the sample is the whole input
    ("remap", (1 << 21) + 16385),         # odd: the pad nibble is remapped back to 0
    ("remap", 3 * (1 << 20) + 8),
    ("full:set", 1 << 22),
    ("full:overflow", (1 << 22) + 3),
    ("full:sample", (1 << 21) + 1),
]


def single_read_encode(torch, sz, x, n, dst, cap, size):
    ws_bytes = sz.sz_workspace_size(n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sz.sz_encode_sample(x, n, ws, ws_bytes)
    sz.sz_encode_first_pass(x, n, ws, ws_bytes, dst, cap)
    sz.sz_encode_finish(x, n, ws, ws_bytes, dst, cap, size)


@pytest.mark.parametrize("case,n", CASES)
def test_single_read_case(torch, sz, case, n):
    label = f"{case} n={n}"
    say(label)
    words = words_for(case, n)
    assert expected_case(words) == case, label
    x = torch.from_numpy(words.view(np.int16)).cuda()
    cap = sz.sz_max_compressed_size(n)
    dst = torch.full((cap,), 0x77, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    want = oracle.encode(words)
    for rep in range(2):                  # the second call finds the first one's bytes
        single_read_encode(torch, sz, x, n, dst, cap, size)
        total = int(size.item())
        assert total == want.size, (label, rep)
        assert np.array_equal(dst[:total].cpu().numpy(), want), (label, rep)
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    sz.sz_decode(dst[:total], total, out, n, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, label
    assert torch.equal(out, x), label


def test_single_read_staged_small_n_refused(torch, sz):
    n = (1 << 20) - 8
    x = torch.zeros(n, dtype=torch.int16, device="cuda")
    cap = sz.sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    ws_bytes = sz.sz_workspace_size(n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    for call in (sz.sz_encode_first_pass, sz.sz_encode_finish):
        with pytest.raises(sz.SplitZipError) as e:
            call(x, n, ws, ws_bytes, dst, cap)
        assert e.value.status == 1
    with pytest.raises(sz.SplitZipError) as e:
        sz.sz_encode_sample(x, n, ws, ws_bytes)
    assert e.value.status == 1


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case,n,page", [("remap", (1 << 27) + 5, 1 << 16),
                                         ("full:sample", (1 << 26) + 7, 1 << 14),
                                         ("full:set", 1 << 26, 1 << 15)])
def test_single_read_pages(torch, sz, case, n, page):
    """sz_encode_pages reads the pages once too (2^26 words and more): codes
    rewritten in a paged tensor, and chunks counted then packed again, or
    packed twice, from pages."""
    assert sz.sz_encode_single_read(n)
    label = f"pages {case} n={n} page={page}"
    say(label)
    words = words_for(case, n)
    assert expected_case(words) == case, label
    pool, table, order = paged(torch, n, page, 12)
    scatter_to_pages(torch, pool, order, words, page)
    cap = sz.sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    sz.sz_encode_pages(table, table.numel(), page, n, dst, cap, size, status)
    total = int(size.item())
    assert int(status.item()) == 0, label
    want = oracle.encode(words)
    assert total == want.size and np.array_equal(dst[:total].cpu().numpy(), want), label
    del pool
    out_pool, out_table, out_order = paged(torch, n, page, 13)
    status.fill_(-1)
    sz.sz_decode_pages(dst[:total], total, out_table, out_table.numel(), page, n, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, label
    assert np.array_equal(gather_pages(out_pool, out_order, n, page), words), label


def narrow_words(case: str, n: int) -> np.ndarray:
    """Ten exponents and no escapes.  "copy": exponent 110 + j drawn with
    weight 10 - j, so that the sample ranks them as the whole input does;
    "remap": equal weights, ranked otherwise by the sample; "full:set": as
    "remap", and exponent 200 too, but only in words the sample does not
    read, so the sampled codebook lacks an exponent the exact one holds."""
    if case == "copy":
        w = pattern(n, 70, [110 + j for j in range(10) for _ in range(10 - j)], 0.0)
    else:
        w = pattern(n, 70, list(range(110, 120)), 0.0)
    if case == "full:set":
        in_sample = np.zeros(n, dtype=bool)
        for s in sample_starts(n):
            in_sample[s:s + SAMPLE_BLOCK_WORDS] = True
        rng = np.random.default_rng([71, n])
        hit = ~in_sample & (rng.random(n) < 0.001)
        w = np.where(hit, (w & np.uint16(0x807F)) | np.uint16(200 << 7), w).astype(np.uint16)
    return w


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case,n", [("copy", (1 << 22) + 9), ("remap", (1 << 22) + 9),
                                    ("full:set", (1 << 22) + 9), ("copy", (1 << 26) + 3),
                                    ("remap", 1 << 26), ("full:set", (1 << 26) + 1)])
def test_single_read_no_escapes(torch, sz, case, n):
    """Fewer than 16 distinct exponents: no escape records, and a codebook
    filled up with exponents of count 0 in ascending order.  The staged
    single-read passes and sz_encode must give the oracle's container, and
    the tile decode (sz_decode's choice from 2^26 words) an index of empty
    tiles that decodes back to the input."""
    from test_gpu_parity import gpu_decode
    label = f"no escapes {case} n={n}"
    say(label)
    words = narrow_words(case, n)
    assert expected_case(words) == case, label
    want = oracle.encode(words)
    assert int(want[16:24].view(np.uint64)[0]) == 0, label  # E in the header
    x = torch.from_numpy(words.view(np.int16)).cuda()
    cap = sz.sz_max_compressed_size(n)
    dst = torch.full((cap,), 0x77, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    single_read_encode(torch, sz, x, n, dst, cap, size)
    total = int(size.item())
    assert total == want.size and np.array_equal(dst[:total].cpu().numpy(), want), label
    got = sz.encode(x).cpu().numpy()
    assert got.size == want.size and np.array_equal(got, want), label
    container = torch.from_numpy(want).cuda()
    for form in ("auto", "tiles"):
        y, status, guard_ok = gpu_decode(torch, sz, container, n, form)
        assert status == 0 and guard_ok, (label, form)
        assert torch.equal(y, x), (label, form)


@pytest.mark.parametrize("fill", [0xA5, 0xFF, 0x00])
def test_single_read_any_workspace_bytes(torch, sz, fill):
    """The staged calls take a workspace in whatever state the caller hands
    it over: arbitrary bytes (0xA5 leaves the sample pass's ticket count out
    of step with its workgroups; 0xFF makes the first workgroup to arrive
    rank a sample it has barely counted), or zeros.  Every call, the first
    included, gives the oracle's container; from the second call on the
    workspace is in step again."""
    n = (1 << 22) + 77
    words = words_for("copy", n)
    x = torch.from_numpy(words.view(np.int16)).cuda()
    cap = sz.sz_max_compressed_size(n)
    dst = torch.full((cap,), 0x77, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws_bytes = sz.sz_workspace_size(n)
    ws = torch.full((ws_bytes,), fill, dtype=torch.uint8, device="cuda")
    want = oracle.encode(words)
    for rep in range(3):
        say(f"workspace fill {fill:#x} call {rep}")
        sz.sz_encode_sample(x, n, ws, ws_bytes)
        sz.sz_encode_first_pass(x, n, ws, ws_bytes, dst, cap)
        sz.sz_encode_finish(x, n, ws, ws_bytes, dst, cap, size)
        total = int(size.item())
        assert total == want.size, (fill, rep)
        assert np.array_equal(dst[:total].cpu().numpy(), want), (fill, rep)


@pytest.mark.timeout(600)
def test_single_read_repack_full_size(torch, sz):
    """The finish's repack branch on the 1 GiB tensor's 4096-chunk plan: the
    llama3-8B-shaped KV tensor with every tenth sampled word moved to
    exponent 200, so the sample ranks 200 into its codebook while the whole
    tensor does not (another set: every chunk packed again)."""
    words = kvgen.generate("llama3_8b_kv_8k")
    n = words.size
    idx = (sample_starts(n)[:, None] + np.arange(SAMPLE_BLOCK_WORDS)[None, :]).ravel()[::10]
    words[idx] = (words[idx] & np.uint16(0x807F)) | np.uint16(200 << 7)
    assert -(-n >> bench.chunk_log2(n)) == 4096
    assert expected_case(words) == "full:set"
    want = oracle.encode(words)
    x = torch.from_numpy(words.view(np.int16)).cuda()
    cap = sz.sz_max_compressed_size(n)
    dst = torch.full((cap,), 0x77, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    say("full:set n=2^29, 4096 chunks")
    single_read_encode(torch, sz, x, n, dst, cap, size)
    total = int(size.item())
    assert total == want.size
    assert np.array_equal(dst[:total].cpu().numpy(), want)
    # and sz_encode takes the same path
    size.zero_()
    sz.sz_encode(x, n, dst, cap, size)
    assert int(size.item()) == want.size
    assert np.array_equal(dst[:want.size].cpu().numpy(), want)
