"""GPU parity on seeded random cases: sizes (mostly ragged), input kinds and
seeds drawn from a fixed generator.  Each container must equal the oracle's
byte for byte, from both encode forms where the single-read one applies, and
sz_decode of the oracle's container must give the input back."""
import numpy as np
import pytest

import oracle
from test_gpu_parity import KINDS, make_words

pytestmark = pytest.mark.gpu

CASES = 80


def draws():
    rng = np.random.default_rng(20261203)
    for i in range(CASES):
        if i % 20 == 0:
            n = int(rng.integers(1 << 20, (1 << 22) + 100))   # single-read staged sizes
        elif rng.random() < 0.5:
            n = int(rng.integers(1, 70000))
        else:
            n = int(rng.integers(70000, 3_000_000))
        yield i, KINDS[int(rng.integers(0, len(KINDS)))], n, int(rng.integers(0, 1 << 30))


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


def test_random_cases(torch, sz):
    for i, kind, n, seed in draws():
        print(f"[gpu-random] case {i} kind={kind} n={n} seed={seed}", flush=True)
        words = make_words(kind, n, seed)
        want = oracle.encode(words)
        x = torch.from_numpy(words.view(np.int16)).cuda()
        got = sz.encode(x).cpu().numpy()
        assert got.size == want.size and np.array_equal(got, want), (i, kind, n, seed)
        if n >= 1 << 20:
            ws_bytes = sz.sz_workspace_size(n)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            cap = sz.sz_max_compressed_size(n)
            dst = torch.empty(cap, dtype=torch.uint8, device="cuda")
            size = torch.zeros(1, dtype=torch.int64, device="cuda")
            sz.sz_encode_sample(x, n, ws, ws_bytes)
            sz.sz_encode_first_pass(x, n, ws, ws_bytes, dst, cap)
            sz.sz_encode_finish(x, n, ws, ws_bytes, dst, cap, size)
            torch.cuda.synchronize()
            assert int(size.item()) == want.size, (i, kind, n, seed)
            assert np.array_equal(dst[:want.size].cpu().numpy(), want), (i, kind, n, seed)
        y = sz.decode(torch.from_numpy(want).cuda(), n, dtype=torch.int16)
        assert torch.equal(y, x), (i, kind, n, seed)
