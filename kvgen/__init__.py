"""Seeded synthetic BF16 KV-cache workloads.

This module only makes inputs: it holds none of the codec's arithmetic and is
shared by the tests, the benchmark and the smoke check.  The explainers
publish no KV dumps, models or datasets, so these synthetic tensors stand in
for the KV caches the SplitZip pages talk about (section "2. La decouverte
secrete": exponents repeat, mantissas scatter).

Every workload is a flat little-endian ``uint16`` array of BF16 bit patterns
in ``[layers, {K,V}, tokens, kv_heads=8, head_dim=128]`` row-major order.

KV recipe (independent PCG64 streams per layer, per K/V slab and per block of
4096 tokens, so any part can be made alone and all parts in parallel):
  * per-layer multiplier ``m_l = exp(U(-1, 1))`` when enabled, else 1;
  * for K then V: per-(head, dim) channel scale ``sigma = exp(N(0, 1))``;
    with outliers, each K channel is multiplied by 30 with probability 1 %;
  * values ``z * float32(sigma * m_l)`` with ``z ~ N(0, 1)`` in float32;
  * rounded to BF16 with round-to-nearest-even on the float32 bits.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

HEADS = 8
HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    n: int
    seed: int


def _kv_n(layers: int, tokens: int) -> int:
    return layers * 2 * tokens * HEADS * HEAD_DIM


WORKLOADS = {
    "single_layer_kv": Workload(
        "single_layer_kv",
        "one layer, K and V [2, 1024 tok, 8 heads, 128 dim], lognormal channel scales",
        _kv_n(1, 1024), 101),
    "llama3_8b_kv_8k": Workload(
        "llama3_8b_kv_8k",
        "32 layers x {K,V} x 8192 tok x 8 heads x 128 dim, 1% x30 K outlier channels",
        _kv_n(32, 8192), 102),
    "llama3_70b_kv_32k": Workload(
        "llama3_70b_kv_32k",
        "80 layers x {K,V} x 32768 tok x 8 heads x 128 dim, outliers, per-layer scale",
        _kv_n(80, 32768), 103),
    "escape_heavy": Workload(
        "escape_heavy",
        "256M words: uniform sign, uniform 7-bit mantissa, exponent uniform in [100,140)",
        1 << 28, 104),
    "special_values": Workload(
        "special_values",
        "512M words of single-layer-style KV plus 0.1% each of +-0, subnormal, +-Inf, NaN",
        1 << 29, 105),
}

# Short aliases used on the command line.
ALIASES = {"c1": "single_layer_kv", "c2": "llama3_8b_kv_8k", "c3": "llama3_70b_kv_32k",
           "c4": "escape_heavy", "c5": "special_values"}


def resolve(name: str) -> Workload:
    name = ALIASES.get(name.lower(), name)
    return WORKLOADS[name]


def rne_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns, round to nearest, ties to even.

    Only finite inputs are produced by the recipes below (no NaN handling).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _threads(threads: int | None) -> int:
    if threads is not None:
        return max(1, threads)
    return max(1, min(16, os.cpu_count() or 1))


TOKEN_BLOCK = 4096  # tokens per independently seeded block of z draws


def _layer_multiplier(seed: int, layer: int, layer_mult: bool) -> float:
    if not layer_mult:
        return 1.0
    return float(np.exp(np.random.default_rng([seed, layer]).uniform(-1.0, 1.0)))


def _channel_scale(seed: int, layer: int, kv: int, outliers: bool, m: float) -> np.ndarray:
    rng = np.random.default_rng([seed, layer, kv + 1])
    sigma = np.exp(rng.standard_normal((HEADS, HEAD_DIM)))
    if outliers and kv == 0:
        sigma = sigma * np.where(rng.random((HEADS, HEAD_DIM)) < 0.01, 30.0, 1.0)
    return (sigma * m).astype(np.float32)


def kv_cache(layers: int, tokens: int, seed: int, outliers: bool, layer_mult: bool,
             out: np.ndarray | None = None, threads: int | None = None) -> np.ndarray:
    """Fill ``[layers, 2, tokens, 8, 128]``.  Streams: ``[seed, l]`` for the
    layer multiplier, ``[seed, l, kv+1]`` for the channel scales and
    ``[seed, l, kv+1, b+1]`` for the z draws of token block ``b``."""
    n = _kv_n(layers, tokens)
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == n
    view = out.reshape(layers, 2, tokens, HEADS, HEAD_DIM)
    scales = {}
    for layer in range(layers):
        m = _layer_multiplier(seed, layer, layer_mult)
        for kv in range(2):
            scales[layer, kv] = _channel_scale(seed, layer, kv, outliers, m)
    blocks = (tokens + TOKEN_BLOCK - 1) // TOKEN_BLOCK
    tasks = [(l, kv, b) for l in range(layers) for kv in range(2) for b in range(blocks)]

    def work(task) -> None:
        layer, kv, b = task
        t0, t1 = b * TOKEN_BLOCK, min(tokens, (b + 1) * TOKEN_BLOCK)
        rng = np.random.default_rng([seed, layer, kv + 1, b + 1])
        z = rng.standard_normal((t1 - t0, HEADS, HEAD_DIM), dtype=np.float32)
        z *= scales[layer, kv]
        view[layer, kv, t0:t1] = rne_bf16(z)

    nt = min(_threads(threads), len(tasks))
    if nt <= 1:
        for t in tasks:
            work(t)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, tasks))
    return out


def escape_heavy(n: int, seed: int, out: np.ndarray | None = None,
                 threads: int | None = None) -> np.ndarray:
    """Uniform sign, uniform 7-bit mantissa, exponent uniform over [100, 140)."""
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 24

    def work(c: int) -> None:
        lo, hi = c * chunk, min(n, (c + 1) * chunk)
        rng = np.random.default_rng([seed, c])
        s = rng.integers(0, 2, hi - lo, dtype=np.uint16)
        e = rng.integers(100, 140, hi - lo, dtype=np.uint16)
        m = rng.integers(0, 128, hi - lo, dtype=np.uint16)
        out[lo:hi] = (s << 15) | (e << 7) | m

    chunks = (n + chunk - 1) // chunk
    with ThreadPoolExecutor(min(_threads(threads), max(1, chunks))) as ex:
        list(ex.map(work, range(chunks)))
    return out


def special_values(seed: int, out: np.ndarray | None = None,
                   threads: int | None = None) -> np.ndarray:
    """Single-layer KV of 2^18 tokens, then 0.1% each of +-0, subnormals,
    +-Inf and NaNs (random payloads) written at seeded distinct positions."""
    out = kv_cache(1, 1 << 18, seed, outliers=False, layer_mult=False, out=out,
                   threads=threads)
    n = out.size
    k = n // 1000
    rng = np.random.default_rng([seed, 1 << 20])
    pos = rng.choice(n, 4 * k, replace=False)
    sign = (rng.integers(0, 2, 4 * k, dtype=np.uint16) << 15).astype(np.uint16)
    payload = rng.integers(1, 128, 2 * k, dtype=np.uint16)
    vals = np.empty(4 * k, dtype=np.uint16)
    vals[0:k] = 0                                   # +-0
    vals[k:2 * k] = payload[:k]                     # subnormal: exponent 0
    vals[2 * k:3 * k] = 0x7F80                      # +-Inf
    vals[3 * k:4 * k] = 0x7F80 | payload[k:]        # NaN, quiet and signalling
    out[pos] = vals | sign
    return out


def generate(name: str, out: np.ndarray | None = None,
             threads: int | None = None) -> np.ndarray:
    """Make a named workload (see ``WORKLOADS``) as a flat uint16 array."""
    w = resolve(name)
    if w.name == "single_layer_kv":
        return kv_cache(1, 1024, w.seed, False, False, out, threads)
    if w.name == "llama3_8b_kv_8k":
        return kv_cache(32, 8192, w.seed, True, False, out, threads)
    if w.name == "llama3_70b_kv_32k":
        return kv_cache(80, 32768, w.seed, True, True, out, threads)
    if w.name == "escape_heavy":
        return escape_heavy(w.n, w.seed, out, threads)
    if w.name == "special_values":
        return special_values(w.seed, out, threads)
    raise KeyError(name)


def small_kv(n: int, seed: int) -> np.ndarray:
    """A KV-like tensor of arbitrary length (ragged sizes for parity tests)."""
    rng = np.random.default_rng([seed, 7])
    channels = HEADS * HEAD_DIM
    sigma = np.exp(rng.standard_normal(channels)).astype(np.float32)
    rows = (n + channels - 1) // channels
    z = rng.standard_normal((max(rows, 1), channels), dtype=np.float32) * sigma
    return rne_bf16(z.reshape(-1)[:n])
