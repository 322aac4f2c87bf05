"""MI355X-native SplitZip BF16 KV-cache codec: Python binding.

A thin ctypes layer over ``libsplitzip.so`` (hand-written HIP for gfx950,
C ABI declared in ``include/splitzip.h``).  The functions named ``sz_*`` are
the C entry points with the same names and arguments; they only marshal
arguments (a torch tensor's data pointer, or a raw integer device pointer,
and the current torch stream by default) and turn a non-zero status into
``SplitZipError``.  Every step of the codec runs in the library's kernels;
PyTorch only provides device memory and streams.

``encode`` and ``decode`` are conveniences that allocate their outputs with
torch and call the entry points.

The method follows the SplitZip explainers (gist.science, arXiv 2605.01708):
top-16 exponent codebook with 4-bit codes two per byte, sign|mantissa bytes,
and (position, exponent) escapes for the remaining exponents (section
"3. La strategie SplitZip"), decoded by lookup, recombination and escape
overwrite (section "4. Pourquoi est-ce rapide ?").
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SplitZipError", "lib_path", "sz_max_compressed_size", "sz_workspace_size", "sz_encode",
    "sz_decode", "sz_encode_noalloc", "sz_encode_histogram", "sz_encode_codebook", "sz_encode_pack",
    "sz_encode_pack_ranked", "sz_encode_single_read", "sz_encode_sample", "sz_encode_first_pass", "sz_encode_finish",
    "sz_decode_unpack", "sz_decode_scatter", "sz_decode_fused", "sz_decode_dense",
    "sz_decode_workspace_size", "sz_decode_index", "sz_decode_tiles",
    "sz_encode_pages", "sz_decode_pages", "sz_blocks_workspace_size", "sz_encode_blocks",
    "sz_decode_blocks", "sz_blocks_decode_workspace_size", "sz_ship_to_host", "sz_ship_from_host", "ShipContext",
    "sz_status_string", "encode",
    "decode", "encode_blocks", "decode_blocks", "BlockContainers",
    "PREFIX_BYTES", "MAX_ELEMENTS", "NOALLOC_WORKSPACE_BYTES",
]

PREFIX_BYTES = 176
MAX_ELEMENTS = 1 << 36
NOALLOC_WORKSPACE_BYTES = 4608 * 1024

SZ_OK = 0
SZ_ERR_INVALID_ARGUMENT = 1
SZ_ERR_CAPACITY = 2
SZ_ERR_TOO_LARGE = 3
SZ_ERR_CORRUPT = 4
SZ_ERR_HIP = 5

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libsplitzip.so")


class SplitZipError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call}: {sz_status_string(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(lib_path):
        raise ImportError(
            f"{lib_path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(lib_path)
    u64, p, i32 = ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int
    L.sz_max_compressed_size.argtypes = [u64]
    L.sz_max_compressed_size.restype = u64
    L.sz_workspace_size.argtypes = [u64]
    L.sz_workspace_size.restype = u64
    L.sz_encode.argtypes = [p, u64, p, u64, p, p]
    L.sz_decode.argtypes = [p, u64, p, u64, p, p]
    L.sz_encode_noalloc.argtypes = [p, u64, p, u64, p, p]
    L.sz_encode_histogram.argtypes = [p, u64, p, u64, p]
    L.sz_encode_codebook.argtypes = [u64, p, u64, p, u64, p, p]
    L.sz_encode_pack.argtypes = [p, u64, p, u64, p, u64, p]
    L.sz_encode_pack_ranked.argtypes = [p, u64, p, u64, p, u64, p, p]
    L.sz_encode_single_read.argtypes = [u64]
    L.sz_encode_single_read.restype = i32
    L.sz_encode_sample.argtypes = [p, u64, p, u64, p]
    L.sz_encode_first_pass.argtypes = [p, u64, p, u64, p, u64, p]
    L.sz_encode_finish.argtypes = [p, u64, p, u64, p, u64, p, p]
    L.sz_decode_unpack.argtypes = [p, u64, p, u64, p, p]
    L.sz_decode_scatter.argtypes = [p, u64, p, u64, p, p]
    L.sz_decode_fused.argtypes = [p, u64, p, u64, p, p]
    L.sz_decode_dense.argtypes = [p, u64, p, u64, p, p]
    L.sz_decode_workspace_size.argtypes = [u64]
    L.sz_decode_workspace_size.restype = u64
    L.sz_decode_index.argtypes = [p, u64, u64, p, u64, p]
    L.sz_decode_tiles.argtypes = [p, u64, p, u64, p, u64, p, p]
    L.sz_encode_pages.argtypes = [p, u64, u64, u64, p, u64, p, p, p]
    L.sz_decode_pages.argtypes = [p, u64, p, u64, u64, u64, p, p]
    L.sz_blocks_workspace_size.argtypes = [u64, u64]
    L.sz_blocks_workspace_size.restype = u64
    L.sz_encode_blocks.argtypes = [p, u64, u64, p, u64, p, p, u64, p, p]
    L.sz_blocks_decode_workspace_size.argtypes = [u64, u64]
    L.sz_blocks_decode_workspace_size.restype = u64
    L.sz_decode_blocks.argtypes = [p, u64, p, u64, u64, p, p, u64, p, p]
    L.sz_ship_to_host.argtypes = [p, u64, u64, p, u64, p, p]
    L.sz_ship_from_host.argtypes = [p, p, u64, u64, p, p, p]
    L.sz_ship_context_create.argtypes = [u64, ctypes.POINTER(ctypes.c_void_p)]
    L.sz_ship_context_destroy.argtypes = [p]
    L.sz_ship_context_destroy.restype = None
    L.sz_ship_to_host_ctx.argtypes = [p, p, u64, p, u64, p, p]
    L.sz_ship_from_host_ctx.argtypes = [p, p, p, u64, p, p, p]
    for name in ("sz_encode", "sz_decode", "sz_encode_noalloc", "sz_encode_histogram", "sz_encode_codebook",
                 "sz_encode_pack", "sz_encode_pack_ranked", "sz_encode_sample",
                 "sz_encode_first_pass", "sz_encode_finish",
                 "sz_decode_unpack", "sz_decode_scatter", "sz_decode_fused",
                 "sz_decode_dense", "sz_decode_index", "sz_decode_tiles", "sz_encode_pages",
                 "sz_decode_pages", "sz_encode_blocks", "sz_decode_blocks", "sz_ship_to_host",
                 "sz_ship_from_host", "sz_ship_context_create", "sz_ship_to_host_ctx",
                 "sz_ship_from_host_ctx"):
        getattr(L, name).restype = i32
    L.sz_status_string.argtypes = [i32]
    L.sz_status_string.restype = ctypes.c_char_p
    return L


_lib = _load()


def _ptr(x) -> int | None:
    """Address of a tensor's data (device, or host for the ship calls' host
    buffers), of a NumPy array's data, or an integer pointer as given
    (None = NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return x.ctypes.data


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, call: str) -> None:
    if status != SZ_OK:
        raise SplitZipError(status, call)


def sz_status_string(status: int) -> str:
    return _lib.sz_status_string(status).decode()


def sz_max_compressed_size(n_elements: int) -> int:
    return int(_lib.sz_max_compressed_size(n_elements))


def sz_workspace_size(n_elements: int) -> int:
    return int(_lib.sz_workspace_size(n_elements))


def sz_encode(src, n_elements: int, dst, dst_capacity: int, d_compressed_size=None,
              stream=None) -> None:
    _check(_lib.sz_encode(_ptr(src), n_elements, _ptr(dst), dst_capacity,
                          _ptr(d_compressed_size), _stream(stream)), "sz_encode")


def sz_encode_noalloc(src, n_elements: int, dst, dst_capacity: int, d_compressed_size=None,
                      stream=None) -> None:
    _check(_lib.sz_encode_noalloc(_ptr(src), n_elements, _ptr(dst), dst_capacity,
                                  _ptr(d_compressed_size), _stream(stream)), "sz_encode_noalloc")


def sz_decode(src, src_bytes: int, dst, n_elements: int, d_status=None, stream=None) -> None:
    _check(_lib.sz_decode(_ptr(src), src_bytes, _ptr(dst), n_elements, _ptr(d_status),
                          _stream(stream)), "sz_decode")


def sz_encode_histogram(src, n_elements: int, workspace, workspace_bytes: int,
                        stream=None) -> None:
    _check(_lib.sz_encode_histogram(_ptr(src), n_elements, _ptr(workspace), workspace_bytes,
                                    _stream(stream)), "sz_encode_histogram")


def sz_encode_codebook(n_elements: int, workspace, workspace_bytes: int, dst,
                       dst_capacity: int, d_compressed_size=None, stream=None) -> None:
    _check(_lib.sz_encode_codebook(n_elements, _ptr(workspace), workspace_bytes, _ptr(dst),
                                   dst_capacity, _ptr(d_compressed_size), _stream(stream)),
           "sz_encode_codebook")


def sz_encode_pack(src, n_elements: int, workspace, workspace_bytes: int, dst,
                   dst_capacity: int, stream=None) -> None:
    _check(_lib.sz_encode_pack(_ptr(src), n_elements, _ptr(workspace), workspace_bytes,
                               _ptr(dst), dst_capacity, _stream(stream)), "sz_encode_pack")


def sz_encode_pack_ranked(src, n_elements: int, workspace, workspace_bytes: int, dst,
                          dst_capacity: int, d_compressed_size=None, stream=None) -> None:
    _check(_lib.sz_encode_pack_ranked(_ptr(src), n_elements, _ptr(workspace), workspace_bytes,
                                      _ptr(dst), dst_capacity, _ptr(d_compressed_size),
                                      _stream(stream)), "sz_encode_pack_ranked")


def sz_encode_single_read(n_elements: int) -> bool:
    return bool(_lib.sz_encode_single_read(n_elements))


def sz_encode_sample(src, n_elements: int, workspace, workspace_bytes: int, stream=None) -> None:
    _check(_lib.sz_encode_sample(_ptr(src), n_elements, _ptr(workspace), workspace_bytes,
                                 _stream(stream)), "sz_encode_sample")


def sz_encode_first_pass(src, n_elements: int, workspace, workspace_bytes: int, dst,
                         dst_capacity: int, stream=None) -> None:
    _check(_lib.sz_encode_first_pass(_ptr(src), n_elements, _ptr(workspace), workspace_bytes,
                                     _ptr(dst), dst_capacity, _stream(stream)),
           "sz_encode_first_pass")


def sz_encode_finish(src, n_elements: int, workspace, workspace_bytes: int, dst,
                     dst_capacity: int, d_compressed_size=None, stream=None) -> None:
    _check(_lib.sz_encode_finish(_ptr(src), n_elements, _ptr(workspace), workspace_bytes,
                                 _ptr(dst), dst_capacity, _ptr(d_compressed_size),
                                 _stream(stream)), "sz_encode_finish")


def sz_decode_unpack(src, src_bytes: int, dst, n_elements: int, d_status=None,
                     stream=None) -> None:
    _check(_lib.sz_decode_unpack(_ptr(src), src_bytes, _ptr(dst), n_elements, _ptr(d_status),
                                 _stream(stream)), "sz_decode_unpack")


def sz_decode_scatter(src, src_bytes: int, dst, n_elements: int, d_status=None,
                      stream=None) -> None:
    _check(_lib.sz_decode_scatter(_ptr(src), src_bytes, _ptr(dst), n_elements, _ptr(d_status),
                                  _stream(stream)), "sz_decode_scatter")


def sz_decode_fused(src, src_bytes: int, dst, n_elements: int, d_status=None,
                    stream=None) -> None:
    _check(_lib.sz_decode_fused(_ptr(src), src_bytes, _ptr(dst), n_elements, _ptr(d_status),
                                _stream(stream)), "sz_decode_fused")


def sz_decode_workspace_size(n_elements: int) -> int:
    return int(_lib.sz_decode_workspace_size(n_elements))


def sz_decode_index(src, src_bytes: int, n_elements: int, workspace, workspace_bytes: int,
                    stream=None) -> None:
    _check(_lib.sz_decode_index(_ptr(src), src_bytes, n_elements, _ptr(workspace),
                                workspace_bytes, _stream(stream)), "sz_decode_index")


def sz_decode_tiles(src, src_bytes: int, workspace, workspace_bytes: int, dst, n_elements: int,
                    d_status=None, stream=None) -> None:
    _check(_lib.sz_decode_tiles(_ptr(src), src_bytes, _ptr(workspace), workspace_bytes,
                                _ptr(dst), n_elements, _ptr(d_status), _stream(stream)),
           "sz_decode_tiles")


def sz_decode_dense(src, src_bytes: int, dst, n_elements: int, d_status=None,
                    stream=None) -> None:
    _check(_lib.sz_decode_dense(_ptr(src), src_bytes, _ptr(dst), n_elements, _ptr(d_status),
                                _stream(stream)), "sz_decode_dense")


def sz_encode_pages(d_pages, n_pages: int, page_elems: int, n_elements: int, dst,
                    dst_capacity: int, d_compressed_size=None, d_status=None, stream=None) -> None:
    """d_pages: device array of page addresses (e.g. an int64 CUDA tensor)."""
    _check(_lib.sz_encode_pages(_ptr(d_pages), n_pages, page_elems, n_elements, _ptr(dst),
                                dst_capacity, _ptr(d_compressed_size), _ptr(d_status),
                                _stream(stream)), "sz_encode_pages")


def sz_decode_pages(src, src_bytes: int, d_pages, n_pages: int, page_elems: int,
                    n_elements: int, d_status=None, stream=None) -> None:
    _check(_lib.sz_decode_pages(_ptr(src), src_bytes, _ptr(d_pages), n_pages, page_elems,
                                n_elements, _ptr(d_status), _stream(stream)), "sz_decode_pages")


def sz_blocks_workspace_size(block_elems: int, n_blocks: int) -> int:
    return int(_lib.sz_blocks_workspace_size(block_elems, n_blocks))


def sz_encode_blocks(d_blocks, n_blocks: int, block_elems: int, dst, dst_pitch: int, d_sizes,
                     workspace, workspace_bytes: int, d_status=None, stream=None) -> None:
    """d_blocks: device array of block addresses (e.g. an int64 CUDA tensor);
    d_sizes: device uint64 array of n_blocks entries (e.g. an int64 tensor)."""
    _check(_lib.sz_encode_blocks(_ptr(d_blocks), n_blocks, block_elems, _ptr(dst), dst_pitch,
                                 _ptr(d_sizes), _ptr(workspace), workspace_bytes, _ptr(d_status),
                                 _stream(stream)), "sz_encode_blocks")


def sz_blocks_decode_workspace_size(block_elems: int, n_blocks: int) -> int:
    return int(_lib.sz_blocks_decode_workspace_size(block_elems, n_blocks))


def sz_decode_blocks(src, src_pitch: int, d_sizes, n_blocks: int, block_elems: int, d_blocks,
                     d_status, workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    """d_status: device int32 array of n_blocks entries (required); with a
    workspace the tile form, without it the single-pass form."""
    _check(_lib.sz_decode_blocks(_ptr(src), src_pitch, _ptr(d_sizes), n_blocks, block_elems,
                                 _ptr(d_blocks), _ptr(workspace), workspace_bytes,
                                 _ptr(d_status), _stream(stream)), "sz_decode_blocks")


def sz_ship_to_host(src, n_elements: int, chunk_elems: int, h_dst, h_capacity: int, h_offsets,
                    stream=None) -> None:
    """h_dst: pinned host buffer; h_offsets: host uint64 array of
    ceil(n / chunk_elems) + 1 entries (a NumPy array or a CPU tensor)."""
    _check(_lib.sz_ship_to_host(_ptr(src), n_elements, chunk_elems, _ptr(h_dst), h_capacity,
                                _ptr(h_offsets), _stream(stream)), "sz_ship_to_host")


def sz_ship_from_host(h_src, h_offsets, n_elements: int, chunk_elems: int, dst, d_status=None,
                      stream=None) -> None:
    _check(_lib.sz_ship_from_host(_ptr(h_src), _ptr(h_offsets), n_elements, chunk_elems,
                                  _ptr(dst), _ptr(d_status), _stream(stream)),
           "sz_ship_from_host")


class ShipContext:
    """A transfer context (sz_ship_context_create) for one chunk size on the
    current device; released by close() or when collected."""

    def __init__(self, chunk_elems: int):
        self.handle = None
        h = ctypes.c_void_p()
        _check(_lib.sz_ship_context_create(chunk_elems, ctypes.byref(h)),
               "sz_ship_context_create")
        self.handle = h.value
        self.chunk_elems = chunk_elems

    def close(self) -> None:
        if getattr(self, "handle", None):
            _lib.sz_ship_context_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()

    def to_host(self, src, n_elements: int, h_dst, h_capacity: int, h_offsets,
                stream=None) -> None:
        _check(_lib.sz_ship_to_host_ctx(self.handle, _ptr(src), n_elements, _ptr(h_dst),
                                        h_capacity, _ptr(h_offsets), _stream(stream)),
               "sz_ship_to_host_ctx")

    def from_host(self, h_src, h_offsets, n_elements: int, dst, d_status=None,
                  stream=None) -> None:
        _check(_lib.sz_ship_from_host_ctx(self.handle, _ptr(h_src), _ptr(h_offsets), n_elements,
                                          _ptr(dst), _ptr(d_status), _stream(stream)),
               "sz_ship_from_host_ctx")


# ---- conveniences (torch allocates; the library computes) -----------------

def encode(x, stream=None):
    """Compress a CUDA tensor of BF16 (or 16-bit integer) words; returns the
    container as a uint8 CUDA tensor trimmed to its exact size (this reads
    the size back, so it synchronises the stream)."""
    import torch
    if x.element_size() != 2 or not x.is_cuda:
        raise ValueError("encode expects a CUDA tensor of 16-bit elements")
    x = x.contiguous()
    n = x.numel()
    cap = sz_max_compressed_size(n)
    dst = torch.empty(cap, dtype=torch.uint8, device=x.device)
    size = torch.zeros(1, dtype=torch.int64, device=x.device)
    sz_encode(x, n, dst, cap, size, stream)
    return dst[: int(size.item())]


def decode(container, n_elements: int, dtype=None, stream=None, check: bool = True):
    """Decompress a uint8 CUDA container into ``n_elements`` words (bfloat16
    unless ``dtype`` says otherwise).  With ``check`` the device status is
    read back (synchronising) and a corrupt container raises."""
    import torch
    out = torch.empty(n_elements, dtype=dtype or torch.bfloat16, device=container.device)
    status = torch.zeros(1, dtype=torch.int32, device=container.device)
    sz_decode(container, container.numel(), out, n_elements, status, stream)
    if check:
        st = int(status.item())
        if st != SZ_OK:
            raise SplitZipError(st, "sz_decode (device check)")
    return out


class BlockContainers:
    """Containers of equal-length blocks as sz_encode_blocks leaves them:
    block b's container is ``data[b * pitch : b * pitch + sizes[b]]``, and
    ``sizes`` stays on the device (a uint64 array held as an int64 tensor)."""

    def __init__(self, data, pitch: int, sizes, block_elems: int):
        self.data, self.pitch, self.sizes, self.block_elems = data, pitch, sizes, block_elems

    def __len__(self) -> int:
        return self.sizes.numel()

    def container(self, b: int):
        """Block b's container, trimmed (reads its size back: synchronises)."""
        return self.data[b * self.pitch: b * self.pitch + int(self.sizes[b].item())]


def _block_table(tensors):
    import torch
    if not tensors:
        raise ValueError("no blocks")
    n = tensors[0].numel()
    for t in tensors:
        if t.element_size() != 2 or not t.is_cuda or t.numel() != n or not t.is_contiguous():
            raise ValueError("blocks must be contiguous CUDA tensors of 16-bit elements, "
                             "all of the same length")
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64,
                        device=tensors[0].device), n


def encode_blocks(tensors, stream=None) -> BlockContainers:
    """Compress equal-length CUDA tensors (one per layer, say), one container
    each, in one launch per pass (sz_encode_blocks); nothing is read back."""
    import torch
    table, n = _block_table(tensors)
    nb = len(tensors)
    dev = tensors[0].device
    pitch = (sz_max_compressed_size(n) + 15) // 16 * 16
    data = torch.empty(nb * pitch, dtype=torch.uint8, device=dev)
    sizes = torch.zeros(nb, dtype=torch.int64, device=dev)
    wb = sz_blocks_workspace_size(n, nb)
    ws = torch.empty(wb, dtype=torch.uint8, device=dev)
    sz_encode_blocks(table, nb, n, data, pitch, sizes, ws, wb, None, stream)
    return BlockContainers(data, pitch, sizes, n)


def decode_blocks(blocks: BlockContainers, outputs, stream=None, check: bool = True):
    """Decompress every container into the matching output tensor (same
    count and length as encoded), with the tile form's workspace; with
    ``check`` the per-block statuses are read back (synchronising) and any
    failure raises, naming the first block that failed."""
    import torch
    table, n = _block_table(outputs)
    nb = len(outputs)
    if nb != len(blocks) or n != blocks.block_elems:
        raise ValueError("outputs do not match the containers' block count and length")
    dev = outputs[0].device
    status = torch.zeros(nb, dtype=torch.int32, device=dev)
    wb = sz_blocks_decode_workspace_size(n, nb)
    ws = torch.empty(wb, dtype=torch.uint8, device=dev)
    sz_decode_blocks(blocks.data, blocks.pitch, blocks.sizes, nb, n, table, status, ws, wb,
                     stream)
    if check:
        st = status.cpu()
        bad = (st != SZ_OK).nonzero()
        if bad.numel():
            b = int(bad[0])
            raise SplitZipError(int(st[b]), f"sz_decode_blocks (block {b})")
    return outputs
