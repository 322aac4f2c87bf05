// ship.hip -- moving a tensor between device and pinned host memory in
// compressed form, chunk by chunk, with the codec and the copies overlapped.
//
// The SplitZip explainers (gist.science pages for arXiv 2605.01708) present
// the codec as a way to shrink the KV transfer between the prefill and the
// decode servers of a disaggregated deployment (introduction and section
// "Les Resultats": the KV transfer gets faster).  On one GPU the transfer
// that exists is the PCIe copy to and from host memory, so these calls wrap
// the codec around it: the tensor is cut into chunks, each chunk is an
// ordinary container (its own codebook), and while chunk c is encoded (or
// decoded) on the caller's stream, earlier chunks' containers are copied on
// a second stream, through a ring of kShipDepth staging buffers.
//
// A transfer context holds everything a transfer needs (the copy stream,
// the staging buffers, the events, the pinned size slots), so that a serving
// loop creates it once and every transfer after that allocates nothing (a
// decode with more chunks than any before it grows the per-chunk status
// array).  The one-shot calls build a context, use it and release it.
#include "splitzip.h"
#include "sz_internal.h"

#include <new>

namespace {

constexpr int kShipDepth = 3;  // staging buffers: chunk groups in flight between codec and copy
// A decode moves chunks in groups of at least this many words: one event
// pair and one wait per stream for a whole group, each chunk still copied to
// its own 16-byte-aligned place in the staging buffer (small chunks are
// otherwise bound by the per-chunk calls on the host).
constexpr uint64_t kShipGroupWords = uint64_t{1} << 24;
constexpr uint64_t kShipGroupBytes = uint64_t{1} << 27;  // staging per buffer, at most

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

uint64_t chunks_of(uint64_t n, uint64_t chunk) { return chunk ? (n + chunk - 1) / chunk : 0; }

bool chunk_size_ok(uint64_t chunk_elems) {
    return chunk_elems > 0 && chunk_elems % 8 == 0 && chunk_elems <= SZ_MAX_ELEMENTS;
}

// The largest status code of `count` chunks (SZ_OK is 0) into *worst: one
// workgroup.
__global__ __launch_bounds__(256) void k_status_worst(const int32_t* __restrict__ st,
                                                      uint64_t count, int32_t* __restrict__ worst) {
    __shared__ int32_t m;
    if (threadIdx.x == 0) m = 0;
    __syncthreads();
    int32_t w = 0;
    for (uint64_t i = threadIdx.x; i < count; i += blockDim.x) w = st[i] > w ? st[i] : w;
    if (w) atomicMax(&m, w);
    __syncthreads();
    if (threadIdx.x == 0) *worst = m;
}

}  // namespace

struct sz_ship_context {
    int device = -1;
    uint64_t chunk_elems = 0;
    uint64_t stage_bytes = 0;                  // sz_max_compressed_size(chunk_elems), 16-aligned
    uint64_t group = 1;                        // chunks a decode stages per buffer
    uint64_t stage_chunks = 0;                 // chunks each staging buffer holds now
    hipStream_t copy = nullptr;                // default priority
    void* stage[kShipDepth] = {};
    hipEvent_t ready[kShipDepth] = {};         // to host: encoded, size copied; from host: arrived
    hipEvent_t done[kShipDepth] = {};          // to host: copied out; from host: decoded
    uint64_t* h_sizes = nullptr;               // pinned, one per staging buffer
    uint64_t* d_sizes = nullptr;               // one per staging buffer
    int32_t* d_status = nullptr;               // one per chunk of a decode
    uint64_t status_cap = 0;
    int32_t* d_worst = nullptr;
    int32_t* h_worst = nullptr;                // pinned

    ~sz_ship_context() {
        if (copy) (void)hipStreamSynchronize(copy);
        for (int i = 0; i < kShipDepth; i++) {
            if (ready[i]) (void)hipEventDestroy(ready[i]);
            if (done[i]) (void)hipEventDestroy(done[i]);
            if (stage[i]) (void)hipFree(stage[i]);
        }
        if (copy) (void)hipStreamDestroy(copy);
        if (h_sizes) (void)hipHostFree(h_sizes);
        if (h_worst) (void)hipHostFree(h_worst);
        if (d_sizes) (void)hipFree(d_sizes);
        if (d_status) (void)hipFree(d_status);
        if (d_worst) (void)hipFree(d_worst);
    }
};

namespace {

// Both streams drained, whatever the outcome.
sz_status drain(sz_ship_context* ctx, hipStream_t stream, sz_status result) {
    if (hipStreamSynchronize(stream) != hipSuccess && result == SZ_OK) result = SZ_ERR_HIP;
    if (hipStreamSynchronize(ctx->copy) != hipSuccess && result == SZ_OK) result = SZ_ERR_HIP;
    return result;
}

// Every chunk's size must be a possible container for its length (then it
// also fits a staging buffer): checked on the host before anything is copied.
sz_status check_offsets(const uint64_t* h_offsets, uint64_t n, uint64_t chunk_elems) {
    const uint64_t chunks = chunks_of(n, chunk_elems);
    for (uint64_t c = 0; c < chunks; c++) {
        const uint64_t len = n - c * chunk_elems < chunk_elems ? n - c * chunk_elems : chunk_elems;
        if (h_offsets[c + 1] < h_offsets[c]) return SZ_ERR_CORRUPT;
        const uint64_t size = h_offsets[c + 1] - h_offsets[c];
        if (size < sz::container_bytes(len, 0) || size > sz_max_compressed_size(len) ||
            (size - sz::container_bytes(len, 0)) % 5 != 0)
            return SZ_ERR_CORRUPT;
    }
    return SZ_OK;
}

sz_status check_context(const sz_ship_context* ctx) {
    if (ctx == nullptr) return SZ_ERR_INVALID_ARGUMENT;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SZ_ERR_HIP;
    return dev == ctx->device ? SZ_OK : SZ_ERR_INVALID_ARGUMENT;
}

}  // namespace

extern "C" {

sz_status sz_ship_context_create(uint64_t chunk_elems, sz_ship_context** out) {
    if (out == nullptr || !chunk_size_ok(chunk_elems)) return SZ_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    sz_ship_context* ctx = new (std::nothrow) sz_ship_context;
    if (ctx == nullptr) return SZ_ERR_HIP;
    bool ok = hipGetDevice(&ctx->device) == hipSuccess;
    ctx->chunk_elems = chunk_elems;
    // each chunk's place 16-byte aligned
    ctx->stage_bytes = (sz_max_compressed_size(chunk_elems) + 15) & ~uint64_t{15};
    {
        const uint64_t by_words = chunk_elems >= kShipGroupWords ? 1 : kShipGroupWords / chunk_elems;
        const uint64_t by_bytes = kShipGroupBytes / ctx->stage_bytes;
        ctx->group = by_words < by_bytes ? by_words : by_bytes;
        if (ctx->group == 0) ctx->group = 1;
    }
    ctx->stage_chunks = 1;  // a decode grows them to `group` chunks
    ok = ok && hipStreamCreateWithFlags(&ctx->copy, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; ok && i < kShipDepth; i++) {
        ok = hipMalloc(&ctx->stage[i], ctx->stage_bytes) == hipSuccess &&
             hipEventCreateWithFlags(&ctx->ready[i], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&ctx->done[i], hipEventDisableTiming) == hipSuccess;
    }
    ok = ok &&
         hipHostMalloc(reinterpret_cast<void**>(&ctx->h_sizes), kShipDepth * sizeof(uint64_t),
                       hipHostMallocDefault) == hipSuccess &&
         hipHostMalloc(reinterpret_cast<void**>(&ctx->h_worst), sizeof(int32_t),
                       hipHostMallocDefault) == hipSuccess &&
         hipMalloc(reinterpret_cast<void**>(&ctx->d_sizes), kShipDepth * sizeof(uint64_t)) ==
             hipSuccess &&
         hipMalloc(reinterpret_cast<void**>(&ctx->d_worst), sizeof(int32_t)) == hipSuccess;
    if (!ok) {
        delete ctx;
        return SZ_ERR_HIP;
    }
    *out = ctx;
    return SZ_OK;
}

void sz_ship_context_destroy(sz_ship_context* ctx) { delete ctx; }

sz_status sz_ship_to_host_ctx(sz_ship_context* ctx, const void* d_src, uint64_t n, void* h_dst,
                              uint64_t h_capacity, uint64_t* h_offsets, hipStream_t stream) {
    if (sz_status s = check_context(ctx)) return s;
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (h_offsets == nullptr || (n > 0 && (d_src == nullptr || h_dst == nullptr)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (n > 0 && !aligned16(d_src)) return SZ_ERR_INVALID_ARGUMENT;
    const uint64_t chunk_elems = ctx->chunk_elems;
    const uint64_t chunks = chunks_of(n, chunk_elems);
    h_offsets[0] = 0;
    if (chunks == 0) return SZ_OK;

    const uint16_t* src = static_cast<const uint16_t*>(d_src);
    uint8_t* dst = static_cast<uint8_t*>(h_dst);

    // copies chunk j's container (its size now known on the host) behind
    // the previous copies; its staging buffer is free again for chunk j +
    // kShipDepth once the copy is done
    auto ship = [&](uint64_t j) -> sz_status {
        const int b = (int)(j % kShipDepth);
        if (hipEventSynchronize(ctx->ready[b]) != hipSuccess) return SZ_ERR_HIP;
        const uint64_t size = ctx->h_sizes[b];
        const uint64_t off = h_offsets[j];
        if (size > h_capacity || off > h_capacity - size) return SZ_ERR_CAPACITY;
        if (hipStreamWaitEvent(ctx->copy, ctx->ready[b], 0) != hipSuccess ||
            hipMemcpyAsync(dst + off, ctx->stage[b], size, hipMemcpyDeviceToHost, ctx->copy) !=
                hipSuccess ||
            hipEventRecord(ctx->done[b], ctx->copy) != hipSuccess)
            return SZ_ERR_HIP;
        h_offsets[j + 1] = off + size;
        return SZ_OK;
    };

    sz_status result = SZ_OK;
    for (uint64_t c = 0; c < chunks && result == SZ_OK; c++) {
        const int b = (int)(c % kShipDepth);
        const uint64_t begin = c * chunk_elems;
        const uint64_t len = n - begin < chunk_elems ? n - begin : chunk_elems;
        // the staging buffer is free once chunk c - kShipDepth's copy is done
        if (c >= kShipDepth && hipStreamWaitEvent(stream, ctx->done[b], 0) != hipSuccess) {
            result = SZ_ERR_HIP;
            break;
        }
        result = sz_encode(src + begin, len, ctx->stage[b], ctx->stage_bytes, ctx->d_sizes + b,
                           stream);
        if (result != SZ_OK) break;
        if (hipMemcpyAsync(ctx->h_sizes + b, ctx->d_sizes + b, sizeof(uint64_t),
                           hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipEventRecord(ctx->ready[b], stream) != hipSuccess) {
            result = SZ_ERR_HIP;
            break;
        }
        // chunk c is queued; ship chunk c - 1 while the device encodes it
        if (c >= 1) result = ship(c - 1);
    }
    if (result == SZ_OK) result = ship(chunks - 1);
    return drain(ctx, stream, result);
}

sz_status sz_ship_from_host_ctx(sz_ship_context* ctx, const void* h_src,
                                const uint64_t* h_offsets, uint64_t n, void* d_dst,
                                int32_t* d_status, hipStream_t stream) {
    if (sz_status s = check_context(ctx)) return s;
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (h_offsets == nullptr || (n > 0 && (h_src == nullptr || d_dst == nullptr)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (n > 0 && !aligned16(d_dst)) return SZ_ERR_INVALID_ARGUMENT;
    const uint64_t chunk_elems = ctx->chunk_elems;
    const uint64_t chunks = chunks_of(n, chunk_elems);
    if (sz_status s = check_offsets(h_offsets, n, chunk_elems)) return s;
    if (chunks == 0) return SZ_OK;
    if (ctx->stage_chunks < ctx->group) {  // the first decode on this context
        if (hipStreamSynchronize(stream) != hipSuccess ||
            hipStreamSynchronize(ctx->copy) != hipSuccess)
            return SZ_ERR_HIP;
        for (int i = 0; i < kShipDepth; i++) {
            (void)hipFree(ctx->stage[i]);
            ctx->stage[i] = nullptr;
        }
        ctx->stage_chunks = 0;
        for (int i = 0; i < kShipDepth; i++)
            if (hipMalloc(&ctx->stage[i], ctx->group * ctx->stage_bytes) != hipSuccess) {
                // back to one chunk per buffer, so that the context stays usable
                for (int j = 0; j < kShipDepth; j++) {
                    if (ctx->stage[j]) (void)hipFree(ctx->stage[j]);
                    ctx->stage[j] = nullptr;
                }
                for (int j = 0; j < kShipDepth; j++)
                    if (hipMalloc(&ctx->stage[j], ctx->stage_bytes) != hipSuccess) return SZ_ERR_HIP;
                ctx->stage_chunks = 1;
                return SZ_ERR_HIP;
            }
        ctx->stage_chunks = ctx->group;
    }
    if (chunks > ctx->status_cap) {  // more chunks than any decode before
        if (hipStreamSynchronize(stream) != hipSuccess) return SZ_ERR_HIP;
        if (ctx->d_status) (void)hipFree(ctx->d_status);
        ctx->d_status = nullptr;
        ctx->status_cap = 0;
        if (hipMalloc(reinterpret_cast<void**>(&ctx->d_status), chunks * sizeof(int32_t)) !=
            hipSuccess)
            return SZ_ERR_HIP;
        ctx->status_cap = chunks;
    }

    const uint8_t* src = static_cast<const uint8_t*>(h_src);
    uint16_t* dst = static_cast<uint16_t*>(d_dst);
    const uint64_t group = ctx->group;
    sz_status result = SZ_OK;
    for (uint64_t g = 0; g * group < chunks && result == SZ_OK; g++) {
        const int b = (int)(g % kShipDepth);
        const uint64_t c0 = g * group, c1 = c0 + group < chunks ? c0 + group : chunks;
        uint8_t* stage = static_cast<uint8_t*>(ctx->stage[b]);
        // the staging buffer is free once group g - kShipDepth's decodes are done
        if (g >= kShipDepth && hipStreamWaitEvent(ctx->copy, ctx->done[b], 0) != hipSuccess) {
            result = SZ_ERR_HIP;
            break;
        }
        for (uint64_t c = c0; c < c1 && result == SZ_OK; c++)
            if (hipMemcpyAsync(stage + (c - c0) * ctx->stage_bytes, src + h_offsets[c],
                               h_offsets[c + 1] - h_offsets[c], hipMemcpyHostToDevice,
                               ctx->copy) != hipSuccess)
                result = SZ_ERR_HIP;
        if (result != SZ_OK || hipEventRecord(ctx->ready[b], ctx->copy) != hipSuccess ||
            hipStreamWaitEvent(stream, ctx->ready[b], 0) != hipSuccess) {
            result = SZ_ERR_HIP;
            break;
        }
        for (uint64_t c = c0; c < c1 && result == SZ_OK; c++) {
            const uint64_t begin = c * chunk_elems;
            const uint64_t len = n - begin < chunk_elems ? n - begin : chunk_elems;
            // every decode form writes its chunk's status word
            result = sz_decode(stage + (c - c0) * ctx->stage_bytes, h_offsets[c + 1] - h_offsets[c],
                               dst + begin, len, ctx->d_status + c, stream);
        }
        if (result == SZ_OK && hipEventRecord(ctx->done[b], stream) != hipSuccess)
            result = SZ_ERR_HIP;
    }
    if (result == SZ_OK) {
        // one status for the whole tensor, the worst chunk's, folded on the
        // device; the host reads that one word
        k_status_worst<<<1, 256, 0, stream>>>(ctx->d_status, chunks, ctx->d_worst);
        if (hipGetLastError() != hipSuccess ||
            (d_status && hipMemcpyAsync(d_status, ctx->d_worst, sizeof(int32_t),
                                        hipMemcpyDeviceToDevice, stream) != hipSuccess) ||
            hipMemcpyAsync(ctx->h_worst, ctx->d_worst, sizeof(int32_t), hipMemcpyDeviceToHost,
                           stream) != hipSuccess)
            result = SZ_ERR_HIP;
    }
    result = drain(ctx, stream, result);
    if (result != SZ_OK) return result;
    return *ctx->h_worst == SZ_OK ? SZ_OK : SZ_ERR_CORRUPT;
}

sz_status sz_ship_to_host(const void* d_src, uint64_t n, uint64_t chunk_elems, void* h_dst,
                          uint64_t h_capacity, uint64_t* h_offsets, hipStream_t stream) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (!chunk_size_ok(chunk_elems)) return SZ_ERR_INVALID_ARGUMENT;
    if (h_offsets == nullptr || (n > 0 && (d_src == nullptr || h_dst == nullptr)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (n > 0 && !aligned16(d_src)) return SZ_ERR_INVALID_ARGUMENT;
    if (n == 0) {
        h_offsets[0] = 0;
        return SZ_OK;
    }
    sz_ship_context* ctx = nullptr;
    if (sz_status s = sz_ship_context_create(chunk_elems, &ctx)) return s;
    const sz_status s = sz_ship_to_host_ctx(ctx, d_src, n, h_dst, h_capacity, h_offsets, stream);
    sz_ship_context_destroy(ctx);
    return s;
}

sz_status sz_ship_from_host(const void* h_src, const uint64_t* h_offsets, uint64_t n,
                            uint64_t chunk_elems, void* d_dst, int32_t* d_status,
                            hipStream_t stream) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (!chunk_size_ok(chunk_elems)) return SZ_ERR_INVALID_ARGUMENT;
    if (h_offsets == nullptr || (n > 0 && (h_src == nullptr || d_dst == nullptr)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (n > 0 && !aligned16(d_dst)) return SZ_ERR_INVALID_ARGUMENT;
    if (sz_status s = check_offsets(h_offsets, n, chunk_elems)) return s;
    if (n == 0) return SZ_OK;
    sz_ship_context* ctx = nullptr;
    if (sz_status s = sz_ship_context_create(chunk_elems, &ctx)) return s;
    const sz_status s = sz_ship_from_host_ctx(ctx, h_src, h_offsets, n, d_dst, d_status, stream);
    sz_ship_context_destroy(ctx);
    return s;
}

}  // extern "C"
