// ship.hip -- moving a tensor between device and pinned host memory in
// compressed form, chunk by chunk, with the codec and the copies overlapped.
//
// The SplitZip explainers (gist.science pages for arXiv 2605.01708) present
// the codec as a way to shrink the KV transfer between the prefill and the
// decode servers of a disaggregated deployment (introduction and section
// "Les Resultats": the KV transfer gets faster).  On one GPU the transfer
// that exists is the PCIe copy to and from host memory, so these two calls
// wrap the codec around it: the tensor is cut into chunks, each chunk is an
// ordinary container (its own codebook), and while chunk c is encoded (or
// decoded) on the caller's stream, chunk c-1's container is copied on a
// second stream.  Host code only: the kernels are the codec's.
#include "splitzip.h"
#include "sz_internal.h"

#include <vector>

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

uint64_t chunks_of(uint64_t n, uint64_t chunk) { return chunk ? (n + chunk - 1) / chunk : 0; }

// Everything a call creates, released on every return path once both
// streams have drained.  The copy stream has the default priority.
struct Resources {
    hipStream_t user = nullptr;    // the caller's stream (not owned)
    hipStream_t copy = nullptr;
    std::vector<hipEvent_t> events;
    void* stage[2] = {nullptr, nullptr};
    uint64_t* h_sizes = nullptr;   // pinned, one per chunk
    int32_t* d_status = nullptr;   // one per chunk

    hipEvent_t new_event() {
        hipEvent_t ev = nullptr;
        if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return nullptr;
        events.push_back(ev);
        return ev;
    }

    ~Resources() {
        // both streams are drained before anything is released
        (void)hipStreamSynchronize(user);
        if (copy) (void)hipStreamSynchronize(copy);
        for (hipEvent_t ev : events) (void)hipEventDestroy(ev);
        if (copy) (void)hipStreamDestroy(copy);
        for (void* p : stage)
            if (p) (void)hipFree(p);
        if (h_sizes) (void)hipHostFree(h_sizes);
        if (d_status) (void)hipFree(d_status);
    }
};

}  // namespace

extern "C" {

sz_status sz_ship_to_host(const void* d_src, uint64_t n, uint64_t chunk_elems, void* h_dst,
                          uint64_t h_capacity, uint64_t* h_offsets, hipStream_t stream) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (chunk_elems == 0 || chunk_elems % 8 != 0 || chunk_elems > SZ_MAX_ELEMENTS)
        return SZ_ERR_INVALID_ARGUMENT;
    if (h_offsets == nullptr || (n > 0 && (d_src == nullptr || h_dst == nullptr)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (n > 0 && !aligned16(d_src)) return SZ_ERR_INVALID_ARGUMENT;
    const uint64_t chunks = chunks_of(n, chunk_elems);
    h_offsets[0] = 0;
    if (chunks == 0) return SZ_OK;

    Resources r;
    r.user = stream;
    const uint64_t stage_bytes = sz_max_compressed_size(chunk_elems);
    if (hipStreamCreateWithFlags(&r.copy, hipStreamNonBlocking) != hipSuccess) return SZ_ERR_HIP;
    for (void*& p : r.stage)
        if (hipMalloc(&p, stage_bytes) != hipSuccess) return SZ_ERR_HIP;
    if (hipHostMalloc(reinterpret_cast<void**>(&r.h_sizes), chunks * sizeof(uint64_t),
                      hipHostMallocDefault) != hipSuccess)
        return SZ_ERR_HIP;
    // the container size of the chunk in each staging buffer
    uint64_t* d_sizes = nullptr;
    if (hipMalloc(reinterpret_cast<void**>(&d_sizes), 2 * sizeof(uint64_t)) != hipSuccess)
        return SZ_ERR_HIP;
    struct FreeOnExit {
        uint64_t* p;
        hipStream_t s;
        ~FreeOnExit() {
            (void)hipStreamSynchronize(s);
            (void)hipFree(p);
        }
    } free_sizes{d_sizes, stream};

    std::vector<hipEvent_t> encoded(chunks), copied(2, nullptr);
    for (uint64_t c = 0; c < chunks; c++)
        if ((encoded[c] = r.new_event()) == nullptr) return SZ_ERR_HIP;
    for (auto& ev : copied)
        if ((ev = r.new_event()) == nullptr) return SZ_ERR_HIP;

    const uint16_t* src = static_cast<const uint16_t*>(d_src);
    uint8_t* dst = static_cast<uint8_t*>(h_dst);
    sz_status result = SZ_OK;

    // copies chunk j's container (its size now known on the host) behind
    // the previous copies, and frees its staging buffer for chunk j + 2
    auto ship = [&](uint64_t j) -> sz_status {
        if (hipEventSynchronize(encoded[j]) != hipSuccess) return SZ_ERR_HIP;
        const uint64_t size = r.h_sizes[j];
        const uint64_t off = h_offsets[j];
        if (size > h_capacity || off > h_capacity - size) return SZ_ERR_CAPACITY;
        if (hipStreamWaitEvent(r.copy, encoded[j], 0) != hipSuccess) return SZ_ERR_HIP;
        if (hipMemcpyAsync(dst + off, r.stage[j % 2], size, hipMemcpyDeviceToHost, r.copy) !=
            hipSuccess)
            return SZ_ERR_HIP;
        if (hipEventRecord(copied[j % 2], r.copy) != hipSuccess) return SZ_ERR_HIP;
        h_offsets[j + 1] = off + size;
        return SZ_OK;
    };

    for (uint64_t c = 0; c < chunks && result == SZ_OK; c++) {
        const uint64_t begin = c * chunk_elems;
        const uint64_t len = n - begin < chunk_elems ? n - begin : chunk_elems;
        // the staging buffer is free once chunk c - 2's copy is done
        if (c >= 2 && hipStreamWaitEvent(stream, copied[c % 2], 0) != hipSuccess) {
            result = SZ_ERR_HIP;
            break;
        }
        result = sz_encode(src + begin, len, r.stage[c % 2], stage_bytes, d_sizes + c % 2, stream);
        if (result != SZ_OK) break;
        if (hipMemcpyAsync(r.h_sizes + c, d_sizes + c % 2, sizeof(uint64_t), hipMemcpyDeviceToHost,
                           stream) != hipSuccess ||
            hipEventRecord(encoded[c], stream) != hipSuccess) {
            result = SZ_ERR_HIP;
            break;
        }
        // chunk c is queued; ship chunk c - 1 while the device encodes it
        if (c >= 1) result = ship(c - 1);
    }
    if (result == SZ_OK) result = ship(chunks - 1);
    if (hipStreamSynchronize(stream) != hipSuccess && result == SZ_OK) result = SZ_ERR_HIP;
    if (hipStreamSynchronize(r.copy) != hipSuccess && result == SZ_OK) result = SZ_ERR_HIP;
    return result;
}

sz_status sz_ship_from_host(const void* h_src, const uint64_t* h_offsets, uint64_t n,
                            uint64_t chunk_elems, void* d_dst, int32_t* d_status,
                            hipStream_t stream) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (chunk_elems == 0 || chunk_elems % 8 != 0 || chunk_elems > SZ_MAX_ELEMENTS)
        return SZ_ERR_INVALID_ARGUMENT;
    if (h_offsets == nullptr || (n > 0 && (h_src == nullptr || d_dst == nullptr)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (n > 0 && !aligned16(d_dst)) return SZ_ERR_INVALID_ARGUMENT;
    const uint64_t chunks = chunks_of(n, chunk_elems);
    // every chunk's size must be a possible container for its length
    uint64_t largest = 0;
    for (uint64_t c = 0; c < chunks; c++) {
        const uint64_t len = n - c * chunk_elems < chunk_elems ? n - c * chunk_elems : chunk_elems;
        if (h_offsets[c + 1] < h_offsets[c]) return SZ_ERR_CORRUPT;
        const uint64_t size = h_offsets[c + 1] - h_offsets[c];
        if (size < sz::container_bytes(len, 0) || size > sz_max_compressed_size(len) ||
            (size - sz::container_bytes(len, 0)) % 5 != 0)
            return SZ_ERR_CORRUPT;
        if (size > largest) largest = size;
    }
    if (chunks == 0) return SZ_OK;

    Resources r;
    r.user = stream;
    if (hipStreamCreateWithFlags(&r.copy, hipStreamNonBlocking) != hipSuccess) return SZ_ERR_HIP;
    for (void*& p : r.stage)
        if (hipMalloc(&p, largest) != hipSuccess) return SZ_ERR_HIP;
    // every decode form writes its chunk's status word, so none is cleared here
    if (hipMalloc(reinterpret_cast<void**>(&r.d_status), chunks * sizeof(int32_t)) != hipSuccess)
        return SZ_ERR_HIP;

    std::vector<hipEvent_t> arrived(chunks), decoded(2, nullptr);
    for (uint64_t c = 0; c < chunks; c++)
        if ((arrived[c] = r.new_event()) == nullptr) return SZ_ERR_HIP;
    for (auto& ev : decoded)
        if ((ev = r.new_event()) == nullptr) return SZ_ERR_HIP;

    const uint8_t* src = static_cast<const uint8_t*>(h_src);
    uint16_t* dst = static_cast<uint16_t*>(d_dst);
    sz_status result = SZ_OK;
    for (uint64_t c = 0; c < chunks && result == SZ_OK; c++) {
        const uint64_t begin = c * chunk_elems;
        const uint64_t len = n - begin < chunk_elems ? n - begin : chunk_elems;
        const uint64_t size = h_offsets[c + 1] - h_offsets[c];
        // the staging buffer is free once chunk c - 2's decode is done
        if (c >= 2 && hipStreamWaitEvent(r.copy, decoded[c % 2], 0) != hipSuccess) {
            result = SZ_ERR_HIP;
            break;
        }
        if (hipMemcpyAsync(r.stage[c % 2], src + h_offsets[c], size, hipMemcpyHostToDevice,
                           r.copy) != hipSuccess ||
            hipEventRecord(arrived[c], r.copy) != hipSuccess ||
            hipStreamWaitEvent(stream, arrived[c], 0) != hipSuccess) {
            result = SZ_ERR_HIP;
            break;
        }
        result = sz_decode(r.stage[c % 2], size, dst + begin, len, r.d_status + c, stream);
        if (result != SZ_OK) break;
        if (hipEventRecord(decoded[c % 2], stream) != hipSuccess) result = SZ_ERR_HIP;
    }
    if (hipStreamSynchronize(stream) != hipSuccess && result == SZ_OK) result = SZ_ERR_HIP;
    if (hipStreamSynchronize(r.copy) != hipSuccess && result == SZ_OK) result = SZ_ERR_HIP;
    if (result != SZ_OK) return result;

    // one status for the whole tensor: the worst chunk's
    std::vector<int32_t> st(chunks, 0);
    if (hipMemcpy(st.data(), r.d_status, chunks * sizeof(int32_t), hipMemcpyDeviceToHost) !=
        hipSuccess)
        return SZ_ERR_HIP;
    int32_t worst = SZ_OK;
    for (int32_t v : st)
        if (v != SZ_OK) worst = v;
    if (d_status && hipMemcpy(d_status, &worst, sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess)
        return SZ_ERR_HIP;
    return worst == SZ_OK ? SZ_OK : SZ_ERR_CORRUPT;
}

}  // extern "C"
