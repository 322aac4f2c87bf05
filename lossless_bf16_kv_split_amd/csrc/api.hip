// api.hip -- extern "C" entry points of libsplitzip.so (declared, with their
// argument contracts, in include/splitzip.h).
//
// Host side only: argument checks that need no device access, the chunk
// plan, a library-owned stream-ordered memory pool for sz_encode's
// workspace, and the kernel launch sequences.  No call synchronises the host.
#include "splitzip.h"
#include "sz_internal.h"

#include <mutex>

namespace {

constexpr int kMaxDevices = 64;

// sz_encode takes the single-read passes from this many words on.  Below,
// their two extra launches (sample ranking, finish) cost more than the
// second read of the input saves: on MI355X the two forms break even
// between 2^25 and 2^26 words of KV data.
constexpr uint64_t kSingleReadAuto = uint64_t{1} << 26;

std::mutex g_mutex;
hipMemPool_t g_pools[kMaxDevices] = {};
int g_num_cus[kMaxDevices] = {};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, uint64_t a_bytes, const void* b, uint64_t b_bytes) {
    if (a_bytes == 0 || b_bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + b_bytes && b0 < a0 + a_bytes;
}

int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    return dev;
}

int num_cus(int dev) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_num_cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        g_num_cus[dev] = v;
    }
    return g_num_cus[dev];
}

// A private pool, so that sz_encode neither changes the process-wide
// default pool nor returns its workspace to the driver after every call.
hipMemPool_t pool_for(int dev) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_pools[dev] == nullptr) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) != hipSuccess) return nullptr;
        uint64_t keep = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        g_pools[dev] = pool;
    }
    return g_pools[dev];
}

sz_status check_encode_args(const void* src, uint64_t n, const void* dst, uint64_t cap) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (dst == nullptr || (n > 0 && src == nullptr)) return SZ_ERR_INVALID_ARGUMENT;
    if (!aligned(dst, 16) || (n > 0 && !aligned(src, 16))) return SZ_ERR_INVALID_ARGUMENT;
    if (cap < sz_max_compressed_size(n)) return SZ_ERR_CAPACITY;
    if (overlap(src, 2 * n, dst, cap)) return SZ_ERR_INVALID_ARGUMENT;
    return SZ_OK;
}

sz_status check_workspace(const void* ws, uint64_t ws_bytes, const sz::EncodePlan& p) {
    if (ws == nullptr || !aligned(ws, 256) || ws_bytes < p.ws_bytes) return SZ_ERR_INVALID_ARGUMENT;
    return SZ_OK;
}

// The single-read passes need n >= 2^20; their scratch area lies inside
// sz_max_compressed_size(n), which check_encode_args demands.
sz_status check_single_read(const sz::EncodePlan& p, uint64_t dst_capacity) {
    if (!p.single_read || p.scratch_end > dst_capacity) return SZ_ERR_INVALID_ARGUMENT;
    return SZ_OK;
}

// Host-side container checks for decode; derives the escape count E from
// the container size alone (total = 176 + ceil(n/2) + n + 5E).
sz_status check_decode_args(const void* src, uint64_t src_bytes, const void* dst, uint64_t n,
                            uint64_t* e_out) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (src == nullptr || (n > 0 && dst == nullptr)) return SZ_ERR_INVALID_ARGUMENT;
    if (!aligned(src, 16) || (n > 0 && !aligned(dst, 16))) return SZ_ERR_INVALID_ARGUMENT;
    const uint64_t fixed = sz::container_bytes(n, 0);
    if (src_bytes < fixed || (src_bytes - fixed) % 5 != 0) return SZ_ERR_CORRUPT;
    const uint64_t e = (src_bytes - fixed) / 5;
    if (e > (15 * n) / 16) return SZ_ERR_CORRUPT;
    if (overlap(src, src_bytes, dst, 2 * n)) return SZ_ERR_INVALID_ARGUMENT;
    *e_out = e;
    return SZ_OK;
}

sz_status hip_status(hipError_t e) { return e == hipSuccess ? SZ_OK : SZ_ERR_HIP; }

// true while `stream` is being captured into a graph (no pool allocation then)
bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &st) != hipSuccess || st != hipStreamCaptureStatusNone;
}

sz::FlatWords flat(const void* p) {
    return sz::FlatWords{const_cast<uint16_t*>(static_cast<const uint16_t*>(p))};
}

// The encode passes sz_encode runs for n words, over the workspace w
template <class Words>
sz_status encode_passes(Words src, uint64_t n, const sz::EncodePlan& p, uint8_t* w, void* d_dst,
                        uint64_t dst_capacity, uint64_t* d_compressed_size, int dev,
                        hipStream_t stream) {
    uint8_t* out = static_cast<uint8_t*>(d_dst);
    sz_status st = SZ_OK;
    if (p.single_read && n >= kSingleReadAuto && p.scratch_end <= dst_capacity) {
        // one read of the input when the sampled codebook holds; the finish
        // pass reads it again only when it does not
        st = hip_status(sz::launch_sample(src, p, w, stream));
        if (st == SZ_OK) st = hip_status(sz::launch_first_pass(src, p, w, out, dst_capacity, stream));
        if (st == SZ_OK)
            st = hip_status(sz::launch_finish(src, p, w, out, dst_capacity, d_compressed_size, stream));
    } else if (p.chunks >= 1 && p.chunks <= sz::kRankedChunks) {
        // few chunks: the pack workgroups rank the counts themselves, with
        // no codebook pass between the two launches
        st = hip_status(sz::launch_histogram(src, p, w, stream));
        if (st == SZ_OK)
            st = hip_status(sz::launch_pack_ranked(src, p, w, out, dst_capacity,
                                                   d_compressed_size, stream));
    } else {
        st = hip_status(sz::launch_histogram(src, p, w, stream));
        // the codebook pass reads counts only, not the words
        if (st == SZ_OK)
            st = hip_status(sz::launch_codebook(sz::FlatWords{nullptr}, p, w, out,
                                                d_compressed_size, stream));
        if (st == SZ_OK)
            st = hip_status(sz::launch_pack(src, p, w, out, dst_capacity, num_cus(dev), stream));
    }
    return st;
}

// the same passes with the workspace from the library pool
template <class Words>
sz_status encode_with_pool(Words src, uint64_t n, void* d_dst, uint64_t dst_capacity,
                           uint64_t* d_compressed_size, int dev, hipMemPool_t pool,
                           hipStream_t stream) {
    const sz::EncodePlan p = sz::plan_encode(n);
    void* ws = nullptr;
    if (hipMallocFromPoolAsync(&ws, p.ws_bytes, pool, stream) != hipSuccess) return SZ_ERR_HIP;
    sz_status st = encode_passes(src, n, p, static_cast<uint8_t*>(ws), d_dst, dst_capacity,
                                 d_compressed_size, dev, stream);
    if (hipFreeAsync(ws, stream) != hipSuccess && st == SZ_OK) st = SZ_ERR_HIP;
    return st;
}

// sz_encode_noalloc's workspace: one array per GPU, loaded with the library
// and held until the process ends.  Its name is a host-side stand-in; the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[SZ_NOALLOC_WORKSPACE_BYTES];
uint8_t* g_scratch_ptr[kMaxDevices] = {};

uint8_t* scratch_for(int dev) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return nullptr;
        g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
    }
    return g_scratch_ptr[dev];
}

sz_status check_decode_workspace(const void* ws, uint64_t ws_bytes, uint64_t n) {
    if (ws == nullptr || !aligned(ws, 256) || ws_bytes < sz::tile_index_layout(n).bytes)
        return SZ_ERR_INVALID_ARGUMENT;
    return SZ_OK;
}

// the decode form sz_decode picks for this escape density
template <class Words>
sz_status decode_by_density(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                            Words dst, int32_t* d_status, hipStream_t stream) {
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    if (n < sz::kTileDecodeMin && e <= n / sz::kScatterDecodeDensity) {
        // small and sparse: stream every word out, then rewrite the escaped ones
        sz_status st = hip_status(sz::launch_unpack(src, src_bytes, n, e, dst, d_status,
                                                    num_cus(dev), stream));
        if (st != SZ_OK) return st;
        return hip_status(sz::launch_scatter(src, n, e, dst, d_status, stream));
    }
    // few escapes in a large tensor: tiles handed out grid-stride after a
    // tile index, in a workspace from the pool (none under graph capture)
    hipMemPool_t pool = e > n / sz::kTileDecodeDensity || n < sz::kTileDecodeMin ||
                                capturing(stream)
                            ? nullptr
                            : pool_for(dev);
    if (pool == nullptr) {
        // many escapes, or no workspace: one pass with a per-word LDS map
        return hip_status(sz::launch_decode_dense(src, src_bytes, n, e, dst, d_status, stream));
    }
    const sz::TileIndexLayout l = sz::tile_index_layout(n);
    void* ws = nullptr;
    if (hipMallocFromPoolAsync(&ws, l.bytes, pool, stream) != hipSuccess) return SZ_ERR_HIP;
    uint8_t* w = static_cast<uint8_t*>(ws);
    sz_status st =
        hip_status(sz::launch_tile_index(src, src_bytes, n, e, w, sz::FlatWords{nullptr}, stream));
    if (st == SZ_OK)
        st = hip_status(sz::launch_decode_tiles(src, n, e, w, dst, d_status, num_cus(dev), stream));
    if (hipFreeAsync(ws, stream) != hipSuccess && st == SZ_OK) st = SZ_ERR_HIP;
    return st;
}

// Host checks of a page description: 2^k-word pages, k >= 14, enough of
// them for n words, and a table pointer; the addresses themselves are on
// the device and are checked there.  Returns the number of pages used.
sz_status check_pages(const void* d_pages, uint64_t n_pages, uint64_t page_elems, uint64_t n,
                      uint32_t* log2_out, uint64_t* used_out) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (page_elems == 0 || (page_elems & (page_elems - 1)) != 0 ||
        page_elems < (uint64_t{1} << sz::kMinPageLog2) || page_elems > SZ_MAX_ELEMENTS)
        return SZ_ERR_INVALID_ARGUMENT;
    uint32_t lg = 0;
    while ((uint64_t{1} << lg) < page_elems) lg++;
    const uint64_t used = (n + page_elems - 1) >> lg;
    if (used > n_pages) return SZ_ERR_INVALID_ARGUMENT;
    if (used > 0 && (d_pages == nullptr || !aligned(d_pages, 8))) return SZ_ERR_INVALID_ARGUMENT;
    *log2_out = lg;
    *used_out = used;
    return SZ_OK;
}

// Per-block calls: at most one block per grid row (HIP's grid height
// limit), a workspace of one encode workspace per block (for the chunk plan
// of all the blocks together), 256-byte strides, and then a flag word per
// block.
constexpr uint64_t kMaxBlocks = 65535;

uint64_t round256(uint64_t x) { return (x + 255) & ~uint64_t{255}; }

struct BlockLayout {
    sz::EncodePlan plan;
    uint64_t stride;     // bytes of workspace per block
    uint64_t flags_off;  // the per-block flags
    uint64_t bytes;
};

BlockLayout block_layout(uint64_t block_elems, uint64_t n_blocks) {
    BlockLayout l;
    l.plan = sz::plan_blocks(block_elems, n_blocks);
    l.stride = round256(l.plan.ws_bytes);
    l.flags_off = n_blocks * l.stride;
    l.bytes = l.flags_off + round256(4 * n_blocks);
    return l;
}

// Host checks shared by the block calls: the block count, the table
// pointer, the container buffer and its pitch, and the size array.  The
// encode needs room for the largest container of a block; the decode only
// a pitch that can hold a container at all (each size is checked against
// the pitch on the device).
sz_status check_blocks(const void* table, uint64_t n_blocks, uint64_t block_elems,
                       const void* containers, uint64_t pitch, const void* sizes, bool encode) {
    if (block_elems > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (n_blocks == 0 || n_blocks > kMaxBlocks) return SZ_ERR_INVALID_ARGUMENT;
    if (table == nullptr || !aligned(table, 8)) return SZ_ERR_INVALID_ARGUMENT;
    if (containers == nullptr || !aligned(containers, 16) || pitch % 16 != 0)
        return SZ_ERR_INVALID_ARGUMENT;
    if (sizes == nullptr || !aligned(sizes, 8)) return SZ_ERR_INVALID_ARGUMENT;
    if (encode && pitch < sz_max_compressed_size(block_elems)) return SZ_ERR_CAPACITY;
    if (!encode && pitch < sz::container_bytes(block_elems, 0)) return SZ_ERR_INVALID_ARGUMENT;
    return SZ_OK;
}

uint16_t* const* block_table(const void* const* t) {
    return reinterpret_cast<uint16_t* const*>(const_cast<void* const*>(t));
}

}  // namespace

extern "C" {

uint64_t sz_max_compressed_size(uint64_t n) {
    if (n > SZ_MAX_ELEMENTS) return 0;
    return sz::container_bytes(n, (15 * n) / 16);
}

uint64_t sz_workspace_size(uint64_t n) {
    if (n > SZ_MAX_ELEMENTS) return 0;
    return sz::plan_encode(n).ws_bytes;
}

sz_status sz_encode_histogram(const void* d_src, uint64_t n, void* d_workspace,
                              uint64_t workspace_bytes, hipStream_t stream) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (n > 0 && (d_src == nullptr || !aligned(d_src, 16))) return SZ_ERR_INVALID_ARGUMENT;
    const sz::EncodePlan p = sz::plan_encode(n);
    if (sz_status s = check_workspace(d_workspace, workspace_bytes, p)) return s;
    return hip_status(sz::launch_histogram(flat(d_src), p,
                                           static_cast<uint8_t*>(d_workspace), stream));
}

sz_status sz_encode_codebook(uint64_t n, void* d_workspace, uint64_t workspace_bytes, void* d_dst,
                             uint64_t dst_capacity, uint64_t* d_compressed_size,
                             hipStream_t stream) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (d_dst == nullptr || !aligned(d_dst, 16)) return SZ_ERR_INVALID_ARGUMENT;
    if (dst_capacity < sz_max_compressed_size(n)) return SZ_ERR_CAPACITY;
    const sz::EncodePlan p = sz::plan_encode(n);
    if (sz_status s = check_workspace(d_workspace, workspace_bytes, p)) return s;
    return hip_status(sz::launch_codebook(sz::FlatWords{nullptr}, p,
                                          static_cast<uint8_t*>(d_workspace),
                                          static_cast<uint8_t*>(d_dst), d_compressed_size,
                                          stream));
}

sz_status sz_encode_pack(const void* d_src, uint64_t n, const void* d_workspace,
                         uint64_t workspace_bytes, void* d_dst, uint64_t dst_capacity,
                         hipStream_t stream) {
    if (sz_status s = check_encode_args(d_src, n, d_dst, dst_capacity)) return s;
    const sz::EncodePlan p = sz::plan_encode(n);
    if (sz_status s = check_workspace(d_workspace, workspace_bytes, p)) return s;
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    return hip_status(sz::launch_pack(flat(d_src), p,
                                      static_cast<const uint8_t*>(d_workspace),
                                      static_cast<uint8_t*>(d_dst), dst_capacity, num_cus(dev),
                                      stream));
}

sz_status sz_encode_pack_ranked(const void* d_src, uint64_t n, const void* d_workspace,
                                uint64_t workspace_bytes, void* d_dst, uint64_t dst_capacity,
                                uint64_t* d_compressed_size, hipStream_t stream) {
    if (sz_status s = check_encode_args(d_src, n, d_dst, dst_capacity)) return s;
    const sz::EncodePlan p = sz::plan_encode(n);
    if (p.chunks < 1 || p.chunks > sz::kRankedChunks) return SZ_ERR_INVALID_ARGUMENT;
    if (sz_status s = check_workspace(d_workspace, workspace_bytes, p)) return s;
    return hip_status(sz::launch_pack_ranked(flat(d_src), p,
                                             static_cast<const uint8_t*>(d_workspace),
                                             static_cast<uint8_t*>(d_dst), dst_capacity,
                                             d_compressed_size, stream));
}

int sz_encode_single_read(uint64_t n) {
    if (n > SZ_MAX_ELEMENTS) return 0;
    return n >= kSingleReadAuto && sz::plan_encode(n).single_read ? 1 : 0;
}

sz_status sz_encode_sample(const void* d_src, uint64_t n, void* d_workspace,
                           uint64_t workspace_bytes, hipStream_t stream) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (d_src == nullptr || !aligned(d_src, 16)) return SZ_ERR_INVALID_ARGUMENT;
    const sz::EncodePlan p = sz::plan_encode(n);
    if (sz_status s = check_workspace(d_workspace, workspace_bytes, p)) return s;
    if (!p.single_read) return SZ_ERR_INVALID_ARGUMENT;
    return hip_status(sz::launch_sample(flat(d_src), p, static_cast<uint8_t*>(d_workspace),
                                        stream));
}

sz_status sz_encode_first_pass(const void* d_src, uint64_t n, void* d_workspace,
                               uint64_t workspace_bytes, void* d_dst, uint64_t dst_capacity,
                               hipStream_t stream) {
    if (sz_status s = check_encode_args(d_src, n, d_dst, dst_capacity)) return s;
    const sz::EncodePlan p = sz::plan_encode(n);
    if (sz_status s = check_workspace(d_workspace, workspace_bytes, p)) return s;
    if (sz_status s = check_single_read(p, dst_capacity)) return s;
    return hip_status(sz::launch_first_pass(flat(d_src), p, static_cast<uint8_t*>(d_workspace),
                                            static_cast<uint8_t*>(d_dst), dst_capacity, stream));
}

sz_status sz_encode_finish(const void* d_src, uint64_t n, void* d_workspace,
                           uint64_t workspace_bytes, void* d_dst, uint64_t dst_capacity,
                           uint64_t* d_compressed_size, hipStream_t stream) {
    if (sz_status s = check_encode_args(d_src, n, d_dst, dst_capacity)) return s;
    const sz::EncodePlan p = sz::plan_encode(n);
    if (sz_status s = check_workspace(d_workspace, workspace_bytes, p)) return s;
    if (sz_status s = check_single_read(p, dst_capacity)) return s;
    return hip_status(sz::launch_finish(flat(d_src), p, static_cast<uint8_t*>(d_workspace),
                                        static_cast<uint8_t*>(d_dst), dst_capacity,
                                        d_compressed_size, stream));
}

sz_status sz_encode(const void* d_src, uint64_t n, void* d_dst, uint64_t dst_capacity,
                    uint64_t* d_compressed_size, hipStream_t stream) {
    if (sz_status s = check_encode_args(d_src, n, d_dst, dst_capacity)) return s;
    // its workspace comes from the pool, which a graph cannot capture
    if (capturing(stream)) return SZ_ERR_INVALID_ARGUMENT;
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    hipMemPool_t pool = pool_for(dev);
    if (pool == nullptr) return SZ_ERR_HIP;
    return encode_with_pool(flat(d_src), n, d_dst, dst_capacity, d_compressed_size, dev, pool,
                            stream);
}

sz_status sz_encode_noalloc(const void* d_src, uint64_t n, void* d_dst, uint64_t dst_capacity,
                            uint64_t* d_compressed_size, hipStream_t stream) {
    if (sz_status s = check_encode_args(d_src, n, d_dst, dst_capacity)) return s;
    const sz::EncodePlan p = sz::plan_encode(n);
    if (p.ws_bytes > SZ_NOALLOC_WORKSPACE_BYTES) return SZ_ERR_TOO_LARGE;
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    uint8_t* ws = scratch_for(dev);
    if (ws == nullptr) return SZ_ERR_HIP;
    return encode_passes(flat(d_src), n, p, ws, d_dst, dst_capacity, d_compressed_size, dev,
                         stream);
}

sz_status sz_decode_unpack(const void* d_src, uint64_t src_bytes, void* d_dst, uint64_t n,
                           int32_t* d_status, hipStream_t stream) {
    uint64_t e = 0;
    if (sz_status s = check_decode_args(d_src, src_bytes, d_dst, n, &e)) return s;
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    return hip_status(sz::launch_unpack(static_cast<const uint8_t*>(d_src), src_bytes, n, e,
                                        flat(d_dst), d_status, num_cus(dev), stream));
}

sz_status sz_decode_scatter(const void* d_src, uint64_t src_bytes, void* d_dst, uint64_t n,
                            int32_t* d_status, hipStream_t stream) {
    uint64_t e = 0;
    if (sz_status s = check_decode_args(d_src, src_bytes, d_dst, n, &e)) return s;
    return hip_status(sz::launch_scatter(static_cast<const uint8_t*>(d_src), n, e, flat(d_dst),
                                         d_status, stream));
}

sz_status sz_decode(const void* d_src, uint64_t src_bytes, void* d_dst, uint64_t n,
                    int32_t* d_status, hipStream_t stream) {
    uint64_t e = 0;
    if (sz_status s = check_decode_args(d_src, src_bytes, d_dst, n, &e)) return s;
    return decode_by_density(static_cast<const uint8_t*>(d_src), src_bytes, n, e, flat(d_dst),
                             d_status, stream);
}

uint64_t sz_decode_workspace_size(uint64_t n) {
    if (n > SZ_MAX_ELEMENTS) return 0;
    return sz::tile_index_layout(n).bytes;
}

sz_status sz_decode_index(const void* d_src, uint64_t src_bytes, uint64_t n, void* d_workspace,
                          uint64_t workspace_bytes, hipStream_t stream) {
    if (n > SZ_MAX_ELEMENTS) return SZ_ERR_TOO_LARGE;
    if (d_src == nullptr || !aligned(d_src, 16)) return SZ_ERR_INVALID_ARGUMENT;
    if (sz_status s = check_decode_workspace(d_workspace, workspace_bytes, n)) return s;
    const uint64_t fixed = sz::container_bytes(n, 0);
    if (src_bytes < fixed || (src_bytes - fixed) % 5 != 0) return SZ_ERR_CORRUPT;
    const uint64_t e = (src_bytes - fixed) / 5;
    if (e > (15 * n) / 16) return SZ_ERR_CORRUPT;
    if (overlap(d_src, src_bytes, d_workspace, workspace_bytes)) return SZ_ERR_INVALID_ARGUMENT;
    return hip_status(sz::launch_tile_index(static_cast<const uint8_t*>(d_src), src_bytes, n, e,
                                            static_cast<uint8_t*>(d_workspace), sz::FlatWords{nullptr}, stream));
}

sz_status sz_decode_tiles(const void* d_src, uint64_t src_bytes, const void* d_workspace,
                          uint64_t workspace_bytes, void* d_dst, uint64_t n, int32_t* d_status,
                          hipStream_t stream) {
    uint64_t e = 0;
    if (sz_status s = check_decode_args(d_src, src_bytes, d_dst, n, &e)) return s;
    if (sz_status s = check_decode_workspace(d_workspace, workspace_bytes, n)) return s;
    if (overlap(d_dst, 2 * n, d_workspace, workspace_bytes) ||
        overlap(d_src, src_bytes, d_workspace, workspace_bytes))
        return SZ_ERR_INVALID_ARGUMENT;
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    return hip_status(sz::launch_decode_tiles(static_cast<const uint8_t*>(d_src), n, e,
                                              static_cast<const uint8_t*>(d_workspace),
                                              flat(d_dst), d_status, num_cus(dev), stream));
}

sz_status sz_decode_fused(const void* d_src, uint64_t src_bytes, void* d_dst, uint64_t n,
                          int32_t* d_status, hipStream_t stream) {
    uint64_t e = 0;
    if (sz_status s = check_decode_args(d_src, src_bytes, d_dst, n, &e)) return s;
    return hip_status(sz::launch_decode_fused(static_cast<const uint8_t*>(d_src), src_bytes, n, e,
                                              flat(d_dst), d_status, stream));
}

sz_status sz_decode_dense(const void* d_src, uint64_t src_bytes, void* d_dst, uint64_t n,
                          int32_t* d_status, hipStream_t stream) {
    uint64_t e = 0;
    if (sz_status s = check_decode_args(d_src, src_bytes, d_dst, n, &e)) return s;
    return hip_status(sz::launch_decode_dense(static_cast<const uint8_t*>(d_src), src_bytes, n, e,
                                              flat(d_dst), d_status, stream));
}

sz_status sz_encode_pages(const void* const* d_pages, uint64_t n_pages, uint64_t page_elems,
                          uint64_t n, void* d_dst, uint64_t dst_capacity,
                          uint64_t* d_compressed_size, int32_t* d_status, hipStream_t stream) {
    uint32_t lg = 0;
    uint64_t used = 0;
    if (sz_status s = check_pages(d_pages, n_pages, page_elems, n, &lg, &used)) return s;
    if (d_dst == nullptr || !aligned(d_dst, 16)) return SZ_ERR_INVALID_ARGUMENT;
    if (dst_capacity < sz_max_compressed_size(n)) return SZ_ERR_CAPACITY;
    if (capturing(stream)) return SZ_ERR_INVALID_ARGUMENT;  // pool memory below
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    hipMemPool_t pool = pool_for(dev);
    if (pool == nullptr) return SZ_ERR_HIP;
    void* flag = nullptr;
    if (hipMallocFromPoolAsync(&flag, 256, pool, stream) != hipSuccess) return SZ_ERR_HIP;
    int32_t* bad = static_cast<int32_t*>(flag);
    const sz::PagedWords src{reinterpret_cast<uint16_t* const*>(const_cast<void* const*>(d_pages)),
                             lg, bad};
    sz_status st = hip_status(sz::launch_check_pages(src.pages, used, bad, d_status, stream));
    if (st == SZ_OK)
        st = encode_with_pool(src, n, d_dst, dst_capacity, d_compressed_size, dev, pool, stream);
    if (hipFreeAsync(flag, stream) != hipSuccess && st == SZ_OK) st = SZ_ERR_HIP;
    return st;
}

sz_status sz_decode_pages(const void* d_src, uint64_t src_bytes, void* const* d_pages,
                          uint64_t n_pages, uint64_t page_elems, uint64_t n, int32_t* d_status,
                          hipStream_t stream) {
    uint32_t lg = 0;
    uint64_t used = 0;
    if (sz_status s = check_pages(d_pages, n_pages, page_elems, n, &lg, &used)) return s;
    uint64_t e = 0;
    // the output pages are checked on the device; here only the container
    if (d_src == nullptr || !aligned(d_src, 16)) return SZ_ERR_INVALID_ARGUMENT;
    const uint64_t fixed = sz::container_bytes(n, 0);
    if (src_bytes < fixed || (src_bytes - fixed) % 5 != 0) return SZ_ERR_CORRUPT;
    e = (src_bytes - fixed) / 5;
    if (e > (15 * n) / 16) return SZ_ERR_CORRUPT;
    if (capturing(stream)) return SZ_ERR_INVALID_ARGUMENT;  // pool memory below
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    hipMemPool_t pool = pool_for(dev);
    if (pool == nullptr) return SZ_ERR_HIP;
    void* flag = nullptr;
    if (hipMallocFromPoolAsync(&flag, 256, pool, stream) != hipSuccess) return SZ_ERR_HIP;
    int32_t* bad = static_cast<int32_t*>(flag);
    const sz::PagedWords dst{reinterpret_cast<uint16_t* const*>(d_pages), lg, bad};
    sz_status st = hip_status(sz::launch_check_pages(dst.pages, used, bad, nullptr, stream));
    if (st == SZ_OK)
        st = decode_by_density(static_cast<const uint8_t*>(d_src), src_bytes, n, e, dst, d_status,
                               stream);
    if (hipFreeAsync(flag, stream) != hipSuccess && st == SZ_OK) st = SZ_ERR_HIP;
    return st;
}

uint64_t sz_blocks_workspace_size(uint64_t block_elems, uint64_t n_blocks) {
    if (block_elems > SZ_MAX_ELEMENTS || n_blocks == 0 || n_blocks > kMaxBlocks) return 0;
    return block_layout(block_elems, n_blocks).bytes;
}

sz_status sz_encode_blocks(const void* const* d_blocks, uint64_t n_blocks, uint64_t block_elems,
                           void* d_dst, uint64_t dst_pitch, uint64_t* d_sizes,
                           void* d_workspace, uint64_t workspace_bytes, int32_t* d_status,
                           hipStream_t stream) {
    if (sz_status s =
            check_blocks(d_blocks, n_blocks, block_elems, d_dst, dst_pitch, d_sizes, true))
        return s;
    const BlockLayout l = block_layout(block_elems, n_blocks);
    if (d_workspace == nullptr || !aligned(d_workspace, 256) || workspace_bytes < l.bytes)
        return SZ_ERR_INVALID_ARGUMENT;
    if (d_status != nullptr && !aligned(d_status, 4)) return SZ_ERR_INVALID_ARGUMENT;
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    uint8_t* ws = static_cast<uint8_t*>(d_workspace);
    uint8_t* out = static_cast<uint8_t*>(d_dst);
    int32_t* flags = reinterpret_cast<int32_t*>(ws + l.flags_off);
    const sz::BlockWords src{block_table(d_blocks), flags, (uint32_t)n_blocks, l.stride,
                             dst_pitch, d_sizes};
    sz_status st = hip_status(sz::launch_check_blocks(src.blocks, n_blocks, flags, d_status, ws,
                                                      l.plan, l.stride, stream));
    if (st != SZ_OK) return st;
    if (l.plan.single_read && block_elems * n_blocks >= kSingleReadAuto &&
        l.plan.scratch_end <= dst_pitch) {
        // as sz_encode on as many words: one read when the sample holds
        st = hip_status(sz::launch_sample(src, l.plan, ws, stream));
        if (st == SZ_OK)
            st = hip_status(sz::launch_first_pass(src, l.plan, ws, out, dst_pitch, stream));
        if (st == SZ_OK)
            st = hip_status(sz::launch_finish(src, l.plan, ws, out, dst_pitch, nullptr, stream));
        return st;
    }
    st = hip_status(sz::launch_histogram(src, l.plan, ws, stream));
    if (l.plan.chunks >= 1 && l.plan.chunks <= sz::kRankedChunks) {
        // few chunks a block: no codebook pass, each pack workgroup ranks
        if (st == SZ_OK)
            st = hip_status(sz::launch_pack_ranked(src, l.plan, ws, out, dst_pitch, nullptr,
                                                   stream));
        return st;
    }
    if (st == SZ_OK) st = hip_status(sz::launch_codebook(src, l.plan, ws, out, nullptr, stream));
    if (st == SZ_OK)
        st = hip_status(sz::launch_pack(src, l.plan, ws, out, dst_pitch, num_cus(dev), stream));
    return st;
}

uint64_t sz_blocks_decode_workspace_size(uint64_t block_elems, uint64_t n_blocks) {
    if (block_elems > SZ_MAX_ELEMENTS || n_blocks == 0 || n_blocks > kMaxBlocks) return 0;
    return n_blocks * round256(sz::tile_index_layout(block_elems, true).bytes);
}

sz_status sz_decode_blocks(const void* d_src, uint64_t src_pitch, const uint64_t* d_sizes,
                           uint64_t n_blocks, uint64_t block_elems, void* const* d_blocks,
                           void* d_workspace, uint64_t workspace_bytes, int32_t* d_status,
                           hipStream_t stream) {
    if (sz_status s =
            check_blocks(d_blocks, n_blocks, block_elems, d_src, src_pitch, d_sizes, false))
        return s;
    if (d_status == nullptr || !aligned(d_status, 4)) return SZ_ERR_INVALID_ARGUMENT;
    const uint64_t ws_stride = round256(sz::tile_index_layout(block_elems, true).bytes);
    if (d_workspace != nullptr &&
        (!aligned(d_workspace, 256) || workspace_bytes < n_blocks * ws_stride))
        return SZ_ERR_INVALID_ARGUMENT;
    const int dev = current_device();
    if (dev < 0) return SZ_ERR_HIP;
    // the statuses start as the address check's flags, which the decode
    // then raises to SZ_ERR_CORRUPT where a container fails its checks
    const sz::BlockWords dst{block_table(d_blocks), d_status, (uint32_t)n_blocks, ws_stride,
                             src_pitch, const_cast<uint64_t*>(d_sizes)};
    const uint8_t* src = static_cast<const uint8_t*>(d_src);
    sz_status st =
        hip_status(sz::launch_check_blocks(dst.blocks, n_blocks, d_status, nullptr, nullptr,
                                           sz::EncodePlan{}, 0, stream));
    if (st != SZ_OK) return st;
    if (d_workspace == nullptr)  // one pass per block range, no workspace
        return hip_status(sz::launch_decode_dense(src, 0, block_elems, 0, dst, d_status, stream));
    // the tile decode: index every block's escape stream, then its tiles
    uint8_t* w = static_cast<uint8_t*>(d_workspace);
    st = hip_status(sz::launch_tile_index(src, 0, block_elems, 0, w, dst, stream));
    if (st == SZ_OK)
        st = hip_status(
            sz::launch_decode_tiles(src, block_elems, 0, w, dst, d_status, num_cus(dev), stream));
    return st;
}

const char* sz_status_string(int status) {
    switch (status) {
        case SZ_OK: return "ok";
        case SZ_ERR_INVALID_ARGUMENT: return "invalid argument (null, misaligned, overlapping or bad workspace)";
        case SZ_ERR_CAPACITY: return "destination capacity below sz_max_compressed_size(n)";
        case SZ_ERR_TOO_LARGE: return "more than 2^36 elements";
        case SZ_ERR_CORRUPT: return "corrupt or inconsistent container";
        case SZ_ERR_HIP: return "HIP launch or allocation failed";
        default: return "unknown status";
    }
}

}  // extern "C"
