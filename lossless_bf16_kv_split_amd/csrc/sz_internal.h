// sz_internal.h -- shared between the kernel and API translation units of
// libsplitzip.so (not installed, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stddef.h>
#include <stdint.h>

namespace sz {

constexpr uint32_t kHeaderBytes = 160;
constexpr uint32_t kPrefixBytes = 176;  // header + 16-byte codebook
constexpr uint32_t kMagic = 0x564B5A53u;
constexpr uint16_t kVersion = 1;
constexpr uint16_t kElementBf16 = 1;
constexpr uint64_t kMaxElements = 1ull << 36;

// Encoding works on power-of-two chunks of the input.  The histogram pass
// counts exponents per chunk, the codebook pass turns those counts into the
// exact number of escapes of every chunk (and so into each chunk's first
// escape slot), and the pack pass lets one workgroup stream one chunk.
// A chunk holds whole pack tiles.  The plan takes the smallest chunk that
// gives at most kPlanChunks chunks, or half of it (then at most kMaxChunks
// chunks) when that leaves less of the pack grid's last wave of resident
// workgroups idle.
constexpr uint32_t kMinChunkLog2 = 14;
constexpr uint32_t kPlanChunks = 2048;
constexpr uint32_t kMaxChunks = 2 * kPlanChunks;
constexpr uint32_t kMinHalvedChunkLog2 = 17;  // a halved chunk keeps >= 2^17 words
// pack workgroups (1024 threads, 8 waves per SIMD) resident at once on
// MI355X: 256 CUs x 2
constexpr uint64_t kResidentPackGroups = 512;

struct EncodePlan {
    uint64_t n = 0;
    uint32_t chunk_log2 = kMinChunkLog2;
    uint32_t chunks = 0;    // G = ceil(n / 2^chunk_log2)
    // workspace layout, byte offsets (256-byte aligned regions)
    uint64_t counts_off = 0;   // u32[256][G]   exponent counts, bin-major
    uint64_t hist_off = 0;     // u64[256]      exponent counts of the whole input
    uint64_t base_off = 0;     // u64[G]        first escape slot of each chunk
    uint64_t totals_off = 0;   // u64[kTotalCopies][256] exponent counts added up by the first pass
    uint64_t esc_off = 0;      // u32[G]        each chunk's escapes under the provisional codebook
    uint64_t sample_off = 0;   // SampleArea (single-read encode)
    uint64_t ws_bytes = 0;
    // Single-read encode (large inputs): the first pass packs with a
    // provisional codebook taken from a sample and puts each chunk's escape
    // records, at most spec_cap of them, in a scratch area of the
    // destination beyond the largest container such a pass can lead to.
    bool single_read = false;
    uint64_t spec_cap = 0;     // records per chunk: chunk size / 16
    uint64_t scratch_pos = 0;  // dst offset of u32 positions[G * spec_cap], 16-byte aligned
    uint64_t scratch_exp = 0;  // dst offset of u8 exponents[G * spec_cap]
    uint64_t scratch_end = 0;  // first dst byte past the scratch area
};

// The sample of the single-read encode: kSampleGroups workgroups add their
// counts into sample_hist and take tickets; the one that arrives last ranks
// the total.  The area also holds the codebook pass's count of workgroups
// done (zeroed, with the whole input's counts, by the pass before it).
constexpr uint32_t kSampleGroups = 64;
// Copies of the whole input's exponent counts that the first pass adds
// into, chunk c into copy c % kTotalCopies: fewer device-wide atomics on
// one address.
constexpr uint32_t kTotalCopies = 4;
struct SampleArea {
    uint32_t sample_hist[256];  // the sample's exponent counts (left zero after ranking)
    uint32_t tickets;       // sample workgroups that added their counts, kSampleGroups a run
    uint32_t overflow;      // set by the first pass: a chunk outgrew its scratch slots
    uint32_t spec_on;       // the sample predicts few escapes: the first pass packs
    uint32_t arrivals;      // codebook-pass workgroups done (the last one ranks)
    uint8_t lut[256];       // provisional exponent -> code, 0x10 = escape
    uint8_t cb[16];         // provisional codebook, code -> exponent
};
static_assert(sizeof(SampleArea) % 16 == 0 && offsetof(SampleArea, lut) % 16 == 0 &&
                  offsetof(SampleArea, cb) % 16 == 0,
              "16-byte loads of the tables");

// The single-read passes take inputs from kSingleReadMin words on (below,
// the sample blocks would overlap).
constexpr uint64_t kSingleReadMin = uint64_t{1} << 20;

EncodePlan plan_encode(uint64_t n);
// The workspace layout and scratch area for n words in chunks of
// 2^chunk_log2 words (plan_encode's own choice of chunk goes through it).
EncodePlan plan_encode_chunks(uint64_t n, uint32_t chunk_log2);
// The plan of each of n_blocks blocks of block_elems words encoded in one
// launch sequence: chunks sized for all the blocks' words together (so
// that the launch holds as many workgroups as one tensor of that size
// would), never smaller than 2^kMinChunkLog2 words, never larger than a
// block needs.
EncodePlan plan_blocks(uint64_t block_elems, uint64_t n_blocks);

// Residency of wide workgroups on MI355X: a wave whose kernel needs more
// than 74 scalar registers of its own (80 with the ones the hardware
// reserves) cannot share a SIMD with seven others, so a CU then holds one
// 16-wave workgroup instead of two -- measured, whatever occupancy the
// compiler reports.  Kernels that rely on eight waves per SIMD cap their
// scalar registers with this attribute (excess values move to VGPR lanes).
#define SZ_EIGHT_WAVE_SGPR_CAP __attribute__((amdgpu_num_sgpr(80)))

// Integer minimum of two 64-bit counts (HIP's overloaded min would take a
// mixed unsigned long / unsigned long long pair through double).
__host__ __device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) {
    return a < b ? a : b;
}

// Word 3 of a buffer resource (raw buffer, 32-bit data) on gfx9-family
// parts, gfx950 included: buffer loads take a 32-bit offset per lane from a
// base in scalar registers and read 0 past num_records bytes.
constexpr int32_t kBufferFlags = 0x00020000;

// 16-byte non-temporal load and store (global_load/store with the nt bit)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Loads and stores through the global address space.  A device address
// read from a table (a page or a block) is a generic pointer to the
// compiler, and accesses through it would be flat instructions; the tables
// hold device memory only, so the accesses to tensor words go through
// these (for a plain tensor argument they are what the compiler emits
// anyway).
// (16 bytes at a time, through the vector type: a uint4 copy would bind a
// generic reference and lose the address space again)
#define SZ_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ uint4 load_global(const uint4* p) {
    const u32x4 v = *(const SZ_GLOBAL u32x4*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_global(uint4* p, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    *(SZ_GLOBAL u32x4*)p = w;
}

__device__ __forceinline__ uint4 load_streaming(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load((const SZ_GLOBAL u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_streaming(uint4* p, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (SZ_GLOBAL u32x4*)p);
}

// sz_decode's choice of decode form, measured on MI355X:
//  - above one escape in kTileDecodeDensity words, the dense decode: over
//    2^28 KV words with escapes injected, tile 178-185 us against dense
//    181-196 us up to one escape in 250, dense ahead from about one in 100
//    (187 against 195 us at 1.2%, 193 against 224 us at 2.7%);
//  - below kTileDecodeMin words, forms that need no workspace (allocating
//    one from the pool costs more host time than such a decode takes):
//    unpack then scatter up to one escape in kScatterDecodeDensity words
//    (10-26 us against 11-28 us for the others from 2^21 to 2^25 words of
//    KV data), else the dense decode;
//  - otherwise the tile decode (the dense one under graph capture).
constexpr uint64_t kTileDecodeDensity = 128;
constexpr uint64_t kScatterDecodeDensity = 256;
constexpr uint64_t kTileDecodeMin = uint64_t{1} << 26;

// Tile decode: one short-lived 256-thread workgroup per 2048-word tile (8
// words per thread), after an index pass that gives every tile its first
// escape record.  On MI355X many small workgroups that each move one
// 16-byte piece per thread and byte stream beat fewer workgroups that
// loop: for the decode's traffic (1.5 B read, 2 B
// written per word) on 2^29 words, 298 us with one 2048-word tile per
// 256-thread workgroup against 328 us for the best persistent grid.
//
// The index pass is search-free and runs one wave per 64 items, the items
// being the E escape records and, as item E, the end of the words (position
// n, tile `tiles`).  An item whose tile differs from its predecessor's is
// the first of its tile: it writes idx[j] = its index for every tile j after
// its predecessor's tile up to its own (the tiles in between have no
// records) and its tile's 64-byte slot: dword 0 the tile's record count (up
// to 16 records ahead are seen, so a count above 15 only says "more than
// 15"), dwords 1..15 the 15 records from its first on as (offset in the
// tile) | exponent << 16 (those past the count belong to later tiles; the
// decode reads only the first count of them).  The decode of a tile loads its slot together with its
// codes and sign|mantissa bytes, so a tile with at most 15 records (on the
// 1 GiB KV tensor all but 0.014% of them, 4 on average) waits for no load
// that depends on another; a tile with more goes through idx and the
// escape stream.  Each launched wave writes its own fault flag (a launch
// holds at most kMaxIndexGroups waves; past that each takes several groups
// of 64 items).
constexpr uint32_t kTileWords = 2048;
constexpr uint32_t kIndexItems = 64;          // items per index wave
constexpr uint64_t kMaxIndexGroups = uint64_t{1} << 20;  // launched; more loop
constexpr uint64_t kMaxTileGroups = uint64_t{1} << 22;   // launched; more loop
constexpr uint32_t kSlotWords = 16;                      // dwords per tile slot
constexpr uint32_t kSlotRecords = kSlotWords - 1;
struct TileIndexLayout {
    uint64_t tiles = 0;       // ceil(n / kTileWords)
    uint64_t max_flags = 0;   // launched index waves for any E <= floor(15n/16)
    uint64_t idx_off = 0;     // u64[tiles + 1]: first record of each tile, then E
    uint64_t flag_off = 0;    // u32[max_flags]: 1 where an index wave found a fault
    uint64_t slot_off = 0;    // u32[tiles][kSlotWords]: each tile's record count and records
    uint64_t bytes = 0;
};
__host__ __device__ inline uint64_t index_groups(uint64_t e) {
    return (e + 1 + kIndexItems - 1) / kIndexItems;
}
// For several blocks in one launch the escape count of each is known only
// on the device, so the index pass runs a number of waves per block fixed
// by the block length -- one per 16384 words (one group of 64 records at
// the KV data's 0.4% escapes), 64 to 4096 of them -- each taking every
// so-many-th group of 64 items.
inline uint64_t block_index_waves(uint64_t n) {
    const uint64_t w = n / 16384;
    return w < 64 ? 64 : (w > 4096 ? 4096 : w);
}
inline TileIndexLayout tile_index_layout(uint64_t n, bool blocks = false) {
    TileIndexLayout l;
    l.tiles = (n + kTileWords - 1) / kTileWords;
    const uint64_t max_groups = index_groups((15 * n) / 16);
    l.max_flags = max_groups < kMaxIndexGroups ? max_groups : kMaxIndexGroups;
    if (blocks) l.max_flags = block_index_waves(n);
    auto align = [](uint64_t x) { return (x + 255) & ~uint64_t{255}; };
    l.idx_off = 0;
    l.flag_off = align(8 * (l.tiles + 1));
    l.slot_off = align(l.flag_off + 4 * l.max_flags);
    l.bytes = align(l.slot_off + 4 * kSlotWords * l.tiles);
    return l;
}

__host__ __device__ inline uint64_t container_bytes(uint64_t n, uint64_t e) {
    return kPrefixBytes + (n + 1) / 2 + n + 5 * e;
}

// Where the uncompressed words live.  Kernels address word i through
// at(i) and walk a range in runs that are contiguous in memory: FlatWords
// is one array (one run); PagedWords is 2^page_log2-word pages at the
// addresses of a device table (runs end at page boundaries).  Pages hold at
// least 2^14 words, so a pack tile (2^14 words), a decode tile or sub-range
// and every 8-word group lie inside one page.
// at_wave(i) is at(i) for callers whose active lanes all address one page
// (a wave's 64 consecutive 8-word groups, 512-word aligned): the page is
// then looked up once per wave, through a scalar load.
struct FlatWords {
    static constexpr bool kPaged = false;
    static constexpr bool kBlocks = false;
    uint16_t* base;
    __device__ __forceinline__ bool invalid() const { return false; }
    __device__ __forceinline__ uint16_t* at(uint64_t i) const { return base + i; }
    __device__ __forceinline__ uint16_t* at_wave(uint64_t i) const { return base + i; }
    __device__ __forceinline__ FlatWords resolve() const { return *this; }
    __device__ __forceinline__ uint64_t run_end(uint64_t, uint64_t end) const { return end; }
};

constexpr uint32_t kMinPageLog2 = 14;

struct PagedWords {
    static constexpr bool kPaged = true;  // at() and at_wave() read the page table
    static constexpr bool kBlocks = false;
    uint16_t* const* pages;   // device table of page addresses
    uint32_t page_log2;
    const int32_t* bad;       // nonzero: the table failed its check, touch no page
    __device__ __forceinline__ bool invalid() const { return *bad != 0; }
    __device__ __forceinline__ uint16_t* at(uint64_t i) const {
        return pages[i >> page_log2] + (i & ((uint64_t{1} << page_log2) - 1));
    }
    __device__ __forceinline__ uint16_t* at_wave(uint64_t i) const {
        const uint64_t page = i >> page_log2;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)page);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(page >> 32));
        return pages[((uint64_t)hi << 32) | lo] + (i & ((uint64_t{1} << page_log2) - 1));
    }
    __device__ __forceinline__ uint64_t run_end(uint64_t i, uint64_t end) const {
        return min_u64(end, ((i >> page_log2) + 1) << page_log2);
    }
    __device__ __forceinline__ PagedWords resolve() const { return *this; }
};

// Several tensors of the same length ("blocks") in one launch, one
// container each: blockIdx.y is the block.  Its words are at blocks[y]; its
// workspace (the encode's, or the tile decode's index) lies y * ws_stride
// bytes after block 0's, its container y * pitch bytes after block 0's,
// and its container size is sizes[y] (written by the encode, read by the
// decode).  flags[y] is kBlockInvalid when the block's address failed its
// check (the encode keeps the flags in its workspace; the decode uses its
// per-block statuses).
constexpr int32_t kBlockInvalid = 1;  // SZ_ERR_INVALID_ARGUMENT
struct BlockWords {
    static constexpr bool kPaged = false;
    static constexpr bool kBlocks = true;
    uint16_t* const* blocks;  // device table of block addresses
    const int32_t* flags;
    uint32_t count;           // blocks (the launch's grid height)
    uint64_t ws_stride;
    uint64_t pitch;
    uint64_t* sizes;
    __device__ __forceinline__ bool invalid() const {
        // other workgroups of the block may raise its decode status meanwhile
        return __hip_atomic_load(flags + blockIdx.y, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT) == kBlockInvalid;
    }
    __device__ __forceinline__ uint16_t* at(uint64_t i) const { return blocks[blockIdx.y] + i; }
    __device__ __forceinline__ uint16_t* at_wave(uint64_t i) const { return blocks[blockIdx.y] + i; }
    __device__ __forceinline__ uint64_t run_end(uint64_t, uint64_t end) const { return end; }
    // the block's words as one flat tensor, its address read once (the
    // workgroup's loops would otherwise read the table entry again for
    // every tile, stores in between keeping it from being hoisted)
    __device__ __forceinline__ FlatWords resolve() const { return FlatWords{blocks[blockIdx.y]}; }
};

// The launch's grid height, and this workgroup's block offsets into the
// workspace and the containers (all 0 for a single tensor).
template <class Words>
inline uint32_t grid_blocks(const Words& w) {
    if constexpr (Words::kBlocks) return w.count;
    else return 1;
}
template <class Words>
__device__ __forceinline__ uint64_t block_ws(const Words& w) {
    if constexpr (Words::kBlocks) return (uint64_t)blockIdx.y * w.ws_stride;
    else return 0;
}
template <class Words>
__device__ __forceinline__ uint64_t block_pitch(const Words& w) {
    if constexpr (Words::kBlocks) return (uint64_t)blockIdx.y * w.pitch;
    else return 0;
}
// p advanced by a byte count, through a char pointer (an integer round
// trip would lose the global address space and turn loads into flat ones)
template <class T>
__device__ __forceinline__ T* byte_offset(T* p, uint64_t bytes) {
    using Byte = typename std::conditional<std::is_const<T>::value, const char, char>::type;
    return reinterpret_cast<T*>(reinterpret_cast<Byte*>(p) + bytes);
}

// Launchers (asynchronous on `stream`; return the launch status).  The
// templates are instantiated for FlatWords and PagedWords, and those of the
// two-read encode and of the dense decode also for BlockWords (one launch
// for all blocks; ws, dst and d_size are block 0's, and src's own fields
// give the other blocks').
template <class Words>
hipError_t launch_histogram(Words src, const EncodePlan& p, uint8_t* ws, hipStream_t stream);
template <class Words>
hipError_t launch_codebook(Words src, const EncodePlan& p, uint8_t* ws, uint8_t* dst,
                           uint64_t* d_size, hipStream_t stream);
template <class Words>
hipError_t launch_pack(Words src, const EncodePlan& p, const uint8_t* ws, uint8_t* dst,
                       uint64_t dst_capacity, int num_cus, hipStream_t stream);
// the codebook and pack passes in one launch, for 1 to kRankedChunks chunks
// (a tensor's or, for BlockWords, each block's): every workgroup ranks the
// counts itself; writes the header and *d_size (for blocks, each block's
// size to src.sizes, 0 for a block it cannot read)
constexpr uint32_t kRankedChunks = 128;
template <class Words>
hipError_t launch_pack_ranked(Words src, const EncodePlan& p, const uint8_t* ws, uint8_t* dst,
                              uint64_t dst_capacity, uint64_t* d_size, hipStream_t stream);
// single-read encode: sample (ranks the provisional codebook), the first
// pass (exact per-chunk and whole-input counts, and the streams under the
// provisional codebook), then the finish pass (takes the exact codebook and
// writes the header and *d_size; moves the escape records into place,
// remaps the codes, or packs again)
template <class Words>
hipError_t launch_sample(Words src, const EncodePlan& p, uint8_t* ws, hipStream_t stream);
template <class Words>
hipError_t launch_first_pass(Words src, const EncodePlan& p, uint8_t* ws, uint8_t* dst,
                             uint64_t dst_capacity, hipStream_t stream);
template <class Words>
hipError_t launch_finish(Words src, const EncodePlan& p, uint8_t* ws, uint8_t* dst,
                         uint64_t dst_capacity, uint64_t* d_size, hipStream_t stream);
template <class Words>
hipError_t launch_unpack(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                         Words dst, int32_t* status, int num_cus, hipStream_t stream);
template <class Words>
hipError_t launch_scatter(const uint8_t* src, uint64_t n, uint64_t e, Words dst,
                          int32_t* status, hipStream_t stream);
template <class Words>
hipError_t launch_decode_fused(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                               Words dst, int32_t* status, hipStream_t stream);
template <class Words>
hipError_t launch_decode_dense(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                               Words dst, int32_t* status, hipStream_t stream);
// tile decode: index the escape stream by tile (header and record-order
// checks included), then decode every tile; the second call writes *status.
// For BlockWords (one launch each for all blocks) src, ws and status are
// block 0's, e is taken from each block's size, and ws_stride in the
// accessor is the per-block workspace (tile_index_layout(n, true).bytes,
// rounded up to 256).
template <class Words>
hipError_t launch_tile_index(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                             uint8_t* ws, Words blocks, hipStream_t stream);
template <class Words>
hipError_t launch_decode_tiles(const uint8_t* src, uint64_t n, uint64_t e, const uint8_t* ws,
                               Words dst, int32_t* status, int num_cus, hipStream_t stream);
// Checks a page table (every address non-NULL and 16-byte aligned) into
// *bad, and mirrors the result into *status when given.
hipError_t launch_check_pages(const uint16_t* const* pages, uint64_t n_pages, int32_t* bad,
                              int32_t* status, hipStream_t stream);
// Checks every block address of a table (non-NULL, 16-byte aligned) into
// flags[b] (0 or kBlockInvalid), and the same into status[b] when given;
// with a workspace (ws != nullptr), also zeroes each block's whole-input
// counts, which the block count pass adds up.
hipError_t launch_check_blocks(const uint16_t* const* blocks, uint64_t n_blocks, int32_t* flags,
                               int32_t* status, uint8_t* ws, const EncodePlan& p,
                               uint64_t ws_stride, hipStream_t stream);

}  // namespace sz
