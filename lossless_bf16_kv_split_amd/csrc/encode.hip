// encode.hip -- the three encode passes of the SplitZip BF16 codec on gfx950.
//
//   histogram  one workgroup per chunk: 256-bin exponent counts in LDS
//              (replicated sub-histograms against same-address conflicts),
//              written out bin-major, counts[bin][chunk]
//   codebook   merge the counts, rank the 256 exponents (count desc, value
//              asc), write header + codebook, and turn every chunk's counts
//              into its exact escape count and first escape slot
//   pack       one workgroup per chunk: 16-byte loads, 256-entry exponent
//              -> code table in LDS, 4-bit codes two per byte, sign|mantissa
//              bytes, ballot/popcount escape ranks, escapes written straight
//              to their final slots in ascending position order
//
// Method: SplitZip explainers (gist.science, arXiv 2605.01708), sections
// "2. La decouverte secrete" (exponents repeat), "3. La strategie SplitZip"
// (top-16 list, fixed 4-bit codes two per byte, rare exponents as
// (position, exponent) notes) and "4. Pourquoi est-ce rapide ?" (fixed-size
// codes make every output slot known in advance).
#include "sz_internal.h"

namespace sz {

// ---------------------------------------------------------------- plan

EncodePlan plan_encode(uint64_t n) {
    EncodePlan p;
    p.n = n;
    uint32_t c = kMinChunkLog2;
    while (c < 40 && ((n + (1ull << c) - 1) >> c) > kMaxChunks) c++;
    p.chunk_log2 = c;
    p.chunks = (uint32_t)((n + (1ull << c) - 1) >> c);
    auto align = [](uint64_t x) { return (x + 255) & ~255ull; };
    p.counts_off = 0;
    p.hist_off = align(p.counts_off + (uint64_t)p.chunks * 256 * 4);
    p.base_off = align(p.hist_off + 256 * 8);
    p.ws_bytes = align(p.base_off + (uint64_t)p.chunks * 8);
    return p;
}

// ---------------------------------------------------------------- pass 1

constexpr int kHistThreads = 256;
// Sub-histograms per workgroup, lane i adding into copy i % 32.  KV
// exponents crowd into a few bins, so fewer copies serialise on same-address
// LDS atomics; from 16 copies up the pass runs at the speed of its loads.
constexpr int kHistCopies = 32;
constexpr int kHistPitch = 257;   // odd pitch: copies of one bin sit in different banks

__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t e) {
    __hip_atomic_fetch_add(h + e, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Two BF16 words per dword: exponents are bits 14..7 and 30..23.
__device__ __forceinline__ void hist_dword(uint32_t* h, uint32_t d) {
    hist_add(h, (d >> 7) & 0xFFu);
    hist_add(h, (d >> 23) & 0xFFu);
}

__device__ __forceinline__ void hist_uint4(uint32_t* h, const uint4& v) {
    hist_dword(h, v.x);
    hist_dword(h, v.y);
    hist_dword(h, v.z);
    hist_dword(h, v.w);
}

// counts[bin * chunks + chunk]: bin-major, so that the codebook pass reads
// every bin's counts, and each chunk's 16 codebook counts, coalesced
template <class Words>
__global__ __launch_bounds__(kHistThreads) void k_histogram(Words src, uint64_t n,
                                                            uint32_t chunk_log2, uint32_t chunks,
                                                            uint32_t* __restrict__ counts) {
    __shared__ uint32_t h[kHistCopies * kHistPitch];
    if (src.invalid()) return;  // the same for every thread
    for (int i = threadIdx.x; i < kHistCopies * kHistPitch; i += kHistThreads) h[i] = 0;
    __syncthreads();

    const uint64_t begin = (uint64_t)blockIdx.x << chunk_log2;
    const uint64_t end = min_u64(begin + (uint64_t{1} << chunk_log2), n);
    uint32_t* mine = h + (threadIdx.x % kHistCopies) * kHistPitch;

    // the chunk in runs contiguous in memory (one run for a flat tensor)
    for (uint64_t r0 = begin; r0 < end;) {
        const uint64_t r1 = src.run_end(r0, end);
        const uint16_t* base = src.at(r0);
        // 8 words per 16-byte load; four loads in flight per thread.  The
        // loads are non-temporal: not allocating the input in the caches
        // leaves the lines already there (often the dirty output of earlier
        // kernels) alone, which measured 25% faster for this pass and 4% for
        // the whole codec.
        const uint4* v = reinterpret_cast<const uint4*>(base);
        const uint32_t groups = (uint32_t)((r1 - r0) >> 3);
        uint32_t g = threadIdx.x;
        for (; g + 3 * kHistThreads < groups; g += 4 * kHistThreads) {
            const uint4 a = load_streaming(v + g);
            const uint4 b = load_streaming(v + g + kHistThreads);
            const uint4 c = load_streaming(v + g + 2 * kHistThreads);
            const uint4 d = load_streaming(v + g + 3 * kHistThreads);
            hist_uint4(mine, a);
            hist_uint4(mine, b);
            hist_uint4(mine, c);
            hist_uint4(mine, d);
        }
        for (; g < groups; g += kHistThreads) hist_uint4(mine, load_streaming(v + g));
        // fewer than 8 words left at the very end of the input
        for (uint64_t i = ((uint64_t)groups << 3) + threadIdx.x; i < r1 - r0; i += kHistThreads)
            hist_add(mine, (base[i] >> 7) & 0xFFu);
        r0 = r1;
    }
    __syncthreads();

    for (int bin = threadIdx.x; bin < 256; bin += kHistThreads) {
        uint32_t s = 0;
#pragma unroll
        for (int c = 0; c < kHistCopies; c++) s += h[c * kHistPitch + bin];
        counts[(uint64_t)bin * chunks + blockIdx.x] = s;
    }
}

template <class Words>
hipError_t launch_histogram(Words src, const EncodePlan& p, uint8_t* ws, hipStream_t stream) {
    if (p.chunks == 0) return hipSuccess;
    k_histogram<Words><<<p.chunks, kHistThreads, 0, stream>>>(
        src, p.n, p.chunk_log2, p.chunks, reinterpret_cast<uint32_t*>(ws + p.counts_off));
    return hipGetLastError();
}
template hipError_t launch_histogram<FlatWords>(FlatWords, const EncodePlan&, uint8_t*,
                                                hipStream_t);
template hipError_t launch_histogram<PagedWords>(PagedWords, const EncodePlan&, uint8_t*,
                                                 hipStream_t);

// One workgroup: every page address must be non-NULL and 16-byte aligned.
__global__ __launch_bounds__(256) void k_check_pages(const uint16_t* const* pages,
                                                     uint64_t n_pages, int32_t* bad,
                                                     int32_t* status) {
    __shared__ int any;
    if (threadIdx.x == 0) any = 0;
    __syncthreads();
    for (uint64_t i = threadIdx.x; i < n_pages; i += 256) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(pages[i]);
        if (a == 0 || (a & 15) != 0) any = 1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        *bad = any;
        if (status) *status = any ? 1 : 0;  // SZ_ERR_INVALID_ARGUMENT or SZ_OK
    }
}

hipError_t launch_check_pages(const uint16_t* const* pages, uint64_t n_pages, int32_t* bad,
                              int32_t* status, hipStream_t stream) {
    k_check_pages<<<1, 256, 0, stream>>>(pages, n_pages, bad, status);
    return hipGetLastError();
}

// ---------------------------------------------------------------- pass 2

// hist[bin] = sum over chunks of counts[bin][chunk]; one workgroup per bin,
// every load coalesced and in flight at once.
constexpr int kMergeThreads = 256;
constexpr uint32_t kMergePerThread = kMaxChunks / kMergeThreads;

__global__ __launch_bounds__(kMergeThreads) void k_merge_counts(const uint32_t* __restrict__ counts,
                                                               uint32_t chunks,
                                                               uint64_t* __restrict__ hist) {
    __shared__ uint64_t wave_sum[kMergeThreads / 64];
    const uint32_t bin = blockIdx.x;
    const uint32_t t = threadIdx.x;
    const uint32_t* row = counts + (uint64_t)bin * chunks;
    uint32_t v[kMergePerThread];
#pragma unroll
    for (uint32_t j = 0; j < kMergePerThread; j++) {
        const uint32_t c = t + j * kMergeThreads;
        v[j] = c < chunks ? row[c] : 0u;
    }
    uint64_t s = 0;
#pragma unroll
    for (uint32_t j = 0; j < kMergePerThread; j++) s += v[j];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) s += __shfl_down(s, d, 64);
    if ((t & 63) == 0) wave_sum[t >> 6] = s;
    __syncthreads();
    if (t == 0) {
        uint64_t total = 0;
        for (int w = 0; w < kMergeThreads / 64; w++) total += wave_sum[w];
        hist[bin] = total;
    }
}

constexpr int kSelectThreads = 1024;
constexpr int kSelectWaves = kSelectThreads / 64;

__device__ __forceinline__ uint64_t wave_inclusive_sum(uint64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// One workgroup.  chunk_base[b] receives the number of escapes in chunks
// before b, which is where chunk b's escape records start.
__global__ __launch_bounds__(kSelectThreads) void k_select(
    uint64_t n, uint32_t chunk_log2, uint32_t chunks, const uint32_t* __restrict__ counts,
    const uint64_t* __restrict__ hist, uint64_t* __restrict__ chunk_base,
    uint8_t* __restrict__ dst, uint64_t* d_size) {
    __shared__ uint64_t key[256];
    __shared__ uint32_t rank_part[4][256];
    __shared__ uint32_t codebook[16];
    __shared__ uint64_t wave_sum[kSelectWaves];
    __shared__ uint64_t wave_off[kSelectWaves];
    __shared__ uint64_t base_lds[kMaxChunks];

    const int t = threadIdx.x;
    const int bin = t & 255;
    const int grp = t >> 8;  // 0..3
    if (t < 16) codebook[t] = 0;

    // key(x) = count << 8 | (255 - x): "more frequent, then smaller exponent"
    // becomes one unsigned comparison (counts stay below 2^37)
    if (t < 256) key[t] = (hist[t] << 8) | (255u - t);
    __syncthreads();

    // rank(x) = #{y : key(y) > key(x)}; group g counts over y in [64g, 64g + 64)
    {
        const uint64_t kx = key[bin];
        uint32_t r = 0;
#pragma unroll 16
        for (int y = grp * 64; y < grp * 64 + 64; y++) r += key[y] > kx ? 1u : 0u;
        rank_part[grp][bin] = r;
    }
    __syncthreads();
    if (t < 256) {
        const uint32_t r = rank_part[0][t] + rank_part[1][t] + rank_part[2][t] + rank_part[3][t];
        if (r < 16) codebook[r] = (uint32_t)t;
    }
    __syncthreads();

    // escapes of chunks 2t and 2t+1 = chunk length - elements whose
    // exponent is in the codebook
    uint32_t cb[16];
#pragma unroll
    for (int c = 0; c < 16; c++) cb[c] = codebook[c] & 255u;
    // chunks 2t and 2t+1: their 16 codebook counts, coalesced across threads
    // (bin-major layout), all in flight at once
    uint32_t v[2][16];
#pragma unroll
    for (int c = 0; c < 16; c++) {
        const uint32_t* row = counts + (uint64_t)cb[c] * chunks;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const uint32_t b = 2 * t + j;
            v[j][c] = b < chunks ? row[b] : 0u;
        }
    }
    uint64_t esc[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const uint32_t b = 2 * t + j;
        if (b < chunks) {
            const uint64_t start = (uint64_t)b << chunk_log2;
            const uint64_t len = min_u64(uint64_t{1} << chunk_log2, n - start);
            uint64_t kept = 0;
#pragma unroll
            for (int c = 0; c < 16; c++) kept += v[j][c];
            esc[j] = len - kept;
        }
    }

    // exclusive scan of the per-chunk escape counts over the workgroup
    const uint64_t mine = esc[0] + esc[1];
    const uint64_t incl = wave_inclusive_sum(mine);
    const int lane = t & 63, wave = t >> 6;
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    if (t == 0) {
        uint64_t run = 0;
        for (int w = 0; w < kSelectWaves; w++) {
            wave_off[w] = run;
            run += wave_sum[w];
        }
    }
    __syncthreads();
    const uint64_t excl = wave_off[wave] + incl - mine;
    if (2 * t < chunks) {
        chunk_base[2 * t] = excl;
        base_lds[2 * t] = excl;
    }
    if (2 * t + 1 < chunks) {
        chunk_base[2 * t + 1] = excl + esc[0];
        base_lds[2 * t + 1] = excl + esc[0];
    }
    const uint64_t E = wave_off[kSelectWaves - 1] + wave_sum[kSelectWaves - 1];
    __syncthreads();
    const uint64_t total = kPrefixBytes + (n + 1) / 2 + n + 5 * E;
    if (t == 0) {
        *reinterpret_cast<uint32_t*>(dst + 0) = kMagic;
        *reinterpret_cast<uint16_t*>(dst + 4) = kVersion;
        *reinterpret_cast<uint16_t*>(dst + 6) = kElementBf16;
        *reinterpret_cast<uint64_t*>(dst + 8) = n;
        *reinterpret_cast<uint64_t*>(dst + 16) = E;
        *reinterpret_cast<uint64_t*>(dst + 24) = total;
        if (d_size) *d_size = total;
    }
    if (t < 16) {
        // seg_end[t]: escapes below element (t+1) * 2^32 -- a chunk boundary,
        // because chunks are powers of two no larger than 2^32
        const uint64_t boundary_chunk = (uint64_t)(t + 1) << (32 - chunk_log2);
        const uint64_t v = boundary_chunk < chunks ? base_lds[boundary_chunk] : E;
        *reinterpret_cast<uint64_t*>(dst + 32 + 8 * t) = v;
        dst[kHeaderBytes + t] = (uint8_t)codebook[t];
    }
}

hipError_t launch_codebook(const EncodePlan& p, uint8_t* ws, uint8_t* dst, uint64_t* d_size,
                           hipStream_t stream) {
    const uint32_t* counts = reinterpret_cast<const uint32_t*>(ws + p.counts_off);
    uint64_t* hist = reinterpret_cast<uint64_t*>(ws + p.hist_off);
    k_merge_counts<<<256, kMergeThreads, 0, stream>>>(counts, p.chunks, hist);
    k_select<<<1, kSelectThreads, 0, stream>>>(p.n, p.chunk_log2, p.chunks, counts, hist,
                                               reinterpret_cast<uint64_t*>(ws + p.base_off),
                                               dst, d_size);
    return hipGetLastError();
}

// ---------------------------------------------------------------- pass 3

// A tile is kPackTile consecutive words; thread t packs kPackWords
// consecutive words of it, so each lane loads, and stores nibbles and
// sign|mantissa bytes, in pieces of 8 or 16 bytes.  16 waves x 16 words
// measured fastest on the 1 GiB KV workload (381 us, against 391 us for
// 16 x 8 and 403 us for 8 x 16); a pure load/store probe of the same byte
// stream takes about 360 us.
constexpr int kPackThreads = 1024;
constexpr int kPackWords = 16;
constexpr int kPackWaves = kPackThreads / 64;
constexpr uint32_t kPackTile = kPackThreads * kPackWords;  // words per workgroup step
constexpr int kPackLoads = kPackWords / 8;                 // 16-byte loads per thread
static_assert(kPackWords == 8 || kPackWords == 16, "one or two 16-byte loads per thread");
static_assert((1u << kMinChunkLog2) % kPackTile == 0, "chunks hold whole tiles");
static_assert(kPackTile <= 65536, "tile offsets fit in 16 bits");
static_assert(kPackThreads >= 256, "one LUT entry per thread");
static_assert(2 * kSelectThreads >= kMaxChunks, "two chunks per select thread");

// Rank of this lane's bits among lower lanes: popcount of mask below lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Split 8 BF16 words (two per dword, little-endian) into 8 sign|mantissa
// bytes and 8 exponent bytes, 4 per dword, element k in byte k % 4.
// v_perm gathers the high and low bytes of 4 words; the sign is bit 7 of
// the high byte, the mantissa bits 6..0 of the low byte, the exponent the
// high byte's low 7 bits above the low byte's bit 7.
__device__ __forceinline__ void split8(const uint32_t* w, uint32_t& sm_lo, uint32_t& sm_hi,
                                       uint32_t& ex_lo, uint32_t& ex_hi) {
    const uint32_t hi0 = __builtin_amdgcn_perm(w[1], w[0], 0x07050301u);
    const uint32_t lo0 = __builtin_amdgcn_perm(w[1], w[0], 0x06040200u);
    const uint32_t hi1 = __builtin_amdgcn_perm(w[3], w[2], 0x07050301u);
    const uint32_t lo1 = __builtin_amdgcn_perm(w[3], w[2], 0x06040200u);
    sm_lo = (hi0 & 0x80808080u) | (lo0 & 0x7F7F7F7Fu);
    sm_hi = (hi1 & 0x80808080u) | (lo1 & 0x7F7F7F7Fu);
    ex_lo = ((hi0 << 1) & 0xFEFEFEFEu) | ((lo0 >> 7) & 0x01010101u);
    ex_hi = ((hi1 << 1) & 0xFEFEFEFEu) | ((lo1 >> 7) & 0x01010101u);
}

// byte k of a little-endian run of dwords (k known at compile time after
// unrolling, so the array stays in registers)
__device__ __forceinline__ uint32_t byte_at(const uint32_t* v, int k) {
    return (v[k >> 2] >> (8 * (k & 3))) & 0xFFu;
}

// The words of one thread, split: sign|mantissa and exponent bytes, the
// 4-bit codes (element k in bits 4(k%8).. of nib[k/8]) and the escape mask.
struct ThreadWords {
    uint32_t sm[kPackWords / 4];
    uint32_t ex[kPackWords / 4];
    uint32_t nib[kPackWords / 8];
    uint32_t mask;
};

__device__ __forceinline__ void encode_words(const uint32_t* w, const uint8_t* lut,
                                             ThreadWords& r) {
#pragma unroll
    for (int h = 0; h < kPackWords / 8; h++)
        split8(w + 4 * h, r.sm[2 * h], r.sm[2 * h + 1], r.ex[2 * h], r.ex[2 * h + 1]);
    r.mask = 0;
#pragma unroll
    for (int h = 0; h < kPackWords / 8; h++) r.nib[h] = 0;
#pragma unroll
    for (int k = 0; k < kPackWords; k++) {
        const uint32_t code = lut[byte_at(r.ex, k)];
        r.nib[k >> 3] |= (code & 0xFu) << (4 * (k & 7));
        r.mask |= (code >> 4) << k;
    }
}

// Escape records of one pack tile go to their final slots: a lane holds at
// most 16 escapes, so five ballots on the bits of its count give its
// exclusive prefix within the wave; wave totals meet in LDS.  A tile with
// few escapes writes them from the lanes that found them.  A tile with many
// first lays them out in LDS in slot order, then stores them with
// consecutive threads on consecutive slots, so that each store instruction
// fills whole cache lines instead of scattering 4- and 1-byte writes.
constexpr uint32_t kStageMin = 1024;  // escapes per tile from which records are staged

struct EscapeOut {
    uint8_t* pos;        // u32 positions (mod 2^32)
    uint8_t* exp;        // u8 exponents
    uint64_t limit;      // slots below this may be written
    bool pos_aligned;    // pos is 4-byte aligned
};

// 16-byte aligned so that a wave reads all wave totals with wide LDS loads
struct alignas(16) PackLds {
    uint32_t wave_escapes[2][kPackWaves];
    uint8_t lut[256];                      // exponent -> code, 0x10 = escape
    uint16_t stage_off[kPackTile];         // tile offset of each staged escape
    uint8_t stage_exp[kPackTile];
};

__device__ __forceinline__ void put_escape(const EscapeOut& out, uint64_t slot, uint32_t pos,
                                           uint32_t exponent) {
    if (slot >= out.limit) return;
    if (out.pos_aligned) {
        *reinterpret_cast<uint32_t*>(out.pos + 4 * slot) = pos;
    } else {
        out.pos[4 * slot + 0] = (uint8_t)(pos & 0xFF);
        out.pos[4 * slot + 1] = (uint8_t)((pos >> 8) & 0xFF);
        out.pos[4 * slot + 2] = (uint8_t)((pos >> 16) & 0xFF);
        out.pos[4 * slot + 3] = (uint8_t)(pos >> 24);
    }
    out.exp[slot] = (uint8_t)exponent;
}

// Positions are stored modulo 2^32, so their sums are taken in 32 bits.
__device__ __forceinline__ uint32_t write_escapes(const ThreadWords& r, uint64_t t0,
                                                  uint64_t slot_base, PackLds& lds, int parity,
                                                  const EscapeOut& out) {
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const uint32_t mask = r.mask;
    const uint32_t cnt = __popc(mask);
    uint32_t lane_prefix = 0, wave_total = 0;
#pragma unroll
    for (int b = 0; b < (kPackWords == 16 ? 5 : 4); b++) {
        const uint64_t bits = __ballot(cnt & (1u << b));
        lane_prefix += lanes_below(bits) << b;
        wave_total += (uint32_t)__popcll(bits) << b;
    }
    if (lane == 0) lds.wave_escapes[parity][wave] = wave_total;
    __syncthreads();
    uint32_t before = 0, tile_total = 0;
#pragma unroll
    for (int v = 0; v < kPackWaves; v++) {
        const uint32_t x = lds.wave_escapes[parity][v];
        before += v < wave ? x : 0u;
        tile_total += x;
    }
    const uint32_t first = before + lane_prefix;  // this lane's first rank in the tile
    if (tile_total >= kStageMin) {
        if (mask) {
            uint32_t q = first;
#pragma unroll
            for (int k = 0; k < kPackWords; k++) {
                if ((mask >> k) & 1u) {
                    lds.stage_off[q] = (uint16_t)(kPackWords * t + k);
                    lds.stage_exp[q] = (uint8_t)byte_at(r.ex, k);
                    q++;
                }
            }
        }
        __syncthreads();
        for (uint32_t q = t; q < tile_total; q += kPackThreads)
            put_escape(out, slot_base + q, (uint32_t)t0 + lds.stage_off[q], lds.stage_exp[q]);
    } else if (mask) {
        uint64_t slot = slot_base + first;
#pragma unroll
        for (int k = 0; k < kPackWords; k++) {
            if ((mask >> k) & 1u) {
                put_escape(out, slot, (uint32_t)t0 + (uint32_t)(kPackWords * t + k),
                           byte_at(r.ex, k));
                slot++;
            }
        }
    }
    return tile_total;
}

// One whole tile: thread t packs words t0 + kPackWords*t onwards, loaded in
// w; returns the tile's escape count.
template <bool kAlignedSm>
__device__ __forceinline__ uint32_t pack_tile(const uint32_t* w, uint64_t t0, const uint8_t* lut,
                                              uint8_t* nib, uint8_t* sm, uint64_t slot_base,
                                              PackLds& lds, int parity, const EscapeOut& esc) {
    const uint64_t i0 = t0 + (uint64_t)threadIdx.x * kPackWords;
    ThreadWords r;
    encode_words(w, lut, r);
    if constexpr (kPackWords == 16) {
        *reinterpret_cast<uint2*>(nib + i0 / 2) = make_uint2(r.nib[0], r.nib[1]);
    } else {
        *reinterpret_cast<uint32_t*>(nib + i0 / 2) = r.nib[0];
    }
    if (kAlignedSm) {
        if constexpr (kPackWords == 16)
            *reinterpret_cast<uint4*>(sm + i0) = make_uint4(r.sm[0], r.sm[1], r.sm[2], r.sm[3]);
        else
            *reinterpret_cast<uint2*>(sm + i0) = make_uint2(r.sm[0], r.sm[1]);
    } else {
#pragma unroll
        for (int k = 0; k < kPackWords; k++) sm[i0 + k] = (uint8_t)byte_at(r.sm, k);
    }
    return write_escapes(r, t0, slot_base, lds, parity, esc);
}

template <bool kAlignedSm, class Words>
__global__ __launch_bounds__(kPackThreads) SZ_EIGHT_WAVE_SGPR_CAP
__attribute__((amdgpu_waves_per_eu(8))) void k_pack(
    Words src, uint64_t n, uint32_t chunk_log2, const uint64_t* __restrict__ chunk_base,
    uint8_t* __restrict__ dst, uint64_t dst_capacity) {
    __shared__ PackLds lds;
    uint8_t* lut = lds.lut;
    if (src.invalid()) return;  // the same for every thread

    const int t = threadIdx.x;
    if (t < 256) lut[t] = 0x10;
    __syncthreads();
    if (t < 16) lut[dst[kHeaderBytes + t]] = (uint8_t)t;
    __syncthreads();

    const uint64_t E = *reinterpret_cast<const uint64_t*>(dst + 16);
    const uint64_t esc_off = kPrefixBytes + (n + 1) / 2 + n;
    // never write an escape record outside the caller's buffer, whatever
    // the workspace and header hold: slots below E, and all 5E escape bytes
    // inside the buffer
    EscapeOut esc;
    esc.pos = dst + esc_off;
    esc.exp = esc.pos + 4 * E;
    esc.limit = (dst_capacity >= esc_off && E <= (dst_capacity - esc_off) / 5) ? E : 0;
    esc.pos_aligned = (esc_off & 3) == 0;
    uint8_t* nib = dst + kPrefixBytes;
    uint8_t* sm = nib + (n + 1) / 2;

    const uint64_t begin = (uint64_t)blockIdx.x << chunk_log2;
    const uint64_t end = min_u64(begin + (uint64_t{1} << chunk_log2), n);
    uint64_t slot_base = chunk_base[blockIdx.x];

    int parity = 0;
    uint64_t t0 = begin;
    // whole tiles, no per-word checks
    for (; t0 + kPackTile <= end; t0 += kPackTile, parity ^= 1) {
        // a tile lies inside one page
        const uint4* p = reinterpret_cast<const uint4*>(src.at(t0) + (uint64_t)t * kPackWords);
        uint32_t w[kPackWords / 2];
#pragma unroll
        for (int h = 0; h < kPackLoads; h++) {
            const uint4 v = p[h];
            w[4 * h + 0] = v.x;
            w[4 * h + 1] = v.y;
            w[4 * h + 2] = v.z;
            w[4 * h + 3] = v.w;
        }
        slot_base += pack_tile<kAlignedSm>(w, t0, lut, nib, sm, slot_base, lds, parity, esc);
    }
    // the ragged last tile of the input (last chunk only); every index below
    // is a compile-time constant after unrolling, so nothing leaves registers
    if (t0 < end) {
        const uint64_t i0 = t0 + (uint64_t)t * kPackWords;
        const uint16_t* mine = src.at(t0) + (uint64_t)t * kPackWords;
        const uint32_t valid =
            i0 + kPackWords <= end ? kPackWords : (i0 < end ? (uint32_t)(end - i0) : 0u);
        uint32_t w[kPackWords / 2];
#pragma unroll
        for (int j = 0; j < kPackWords / 2; j++) {
            const uint32_t lo = 2 * j < (int)valid ? mine[2 * j] : 0u;
            const uint32_t hi = 2 * j + 1 < (int)valid ? mine[2 * j + 1] : 0u;
            w[j] = lo | (hi << 16);
        }
        ThreadWords r;
        encode_words(w, lut, r);
        // words past the end have no code (the pad nibble of an odd n is 0)
        // and are no escapes
        r.mask &= (1u << valid) - 1u;  // valid <= 16
#pragma unroll
        for (int k = 0; k < kPackWords; k++)
            if (k >= (int)valid) r.nib[k >> 3] &= ~(0xFu << (4 * (k & 7)));
#pragma unroll
        for (int j = 0; j < kPackWords / 2; j++)
            if (2 * j < (int)valid) nib[i0 / 2 + j] = (uint8_t)byte_at(r.nib, j);
#pragma unroll
        for (int k = 0; k < kPackWords; k++)
            if (k < (int)valid) sm[i0 + k] = (uint8_t)byte_at(r.sm, k);
        write_escapes(r, t0, slot_base, lds, parity, esc);
    }
}

template <class Words>
hipError_t launch_pack(Words src, const EncodePlan& p, const uint8_t* ws, uint8_t* dst,
                       uint64_t dst_capacity, int /*num_cus*/, hipStream_t stream) {
    if (p.chunks == 0) return hipSuccess;
    const uint64_t* base = reinterpret_cast<const uint64_t*>(ws + p.base_off);
    // the sign|mantissa stream starts at 176 + ceil(n/2): 16-byte aligned
    // exactly when n is a multiple of 32
    const bool aligned = ((kPrefixBytes + (p.n + 1) / 2) & 15) == 0;
    if (aligned)
        k_pack<true, Words><<<p.chunks, kPackThreads, 0, stream>>>(src, p.n, p.chunk_log2, base,
                                                                   dst, dst_capacity);
    else
        k_pack<false, Words><<<p.chunks, kPackThreads, 0, stream>>>(src, p.n, p.chunk_log2, base,
                                                                    dst, dst_capacity);
    return hipGetLastError();
}
template hipError_t launch_pack<FlatWords>(FlatWords, const EncodePlan&, const uint8_t*,
                                           uint8_t*, uint64_t, int, hipStream_t);
template hipError_t launch_pack<PagedWords>(PagedWords, const EncodePlan&, const uint8_t*,
                                            uint8_t*, uint64_t, int, hipStream_t);

}  // namespace sz
