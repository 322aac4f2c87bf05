// encode.hip -- the three encode passes of the SplitZip BF16 codec on gfx950.
//
//   histogram  one workgroup per chunk: 256-bin exponent counts in LDS
//              (replicated sub-histograms against same-address conflicts),
//              written out bin-major, counts[bin][chunk]
//   codebook   merge the counts, rank the 256 exponents (count desc, value
//              asc), write header + codebook, and turn every chunk's counts
//              into its exact escape count and first escape slot
//   pack       one workgroup per chunk: 16-byte loads, 256-entry exponent
//              -> code table in LDS whose 16-bit entries combine four at a
//              time into two nibble bytes and four escape flags, sign|mantissa
//              bytes, ballot/popcount escape ranks, escapes written straight
//              to their final slots in ascending position order
//
// and the single-read form of the same encode (large inputs), which reads
// the input once when a sample predicts the codebook:
//
//   sample     512 blocks of 2048 words counted by 64 workgroups; one more
//              ranks them into a provisional codebook
//   first      the pack kernel with the provisional code table, counting
//              the exact exponents of its chunk as it packs; escape records
//              to per-chunk scratch slots past the container
//   codebook   as above, from the first pass's counts
//   finish     the pack kernel again: records moved into place (same
//              codebook), codes rewritten (same 16 exponents, other order),
//              or the chunk packed again from the input (anything else)
//
// The container is the same either way; the sample only decides how much
// of the work the first pass can keep.
// Method: SplitZip explainers (gist.science, arXiv 2605.01708), sections
// "2. La decouverte secrete" (exponents repeat), "3. La strategie SplitZip"
// (top-16 list, fixed 4-bit codes two per byte, rare exponents as
// (position, exponent) notes) and "4. Pourquoi est-ce rapide ?" (fixed-size
// codes make every output slot known in advance).
#include "sz_internal.h"

namespace sz {

// ---------------------------------------------------------------- plan

EncodePlan plan_encode(uint64_t n) {
    uint32_t c = kMinChunkLog2;
    while (c < 40 && ((n + (1ull << c) - 1) >> c) > kPlanChunks) c++;
    // Halve the chunk (on MI355X):
    //  - when that fills the pack grid's last wave better: the pack kernels
    //    give each workgroup one chunk, so a grid ending in a partly filled
    //    wave leaves CUs idle (1280 chunks of 2^22 words ran the first pass
    //    6% below the per-byte rate of 2048 chunks).  Test: the idle share of
    //    the slots, (slots - G) / slots, drops by more than 1/50;
    //  - when the halved plan has more than 3072 chunks, a multiple of 4: the
    //    select then reads four chunks' counts per load, as fast as it reads
    //    2048 chunks, and the smaller chunks stream faster (1 GiB tensor:
    //    first pass 370 -> 359 us with 4096 chunks of 2^17 words);
    // and only into chunks of at least 2^17 words: below, the per-chunk
    // costs (count flushes, a larger merge and select) outweigh either gain
    // (whole sz_encode calls on 2^25 to 2^27 words ran 3-22% slower).
    if (c > kMinHalvedChunkLog2) {
        const uint64_t g0 = (n + (1ull << c) - 1) >> c, g1 = (n + (1ull << (c - 1)) - 1) >> (c - 1);
        const uint64_t s0 = (g0 + kResidentPackGroups - 1) / kResidentPackGroups * kResidentPackGroups;
        const uint64_t s1 = (g1 + kResidentPackGroups - 1) / kResidentPackGroups * kResidentPackGroups;
        const bool fills = 50 * (s1 - g1) * s0 + s1 * s0 < 50 * (s0 - g0) * s1;
        const bool wide_select = g1 > 3 * kMaxChunks / 4 && g1 % 4 == 0;
        if (fills || wide_select) c--;
    }
    return plan_encode_chunks(n, c);
}

EncodePlan plan_encode_chunks(uint64_t n, uint32_t c) {
    EncodePlan p;
    p.n = n;
    p.chunk_log2 = c;
    p.chunks = (uint32_t)((n + (1ull << c) - 1) >> c);
    auto align = [](uint64_t x) { return (x + 255) & ~255ull; };
    p.counts_off = 0;
    p.hist_off = align(p.counts_off + (uint64_t)p.chunks * 256 * 4);
    p.base_off = align(p.hist_off + 256 * 8);
    p.totals_off = align(p.base_off + (uint64_t)p.chunks * 8);
    p.esc_off = align(p.totals_off + kTotalCopies * 256 * 8);
    p.sample_off = align(p.esc_off + (uint64_t)p.chunks * 4);
    p.ws_bytes = align(p.sample_off + sizeof(SampleArea));
    // scratch for the provisional escape records: past every container
    // whose chunks each hold at most spec_cap escapes, inside the worst-case
    // container size the caller must provide
    p.spec_cap = (uint64_t{1} << c) / 16;
    const uint64_t e_max = (uint64_t)p.chunks * p.spec_cap;
    const uint64_t esc_off = kPrefixBytes + (n + 1) / 2 + n;
    p.scratch_pos = (esc_off + 5 * e_max + 15) & ~uint64_t{15};
    p.scratch_exp = p.scratch_pos + 4 * e_max;
    p.scratch_end = p.scratch_exp + e_max;
    p.single_read = n >= kSingleReadMin && p.scratch_end <= container_bytes(n, (15 * n) / 16);
    return p;
}

EncodePlan plan_blocks(uint64_t block_elems, uint64_t n_blocks) {
    uint32_t c = plan_encode(block_elems * n_blocks).chunk_log2;
    uint32_t fit = kMinChunkLog2;  // the smallest chunk that holds a whole block
    while (fit < 32 && (uint64_t{1} << fit) < block_elems) fit++;
    if (c > fit) c = fit;
    return plan_encode_chunks(block_elems, c);
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

// Adds the exponents of words [begin, end) into this thread's copy `mine`,
// kThreads threads striding over each run that is contiguous in memory
// (one run for a flat tensor).  8 words per 16-byte load; four loads in
// flight per thread.  The loads are non-temporal: not allocating the input
// in the caches leaves the lines already there (often the dirty output of
// earlier kernels) alone, which measured 25% faster for this pass and 4%
// for the whole codec.
template <int kThreads, class Words>
__device__ __forceinline__ void count_exponents(Words src, uint64_t begin, uint64_t end,
                                                uint32_t* mine) {
    for (uint64_t r0 = begin; r0 < end;) {
        const uint64_t r1 = src.run_end(r0, end);
        const uint16_t* base = src.at(r0);
        const uint4* v = reinterpret_cast<const uint4*>(base);
        const uint32_t groups = (uint32_t)((r1 - r0) >> 3);
        uint32_t g = threadIdx.x;
        for (; g + 3 * kThreads < groups; g += 4 * kThreads) {
            const uint4 a = load_streaming(v + g);
            const uint4 b = load_streaming(v + g + kThreads);
            const uint4 c = load_streaming(v + g + 2 * kThreads);
            const uint4 d = load_streaming(v + g + 3 * kThreads);
            hist_uint4(mine, a);
            hist_uint4(mine, b);
            hist_uint4(mine, c);
            hist_uint4(mine, d);
        }
        for (; g < groups; g += kThreads) hist_uint4(mine, load_streaming(v + g));
        // fewer than 8 words left at the very end of the input
        for (uint64_t i = ((uint64_t)groups << 3) + threadIdx.x; i < r1 - r0; i += kThreads)
            hist_add(mine, (base[i] >> 7) & 0xFFu);
        r0 = r1;
    }
}

// counts[bin * chunks + chunk]: bin-major, so that the codebook pass reads
// every bin's counts, and each chunk's 16 codebook counts, coalesced
// Workgroup 0 also zeroes what the codebook pass counts up: the whole
// input's counts and the number of its workgroups done.  For blocks, every
// workgroup adds its counts to its block's whole-input counts instead,
// which the address check zeroed.
template <class Words>
__global__ __launch_bounds__(kHistThreads) void k_histogram(Words src, uint64_t n,
                                                            uint32_t chunk_log2, uint32_t chunks,
                                                            uint32_t* __restrict__ counts,
                                                            uint64_t* __restrict__ hist,
                                                            uint32_t* __restrict__ arrivals) {
    __shared__ uint32_t h[kHistCopies * kHistPitch];
    if constexpr (Words::kBlocks) {
        const uint64_t off = block_ws(src);
        counts = byte_offset(counts, off);
        hist = byte_offset(hist, off);
        arrivals = byte_offset(arrivals, off);
    }
    if (blockIdx.x == 0 && !Words::kBlocks) {
        for (int b = threadIdx.x; b < 256; b += kHistThreads) hist[b] = 0;
        if (threadIdx.x == 0) *arrivals = 0;
    }
    if (blockIdx.x >= chunks || src.invalid()) return;  // the same for every thread
    for (int i = threadIdx.x; i < kHistCopies * kHistPitch; i += kHistThreads) h[i] = 0;
    __syncthreads();

    const uint64_t begin = (uint64_t)blockIdx.x << chunk_log2;
    const uint64_t end = min_u64(begin + (uint64_t{1} << chunk_log2), n);
    count_exponents<kHistThreads>(src.resolve(), begin, end,
                                  h + (threadIdx.x % kHistCopies) * kHistPitch);
    __syncthreads();

    for (int bin = threadIdx.x; bin < 256; bin += kHistThreads) {
        uint32_t s = 0;
#pragma unroll
        for (int c = 0; c < kHistCopies; c++) s += h[c * kHistPitch + bin];
        counts[(uint64_t)bin * chunks + blockIdx.x] = s;
        if constexpr (Words::kBlocks)
            __hip_atomic_fetch_add(hist + bin, (uint64_t)s, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <class Words>
hipError_t launch_histogram(Words src, const EncodePlan& p, uint8_t* ws, hipStream_t stream) {
    const uint32_t groups = p.chunks > 0 ? p.chunks : 1;  // the accumulators are zeroed
    k_histogram<Words><<<dim3(groups, grid_blocks(src)), kHistThreads, 0, stream>>>(
        src, p.n, p.chunk_log2, p.chunks, reinterpret_cast<uint32_t*>(ws + p.counts_off),
        reinterpret_cast<uint64_t*>(ws + p.hist_off),
        &reinterpret_cast<SampleArea*>(ws + p.sample_off)->arrivals);
    return hipGetLastError();
}
template hipError_t launch_histogram<FlatWords>(FlatWords, const EncodePlan&, uint8_t*,
                                                hipStream_t);
template hipError_t launch_histogram<PagedWords>(PagedWords, const EncodePlan&, uint8_t*,
                                                 hipStream_t);
template hipError_t launch_histogram<BlockWords>(BlockWords, const EncodePlan&, uint8_t*,
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

// One workgroup per block: its address must be non-NULL and 16-byte
// aligned, else the block is flagged and its workgroups touch none of its
// memory; with a workspace, the block's whole-input counts start at zero.
__global__ __launch_bounds__(256) void k_check_blocks(const uint16_t* const* blocks,
                                                      int32_t* flags, int32_t* status,
                                                      uint64_t* hist, uint64_t ws_stride) {
    const uint32_t b = blockIdx.x;
    if (hist) byte_offset(hist, (uint64_t)b * ws_stride)[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(blocks[b]);
        const int32_t f = (a == 0 || (a & 15) != 0) ? kBlockInvalid : 0;
        flags[b] = f;
        if (status) status[b] = f;
    }
}

hipError_t launch_check_blocks(const uint16_t* const* blocks, uint64_t n_blocks, int32_t* flags,
                               int32_t* status, uint8_t* ws, const EncodePlan& p,
                               uint64_t ws_stride, hipStream_t stream) {
    if (n_blocks == 0) return hipSuccess;
    uint64_t* hist = ws ? reinterpret_cast<uint64_t*>(ws + p.hist_off) : nullptr;
    k_check_blocks<<<(uint32_t)n_blocks, 256, 0, stream>>>(blocks, flags, status, hist, ws_stride);
    return hipGetLastError();
}

// ---------------------------------------------------------------- pass 2

constexpr int kSelectThreads = 1024;
constexpr int kSelectWaves = kSelectThreads / 64;
constexpr int kSelectChunks = kMaxChunks / kSelectThreads;  // chunks per select thread

__device__ __forceinline__ uint64_t wave_inclusive_sum(uint64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// Rank of this lane's bits among lower lanes: popcount of mask below lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// LDS of top16_ranks (keys of type K: 64-bit, or 32-bit where every count
// is below 2^24).
template <class K>
struct alignas(16) RankLds {
    uint32_t full[4][256];   // partial counts of the full ranking
    K gmax[4][16];           // per wave of the first four, each group's largest key
    K cand[64];              // the candidates' keys
    uint32_t wave_cand[4];   // candidates per wave
};

template <class K>
__device__ __forceinline__ K max_key(K a, K b) {
    return a > b ? a : b;
}
template <class K>
__device__ __forceinline__ K min_key(K a, K b) {
    return a < b ? a : b;
}

// Every exponent's rank as the number of larger keys, four groups of 256
// threads each comparing against 64 of the keys, 16-byte LDS loads (key
// 16-byte aligned).  Returns the rank of exponent t to threads t < 256.
template <class K>
__device__ __forceinline__ uint32_t full_rank(const K* key, RankLds<K>& s) {
    const int t = threadIdx.x;
    const int bin = t & 255, grp = t >> 8;  // 0..3
    const K kx = key[bin];
    const uint4* k4 = reinterpret_cast<const uint4*>(key + grp * 64);
    uint32_t r = 0;
#pragma unroll
    for (int y = 0; y < (int)(64 * sizeof(K) / 16); y++) {
        const uint4 v = k4[y];
        if constexpr (sizeof(K) == 8) {
            r += ((uint64_t)v.y << 32 | v.x) > kx ? 1u : 0u;
            r += ((uint64_t)v.w << 32 | v.z) > kx ? 1u : 0u;
        } else {
            r += (v.x > kx ? 1u : 0u) + (v.y > kx ? 1u : 0u) + (v.z > kx ? 1u : 0u) +
                 (v.w > kx ? 1u : 0u);
        }
    }
    s.full[grp][bin] = r;
    __syncthreads();
    return t < 256 ? s.full[0][t] + s.full[1][t] + s.full[2][t] + s.full[3][t] : 0u;
}

// The 16 most frequent exponents' ranks (the codebook rule: key = count << 8
// | 255 - exponent, larger key earlier; the keys are distinct), from the
// keys in LDS, which the caller has synchronised.  Returns to thread t < 256
// the number of keys larger than exponent t's when that is below 16, and 16
// or more otherwise.  Candidates first: with the exponents in 16 interleaved
// groups (e, e + 16, ..., e + 240), the smallest of the groups' largest
// keys, L, has at least 16 keys at or above it (those maxima), so the top 16
// are among the keys >= L, and a candidate's rank counts candidates only.
// The exponents of real data crowd into one run of consecutive bins, one
// bin of it per group, so about 16 keys are candidates; with more than 64
// every key is ranked against all 256 instead.
template <class K>
__device__ __forceinline__ uint32_t top16_ranks(const K* key, RankLds<K>& s) {
    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6;
    K kx = 0;
    if (t < 256) {
        // lanes l, l ^ 16, l ^ 32, l ^ 48 of a wave hold one group's bins
        kx = key[t];
        K m = max_key<K>(kx, __shfl_xor(kx, 16, 64));
        m = max_key<K>(m, __shfl_xor(m, 32, 64));
        if (lane < 16) s.gmax[w][lane] = m;
    }
    __syncthreads();
    bool cand = false;
    uint32_t in_wave = 0;
    if (t < 256) {
        // each of the four waves works out L itself
        const int g = lane & 15;
        K l = max_key<K>(max_key<K>(s.gmax[0][g], s.gmax[1][g]),
                         max_key<K>(s.gmax[2][g], s.gmax[3][g]));
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) l = min_key<K>(l, __shfl_xor(l, d, 64));
        cand = kx >= l;
        const uint64_t bits = __ballot(cand);
        in_wave = lanes_below(bits);
        if (lane == 0) s.wave_cand[w] = (uint32_t)__popcll(bits);
    }
    __syncthreads();
    const uint32_t total = s.wave_cand[0] + s.wave_cand[1] + s.wave_cand[2] + s.wave_cand[3];
    if (total > 64) return full_rank(key, s);  // the same for every thread
    if (cand) {
        uint32_t before = 0;
        for (int v = 0; v < w; v++) before += s.wave_cand[v];
        s.cand[before + in_wave] = kx;
    }
    __syncthreads();
    uint32_t r = 16;  // below every candidate: not in the top 16
    if (cand) {
        r = 0;
        for (uint32_t i = 0; i < total; i++) r += s.cand[i] > kx ? 1u : 0u;
    }
    return t < 256 ? r : 0u;
}

// The sums over the 64 lanes of each of the 16 values part[0..15] a lane
// holds, by halving exchanges, as in a reduce-scatter: at each of four
// steps the lanes whose bit log2(4 * half) is set keep the upper half of
// their values and send the lower, the others the reverse; two more
// exchanges add the four lanes that end up with the same value.  Value i's
// sum is returned to lanes 4i .. 4i + 3, i's bits taken from lane bits
// 5, 4, 3, 2; part is overwritten.  (Mask arithmetic picks the halves: a
// select of two array elements is turned by the compiler into a dynamic
// index over the array, a chain of hundreds of selects.)
__device__ __forceinline__ uint32_t sum16_across_lanes(uint32_t (&part)[16], int lane) {
#pragma unroll
    for (int half = 8; half >= 1; half >>= 1) {
        const uint32_t upper = (lane & (4 * half)) != 0 ? ~0u : 0u;
#pragma unroll
        for (int i = 0; i < half; i++) {
            const uint32_t a = part[i], b = part[half + i], flip = (a ^ b) & upper;
            part[i] = (a ^ flip) + __shfl_xor(b ^ flip, 4 * half, 64);
        }
    }
    uint32_t sum = part[0];
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    return sum;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// Escape counts of chunks per * t .. per * t + per - 1 (per = ceil(chunks /
// 1024), the same for the whole workgroup) under the codebook in LDS: chunk
// length - elements whose exponent is in the codebook, from the bin-major
// per-chunk counts.  Four chunks a thread, 16-byte aligned, are read with
// 16-byte loads; otherwise two chunks per round of loads (one round up to
// 2048 chunks; two keep the counts of up to four chunks from spilling).  The
// codebook is the same in every lane: scalar row addresses.
__device__ __forceinline__ void exact_chunk_escapes(const uint32_t* __restrict__ counts,
                                                    uint32_t chunks, uint32_t chunk_log2,
                                                    uint64_t n, const uint32_t* codebook,
                                                    uint64_t (&esc)[kSelectChunks]) {
    const int t = threadIdx.x;
    uint32_t cb[16];
#pragma unroll
    for (int c = 0; c < 16; c++) cb[c] = __builtin_amdgcn_readfirstlane(codebook[c] & 255u);
    const uint32_t per = (chunks + kSelectThreads - 1) / kSelectThreads;  // <= kSelectChunks
    if (per == 4 && chunks % 4 == 0) {
        // four contiguous chunks per thread, 16-byte aligned: one 16-byte
        // load per codebook row, the rows in two halves of eight
        const uint32_t b0 = 4 * t;
        if (b0 < chunks) {
            uint32_t kept[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int h = 0; h < 2; h++) {
                uint4 v[8];
#pragma unroll
                for (int c = 0; c < 8; c++)
                    v[c] = *reinterpret_cast<const uint4*>(counts + (uint64_t)cb[8 * h + c] * chunks + b0);
#pragma unroll
                for (int c = 0; c < 8; c++) {
                    kept[0] += v[c].x;
                    kept[1] += v[c].y;
                    kept[2] += v[c].z;
                    kept[3] += v[c].w;
                }
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint64_t start = (uint64_t)(b0 + j) << chunk_log2;
                esc[j] = min_u64(uint64_t{1} << chunk_log2, n - start) - kept[j];
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < kSelectChunks / 2; r++) {
            if ((uint32_t)(2 * r) >= per) break;
            // the two chunks' 16 codebook counts, coalesced across threads
            // (bin-major layout), all in flight at once
            uint32_t v[2][16];
#pragma unroll
            for (int c = 0; c < 16; c++) {
                const uint32_t* row = counts + (uint64_t)cb[c] * chunks;
#pragma unroll
                for (int jj = 0; jj < 2; jj++) {
                    const uint32_t j = 2 * r + jj, b = per * t + j;
                    v[jj][c] = j < per && b < chunks ? row[b] : 0u;
                }
            }
#pragma unroll
            for (int jj = 0; jj < 2; jj++) {
                const uint32_t j = 2 * r + jj, b = per * t + j;
                if (j < per && b < chunks) {
                    const uint64_t start = (uint64_t)b << chunk_log2;
                    const uint64_t len = min_u64(uint64_t{1} << chunk_log2, n - start);
                    uint64_t kept = 0;
#pragma unroll
                    for (int c = 0; c < 16; c++) kept += v[jj][c];
                    esc[2 * r + jj] = len - kept;
                }
            }
        }
    }
}

// The same escape counts one chunk at a time (its 16 codebook rows in
// flight together), for a kernel held to 64 registers a lane.
__device__ __forceinline__ void exact_chunk_escapes_narrow(const uint32_t* __restrict__ counts,
                                                           uint32_t chunks, uint32_t chunk_log2,
                                                           uint64_t n, const uint32_t* codebook,
                                                           uint64_t (&esc)[kSelectChunks]) {
    const int t = threadIdx.x;
    const uint32_t per = (chunks + kSelectThreads - 1) / kSelectThreads;  // <= kSelectChunks
#pragma unroll
    for (int j = 0; j < kSelectChunks; j++) {
        const uint32_t b = per * t + j;
        if ((uint32_t)j < per && b < chunks) {
            uint64_t kept = 0;
#pragma unroll
            for (int c = 0; c < 16; c++) kept += counts[(uint64_t)codebook[c] * chunks + b];
            const uint64_t start = (uint64_t)b << chunk_log2;
            esc[j] = min_u64(uint64_t{1} << chunk_log2, n - start) - kept;
        }
    }
}

// The same from chunk-major counts (chunk b's 256 at counts + 256 b): a
// lane's 16 loads hit its own chunk's row, so they do not coalesce across
// the wave; for the rare case that needs them.
__device__ __forceinline__ void exact_chunk_escapes_chunk_major(const uint32_t* __restrict__ counts,
                                                                uint32_t chunks, uint32_t chunk_log2,
                                                                uint64_t n, const uint32_t* codebook,
                                                                uint64_t (&esc)[kSelectChunks]) {
    const int t = threadIdx.x;
    const uint32_t per = (chunks + kSelectThreads - 1) / kSelectThreads;  // <= kSelectChunks
#pragma unroll
    for (int j = 0; j < kSelectChunks; j++) {
        const uint32_t b = per * t + j;
        if ((uint32_t)j < per && b < chunks) {
            const uint32_t* mine = counts + (uint64_t)b * 256;
            uint64_t kept = 0;
#pragma unroll
            for (int c = 0; c < 16; c++) kept += mine[codebook[c]];
            const uint64_t start = (uint64_t)b << chunk_log2;
            esc[j] = min_u64(uint64_t{1} << chunk_log2, n - start) - kept;
        }
    }
}

// Exclusive scan of the chunks' escape counts (each thread's kSelectChunks
// in order) over the 1024-thread workgroup: returns the escapes before this
// thread's first chunk, and the total E to every thread.
__device__ __forceinline__ uint64_t scan_chunk_escapes(const uint64_t (&esc)[kSelectChunks],
                                                       uint64_t* wave_sum, uint64_t* wave_off,
                                                       uint64_t& E) {
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    uint64_t mine = 0;
#pragma unroll
    for (int j = 0; j < kSelectChunks; j++) mine += esc[j];
    const uint64_t incl = wave_inclusive_sum(mine);
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
    E = wave_off[kSelectWaves - 1] + wave_sum[kSelectWaves - 1];
    return wave_off[wave] + incl - mine;
}

// Up to this many chunks (tensors of up to 2^22 words) the codebook pass is
// one workgroup.
constexpr uint32_t kSmallCodebookChunks = 256;

// The codebook pass, one launch of 256 workgroups: workgroup b sums bin b's
// counts over the chunks (every load in flight at once, bin-major layout)
// and adds the total to hist[b], which the pass before zeroed; device-wide
// atomics whose returned value is waited for, so the bin is in before the
// workgroup counts itself done.  The workgroup that arrives last reads the
// 256 totals back through atomics and ranks them; turns every chunk's counts
// into its escape count and first escape slot (chunk_base); writes header,
// codebook, seg_end and *d_size; and zeroes hist and the arrival count
// again, so the pass can run twice on one workspace, and the sample pass's
// tickets and counts, which puts a workspace that came in with other values
// in step for the next sample pass.  For blocks, one workgroup per block,
// each on its block's workspace and container: the count pass has already
// added up the whole block's counts, so the workgroup goes straight to the
// ranking.  With at most kSmallCodebookChunks chunks one workgroup sums the
// 256 rows itself and ranks them, with no device-wide adds, arrivals or
// read-back in between.
template <class Words>
__global__ __launch_bounds__(kSelectThreads) void k_codebook(
    Words src, uint64_t n, uint32_t chunk_log2, uint32_t chunks, const uint32_t* __restrict__ counts,
    uint64_t* __restrict__ hist, SampleArea* __restrict__ sample, uint64_t* __restrict__ chunk_base,
    uint8_t* __restrict__ dst, uint64_t* d_size) {
    __shared__ alignas(16) uint64_t key[256];
    __shared__ RankLds<uint64_t> rank_lds;
    __shared__ uint32_t codebook[16];
    __shared__ uint64_t wave_sum[kSelectWaves];
    __shared__ uint64_t wave_off[kSelectWaves];
    __shared__ uint64_t base_lds[kMaxChunks];
    __shared__ uint32_t last;

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    if constexpr (Words::kBlocks) {
        const uint64_t off = block_ws(src);
        counts = byte_offset(counts, off);
        hist = byte_offset(hist, off);
        sample = byte_offset(sample, off);
        chunk_base = byte_offset(chunk_base, off);
        dst = byte_offset(dst, block_pitch(src));
        d_size = src.sizes + blockIdx.y;
        if (src.invalid()) {  // the same for every thread: no counts to read
            if (t == 0) *d_size = 0;
            return;
        }
    } else if (gridDim.x == 1) {
        // at most kSmallCodebookChunks chunks: this one workgroup reads every
        // count itself (no device-wide adds, arrivals or read-back between
        // the counts and the ranking).  Wave w sums bins 16w .. 16w + 15,
        // consecutive lanes on consecutive chunks of a row, 128 chunks of
        // each of its rows per round of loads; then the sums across lanes.
        const uint32_t w = __builtin_amdgcn_readfirstlane(t >> 6);  // scalar row addresses
        const uint32_t* rows = counts + (uint64_t)16 * w * chunks;
        uint32_t part[16];
#pragma unroll
        for (int i = 0; i < 16; i++) part[i] = 0;
        for (uint32_t c0 = 0; c0 < chunks; c0 += 128) {
            uint32_t v[2][16];
            if (c0 + 128 <= chunks) {  // a whole round: no per-load checks
#pragma unroll
                for (int h = 0; h < 2; h++)
#pragma unroll
                    for (int i = 0; i < 16; i++)
                        v[h][i] = rows[(uint64_t)i * chunks + c0 + 64 * h + lane];
            } else {
#pragma unroll
                for (int h = 0; h < 2; h++)
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        const uint32_t c = c0 + 64 * h + lane;
                        v[h][i] = c < chunks ? rows[(uint64_t)i * chunks + c] : 0u;
                    }
            }
#pragma unroll
            for (int i = 0; i < 16; i++) part[i] += v[0][i] + v[1][i];
        }
        const uint32_t sum = sum16_across_lanes(part, lane);
        if ((lane & 3) == 0) {
            const uint32_t bin = 16 * w + ((lane >> 2) & 15);
            key[bin] = ((uint64_t)sum << 8) | (255u - bin);
        }
    } else {
        const uint32_t bin = blockIdx.x;
        const uint32_t* row = counts + (uint64_t)bin * chunks;
        uint32_t v[kSelectChunks];
#pragma unroll
        for (int j = 0; j < kSelectChunks; j++) {
            const uint32_t c = t + j * kSelectThreads;
            v[j] = c < chunks ? row[c] : 0u;
        }
        uint64_t s = 0;
#pragma unroll
        for (int j = 0; j < kSelectChunks; j++) s += v[j];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) s += __shfl_down(s, d, 64);
        if (lane == 0) wave_sum[wave] = s;
        __syncthreads();
        if (t == 0) {
            uint64_t total = 0;
            for (int w = 0; w < kSelectWaves; w++) total += wave_sum[w];
            const uint64_t before = __hip_atomic_fetch_add(hist + bin, total, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
            // the add has returned before the arrival is counted: the empty
            // asm reads the returned value, so the wave waits for it
            asm volatile("" ::"v"(before));
            const uint32_t done = __hip_atomic_fetch_add(&sample->arrivals, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            last = done == gridDim.x - 1 ? 1u : 0u;
        }
        __syncthreads();
        if (!last) return;
    }

    // the last workgroup: key(x) = count << 8 | (255 - x) turns "more
    // frequent, then smaller exponent" into one unsigned comparison (counts
    // stay below 2^37)
    if (t < 256 && (Words::kBlocks || gridDim.x > 1))
        key[t] = (__hip_atomic_fetch_add(hist + t, uint64_t{0}, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) << 8) | (255u - t);
    __syncthreads();
    {
        const uint32_t r = top16_ranks(key, rank_lds);
        if (t < 256 && r < 16) codebook[r] = (uint32_t)t;
    }
    __syncthreads();
    uint64_t esc[kSelectChunks] = {};
    exact_chunk_escapes(counts, chunks, chunk_log2, n, codebook, esc);
    const uint32_t per = (chunks + kSelectThreads - 1) / kSelectThreads;
    uint64_t E;
    uint64_t excl = scan_chunk_escapes(esc, wave_sum, wave_off, E);
#pragma unroll
    for (int j = 0; j < kSelectChunks; j++) {
        const uint32_t b = per * t + j;
        if ((uint32_t)j < per && b < chunks) {
            chunk_base[b] = excl;
            base_lds[b] = excl;
        }
        excl += esc[j];
    }
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
    // ready for another run of this pass on the same workspace, and the
    // sample pass's tickets and counts back in step
    if (t < 256) {
        hist[t] = 0;
        sample->sample_hist[t] = 0;
    }
    if (t == 0) {
        sample->arrivals = 0;
        sample->tickets = 0;
    }
}

template <class Words>
hipError_t launch_codebook(Words src, const EncodePlan& p, uint8_t* ws, uint8_t* dst,
                           uint64_t* d_size, hipStream_t stream) {
    const uint32_t* counts = reinterpret_cast<const uint32_t*>(ws + p.counts_off);
    uint64_t* hist = reinterpret_cast<uint64_t*>(ws + p.hist_off);
    SampleArea* sample = reinterpret_cast<SampleArea*>(ws + p.sample_off);
    const uint32_t groups = Words::kBlocks || p.chunks <= kSmallCodebookChunks ? 1 : 256;
    k_codebook<Words><<<dim3(groups, grid_blocks(src)), kSelectThreads, 0, stream>>>(
        src, p.n, p.chunk_log2, p.chunks, counts, hist, sample,
        reinterpret_cast<uint64_t*>(ws + p.base_off), dst, d_size);
    return hipGetLastError();
}
template hipError_t launch_codebook<FlatWords>(FlatWords, const EncodePlan&, uint8_t*, uint8_t*,
                                               uint64_t*, hipStream_t);
template hipError_t launch_codebook<BlockWords>(BlockWords, const EncodePlan&, uint8_t*, uint8_t*,
                                                uint64_t*, hipStream_t);

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
static_assert(kSelectChunks * kSelectThreads == kMaxChunks, "whole chunks per select thread");

// byte k of a little-endian run of dwords (k known at compile time after
// unrolling, so the array stays in registers)
__device__ __forceinline__ uint32_t byte_at(const uint32_t* v, int k) {
    return (v[k >> 2] >> (8 * (k & 3))) & 0xFFu;
}

// The code table the pack kernels read: one u16 per exponent, the code
// (0..15) in bits 3..0 and, for an exponent outside the codebook, code 0
// with bit 8 set.  Four entries of words 4j..4j+3, placed at bits 0, 4, 16
// and 20 of one dword (entry m shifted by 4(m % 2) + 16(m / 2)), give that
// dword's bytes 0 and 2 = the two nibble bytes of the four words, and their
// escape flags at bits 8, 12, 24 and 28 -- no per-word code arithmetic.
constexpr uint16_t kEscapeEntry = 0x100;
constexpr uint32_t kFlagBits = 0x11001100u;

__device__ __forceinline__ uint32_t flag_shift(int m) {
    return m == 0 ? 8u : m == 1 ? 12u : m == 2 ? 24u : 28u;
}

// Table entry at byte offset x (twice the exponent).
__device__ __forceinline__ uint32_t code_entry(const uint16_t* table, uint32_t x) {
    return *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(table) + x);
}

// Exponent of the thread's word k (two words per dword, little-endian).
__device__ __forceinline__ uint32_t exponent_of(const uint32_t* w, int k) {
    return (w[k >> 1] >> ((k & 1) ? 23 : 7)) & 0xFFu;
}

// The words of one thread, split: sign|mantissa bytes, the 4-bit codes
// (element k in bits 4(k%8).. of nib[k/8]), per four words the combined
// table entries (word 4j+m escapes when bit flag_shift(m) of quad[j] is
// set; other bits are code bits) and the number of escapes.
struct ThreadWords {
    uint32_t sm[kPackWords / 4];
    uint32_t nib[kPackWords / 8];
    uint32_t quad[kPackWords / 4];
    uint32_t count;
};

__device__ __forceinline__ bool escaped(const ThreadWords& r, int k) {
    return (r.quad[k >> 2] >> flag_shift(k & 3)) & 1u;
}

// With kCount, every exponent is also counted into hmine (its u32 count at
// byte offset 2x from hmine, x being twice the exponent).
template <bool kCount>
__device__ __forceinline__ void encode_words(const uint32_t* w, const uint16_t* table,
                                             ThreadWords& r, uint32_t* hmine) {
#pragma unroll
    for (int h = 0; h < kPackWords / 8; h++) {
        // sign bit of the high byte, mantissa bits of the low byte
        const uint32_t* v = w + 4 * h;
        const uint32_t hi0 = __builtin_amdgcn_perm(v[1], v[0], 0x07050301u);
        const uint32_t lo0 = __builtin_amdgcn_perm(v[1], v[0], 0x06040200u);
        const uint32_t hi1 = __builtin_amdgcn_perm(v[3], v[2], 0x07050301u);
        const uint32_t lo1 = __builtin_amdgcn_perm(v[3], v[2], 0x06040200u);
        r.sm[2 * h] = (hi0 & 0x80808080u) | (lo0 & 0x7F7F7F7Fu);
        r.sm[2 * h + 1] = (hi1 & 0x80808080u) | (lo1 & 0x7F7F7F7Fu);
    }
    r.count = 0;
#pragma unroll
    for (int j = 0; j < kPackWords / 4; j++) {
        const uint32_t d0 = w[2 * j], d1 = w[2 * j + 1];  // words 4j, 4j+1 | 4j+2, 4j+3
        const uint32_t x0 = (d0 >> 6) & 0x1FEu, x1 = (d0 >> 22) & 0x1FEu;
        const uint32_t x2 = (d1 >> 6) & 0x1FEu, x3 = (d1 >> 22) & 0x1FEu;
        if (kCount) {
            hist_add(hmine, x0 >> 1);
            hist_add(hmine, x1 >> 1);
            hist_add(hmine, x2 >> 1);
            hist_add(hmine, x3 >> 1);
        }
        const uint32_t a = code_entry(table, x0) | (code_entry(table, x2) << 16);
        const uint32_t b = code_entry(table, x1) | (code_entry(table, x3) << 16);
        r.quad[j] = a | (b << 4);
        r.count += __popc(r.quad[j] & kFlagBits);
    }
#pragma unroll
    for (int h = 0; h < kPackWords / 8; h++)
        r.nib[h] = __builtin_amdgcn_perm(r.quad[2 * h + 1], r.quad[2 * h], 0x06040200u);
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
    uint16_t code[256];                    // exponent -> table entry (see encode_words)
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
// w: the thread's words (for the escaped exponents).
__device__ __forceinline__ uint32_t write_escapes(const ThreadWords& r, const uint32_t* w,
                                                  uint64_t t0, uint64_t slot_base, PackLds& lds,
                                                  int parity, const EscapeOut& out) {
    const int t = threadIdx.x;
    const int lane = t & 63;
    // the wave index as a scalar: "v < wave" below is then one scalar
    // compare per v, not a lane mask per v kept in scalar registers across
    // the tile loop (sixteen 64-bit masks, which pushed the finish kernel's
    // pack loop into reloading spilled registers on every tile)
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const uint32_t cnt = r.count;
    uint32_t lane_prefix = 0, wave_total = 0;
    if (__ballot(cnt > 1) == 0) {
        // at most one escape per lane (the usual case on KV data): one ballot
        const uint64_t bits = __ballot(cnt != 0);
        lane_prefix = lanes_below(bits);
        wave_total = (uint32_t)__popcll(bits);
    } else {
#pragma unroll
        for (int b = 0; b < (kPackWords == 16 ? 5 : 4); b++) {
            const uint64_t bits = __ballot(cnt & (1u << b));
            lane_prefix += lanes_below(bits) << b;
            wave_total += (uint32_t)__popcll(bits) << b;
        }
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
        if (cnt) {
            uint32_t q = first;
#pragma unroll
            for (int k = 0; k < kPackWords; k++) {
                if (escaped(r, k)) {
                    lds.stage_off[q] = (uint16_t)(kPackWords * t + k);
                    lds.stage_exp[q] = (uint8_t)exponent_of(w, k);
                    q++;
                }
            }
        }
        __syncthreads();
        for (uint32_t q = t; q < tile_total; q += kPackThreads)
            put_escape(out, slot_base + q, (uint32_t)t0 + lds.stage_off[q], lds.stage_exp[q]);
    } else if (cnt) {
        uint64_t slot = slot_base + first;
#pragma unroll
        for (int k = 0; k < kPackWords; k++) {
            if (escaped(r, k)) {
                put_escape(out, slot, (uint32_t)t0 + (uint32_t)(kPackWords * t + k),
                           exponent_of(w, k));
                slot++;
            }
        }
    }
    return tile_total;
}

// One whole tile: thread t packs words t0 + kPackWords*t onwards, loaded in
// w (with kCount also counting their exponents into hmine); returns the
// tile's escape count.
template <bool kAlignedSm, bool kCount>
__device__ __forceinline__ uint32_t pack_tile(const uint32_t* w, uint64_t t0,
                                              const uint16_t* table, uint8_t* nib, uint8_t* sm,
                                              uint64_t slot_base, PackLds& lds, int parity,
                                              const EscapeOut& esc, uint32_t* hmine) {
    const uint64_t i0 = t0 + (uint64_t)threadIdx.x * kPackWords;
    ThreadWords r;
    encode_words<kCount>(w, table, r, hmine);
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
    return write_escapes(r, w, t0, slot_base, lds, parity, esc);
}

// The pack kernel serves three passes:
//   kClassic  codes from the exact codebook in the header; escape records to
//             their final slots (chunk_base).
//   kRanked   the same for at most kRankedChunks chunks, with no codebook
//             pass before it: every workgroup ranks the histogram pass's
//             counts itself and works out its chunk's first escape slot
//             (ranked_codebook, below); workgroup 0 writes the header.
//   kFirst    first pass of the single-read encode: the exact exponent counts
//             of the chunk (for the finish pass) and, when the
//             sample predicts few escapes, the streams under the provisional
//             codebook, escape records to the chunk's scratch slots.
// k_finish (below) completes the single-read encode.
enum class PackRole { kClassic, kRanked, kFirst };

// LDS of ranked_codebook.
struct RankedLds {
    alignas(16) uint32_t key[256];
    RankLds<uint32_t> rank;
    uint32_t codebook[16];
    uint32_t kept[kRankedChunks];  // per chunk: words whose exponent is in the codebook
    uint8_t lut[256];              // exponent -> code, 16 = escape
    uint64_t sums[2][2];           // escapes of all chunks and of those below, per wave
};

// The exact codebook from every chunk's counts (bin-major, as the histogram
// pass leaves them; counts below 2^24), the escapes below chunk `chunk` (its
// first escape slot, returned) and E.  Wave w loads bins 16w .. 16w + 15
// with consecutive lanes on consecutive chunks (all 32 loads a lane in
// flight at once) and sums them across lanes; after the ranking the same
// registers give each chunk's count of codebook exponents.
__device__ __forceinline__ uint64_t ranked_codebook(const uint32_t* __restrict__ counts, uint64_t n,
                                                    uint32_t chunk_log2, uint32_t chunks,
                                                    uint32_t chunk, RankedLds& o, uint64_t& E) {
    const int t = threadIdx.x;
    const int lane = t & 63;
    const uint32_t w = __builtin_amdgcn_readfirstlane(t >> 6);  // scalar row addresses
    const uint32_t* rows = counts + (uint64_t)16 * w * chunks;
    uint32_t v[2][16];
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t c = 64 * h + lane;
            v[h][i] = c < chunks ? rows[(uint64_t)i * chunks + c] : 0u;
        }
    uint32_t part[16];
#pragma unroll
    for (int i = 0; i < 16; i++) part[i] = v[0][i] + v[1][i];
    const uint32_t sum = sum16_across_lanes(part, lane);
    if ((lane & 3) == 0) {
        const uint32_t bin = 16 * w + ((lane >> 2) & 15);
        o.key[bin] = (min(sum, (1u << 24) - 1) << 8) | (255u - bin);
    }
    if (t < (int)kRankedChunks) o.kept[t] = 0;
    __syncthreads();
    const uint32_t r = top16_ranks(o.key, o.rank);
    if (t < 256) {
        o.lut[t] = r < 16 ? (uint8_t)r : (uint8_t)16;
        if (r < 16) o.codebook[r] = (uint32_t)t;
    }
    __syncthreads();
    uint32_t k0 = 0, k1 = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        if (o.lut[16 * w + i] < 16) {  // the same for the wave
            k0 += v[0][i];
            k1 += v[1][i];
        }
    }
    if (k0) atomicAdd(&o.kept[lane], k0);  // nonzero only for chunks that exist
    if (k1) atomicAdd(&o.kept[64 + lane], k1);
    __syncthreads();
    uint64_t all = 0, below = 0;
    if ((uint32_t)t < chunks) {
        const uint64_t start = (uint64_t)t << chunk_log2;
        all = min_u64(uint64_t{1} << chunk_log2, n - start) - o.kept[t];
        below = (uint32_t)t < chunk ? all : 0;
    }
    if (t < 128) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            all += __shfl_xor(all, d, 64);
            below += __shfl_xor(below, d, 64);
        }
        if (lane == 0) {
            o.sums[w][0] = all;
            o.sums[w][1] = below;
        }
    }
    __syncthreads();
    E = o.sums[0][0] + o.sums[1][0];
    return o.sums[0][1] + o.sums[1][1];
}

constexpr int kSpecCopies = 16;    // exponent sub-histograms of the first pass
constexpr int kSpecPitch = 257;

// The container's escape stream.  Never writes a record outside the caller's
// buffer, whatever the workspace and header hold: slots below E, and all 5E
// escape bytes inside the buffer.
__device__ __forceinline__ EscapeOut escape_slots(uint8_t* dst, uint64_t n, uint64_t dst_capacity,
                                                  uint64_t E) {
    const uint64_t esc_off = kPrefixBytes + (n + 1) / 2 + n;
    EscapeOut esc;
    esc.pos = dst + esc_off;
    esc.exp = esc.pos + 4 * E;
    esc.limit = (dst_capacity >= esc_off && E <= (dst_capacity - esc_off) / 5) ? E : 0;
    esc.pos_aligned = (esc_off & 3) == 0;
    return esc;
}

// The same, E read from the header.
__device__ __forceinline__ EscapeOut final_slots(uint8_t* dst, uint64_t n, uint64_t dst_capacity) {
    return escape_slots(dst, n, dst_capacity, *reinterpret_cast<const uint64_t*>(dst + 16));
}

// Exponent -> code tables from a codebook (code -> exponent, 16 entries in
// LDS or global memory): lds.lut (0x10 = escape) and lds.code (encode_words'
// entries); the caller synchronises before using them.
template <class Entry>
__device__ __forceinline__ void code_table(const Entry* cb, PackLds& lds) {
    const int t = threadIdx.x;
    if (t < 256) {
        lds.lut[t] = 0x10;
        lds.code[t] = kEscapeEntry;
    }
    __syncthreads();
    if (t < 16) {
        const uint8_t e = (uint8_t)cb[t];
        lds.lut[e] = (uint8_t)t;
        lds.code[e] = (uint16_t)t;
    }
}

// The same from the header's codebook.
__device__ __forceinline__ void exact_code_table(const uint8_t* dst, PackLds& lds) {
    code_table(dst + kHeaderBytes, lds);
}

// Packs words [begin, end) with the code table in lds.code, escape records to
// esc from slot slot_base on; with kCount, every exponent is also counted
// into hmine, and with write false only that.  parity selects the next
// tile's wave-total buffer and carries over from chunk to chunk when one
// workgroup packs several.  Returns the number of escapes.
template <bool kAlignedSm, bool kCount, class Words>
__device__ __forceinline__ uint64_t pack_range(Words src, uint64_t n, uint64_t begin,
                                               uint64_t end, uint8_t* dst, const EscapeOut& esc,
                                               uint64_t slot_base, bool write, uint32_t* hmine,
                                               PackLds& lds, int& parity) {
    const int t = threadIdx.x;
    const uint16_t* table = lds.code;
    uint8_t* nib = dst + kPrefixBytes;
    uint8_t* sm = nib + (n + 1) / 2;
    const uint64_t first_slot = slot_base;
    uint64_t t0 = begin;
    if (kCount && !write) {
        // counts only, at the speed of the histogram pass
        count_exponents<kPackThreads>(src, begin, end, hmine);
        t0 = end;
    }
    // whole tiles, no per-word checks (with kCount, only entered when the
    // streams are written: the exponents are counted while packing).  A tile
    // lies inside one page; for a paged tensor the next tile's page address
    // is looked up while this tile is packed, after this tile's loads are
    // issued, so that no tile waits for its page-table entry.
    const uint16_t* tile_words = nullptr;
    if constexpr (Words::kPaged) {
        if (t0 + kPackTile <= end) tile_words = src.at(t0);
    }
    for (; t0 + kPackTile <= end; t0 += kPackTile, parity ^= 1) {
        if constexpr (!Words::kPaged) tile_words = src.at(t0);
        const uint4* p = reinterpret_cast<const uint4*>(tile_words + (uint64_t)t * kPackWords);
        uint32_t w[kPackWords / 2];
#pragma unroll
        for (int h = 0; h < kPackLoads; h++) {
            const uint4 v = load_global(p + h);
            w[4 * h + 0] = v.x;
            w[4 * h + 1] = v.y;
            w[4 * h + 2] = v.z;
            w[4 * h + 3] = v.w;
        }
        if constexpr (Words::kPaged) {
            if (t0 + 2 * kPackTile <= end) tile_words = src.at(t0 + kPackTile);
        }
        slot_base += pack_tile<kAlignedSm, kCount>(w, t0, table, nib, sm, slot_base, lds, parity,
                                                   esc, hmine);
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
            if (kCount) {
                if (2 * j < (int)valid) hist_add(hmine, (lo >> 7) & 0xFFu);
                if (2 * j + 1 < (int)valid) hist_add(hmine, (hi >> 7) & 0xFFu);
            }
        }
        if (!kCount || write) {
            ThreadWords r;
            encode_words<false>(w, table, r, nullptr);
            // words past the end have no code (the pad nibble of an odd n is
            // 0) and are no escapes
            r.count = 0;
#pragma unroll
            for (int k = 0; k < kPackWords; k++) {
                if (k >= (int)valid) {
                    r.nib[k >> 3] &= ~(0xFu << (4 * (k & 7)));
                    r.quad[k >> 2] &= ~(1u << flag_shift(k & 3));
                }
            }
#pragma unroll
            for (int j = 0; j < kPackWords / 4; j++) r.count += __popc(r.quad[j] & kFlagBits);
#pragma unroll
            for (int j = 0; j < kPackWords / 2; j++)
                if (2 * j < (int)valid) nib[i0 / 2 + j] = (uint8_t)byte_at(r.nib, j);
#pragma unroll
            for (int k = 0; k < kPackWords; k++)
                if (k < (int)valid) sm[i0 + k] = (uint8_t)byte_at(r.sm, k);
            slot_base += write_escapes(r, w, t0, slot_base, lds, parity, esc);
        }
        parity ^= 1;
    }
    return slot_base - first_slot;
}

// One workgroup per chunk.
template <bool kAlignedSm, class Words, PackRole kRole>
__global__ __launch_bounds__(kPackThreads) SZ_EIGHT_WAVE_SGPR_CAP
__attribute__((amdgpu_waves_per_eu(8))) void k_pack(
    Words src, uint64_t n, uint32_t chunk_log2, const uint64_t* __restrict__ chunk_base,
    uint8_t* __restrict__ dst, uint64_t dst_capacity, uint32_t* __restrict__ counts,
    uint64_t* __restrict__ totals, uint32_t* __restrict__ chunk_esc,
    SampleArea* __restrict__ area, uint64_t spec_cap, uint64_t scratch_pos,
    uint64_t scratch_exp, uint64_t* d_size) {
    constexpr bool kFirst = kRole == PackRole::kFirst;
    constexpr bool kRanked = kRole == PackRole::kRanked;
    __shared__ PackLds lds;
    __shared__ uint32_t hist[kFirst ? kSpecCopies * kSpecPitch : 1];
    __shared__ std::conditional_t<kRanked, RankedLds, char> ranked;
    if constexpr (kRanked && Words::kBlocks) {
        // this pass writes the block's size: 0 for a block it cannot read
        d_size = src.sizes + blockIdx.y;
        if (src.invalid()) {  // the same for every thread
            if (blockIdx.x == 0 && threadIdx.x == 0) *d_size = 0;
            return;
        }
    }
    if (src.invalid()) return;  // the same for every thread
    if constexpr (Words::kBlocks) {
        const uint64_t off = block_ws(src);
        chunk_base = byte_offset(chunk_base, off);
        counts = byte_offset(counts, off);
        totals = byte_offset(totals, off);
        chunk_esc = byte_offset(chunk_esc, off);
        area = byte_offset(area, off);
        dst = byte_offset(dst, block_pitch(src));
    }

    const int t = threadIdx.x;
    const uint32_t chunk = blockIdx.x;
    const uint64_t begin = (uint64_t)chunk << chunk_log2;
    const uint64_t end = min_u64(begin + (uint64_t{1} << chunk_log2), n);

    bool write = true;
    uint32_t* hmine = nullptr;
    EscapeOut esc;
    uint64_t slot_base;
    if (kFirst) {
        // the provisional code table the sample pass left; the streams are
        // written only when the sample predicts few escapes, otherwise this
        // pass only counts and the finish pass packs
        if (t < 256) {
            const uint8_t c = area->lut[t];
            lds.code[t] = c < 16 ? (uint16_t)c : kEscapeEntry;
        }
        write = area->spec_on != 0;
        for (int i = t; i < kSpecCopies * kSpecPitch; i += kPackThreads) hist[i] = 0;
        hmine = hist + (t % kSpecCopies) * kSpecPitch;
        // this chunk's scratch slots
        esc.pos = dst + scratch_pos + 4 * (uint64_t)chunk * spec_cap;
        esc.exp = dst + scratch_exp + (uint64_t)chunk * spec_cap;
        esc.limit = spec_cap;
        esc.pos_aligned = true;
        slot_base = 0;
    } else if constexpr (kRanked) {
        uint64_t E;
        slot_base = ranked_codebook(counts, n, chunk_log2, gridDim.x, chunk, ranked, E);
        if (chunk == 0) {
            // the header, as the codebook pass writes it (n < 2^32: every
            // seg_end entry is E)
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
                *reinterpret_cast<uint64_t*>(dst + 32 + 8 * t) = E;
                dst[kHeaderBytes + t] = (uint8_t)ranked.codebook[t];
            }
        }
        code_table(ranked.codebook, lds);
        esc = escape_slots(dst, n, dst_capacity, E);
    } else {
        exact_code_table(dst, lds);
        esc = final_slots(dst, n, dst_capacity);
        slot_base = chunk_base[chunk];
    }
    __syncthreads();

    int parity = 0;
    const uint64_t escapes = pack_range<kAlignedSm, kFirst>(src.resolve(), n, begin, end, dst, esc,
                                                            slot_base, write, hmine, lds, parity);
    if (kFirst) {
        __syncthreads();
        // the chunk's exact counts: when the streams were written (the
        // finish then rarely needs them), chunk-major, its 256 counts in one
        // coalesced store (bin-major they are 256 words on 256 lines shared
        // with other chunks' workgroups: 5-6 us of the 1 GiB pass); when the
        // pass only counted, bin-major as the histogram pass lays them, so
        // that the finish, which then needs every chunk's escape count,
        // reads a codebook row of them with one coalesced load
        for (int b = t; b < 256; b += kPackThreads) {
            uint32_t s = 0;
#pragma unroll
            for (int c = 0; c < kSpecCopies; c++) s += hist[c * kSpecPitch + b];
            counts[write ? (uint64_t)chunk * 256 + b : (uint64_t)b * gridDim.x + chunk] = s;
            // and into the whole input's counts (nothing waits for the add:
            // the finish pass, a later launch, reads the sums)
            __hip_atomic_fetch_add(totals + (chunk % kTotalCopies) * 256 + b, (uint64_t)s,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (t == 0) chunk_esc[chunk] = (uint32_t)min_u64(escapes, ~0u);
        // more escapes than scratch slots: the finish pass must pack again
        if (t == 0 && write && escapes > spec_cap) atomicOr(&area->overflow, 1u);
    }
}

// Workgroups of the finish pass: two per CU of MI355X.
constexpr uint32_t kFinishGroups = 512;
// Escape records a finish thread moves per round of loads.
constexpr int kFinishBatch = 4;
constexpr uint32_t kFinishChunks = kMaxChunks / kFinishGroups;  // chunks per workgroup, at most
static_assert(kFinishChunks * kFinishGroups == kMaxChunks, "whole chunks per finish workgroup");
static_assert(kPackThreads == kSelectThreads, "the finish pass ranks and scans as the codebook pass");

// The finish pass of the single-read encode; it also takes the exact
// codebook, with no pass of its own.  Every workgroup sums the whole input's
// counts that the first pass added up, ranks the 256 exponents by the
// codebook rule, and scans the chunks' escape counts -- the first pass's own
// when it wrote the streams, no chunk outgrew its scratch slots and the
// exact codebook holds the same 16 exponents as the provisional one (the
// same escapes then); otherwise chunk length minus the chunk's counts of the
// 16 codebook exponents -- so that it knows the codebook, E and the first
// escape slot of each of its chunks without waiting for another workgroup.
// Workgroup 0 writes header, seg_end, codebook and *d_size, and puts the
// sample pass's tickets and counts back to zero.  Then, the same decision in
// every workgroup:
//  - same 16 exponents, streams written, no overflow: the streams stand.
//    The escape records of the workgroup's chunks (chunk b, b + gridDim.x,
//    ...) move from their scratch slots to their final slots in one sweep;
//    when the order differs too, each chunk's 4-bit codes are rewritten
//    (provisional code -> exact code, both nibbles of a byte at once) and
//    the codes of its escaped words and of an odd n's pad nibble set back
//    to 0;
//  - otherwise the workgroup packs its chunks again from the input.
template <bool kAlignedSm, class Words>
__global__ __launch_bounds__(kPackThreads) SZ_EIGHT_WAVE_SGPR_CAP
__attribute__((amdgpu_waves_per_eu(8))) void k_finish(
    Words src, uint64_t n, uint32_t chunk_log2, uint32_t chunks,
    const uint32_t* __restrict__ counts, const uint64_t* __restrict__ totals,
    const uint32_t* __restrict__ chunk_esc, uint8_t* __restrict__ dst, uint64_t dst_capacity,
    SampleArea* __restrict__ area, uint64_t spec_cap, uint64_t scratch_pos, uint64_t scratch_exp,
    uint64_t* d_size) {
    __shared__ PackLds lds;
    __shared__ uint8_t remap[256];  // provisional code pair -> exact code pair
    __shared__ alignas(16) uint64_t key[256];
    __shared__ RankLds<uint64_t> rank_lds;
    __shared__ uint32_t codebook[16];
    __shared__ uint64_t wave_sum[kSelectWaves];
    __shared__ uint64_t wave_off[kSelectWaves];
    __shared__ uint64_t my_first[kFinishChunks];  // this workgroup's chunks' first slots
    __shared__ uint32_t my_count[kFinishChunks];  // and record counts (copy case)
    __shared__ uint32_t mismatch;
    __shared__ uint32_t reranked;  // the provisional codebook failed its check
    if constexpr (Words::kBlocks) {
        const uint64_t off = block_ws(src);
        counts = byte_offset(counts, off);
        totals = byte_offset(totals, off);
        chunk_esc = byte_offset(chunk_esc, off);
        area = byte_offset(area, off);
        dst = byte_offset(dst, block_pitch(src));
        d_size = src.sizes + blockIdx.y;
        if (src.invalid()) {  // the same for every thread
            if (blockIdx.x == 0 && threadIdx.x == 0) *d_size = 0;
            return;
        }
    }
    if (src.invalid()) return;  // the same for every thread
    const int t = threadIdx.x;

    // every load the decision needs, issued at once: the provisional
    // codebook, the first pass's flags, the whole input's counts, and the
    // first pass's escape counts of chunks per * t .. per * t + per - 1
    // (every chunk's entry is written by the first pass, so they are read
    // before it is known whether they count)
    const uint4 prov = *reinterpret_cast<const uint4*>(area->cb);
    const uint32_t spec_on = area->spec_on, overflow = area->overflow;
    const uint32_t per = (chunks + kPackThreads - 1) / kPackThreads;  // <= kSelectChunks
    uint64_t esc[kSelectChunks] = {};
    if (per == 4 && chunks % 4 == 0) {
        if (4 * (uint32_t)t < chunks) {
            const uint4 v = *reinterpret_cast<const uint4*>(chunk_esc + 4 * t);
            esc[0] = v.x;
            esc[1] = v.y;
            esc[2] = v.z;
            esc[3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kSelectChunks; j++) {
            const uint32_t b = per * t + j;
            if ((uint32_t)j < per && b < chunks) esc[j] = chunk_esc[b];
        }
    }
    if (t < 256) {
        uint64_t c = 0;
#pragma unroll
        for (int k = 0; k < (int)kTotalCopies; k++) c += totals[k * 256 + t];
        key[t] = (c << 8) | (255u - (uint32_t)t);
    }
    if (t == 0) {
        mismatch = 0;
        reranked = 0;
    }
    __syncthreads();
    // The provisional codebook is the exact one when its 16 keys descend and
    // every other exponent's key lies below its last (the keys are
    // distinct): two keys a thread to compare instead of a ranking of all
    // 256, which runs only when this check fails.
    const uint32_t pw[4] = {prov.x, prov.y, prov.z, prov.w};
    {
        bool bad = false;
        if (t < 15) {
            bad = key[byte_at(pw, t)] <= key[byte_at(pw, t + 1)];
        } else if (t >= 256 && t < 512) {
            const uint32_t e = t - 256;
            bool found = false;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t v = pw[k] ^ (0x01010101u * e);
                found |= ((v - 0x01010101u) & ~v & 0x80808080u) != 0;
            }
            bad = !found && key[e] > key[byte_at(pw, 15)];
        }
        if (bad) reranked = 1;
    }
    __syncthreads();
    if (reranked == 0) {
        if (t < 16) codebook[t] = byte_at(pw, t);
    } else {
        const uint32_t r = top16_ranks(key, rank_lds);
        if (t < 256 && r < 16) codebook[r] = (uint32_t)t;
    }
    __syncthreads();
    // the same set: every exact codebook entry is one of the 16 provisional
    // ones (a byte of prov equal to it: a zero byte of prov ^ 0x01010101 * e);
    // the same order: entry t is provisional entry t.  Misses are or-ed into
    // mismatch: bit 0 another set, bit 1 another order.
    if (t < 16) {
        const uint32_t e = codebook[t];
        const uint32_t word = t < 4 ? prov.x : t < 8 ? prov.y : t < 12 ? prov.z : prov.w;
        const bool in_place = ((word >> (8 * (t & 3))) & 0xFFu) == e;
        const uint32_t v[4] = {prov.x ^ (0x01010101u * e), prov.y ^ (0x01010101u * e),
                               prov.z ^ (0x01010101u * e), prov.w ^ (0x01010101u * e)};
        bool found = false;
#pragma unroll
        for (int k = 0; k < 4; k++) found |= ((v[k] - 0x01010101u) & ~v[k] & 0x80808080u) != 0;
        const uint32_t miss = (found ? 0u : 1u) | (in_place ? 0u : 2u);
        if (miss) atomicOr(&mismatch, miss);
    }
    __syncthreads();
    const bool same_order = (mismatch & 2u) == 0;
    const bool keep = spec_on != 0 && overflow == 0 && (mismatch & 1u) == 0;
    if (!keep) {
        // the first pass left chunk-major counts when it wrote the streams,
        // bin-major when it only counted
        if (spec_on)
            exact_chunk_escapes_chunk_major(counts, chunks, chunk_log2, n, codebook, esc);
        else
            exact_chunk_escapes_narrow(counts, chunks, chunk_log2, n, codebook, esc);
    }
    uint64_t E;
    uint64_t excl = scan_chunk_escapes(esc, wave_sum, wave_off, E);
    const uint32_t seg_shift = 32 - chunk_log2;  // chunks per 2^32 elements: 2^seg_shift
#pragma unroll
    for (int j = 0; j < kSelectChunks; j++) {
        const uint32_t b = per * t + j;
        if ((uint32_t)j < per && b < chunks) {
            if (b % gridDim.x == blockIdx.x) {
                my_first[b / gridDim.x] = excl;
                my_count[b / gridDim.x] = (uint32_t)min_u64(esc[j], spec_cap);
            }
            // seg_end[k]: escapes below element (k + 1) * 2^32, a chunk boundary
            const uint32_t k = (b >> seg_shift) - 1;
            if (blockIdx.x == 0 && b != 0 && (b & ((1u << seg_shift) - 1)) == 0 && k < 16)
                *reinterpret_cast<uint64_t*>(dst + 32 + 8 * k) = excl;
        }
        excl += esc[j];
    }
    const uint64_t total = kPrefixBytes + (n + 1) / 2 + n + 5 * E;
    if (blockIdx.x == 0) {
        if (t == 0) {
            *reinterpret_cast<uint32_t*>(dst + 0) = kMagic;
            *reinterpret_cast<uint16_t*>(dst + 4) = kVersion;
            *reinterpret_cast<uint16_t*>(dst + 6) = kElementBf16;
            *reinterpret_cast<uint64_t*>(dst + 8) = n;
            *reinterpret_cast<uint64_t*>(dst + 16) = E;
            *reinterpret_cast<uint64_t*>(dst + 24) = total;
            if (d_size) *d_size = total;
            area->tickets = 0;
        }
        if (t < 16) {
            if (((uint64_t)(t + 1) << seg_shift) >= chunks)
                *reinterpret_cast<uint64_t*>(dst + 32 + 8 * t) = E;
            dst[kHeaderBytes + t] = (uint8_t)codebook[t];
        }
        if (t < 256) area->sample_hist[t] = 0;
    }
    __syncthreads();
    const EscapeOut esc_out = escape_slots(dst, n, dst_capacity, E);
    const uint32_t mine = (chunks - blockIdx.x + gridDim.x - 1) / gridDim.x;  // <= kFinishChunks

    if (keep) {
        // the records of this workgroup's chunks move in one sweep,
        // consecutive threads on consecutive records of a chunk, and
        // kFinishBatch records a thread per round, all loaded before any is
        // stored (one memory round trip a round)
        const uint32_t* spos = reinterpret_cast<const uint32_t*>(dst + scratch_pos);
        const uint8_t* sexp = dst + scratch_exp;
        uint32_t count = 0;
        for (uint32_t j = 0; j < mine; j++) count += my_count[j];
        for (uint32_t r0 = 0; r0 < count; r0 += kFinishBatch * kPackThreads) {
            uint32_t pos[kFinishBatch], ex[kFinishBatch];
            uint64_t slot[kFinishBatch];
#pragma unroll
            for (int k = 0; k < kFinishBatch; k++) {
                const uint32_t r = r0 + t + k * kPackThreads;
                slot[k] = ~uint64_t{0};
                if (r < count) {
                    uint32_t j = 0, q = r;
                    while (q >= my_count[j]) q -= my_count[j++];
                    const uint64_t from = (uint64_t)(blockIdx.x + j * gridDim.x) * spec_cap + q;
                    pos[k] = spos[from];
                    ex[k] = sexp[from];
                    slot[k] = my_first[j] + q;
                }
            }
#pragma unroll
            for (int k = 0; k < kFinishBatch; k++)
                if (slot[k] != ~uint64_t{0}) put_escape(esc_out, slot[k], pos[k], ex[k]);
        }
        if (same_order) return;

        uint8_t* lut = lds.lut;
        code_table(codebook, lds);
        __syncthreads();
        if (t < 256)
            remap[t] = (uint8_t)((lut[area->cb[t & 15]] & 0xF) |
                                 ((lut[area->cb[t >> 4]] & 0xF) << 4));
        __syncthreads();
        uint8_t* nib = dst + kPrefixBytes;
        for (uint32_t c = blockIdx.x; c < chunks; c += gridDim.x) {
            const uint64_t begin = (uint64_t)c << chunk_log2;
            const uint64_t end = min_u64(begin + (uint64_t{1} << chunk_log2), n);
            const uint64_t b0 = begin / 2, b1 = (end + 1) / 2;  // the chunk's nibble bytes
            for (uint64_t b = b0 + (uint64_t)t * 16; b < b1; b += (uint64_t)kPackThreads * 16) {
                if (b + 16 <= b1) {
                    const uint4 v = *reinterpret_cast<const uint4*>(nib + b);
                    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const uint32_t x = w[j];
                        w[j] = (uint32_t)remap[x & 0xFF] | ((uint32_t)remap[(x >> 8) & 0xFF] << 8) |
                               ((uint32_t)remap[(x >> 16) & 0xFF] << 16) |
                               ((uint32_t)remap[x >> 24] << 24);
                    }
                    *reinterpret_cast<uint4*>(nib + b) = make_uint4(w[0], w[1], w[2], w[3]);
                } else {
                    for (uint64_t k = b; k < b1; k++) nib[k] = remap[nib[k]];
                }
            }
            __syncthreads();
            // escaped words keep code 0: one thread per byte, the one of the
            // byte's first record
            const uint64_t cnt = my_count[(c - blockIdx.x) / gridDim.x];
            const uint32_t* cpos = spos + (uint64_t)c * spec_cap;
            const uint64_t seg = begin & ~uint64_t{0xFFFFFFFF};  // a chunk lies in one segment
            for (uint64_t q = t; q < cnt; q += kPackThreads) {
                const uint64_t p = seg | cpos[q];
                if (q > 0 && (seg | cpos[q - 1]) / 2 == p / 2) continue;
                uint32_t clear = (p & 1) ? 0xF0u : 0x0Fu;
                if (q + 1 < cnt && (seg | cpos[q + 1]) / 2 == p / 2) clear = 0xFFu;
                nib[p / 2] &= (uint8_t)~clear;
            }
            __syncthreads();
            // and so does the pad nibble of an odd n
            if (t == 0 && end == n && (n & 1)) nib[n / 2] &= 0x0F;
        }
        return;
    }

    code_table(codebook, lds);
    __syncthreads();
    const auto words = src.resolve();
    int parity = 0;
    for (uint32_t c = blockIdx.x, j = 0; c < chunks; c += gridDim.x, j++) {
        const uint64_t begin = (uint64_t)c << chunk_log2;
        const uint64_t end = min_u64(begin + (uint64_t{1} << chunk_log2), n);
        pack_range<kAlignedSm, false>(words, n, begin, end, dst, esc_out, my_first[j], true, nullptr,
                                      lds, parity);
    }
}

template <class Words, PackRole kRole>
hipError_t launch_pack_role(Words src, const EncodePlan& p, const uint8_t* ws, uint8_t* dst,
                            uint64_t dst_capacity, uint64_t* d_size, hipStream_t stream) {
    if (p.chunks == 0) return hipSuccess;
    const uint64_t* base = reinterpret_cast<const uint64_t*>(ws + p.base_off);
    uint32_t* counts = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(ws) + p.counts_off);
    SampleArea* area = reinterpret_cast<SampleArea*>(const_cast<uint8_t*>(ws) + p.sample_off);
    uint64_t* totals = reinterpret_cast<uint64_t*>(const_cast<uint8_t*>(ws) + p.totals_off);
    uint32_t* chunk_esc = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(ws) + p.esc_off);
    // the sign|mantissa stream starts at 176 + ceil(n/2): 16-byte aligned
    // exactly when n is a multiple of 32
    const bool aligned = ((kPrefixBytes + (p.n + 1) / 2) & 15) == 0;
    if (aligned)
        k_pack<true, Words, kRole><<<dim3(p.chunks, grid_blocks(src)), kPackThreads, 0, stream>>>(
            src, p.n, p.chunk_log2, base, dst, dst_capacity, counts, totals, chunk_esc, area,
            p.spec_cap, p.scratch_pos, p.scratch_exp, d_size);
    else
        k_pack<false, Words, kRole><<<dim3(p.chunks, grid_blocks(src)), kPackThreads, 0, stream>>>(
            src, p.n, p.chunk_log2, base, dst, dst_capacity, counts, totals, chunk_esc, area,
            p.spec_cap, p.scratch_pos, p.scratch_exp, d_size);
    return hipGetLastError();
}

template <class Words>
hipError_t launch_pack(Words src, const EncodePlan& p, const uint8_t* ws, uint8_t* dst,
                       uint64_t dst_capacity, int /*num_cus*/, hipStream_t stream) {
    return launch_pack_role<Words, PackRole::kClassic>(src, p, ws, dst, dst_capacity, nullptr,
                                                       stream);
}

template <class Words>
hipError_t launch_pack_ranked(Words src, const EncodePlan& p, const uint8_t* ws, uint8_t* dst,
                              uint64_t dst_capacity, uint64_t* d_size, hipStream_t stream) {
    if (p.chunks == 0 || p.chunks > kRankedChunks) return hipErrorInvalidValue;
    return launch_pack_role<Words, PackRole::kRanked>(src, p, ws, dst, dst_capacity, d_size,
                                                      stream);
}

template <class Words>
hipError_t launch_first_pass(Words src, const EncodePlan& p, uint8_t* ws, uint8_t* dst,
                             uint64_t dst_capacity, hipStream_t stream) {
    return launch_pack_role<Words, PackRole::kFirst>(src, p, ws, dst, dst_capacity, nullptr,
                                                     stream);
}

template <class Words>
hipError_t launch_finish(Words src, const EncodePlan& p, uint8_t* ws, uint8_t* dst,
                         uint64_t dst_capacity, uint64_t* d_size, hipStream_t stream) {
    if (p.chunks == 0) return hipSuccess;
    const uint32_t* counts = reinterpret_cast<const uint32_t*>(ws + p.counts_off);
    const uint64_t* totals = reinterpret_cast<const uint64_t*>(ws + p.totals_off);
    const uint32_t* chunk_esc = reinterpret_cast<const uint32_t*>(ws + p.esc_off);
    SampleArea* area = reinterpret_cast<SampleArea*>(ws + p.sample_off);
    // up to kFinishGroups workgroups per tensor or block: for blocks, one per
    // chunk of each (fewer, with several chunks each, leave a block that has
    // to be packed again to too few workgroups: 32 blocks of 2^24 words
    // with 16 workgroups each took 203 us for this pass, against about 120
    // with one per chunk)
    const dim3 grid(p.chunks < kFinishGroups ? p.chunks : kFinishGroups, grid_blocks(src));
    const bool aligned = ((kPrefixBytes + (p.n + 1) / 2) & 15) == 0;
    if (aligned)
        k_finish<true, Words><<<grid, kPackThreads, 0, stream>>>(
            src, p.n, p.chunk_log2, p.chunks, counts, totals, chunk_esc, dst, dst_capacity, area,
            p.spec_cap, p.scratch_pos, p.scratch_exp, d_size);
    else
        k_finish<false, Words><<<grid, kPackThreads, 0, stream>>>(
            src, p.n, p.chunk_log2, p.chunks, counts, totals, chunk_esc, dst, dst_capacity, area,
            p.spec_cap, p.scratch_pos, p.scratch_exp, d_size);
    return hipGetLastError();
}

// ---------------------------------------------------------------- sample

// 512 blocks of 2048 consecutive words, evenly spread over the input (block
// j starts at the 2048-word boundary at or below j * n / 512): whole blocks,
// so that a layout with a short period (a KV cache's heads x dims) is
// sampled evenly.  Eight blocks per 1024-thread workgroup.
constexpr uint32_t kSampleBlocks = 512;
constexpr uint32_t kSampleBlockWords = 2048;
constexpr uint32_t kSampleThreads = 1024;
constexpr uint32_t kSampleBlocksPerGroup = kSampleBlocks / kSampleGroups;
constexpr uint32_t kSampleLoads = kSampleBlocksPerGroup * kSampleBlockWords / 8 / kSampleThreads;
static_assert(kSampleBlocks % kSampleGroups == 0, "whole blocks per workgroup");
static_assert(kSingleReadMin / kSampleBlocks >= kSampleBlockWords, "blocks do not overlap");
static_assert(kSampleThreads == 1024, "four groups of 256 threads rank the exponents");
static_assert((kSampleGroups & (kSampleGroups - 1)) == 0, "tickets wrap at a multiple of a run");
// Per-layer blocks are sampled in proportion to their length: one
// workgroup (8 runs of 2048 words) per 2^19 words of a block, a power of two
// from 4 to 32, so about 1/32 of every block (a fixed 32 runs made 1/256 of
// a 2^24-word block, whose finish then rewrote the codes of 13 of 32 blocks
// and packed one again; 256 runs, 6 and none).
constexpr uint32_t kBlockSampleGroups = 4;
constexpr uint32_t kBlockSampleGroupsMax = 32;
static_assert((kBlockSampleGroups & (kBlockSampleGroups - 1)) == 0, "tickets wrap at a multiple of a run");
static_assert(kSingleReadMin / (kBlockSampleGroups * kSampleBlocksPerGroup) >= kSampleBlockWords,
              "blocks do not overlap");

template <class Words>
uint32_t sample_groups(uint64_t n) {
    if constexpr (!Words::kBlocks) {
        return kSampleGroups;
    } else {
        // groups * 2^19 <= n keeps the runs apart: n / (groups * 8) >= 2^16
        uint32_t g = kBlockSampleGroups;
        while (g < kBlockSampleGroupsMax && (uint64_t{2} * g << 19) <= n) g *= 2;
        return g;
    }
}

// The sample pass, one launch.  Each workgroup counts its blocks, adds the
// counts into area->sample_hist (device-wide atomics whose returned values
// a barrier waits for) and then takes a ticket.  Tickets count on from run
// to run, a run being the launch's workgroups per tensor or block (a power of
// two; each block on its own area), so the workgroup whose ticket completes a
// multiple of the run arrives last; the codebook pass puts tickets and
// counts back to zero, so a workspace that came in with other values is in
// step from its second encode on (until then the provisional codebook may
// be ranked from part of the sample: a slower finish, never another
// container).  The last workgroup reads the totals back, zeroing them, and
// ranks the 256 exponents by the codebook rule (count descending, exponent
// ascending); it leaves the provisional code table and decides whether the
// first pass packs (at most one escape in 32 sampled words).  Workgroup 0
// first clears what the later passes count up from zero (the first pass's
// counts and overflow flag, the codebook pass's counts and workgroups
// done), off the last workgroup's path.
template <class Words>
__global__ __launch_bounds__(kSampleThreads) void k_sample(Words src, uint64_t n,
                                                           SampleArea* __restrict__ area,
                                                           uint64_t* __restrict__ hist,
                                                           uint64_t* __restrict__ totals) {
    const uint32_t kGroups = gridDim.x;  // a power of two
    constexpr uint32_t kBlocksPerGroup = kSampleBlocksPerGroup;
    constexpr uint32_t kLoadsPerBlock = kSampleBlockWords / 8;
    __shared__ uint32_t h[kSpecCopies * kSpecPitch];
    __shared__ RankLds<uint32_t> rank_lds;
    __shared__ alignas(16) uint32_t key[256];
    __shared__ uint32_t sums[2][4];
    __shared__ uint32_t last;
    if constexpr (Words::kBlocks) {
        const uint64_t off = block_ws(src);
        area = byte_offset(area, off);
        hist = byte_offset(hist, off);
        totals = byte_offset(totals, off);
    }
    if (src.invalid()) return;
    const int t = threadIdx.x;
    if (blockIdx.x == 0) {
        // what the later passes count up from zero: the codebook pass's
        // whole-input counts and arrivals, the first pass's counts and its
        // overflow flag
        if (t < 256) hist[t] = 0;
        for (uint32_t i = t; i < kTotalCopies * 256; i += kSampleThreads) totals[i] = 0;
        if (t == 0) {
            area->overflow = 0;
            area->arrivals = 0;
        }
    }
    for (int i = t; i < kSpecCopies * kSpecPitch; i += kSampleThreads) h[i] = 0;
    __syncthreads();
    uint32_t* mine = h + (t % kSpecCopies) * kSpecPitch;
    const uint64_t spacing = n / (kGroups * kBlocksPerGroup);
    const auto words = src.resolve();
#pragma unroll
    for (uint32_t k = 0; k < kSampleLoads; k++) {
        const uint32_t g = t + k * kSampleThreads;  // 16-byte group in this workgroup's share
        const uint64_t block = (uint64_t)blockIdx.x * kBlocksPerGroup + g / kLoadsPerBlock;
        const uint64_t start = block * spacing / kSampleBlockWords * kSampleBlockWords;
        const uint64_t word = start + (uint64_t)(g % kLoadsPerBlock) * 8;
        // a block lies inside one page
        hist_uint4(mine, load_global(reinterpret_cast<const uint4*>(words.at(word))));
    }
    __syncthreads();
    uint32_t before = 0;
    if (t < 256) {
        uint32_t s = 0;
#pragma unroll
        for (int c = 0; c < kSpecCopies; c++) s += h[c * kSpecPitch + t];
        before = __hip_atomic_fetch_add(area->sample_hist + t, s, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    }
    // every add has returned before the ticket is taken: the empty asm reads
    // the returned value, so the wave waits for it ahead of the barrier
    asm volatile("" ::"v"(before));
    __syncthreads();
    if (t == 0) {
        const uint32_t ticket = __hip_atomic_fetch_add(&area->tickets, 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        last = (ticket + 1) % kGroups == 0 ? 1u : 0u;
    }
    __syncthreads();
    if (!last) return;

    uint32_t c = 0;
    if (t < 256) {
        c = __hip_atomic_exchange(area->sample_hist + t, 0u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        // 32-bit keys: a sample count is below 2^24 (a workspace that came
        // in with other counts is clamped there; the keys stay distinct)
        key[t] = (min(c, (1u << 24) - 1) << 8) | (255u - (uint32_t)t);
    }
    __syncthreads();
    const uint32_t r = top16_ranks(key, rank_lds);
    if (t < 256) {
        area->lut[t] = r < 16 ? (uint8_t)r : (uint8_t)0x10;
        if (r < 16) area->cb[r] = (uint8_t)t;
        const uint32_t all = wave_sum_u32(c), top = wave_sum_u32(r < 16 ? c : 0u);
        if ((t & 63) == 0) {
            sums[0][t >> 6] = all;
            sums[1][t >> 6] = top;
        }
    }
    __syncthreads();
    if (t == 0) {
        const uint32_t all = sums[0][0] + sums[0][1] + sums[0][2] + sums[0][3];
        const uint32_t top = sums[1][0] + sums[1][1] + sums[1][2] + sums[1][3];
        area->spec_on = all > 0 && (uint64_t)(all - top) * 32 <= all ? 1u : 0u;
    }
}

template <class Words>
hipError_t launch_sample(Words src, const EncodePlan& p, uint8_t* ws, hipStream_t stream) {
    SampleArea* area = reinterpret_cast<SampleArea*>(ws + p.sample_off);
    k_sample<Words><<<dim3(sample_groups<Words>(p.n), grid_blocks(src)), kSampleThreads, 0, stream>>>(
        src, p.n, area, reinterpret_cast<uint64_t*>(ws + p.hist_off),
        reinterpret_cast<uint64_t*>(ws + p.totals_off));
    return hipGetLastError();
}

#define SZ_ENCODE_INSTANCES(W)                                                                  \
    template hipError_t launch_pack<W>(W, const EncodePlan&, const uint8_t*, uint8_t*,          \
                                       uint64_t, int, hipStream_t);                             \
    template hipError_t launch_first_pass<W>(W, const EncodePlan&, uint8_t*, uint8_t*,          \
                                             uint64_t, hipStream_t);                            \
    template hipError_t launch_finish<W>(W, const EncodePlan&, uint8_t*, uint8_t*, uint64_t,     \
                                         uint64_t*, hipStream_t);                               \
    template hipError_t launch_sample<W>(W, const EncodePlan&, uint8_t*, hipStream_t);
SZ_ENCODE_INSTANCES(FlatWords)
SZ_ENCODE_INSTANCES(PagedWords)
SZ_ENCODE_INSTANCES(BlockWords)
#undef SZ_ENCODE_INSTANCES
template hipError_t launch_pack_ranked<FlatWords>(FlatWords, const EncodePlan&, const uint8_t*,
                                                  uint8_t*, uint64_t, uint64_t*, hipStream_t);
template hipError_t launch_pack_ranked<PagedWords>(PagedWords, const EncodePlan&, const uint8_t*,
                                                   uint8_t*, uint64_t, uint64_t*, hipStream_t);
template hipError_t launch_pack_ranked<BlockWords>(BlockWords, const EncodePlan&, const uint8_t*,
                                                   uint8_t*, uint64_t, uint64_t*, hipStream_t);

}  // namespace sz
