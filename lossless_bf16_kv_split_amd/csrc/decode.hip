// decode.hip -- the two decode passes of the SplitZip BF16 codec on gfx950.
//
//   unpack   stream 16 codes (8 bytes) and 16 sign|mantissa bytes per thread
//            step into 16 BF16 words (32 bytes); the codebook lives in four
//            registers; block 0 also checks the header
//   scatter  one thread per escape record: rebuild its word with the stored
//            exponent, after checking the position is in range and above
//            the previous one
//
// Method: SplitZip explainers (gist.science, arXiv 2605.01708), section
// "4. Pourquoi est-ce rapide ?", decoding bullet: look the 4-bit code up,
// put the exponent back next to sign and mantissa, and overwrite the slot of
// every escape note; linear work with no detours.
#include "sz_internal.h"

#include <type_traits>

namespace sz {

constexpr int kUnpackThreads = 256;
constexpr int kScatterThreads = 256;
constexpr uint64_t kMaxDecodeRanges = 8192;  // workgroups of a single-pass decode
constexpr int32_t kStatusInvalid = 1;   // SZ_ERR_INVALID_ARGUMENT: a bad page table
constexpr int32_t kStatusCorrupt = 4;

// v_perm_b32: byte i of the result is byte sel[i] of the 8-byte value
// {hi (bytes 4..7), lo (bytes 0..3)}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// bitwise select: bits of a where m is set, bits of b elsewhere (v_bfi_b32)
__device__ __forceinline__ uint32_t bitselect(uint32_t m, uint32_t a, uint32_t b) {
    return (m & a) | (~m & b);
}

// Four 4-bit codes, one per byte of x, to their four exponent bytes; the
// 16-byte codebook sits in four registers cb0..cb3.  Codes 0..7 come from
// cb0:cb1, codes 8..15 from cb2:cb3, chosen per byte by bit 3 of the code.
__device__ __forceinline__ uint32_t lookup4(uint32_t x, uint4 cb) {
    const uint32_t sel = x & 0x07070707u;
    const uint32_t lo = perm(cb.y, cb.x, sel);
    const uint32_t hi = perm(cb.w, cb.z, sel);
    const uint32_t bit3 = (x >> 3) & 0x01010101u;
    return bitselect((bit3 << 8) - bit3, hi, lo);  // 0xFF in every byte with bit 3 set
}

// Exponent bytes of eight words from one dword of codes (element 2j in the
// low nibble of byte j): e0 holds elements 0..3, e1 elements 4..7.
__device__ __forceinline__ void exponents8(uint32_t codes, uint4 cb, uint32_t& e0, uint32_t& e1) {
    const uint32_t even = lookup4(codes & 0x0F0F0F0Fu, cb);         // elements 0,2,4,6
    const uint32_t odd = lookup4((codes >> 4) & 0x0F0F0F0Fu, cb);   // elements 1,3,5,7
    e0 = perm(odd, even, 0x05010400u);
    e1 = perm(odd, even, 0x07030602u);
}

// Eight words from their exponent bytes (e0, e1) and sign|mantissa bytes
// (s0 elements 0..3, s1 elements 4..7).  Per byte lane: high byte of the
// word = sign | exponent >> 1, low byte = (exponent & 1) << 7 | mantissa;
// the two byte streams are then interleaved into words.
__device__ __forceinline__ uint4 words8(uint32_t e0, uint32_t e1, uint32_t s0, uint32_t s1) {
    const uint32_t h0 = bitselect(0x80808080u, s0, e0 >> 1);
    const uint32_t l0 = bitselect(0x80808080u, e0 << 7, s0);
    const uint32_t h1 = bitselect(0x80808080u, s1, e1 >> 1);
    const uint32_t l1 = bitselect(0x80808080u, e1 << 7, s1);
    return make_uint4(perm(h0, l0, 0x05010400u), perm(h0, l0, 0x07030602u),
                      perm(h1, l1, 0x05010400u), perm(h1, l1, 0x07030602u));
}

__device__ __forceinline__ uint4 decode8(uint32_t codes, uint32_t s0, uint32_t s1, uint4 cb) {
    uint32_t e0, e1;
    exponents8(codes, cb, e0, e1);
    return words8(e0, e1, s0, s1);
}

// one word, for the last n % 8 elements
__device__ __forceinline__ uint32_t recombine(uint32_t sm, uint32_t e) {
    return ((sm & 0x80u) << 8) | (e << 7) | (sm & 0x7Fu);
}

__device__ __forceinline__ uint32_t codebook_byte(uint4 cb, uint32_t c) {
    return lookup4(c, cb) & 0xFFu;
}

__device__ __forceinline__ uint32_t load4_unaligned(const uint8_t* q) {
    return (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) |
           ((uint32_t)q[3] << 24);
}

// The header's fields against n, e and the container size.  All 160 bytes
// are loaded first (ten 16-byte loads in flight together; every container
// holds at least 176 bytes, checked on the host), then compared, so the
// check costs one memory round trip.
__device__ bool header_ok(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e) {
    uint64_t h[20];
#pragma unroll
    for (int q = 0; q < 10; q++) {
        const uint4 v = reinterpret_cast<const uint4*>(src)[q];
        h[2 * q] = ((uint64_t)v.y << 32) | v.x;
        h[2 * q + 1] = ((uint64_t)v.w << 32) | v.z;
    }
    bool ok = (uint32_t)h[0] == kMagic && (uint16_t)(h[0] >> 32) == kVersion &&
              (uint16_t)(h[0] >> 48) == kElementBf16 && h[1] == n && h[2] == e &&
              h[3] == src_bytes;
    // seg_end[s] (h[4 + s]) never decreases, and equals e from the last
    // segment holding words on
    const uint64_t segments_used = (n + 0xFFFFFFFFull) >> 32;
    uint64_t prev = 0;
#pragma unroll
    for (uint32_t sg = 0; sg < 16; sg++) {
        const uint64_t v = h[4 + sg];
        ok = ok && v >= prev && ((uint64_t)sg + 1 < segments_used || v == e);
        prev = v;
    }
    return ok;
}

template <bool kAlignedSm, class Words>
__global__ __launch_bounds__(kUnpackThreads) void k_unpack(const uint8_t* __restrict__ src,
                                                          uint64_t src_bytes, uint64_t n,
                                                          uint64_t e, Words out,
                                                          int32_t* status) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && status)
        *status = out.invalid() ? kStatusInvalid
                                : (header_ok(src, src_bytes, n, e) ? 0 : kStatusCorrupt);
    if (out.invalid()) return;

    const uint4 cb = *reinterpret_cast<const uint4*>(src + kHeaderBytes);
    const uint8_t* nib = src + kPrefixBytes;
    const uint8_t* sm = nib + (n + 1) / 2;

    // 8 words per thread step: 4 code bytes + 8 sm bytes in, 16 bytes out
    const uint64_t groups = n / 8;
    const uint64_t stride = (uint64_t)gridDim.x * kUnpackThreads;
    for (uint64_t g = (uint64_t)blockIdx.x * kUnpackThreads + threadIdx.x; g < groups; g += stride) {
        const uint32_t codes = *reinterpret_cast<const uint32_t*>(nib + 4 * g);
        uint32_t s0, s1;
        if (kAlignedSm) {
            const uint2 v = *reinterpret_cast<const uint2*>(sm + 8 * g);
            s0 = v.x;
            s1 = v.y;
        } else {
            s0 = load4_unaligned(sm + 8 * g);
            s1 = load4_unaligned(sm + 8 * g + 4);
        }
        // non-temporal: the words are not kept dirty in the caches, so later
        // kernels do not pay for writing them back
        // a wave's 64 groups are 512 consecutive words: one page
        store_streaming(reinterpret_cast<uint4*>(out.at_wave(8 * g)), decode8(codes, s0, s1, cb));
    }

    // the last n % 8 words
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = groups * 8 + threadIdx.x; i < n; i += kUnpackThreads) {
            const uint32_t code = (nib[i / 2] >> (4 * (i & 1))) & 0xFu;
            *out.at(i) = (uint16_t)recombine(sm[i], codebook_byte(cb, code));
        }
    }
}

template <class Words>
hipError_t launch_unpack(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                         Words dst, int32_t* status, int num_cus, hipStream_t stream) {
    const uint64_t groups = n / 8;
    uint64_t blocks = (groups + kUnpackThreads - 1) / kUnpackThreads;
    // four workgroups per CU: measured fastest for this read 1.5 / write 2
    // byte stream (more resident waves only add DRAM page conflicts)
    const uint64_t cap = (uint64_t)(num_cus > 0 ? num_cus : 256) * 4;
    if (blocks > cap) blocks = cap;
    if (blocks == 0) blocks = 1;  // header check and tail still run
    const bool aligned = ((kPrefixBytes + (n + 1) / 2) & 7) == 0;
    if (aligned)
        k_unpack<true, Words><<<(uint32_t)blocks, kUnpackThreads, 0, stream>>>(
            src, src_bytes, n, e, dst, status);
    else
        k_unpack<false, Words><<<(uint32_t)blocks, kUnpackThreads, 0, stream>>>(
            src, src_bytes, n, e, dst, status);
    return hipGetLastError();
}

// position of escape k: segment = #{s : seg_end[s] <= k}, low 32 bits stored
__device__ __forceinline__ uint64_t escape_position(const uint64_t* seg_end, uint64_t k,
                                                    const uint8_t* pos_lo, bool aligned) {
    uint64_t seg = 0;
#pragma unroll
    for (int s = 0; s < 16; s++) seg += seg_end[s] <= k ? 1u : 0u;
    uint32_t lo;
    if (aligned) {
        lo = reinterpret_cast<const uint32_t*>(pos_lo)[k];
    } else {
        const uint8_t* q = pos_lo + 4 * k;
        lo = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) |
             ((uint32_t)q[3] << 24);
    }
    return (seg << 32) | lo;
}

template <class Words>
__global__ __launch_bounds__(kScatterThreads) void k_scatter(const uint8_t* __restrict__ src,
                                                            uint64_t n, uint64_t e, Words out,
                                                            int32_t* status) {
    const uint64_t k = (uint64_t)blockIdx.x * kScatterThreads + threadIdx.x;
    if (k >= e || out.invalid()) return;
    const uint64_t* seg_end = reinterpret_cast<const uint64_t*>(src + 32);
    const uint64_t esc_off = kPrefixBytes + (n + 1) / 2 + n;
    const uint8_t* pos_lo = src + esc_off;
    const uint8_t* exps = pos_lo + 4 * e;
    const bool aligned = (esc_off & 3) == 0;

    const uint64_t p = escape_position(seg_end, k, pos_lo, aligned);
    bool ok = p < n;
    if (k > 0) ok = ok && p > escape_position(seg_end, k - 1, pos_lo, aligned);
    if (!ok) {
        if (status)
            __hip_atomic_fetch_max(status, kStatusCorrupt, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    // the unpack pass already wrote sign and mantissa: replace the exponent
    // field in place (reading the word's own line, not the sm stream's)
    uint16_t* q = out.at(p);
    const uint32_t w = *q;
    *q = (uint16_t)((w & 0x807Fu) | ((uint32_t)exps[k] << 7));
}

template <class Words>
hipError_t launch_scatter(const uint8_t* src, uint64_t n, uint64_t e, Words dst,
                          int32_t* status, hipStream_t stream) {
    if (e == 0) return hipSuccess;
    const uint64_t blocks = (e + kScatterThreads - 1) / kScatterThreads;
    k_scatter<Words><<<(uint32_t)blocks, kScatterThreads, 0, stream>>>(src, n, e, dst, status);
    return hipGetLastError();
}

// ------------------------------------------------------------------------
// Fused decode: unpack and escape overwrite in one pass, so every word is
// written once.  One workgroup per power-of-two range of words.

constexpr int kFusedThreads = 512;
constexpr uint32_t kFusedTile = kFusedThreads * 8;   // words per workgroup step
constexpr int kBatchPerThread = 2;
static_assert(kBatchPerThread >= 1 && kBatchPerThread <= 4, "prefetched exponents share one register");
constexpr uint32_t kBatch = kFusedThreads * kBatchPerThread;  // escape records in LDS
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;

// Escape positions: low 32 bits stored, segment from the header's seg_end
// (kept in LDS; with n <= 2^32 every escape is in segment 0).
struct EscapeReader {
    const uint8_t* pos_lo;
    const uint8_t* exps;
    const uint64_t* seg_end;  // LDS copy of the header table
    bool one_segment;
    bool aligned;

    __device__ uint32_t low32(uint64_t k) const {
        return aligned ? reinterpret_cast<const uint32_t*>(pos_lo)[k]
                       : load4_unaligned(pos_lo + 4 * k);
    }

    __device__ uint64_t position(uint64_t k) const {
        uint64_t seg = 0;
        if (!one_segment) {
#pragma unroll
            for (int s = 0; s < 16; s++) seg += seg_end[s] <= k ? 1u : 0u;
        }
        return (seg << 32) | low32(k);
    }
};

// First k in [first, last] whose position is >= target (last when none
// is), for one wavefront: every step probes 64 evenly spaced records and
// keeps the bracket where the predicate turns true, so the interval shrinks
// on every step and the loop ends on any input (sorted input gives the
// exact lower bound).
__device__ uint64_t wave_lower_bound(const EscapeReader& r, uint64_t first, uint64_t last,
                                     uint64_t target) {
    const uint64_t lane = threadIdx.x & 63;
    uint64_t lo = first, hi = last;
    while (hi - lo > 64) {
        const uint64_t step = (hi - lo + 63) / 64;
        const uint64_t k = lo + lane * step;
        const bool ge = k < hi ? r.position(k) >= target : true;
        const uint64_t m = __ballot(ge);
        const uint64_t f = m ? (uint64_t)(__ffsll((long long)m) - 1) : 64;
        const uint64_t new_hi = f < 64 ? min_u64(hi, lo + f * step) : hi;
        const uint64_t new_lo = f > 0 ? lo + (f - 1) * step + 1 : lo;
        lo = new_lo;
        hi = new_hi;
    }
    const uint64_t k = lo + lane;
    const bool ge = k < hi ? r.position(k) >= target : true;
    const uint64_t m = __ballot(ge);
    return m ? min_u64(lo + (uint64_t)(__ffsll((long long)m) - 1), hi) : hi;
}

// a value every lane holds, moved to scalar registers
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// bits 0..3 of x -> bytes 0..3 set to 0xFF or 0x00
__device__ __forceinline__ uint32_t bits_to_bytes(uint32_t x) {
    const uint32_t spread = ((x & 0xFu) * 0x00204081u) & 0x01010101u;
    return (spread << 8) - spread;
}

__global__ void k_status_clear(int32_t* status) { *status = 0; }

// Eight waves per SIMD (four workgroups per CU) need at most 64 VGPRs and
// the scalar-register cap; two prefetched records per thread and no
// register prefetch of the next tile keep the kernel inside both.
template <bool kAlignedSm, class Words>
__global__ __launch_bounds__(kFusedThreads) SZ_EIGHT_WAVE_SGPR_CAP
__attribute__((amdgpu_waves_per_eu(8))) void k_decode_fused(
    const uint8_t* __restrict__ src, uint64_t src_bytes, uint64_t n, uint64_t e,
    uint32_t range_log2, Words out, int32_t* status) {
    __shared__ uint32_t batch_pos[kBatch];            // offsets from the range start
    __shared__ uint8_t batch_exp[kBatch];
    __shared__ uint8_t patch_exp[2][kFusedTile];      // exponent of each escaped word
    __shared__ uint32_t patch_bits[2][kFusedTile / 32];
    __shared__ uint64_t bounds[2];
    __shared__ uint64_t seg_table[16];
    __shared__ int bad;

    const int t = threadIdx.x;
    const int wave = t >> 6;
    if (out.invalid()) {  // the same for every thread
        if (blockIdx.x == 0 && t == 0 && status)
            __hip_atomic_fetch_max(status, kStatusInvalid, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    if (t == 0) bad = 0;
    if (blockIdx.x == 0 && t == 0 && !header_ok(src, src_bytes, n, e)) bad = 1;

    const uint4 cb = *reinterpret_cast<const uint4*>(src + kHeaderBytes);
    const uint8_t* nib = src + kPrefixBytes;
    const uint8_t* sm = nib + (n + 1) / 2;
    const uint64_t esc_off = kPrefixBytes + (n + 1) / 2 + n;
    EscapeReader rd;
    rd.pos_lo = src + esc_off;
    rd.exps = rd.pos_lo + 4 * e;
    rd.aligned = (esc_off & 3) == 0;
    rd.one_segment = n <= (1ull << 32);
    rd.seg_end = seg_table;
    if (t < 16) seg_table[t] = reinterpret_cast<const uint64_t*>(src + 32)[t];
    __syncthreads();

    const uint64_t begin = min_u64((uint64_t)blockIdx.x << range_log2, n);
    const uint64_t end = min_u64(begin + (uint64_t{1} << range_log2), n);

    // escapes of this range: [k_lo, k_hi)
    if (wave < 2) {
        const uint64_t b = wave_lower_bound(rd, 0, e, wave == 0 ? begin : end);
        if ((t & 63) == 0) bounds[wave] = b;
    }
    __syncthreads();
    const uint64_t k_lo = uniform64(bounds[0]);
    const uint64_t k_hi = uniform64(bounds[1] > k_lo ? bounds[1] : k_lo);
    if (t == 0 && blockIdx.x == gridDim.x - 1 && bounds[1] != e) bad = 1;  // positions >= n

    // batch of escape records in LDS, the next batch prefetched in registers
    uint64_t kb = k_lo;
    uint32_t cnt = (uint32_t)min_u64(kBatch, k_hi - kb);
    uint64_t next_kb = kb + cnt;
    uint32_t pre_off[kBatchPerThread];   // offset from begin, or kNoSlot
    uint32_t pre_exp = 0;                // the records' exponents, one per byte
    bool pre_first_ok = true;            // first record of the batch above its predecessor

    auto fetch = [&](uint64_t base) {
        pre_exp = 0;
#pragma unroll
        for (int i = 0; i < kBatchPerThread; i++) {
            const uint64_t k = base + (uint64_t)(t + i * kFusedThreads);
            pre_off[i] = kNoSlot;
            if (k < k_hi) {
                const uint64_t p = rd.position(k);
                if (p >= begin && p < end) pre_off[i] = (uint32_t)(p - begin);
                pre_exp |= (uint32_t)rd.exps[k] << (8 * i);
                if (i == 0 && t == 0 && k > 0) pre_first_ok = p > rd.position(k - 1);
            }
        }
    };
    // install the fetched records (batch starting at kb, cnt records), then
    // check they ascend: against the neighbour, and the first against the
    // record before the batch; a record outside the range is corrupt too
    auto install = [&]() {
#pragma unroll
        for (int i = 0; i < kBatchPerThread; i++) {
            const uint32_t q = t + i * kFusedThreads;
            if (q < cnt) {
                batch_pos[q] = pre_off[i];
                batch_exp[q] = (uint8_t)(pre_exp >> (8 * i));
                if (pre_off[i] == kNoSlot) bad = 1;
            }
        }
        if (t == 0 && cnt > 0 && !pre_first_ok) bad = 1;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kBatchPerThread; i++) {
            const uint32_t q = t + i * kFusedThreads;
            if (q > 0 && q < cnt && !(batch_pos[q] > batch_pos[q - 1])) bad = 1;
        }
    };

    fetch(kb);
    install();
    fetch(next_kb);

    // a tile's codes and sign|mantissa bytes; their loads stay in flight
    // while the tile's escapes are marked
    auto load_tile = [&](uint64_t i0, uint32_t& codes, uint32_t& s0, uint32_t& s1) {
        if (i0 + 8 <= end) {
            codes = *reinterpret_cast<const uint32_t*>(nib + i0 / 2);
            if (kAlignedSm) {
                const uint2 v = *reinterpret_cast<const uint2*>(sm + i0);
                s0 = v.x;
                s1 = v.y;
            } else {
                s0 = load4_unaligned(sm + i0);
                s1 = load4_unaligned(sm + i0 + 4);
            }
        }
    };

    int parity = 0;
    for (uint64_t t0 = begin; t0 < end; t0 += kFusedTile, parity ^= 1) {
        const uint64_t i0 = t0 + (uint64_t)t * 8;
        const bool full = i0 + 8 <= end;
        uint32_t codes = 0, s0 = 0, s1 = 0;
        load_tile(i0, codes, s0, s1);
        for (int q = t; q < (int)(kFusedTile / 32); q += kFusedThreads) patch_bits[parity][q] = 0;
        __syncthreads();

        // mark this tile's escapes; refill the batch while it ends inside the tile
        const uint32_t off0 = (uint32_t)(t0 - begin);
        while (true) {
#pragma unroll
            for (int i = 0; i < kBatchPerThread; i++) {
                const uint32_t q = t + i * kFusedThreads;
                if (q < cnt) {
                    const uint32_t d = batch_pos[q] - off0;
                    if (d < kFusedTile) {
                        patch_exp[parity][d] = batch_exp[q];
                        atomicOr(&patch_bits[parity][d >> 5], 1u << (d & 31));
                    }
                }
            }
            const bool more = kb + cnt < k_hi;
            const bool ends_here = cnt == 0 || batch_pos[cnt - 1] - off0 < kFusedTile ||
                                   batch_pos[cnt - 1] < off0;
            if (!(more && ends_here)) break;
            __syncthreads();
            kb = next_kb;
            cnt = (uint32_t)min_u64(kBatch, k_hi - kb);
            next_kb = kb + cnt;
            install();
            fetch(next_kb);
        }
        __syncthreads();

        // patch the exponents of escaped words, then rebuild the words
        const uint32_t present = (patch_bits[parity][t >> 2] >> (8 * (t & 3))) & 0xFFu;
        if (full) {
            uint32_t e0, e1;
            exponents8(codes, cb, e0, e1);
            if (present) {
                const uint2 pe = *reinterpret_cast<const uint2*>(&patch_exp[parity][8 * t]);
                e0 = bitselect(bits_to_bytes(present), pe.x, e0);
                e1 = bitselect(bits_to_bytes(present >> 4), pe.y, e1);
            }
            // a wave's words are 512 consecutive words: one page
            store_global(reinterpret_cast<uint4*>(out.at_wave(i0)), words8(e0, e1, s0, s1));
        } else {
            for (uint32_t k = 0; k < 8 && i0 + k < end; k++) {
                const uint64_t i = i0 + k;
                const uint32_t code = (nib[i / 2] >> (4 * (i & 1))) & 0xFu;
                const uint32_t ex = (present >> k) & 1u ? patch_exp[parity][8 * t + k]
                                                        : codebook_byte(cb, code);
                *out.at(i) = (uint16_t)recombine(sm[i], ex);
            }
        }
    }
    __syncthreads();
    if (t == 0 && bad && status)
        __hip_atomic_fetch_max(status, kStatusCorrupt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class Words>
hipError_t launch_decode_fused(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                               Words dst, int32_t* status, hipStream_t stream) {
    uint32_t r = 13;
    // at most kMaxDecodeRanges workgroups: enough for several waves of
    // resident workgroups (a 10.7 GB input with 2048 ranges left the last
    // wave a quarter full: 16% slower)
    while (r < 40 && ((n + (1ull << r) - 1) >> r) > kMaxDecodeRanges) r++;
    uint64_t blocks = (n + (1ull << r) - 1) >> r;
    if (blocks == 0) blocks = 1;  // the header check still runs
    if (status) k_status_clear<<<1, 1, 0, stream>>>(status);
    const bool aligned = ((kPrefixBytes + (n + 1) / 2) & 7) == 0;
    if (aligned)
        k_decode_fused<true, Words><<<(uint32_t)blocks, kFusedThreads, 0, stream>>>(
            src, src_bytes, n, e, r, dst, status);
    else
        k_decode_fused<false, Words><<<(uint32_t)blocks, kFusedThreads, 0, stream>>>(
            src, src_bytes, n, e, r, dst, status);
    return hipGetLastError();
}

// ------------------------------------------------------------------------
// Tile decode: one 256-thread workgroup per 2048-word tile, after an index
// pass that gives every tile its first escape record (the layout and the
// measurements are described with kTileWords).

constexpr int kTileThreads = kTileWords / 8;   // 8 words per thread
constexpr uint32_t kAhead = 16;   // records a tile's first record looks ahead
static_assert(kAhead > kSlotRecords && kAhead <= 64, "look-ahead past a full slot, within a wave");
constexpr uint32_t kNoTile = 0xFFFFFFFFu;
constexpr uint64_t kShortGap = 32;  // tile entries a lane fills alone

// Set bits of a wave mask below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// An item of the index pass: record k < e, the end item k == e (position
// n, tile `tiles`), or nothing past it (tile kNoTile).
struct IndexItem {
    uint64_t pos;
    uint32_t tile;
    uint32_t rec;  // offset in its tile | exponent << 16 (records only)
};

// Position of record k (its stored low 32 bits, with the segment number
// above them past 2^32 words), read with no branch so that the loads of a
// group go out together.
template <bool kOneSegment, bool kAlignedPos>
__device__ __forceinline__ uint64_t record_position(const EscapeReader& rd, uint64_t k) {
    const uint32_t lo = kAlignedPos ? reinterpret_cast<const uint32_t*>(rd.pos_lo)[k]
                                    : load4_unaligned(rd.pos_lo + 4 * k);
    if (kOneSegment) return lo;
    uint64_t seg = 0;
#pragma unroll
    for (int sg = 0; sg < 16; sg++) seg += rd.seg_end[sg] <= k ? 1u : 0u;
    return (seg << 32) | lo;
}

// Item k from its loaded position p and exponent x (both unused past the
// records).
__device__ __forceinline__ IndexItem make_item(uint64_t n, uint64_t e, uint64_t tiles, uint64_t k,
                                               uint64_t p, uint32_t x) {
    IndexItem it{0, kNoTile, 0};
    if (k < e) {
        it.pos = p;
        it.tile = (uint32_t)min_u64(p / kTileWords, tiles);
        it.rec = (uint32_t)(p - (uint64_t)it.tile * kTileWords) | (x << 16);
    } else if (k == e) {
        it.pos = n;
        it.tile = (uint32_t)tiles;
    }
    return it;
}

// A block's container (at src + y * pitch) and its escape count from its
// size, size = 176 + ceil(n/2) + n + 5E: false when the size cannot be a
// container of n words or runs past the pitch (nothing of it may be read).
struct BlockContainer {
    const uint8_t* src;
    uint64_t bytes;
    uint64_t e;
    bool ok;
};
__device__ __forceinline__ BlockContainer block_container(const BlockWords& blk, uint64_t n,
                                                          const uint8_t* src) {
    BlockContainer c;
    c.src = byte_offset(src, block_pitch(blk));
    c.bytes = blk.sizes[blockIdx.y];
    const uint64_t fixed = container_bytes(n, 0);
    const uint64_t extra = c.bytes - fixed;
    c.e = extra / 5;
    c.ok = !(c.bytes < fixed || c.bytes > blk.pitch || extra % 5 != 0 || c.e > (15 * n) / 16);
    return c;
}

// One wave per group of 64 items: lane L holds item k0 + L, and lanes
// 0..15 also load item k0 + 64 + L, so that the 16 items after the group
// are at hand.
// A lane whose item is the first of its tile fills idx over the gap back to
// its predecessor's tile (a short gap alone, a long one with the whole
// wave), sets the record count of the empty tiles in it to 0, and has its
// tile's slot written: the run of the tile's items (from a ballot of where
// the tile changes), then the 15 records from its own on, taken from LDS.
// Every global load of a group is issued before any is used (indices
// clamped to the last record), so a wave waits for memory once.  Faults: a
// position not above
// its predecessor, or not below n; the header (wave 0).  kOneSegment:
// n <= 2^32, every position is its stored low 32 bits.  kAlignedPos: the
// positions are 4-byte aligned.  For blocks (blockIdx.y the block) the
// container, E and the workspace are the block's, and a block whose size
// is no container is left to the decode pass to report.
template <bool kOneSegment, bool kAlignedPos, class Words>
__global__ __launch_bounds__(64) void k_tile_index(
    const uint8_t* __restrict__ src, uint64_t src_bytes, uint64_t n, uint64_t e, uint64_t groups,
    uint64_t* __restrict__ idx, uint32_t* __restrict__ flags, uint32_t* __restrict__ slots,
    Words blk) {
    __shared__ uint64_t seg_table[16];
    __shared__ uint32_t rec_lds[64 + kAhead];  // the items' records, then the 16 after them
    __shared__ uint32_t lead_lds[64];  // lane of each slot's first record, in tile order
    __shared__ uint32_t run_lds[64];   // and its tile's run
    __shared__ uint32_t tile_lds[64];  // and its tile
    const uint32_t lane = threadIdx.x;
    if constexpr (Words::kBlocks) {
        const BlockContainer c = block_container(blk, n, src);
        if (!c.ok) return;  // the same for the wave
        src = c.src;
        src_bytes = c.bytes;
        e = c.e;
        groups = index_groups(e);
        const uint64_t off = block_ws(blk);
        idx = byte_offset(idx, off);
        flags = byte_offset(flags, off);
        slots = byte_offset(slots, off);
    }
    bool bad = false;
    if (blockIdx.x == 0 && lane == 0) bad = !header_ok(src, src_bytes, n, e);
    const uint64_t esc_off = kPrefixBytes + (n + 1) / 2 + n;
    EscapeReader rd;
    rd.pos_lo = src + esc_off;
    rd.exps = rd.pos_lo + 4 * e;
    rd.aligned = kAlignedPos;
    rd.one_segment = kOneSegment;
    rd.seg_end = seg_table;
    if (!kOneSegment) {  // the segment table is read only past 2^32 words
        if (lane < 16) seg_table[lane] = reinterpret_cast<const uint64_t*>(src + 32)[lane];
        __syncthreads();
    }
    const uint64_t tiles = (n + kTileWords - 1) / kTileWords;
    const uint64_t last = e > 0 ? e - 1 : 0;
    for (uint64_t g = blockIdx.x; g < groups; g += gridDim.x) {
        const uint64_t k = g * kIndexItems + lane;
        const uint64_t ka = k + kIndexItems;  // the item 64 on, for the look-ahead
        uint64_t p = 0, pp = 0, pa = 0;
        uint32_t x = 0, xa = 0;
        if (e > 0) {  // the same for the whole grid
            // (only lanes 0..15 need the item 64 on; the others read their
            // own again, from lines already fetched)
            const uint64_t kc = min_u64(k, last);
            const uint64_t kac = lane < kAhead ? min_u64(ka, last) : kc;
            const uint64_t kpc = min_u64(k > 0 ? k - 1 : 0, last);
            p = record_position<kOneSegment, kAlignedPos>(rd, kc);
            pp = record_position<kOneSegment, kAlignedPos>(rd, kpc);
            pa = record_position<kOneSegment, kAlignedPos>(rd, kac);
            x = rd.exps[kc];
            xa = rd.exps[kac];
        }
        const IndexItem it = make_item(n, e, tiles, k, p, x);
        const IndexItem ahead = make_item(n, e, tiles, ka, pa, xa);
        const bool has_prev = k > 0 && k <= e;
        const uint32_t prev_tile = has_prev ? (uint32_t)min_u64(pp / kTileWords, tiles) : kNoTile;
        if (k < e && (it.pos >= n || (k > 0 && !(it.pos > pp)))) bad = true;
        const bool first = k <= e && (k == 0 || it.tile != prev_tile);

        // a tile's run: its items from the first on, up to the next item of
        // another tile (the group's 64 items and the 16 after it); bit i of
        // starts (i < 64) and of starts_ahead (item 64 + i) is set where an
        // item's tile differs from its predecessor's
        // (both shuffles run with every lane active, then one is picked)
        const uint32_t last_tile = (uint32_t)__shfl(it.tile, 63, 64);
        const uint32_t prev_ahead_tile = (uint32_t)__shfl_up(ahead.tile, 1, 64);
        const uint32_t before_ahead = lane == 0 ? last_tile : prev_ahead_tile;
        const uint64_t starts = __ballot(it.tile != (uint32_t)__shfl_up(it.tile, 1, 64));
        const uint64_t starts_ahead = __ballot(lane < kAhead && ahead.tile != before_ahead);
        const uint64_t later = lane < 63 ? starts >> (lane + 1) : 0;
        const uint32_t next = later ? lane + 1 + (uint32_t)__builtin_ctzll(later)
                                    : (starts_ahead ? 64u + (uint32_t)__builtin_ctzll(starts_ahead)
                                                    : 64u + kAhead);
        const uint32_t run = min(next - lane, kAhead + 1);  // above 15: "more than 15"

        // the gap: tiles (prev_tile, tile], the tiles before this one empty
        const uint64_t lo = k == 0 ? 0 : (uint64_t)prev_tile + 1;
        const uint64_t hi = it.tile;  // <= tiles for items up to the end item
        const bool has_gap = first && hi >= lo;
        if (has_gap && hi - lo < kShortGap) {
            for (uint64_t jt = lo; jt <= hi; jt++) {
                idx[jt] = k;
                if (jt < hi && jt < tiles) slots[jt * kSlotWords] = 0;
            }
        }
        uint64_t wide = __ballot(has_gap && hi - lo >= kShortGap);
        while (wide) {  // long gaps: the whole wave fills one at a time
            const int src_lane = __builtin_ctzll(wide);
            wide &= wide - 1;
            const uint64_t wlo = uniform64(__shfl(lo, src_lane, 64));
            const uint64_t whi = uniform64(__shfl(hi, src_lane, 64));
            const uint64_t wk = uniform64(__shfl(k, src_lane, 64));
            for (uint64_t jt = wlo + lane; jt <= whi; jt += 64) {
                idx[jt] = wk;
                if (jt < whi && jt < tiles) slots[jt * kSlotWords] = 0;
            }
        }
        // the slots of the group's first-of-tile records (the run, then the
        // records from this one on; those past the run belong to later
        // tiles and are never read), stored in tile order by consecutive
        // lanes on consecutive 16-byte pieces, so that the tiles of a group,
        // mostly consecutive, are written in whole lines
        const bool writes = first && k < e && it.tile < tiles;
        const uint64_t wmask = __ballot(writes);
        __syncthreads();  // the previous group's pieces are stored
        rec_lds[lane] = it.rec;
        if (lane < kAhead) rec_lds[64 + lane] = ahead.rec;
        if (writes) {
            const uint32_t jw = lanes_below(wmask);
            lead_lds[jw] = lane;
            run_lds[jw] = run;
            tile_lds[jw] = it.tile;
        }
        __syncthreads();
        const uint32_t pieces = 4u * (uint32_t)__popcll(wmask);
        for (uint32_t pc = lane; pc < pieces; pc += 64) {
            const uint32_t jw = pc / 4, w0 = 4 * (pc % 4);  // slot words w0 .. w0 + 3
            const uint32_t* recs = rec_lds + lead_lds[jw];   // word w >= 1 is recs[w - 1]
            const uint32_t head = recs[w0 == 0 ? 0 : w0 - 1];
            const uint4 v = make_uint4(w0 == 0 ? run_lds[jw] : head, recs[w0], recs[w0 + 1],
                                       recs[w0 + 2]);
            reinterpret_cast<uint4*>(slots + (uint64_t)tile_lds[jw] * kSlotWords)[pc % 4] = v;
        }
    }
    bad = __ballot(bad) != 0;
    if (lane == 0) flags[blockIdx.x] = bad ? 1u : 0u;
}

template <class Words>
hipError_t launch_tile_index(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                             uint8_t* ws, Words blk, hipStream_t stream) {
    const TileIndexLayout l = tile_index_layout(n, Words::kBlocks);
    const uint64_t groups = index_groups(e);
    const dim3 grid((uint32_t)(Words::kBlocks ? l.max_flags : min_u64(groups, l.max_flags)),
                    grid_blocks(blk));
    uint64_t* idx = reinterpret_cast<uint64_t*>(ws + l.idx_off);
    uint32_t* flags = reinterpret_cast<uint32_t*>(ws + l.flag_off);
    uint32_t* slots = reinterpret_cast<uint32_t*>(ws + l.slot_off);
    const bool one = n <= (uint64_t{1} << 32);
    const bool aligned = ((kPrefixBytes + (n + 1) / 2 + n) & 3) == 0;
#define SZ_INDEX(O, A)                                                                     \
    k_tile_index<O, A, Words><<<grid, 64, 0, stream>>>(src, src_bytes, n, e, groups, idx, \
                                                       flags, slots, blk)
    if (one && aligned) SZ_INDEX(true, true);
    else if (one) SZ_INDEX(true, false);
    else if (aligned) SZ_INDEX(false, true);
    else SZ_INDEX(false, false);
#undef SZ_INDEX
    return hipGetLastError();
}
template hipError_t launch_tile_index<FlatWords>(const uint8_t*, uint64_t, uint64_t, uint64_t,
                                                 uint8_t*, FlatWords, hipStream_t);
template hipError_t launch_tile_index<BlockWords>(const uint8_t*, uint64_t, uint64_t, uint64_t,
                                                  uint8_t*, BlockWords, hipStream_t);

// Exponent byte k (0..7) of the pair (e0: words 0..3, e1: words 4..7) set to x.
__device__ __forceinline__ void set_exponent(uint32_t& e0, uint32_t& e1, uint32_t k, uint32_t x) {
    const uint32_t sh = 8 * (k & 3);
    const uint32_t m = 0xFFu << sh;
    if (k < 4) e0 = (e0 & ~m) | (x << sh);
    else e1 = (e1 & ~m) | (x << sh);
}

// One lane's candidate record (offset in the tile in bits 10..0, exponent
// in bits 23..16) where `mine` (a wave ballot) has its bit set: the wave
// walks only the records inside its own 512 words, by lane reads, and the
// thread whose 8 words hold a record patches that exponent.  Offsets are
// masked to the tile, so any record content patches only this tile.
__device__ __forceinline__ void patch_wave(uint32_t v, uint64_t mine, uint32_t& e0, uint32_t& e1) {
    const uint32_t first = 8u * (threadIdx.x % kTileThreads);
    while (mine) {
        const int j = __builtin_ctzll(mine);
        mine &= mine - 1;
        const uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
        const uint32_t d = (r & (kTileWords - 1)) - first;
        if (d < 8) set_exponent(e0, e1, d, (r >> 16) & 0xFFu);
    }
}

// The wave's 512-word quarter of the tile, as bits 10..9 of an offset.
__device__ __forceinline__ uint32_t wave_quarter() { return (threadIdx.x % kTileThreads) >> 6; }

// The records [ks, ke) of the tile starting at word t0, 64 at a time: each
// lane loads one record, the wave keeps those inside its own words.
// rd.pos_lo holds 4-byte aligned positions when `aligned`; only the low 32
// bits are compared, a tile lying inside one 2^32-word segment.
__device__ __forceinline__ void patch_records(const EscapeReader& rd, uint64_t ks, uint64_t ke,
                                              uint64_t t0, uint32_t& e0, uint32_t& e1) {
    const uint32_t lane = threadIdx.x & 63;
    for (uint64_t q0 = ks; q0 < ke; q0 += 64) {
        const uint64_t q = q0 + lane;
        uint32_t v = 0;
        bool in = false;
        if (q < ke) {
            const uint32_t d = rd.low32(q) - (uint32_t)t0;
            in = d < kTileWords && (d >> 9) == wave_quarter();
            v = d | ((uint32_t)rd.exps[q] << 16);
        }
        patch_wave(v, __ballot(in), e0, e1);
    }
}

// A tile's records [ks, ke) marked in an LDS exponent map between two
// barriers (every thread of the workgroup calls it), then patched into this
// thread's 8 exponents: for tiles with many records, where a walk through
// lane reads would take one step per record.
struct TileMap {
    uint8_t exp[kTileWords];
    uint32_t bits[kTileWords / 32];
};

__device__ __forceinline__ void patch_mapped(const EscapeReader& rd, uint64_t ks, uint64_t ke,
                                             uint64_t t0, uint32_t& e0, uint32_t& e1,
                                             TileMap& map) {
    const int t = threadIdx.x;
    if (t < (int)(kTileWords / 32)) map.bits[t] = 0;
    __syncthreads();
    for (uint64_t q = ks + t; q < ke; q += kTileThreads) {
        const uint32_t d = rd.low32(q) - (uint32_t)t0;
        if (d < kTileWords) {
            map.exp[d] = rd.exps[q];
            atomicOr(&map.bits[d >> 5], 1u << (d & 31));
        }
    }
    __syncthreads();
    const uint32_t present = (map.bits[t >> 2] >> (8 * (t & 3))) & 0xFFu;
    if (present) {
        const uint2 pe = *reinterpret_cast<const uint2*>(&map.exp[8 * t]);
        e0 = bitselect(bits_to_bytes(present), pe.x, e0);
        e1 = bitselect(bits_to_bytes(present >> 4), pe.y, e1);
    }
    __syncthreads();  // the map is reused by the next tile
}

// Workgroup 0 folds the index waves' fault flags into the status; workgroup
// b > 0 decodes tile b - 1 (a launch holds at most kMaxTileGroups + 1; past
// that each takes tiles b - 1, b - 1 + grid - 1, ...).  Per tile: the
// slot, the codes and sign|mantissa bytes, all loaded before anything waits
// on one; the slot's records patched in (or, for a tile with more records
// than its slot, the index entries, clamped to [0, E] and to one tile's
// worth of records, and the escape stream); one 16-byte non-temporal store
// per thread.  kDense (containers averaging more records per tile than a
// slot holds): a tile beyond its slot marks an LDS exponent map; otherwise
// no LDS, no barrier, no atomic.
template <bool kAlignedSm, class Words, bool kDense>
__global__ __launch_bounds__(kTileThreads) void k_decode_tiles(
    const uint8_t* __restrict__ src, uint64_t n, uint64_t e, const uint64_t* __restrict__ idx,
    const uint32_t* __restrict__ flags, uint64_t n_flags, const uint32_t* __restrict__ slots,
    Words out, int32_t* status) {
    struct NoMap {};
    __shared__ typename std::conditional<kDense, TileMap, NoMap>::type map;
    const int t = threadIdx.x;
    const uint32_t lane = t & 63;
    const uint64_t workers = gridDim.x - 1;  // workgroup 0 folds the flags
    // For blocks: this block's container, workspace and status.  A tile
    // workgroup waits on nothing of the block's before its tile's own loads
    // go out (a dependent load first would make every short-lived
    // workgroup wait for memory twice): the block's words address is a
    // scalar load first waited for at the store, which skips a NULL or
    // misaligned one; the size, which gives E, is read only on the way to
    // the escape stream, for a tile with more records than its slot, and a
    // size that is no container then leaves the tile unpatched (its words
    // are unspecified, the status says corrupt, and nothing outside the
    // block's pitch is read).  Workgroup 0 checks the size and reports.
    const uint8_t* const src0 = src;
    if constexpr (Words::kBlocks) {
        status += blockIdx.y;
        src = byte_offset(src, block_pitch(out));
        const uint64_t off = block_ws(out);
        idx = byte_offset(idx, off);
        flags = byte_offset(flags, off);
        slots = byte_offset(slots, off);
    }
    if (blockIdx.x == 0) {
        if constexpr (Words::kBlocks) {
            if (!block_container(out, n, src0).ok) {  // the same for every thread
                if (t == 0) *status = out.invalid() ? kStatusInvalid : kStatusCorrupt;
                return;
            }
        }
        uint32_t any = 0;
#pragma unroll 8
        for (uint64_t f = t; f < n_flags; f += kTileThreads) any |= flags[f];
        any = __syncthreads_or(any);
        if (t == 0 && status) *status = out.invalid() ? kStatusInvalid : (any ? kStatusCorrupt : 0);
        return;
    }
    if constexpr (!Words::kBlocks && !Words::kPaged) {
        if (out.invalid()) return;  // the same for every thread
    }
    // blocks: the block's address, a scalar load first waited for at the
    // tile's store, together with the codebook's
    const auto words = out.resolve();

    const uint8_t* nib = src + kPrefixBytes;
    const uint8_t* sm = nib + (n + 1) / 2;
    const uint64_t tiles = (n + kTileWords - 1) / kTileWords;
    const uint64_t whole = n / kTileWords;  // tiles with all kTileWords words
    const uint64_t esc_off = kPrefixBytes + (n + 1) / 2 + n;

    // the tile's records into e0/e1: from its slot, or, past the slot's
    // capacity, from the escape stream
    auto patch = [&](uint64_t tile, uint64_t t0, uint32_t sv, uint32_t& e0, uint32_t& e1) {
        const uint32_t cnt = (uint32_t)__builtin_amdgcn_readfirstlane((int)sv);
        if (cnt <= kSlotRecords) {
            const bool in = lane >= 1 && lane <= cnt && ((sv >> 9) & 3u) == wave_quarter();
            patch_wave(sv, __ballot(in), e0, e1);
            return;
        }
        if constexpr (Words::kBlocks) {
            const BlockContainer c = block_container(out, n, src0);
            if (!c.ok) return;  // the same for every thread: reported by workgroup 0
            e = c.e;
        }
        EscapeReader rd;
        rd.pos_lo = src + esc_off;
        rd.exps = rd.pos_lo + 4 * e;
        rd.aligned = (esc_off & 3) == 0;
        rd.one_segment = n <= (1ull << 32);
        rd.seg_end = nullptr;  // unused: tiles compare the low 32 bits only
        const uint64_t ks = min_u64(uniform64(idx[tile]), e);
        uint64_t ke = min_u64(uniform64(idx[tile + 1]), e);
        if (ke < ks) ke = ks;                              // a faulty index: flagged
        if (ke - ks > kTileWords) ke = ks + kTileWords;
        if constexpr (kDense) patch_mapped(rd, ks, ke, t0, e0, e1, map);
        else patch_records(rd, ks, ke, t0, e0, e1);
    };

    for (uint64_t tile = blockIdx.x - 1; tile < tiles; tile += workers) {
        const uint64_t t0 = tile * kTileWords;
        const uint64_t i0 = t0 + (uint64_t)t * 8;
        // every load of the tile goes out before anything waits on one
        const uint32_t sv = lane < kSlotWords ? slots[tile * kSlotWords + lane] : 0u;
        // a paged tensor's table check, read with the tile's loads and
        // tested only at the store (the empty asm there keeps the compiler
        // from testing, and so waiting for, it any earlier)
        int32_t table_flag = 0;
        if constexpr (Words::kPaged) table_flag = *out.bad;

        if (tile < whole) {
            const uint32_t codes = *reinterpret_cast<const uint32_t*>(nib + i0 / 2);
            uint32_t s0, s1;
            if (kAlignedSm) {
                const uint2 v = *reinterpret_cast<const uint2*>(sm + i0);
                s0 = v.x;
                s1 = v.y;
            } else {
                s0 = load4_unaligned(sm + i0);
                s1 = load4_unaligned(sm + i0 + 4);
            }
            // a wave's words are 512 consecutive words: one page
            uint16_t* words_out = nullptr;
            if constexpr (Words::kPaged) words_out = out.at_wave(i0);
            const uint4 cb = *reinterpret_cast<const uint4*>(src + kHeaderBytes);
            uint32_t e0, e1;
            exponents8(codes, cb, e0, e1);
            patch(tile, t0, sv, e0, e1);
            bool write = true;
            if constexpr (Words::kBlocks) {
                // a NULL or misaligned block address: nothing written
                const uintptr_t a = reinterpret_cast<uintptr_t>(words.base);
                write = a != 0 && (a & 15) == 0;
                words_out = words.at(i0);
            } else if constexpr (Words::kPaged) {
                asm volatile("" : "+v"(table_flag));
                write = table_flag == 0;
            } else {
                words_out = out.at_wave(i0);
            }
            // written past the caches: a decode's output is larger than they
            // are, and lines left dirty cost the next kernel their write-back
            if (write) store_streaming(reinterpret_cast<uint4*>(words_out), words8(e0, e1, s0, s1));
        } else {
            // the partial last tile: words past n are neither read nor written
            if constexpr (Words::kBlocks) {
                const uintptr_t a = reinterpret_cast<uintptr_t>(words.base);
                if (a == 0 || (a & 15) != 0) return;
            }
            const uint4 cb = *reinterpret_cast<const uint4*>(src + kHeaderBytes);
            uint32_t ex[8];
            for (uint32_t k = 0; k < 8; k++) {
                const uint64_t i = i0 + k;
                ex[k] = i < n ? codebook_byte(cb, (nib[i / 2] >> (4 * (i & 1))) & 0xFu) : 0u;
            }
            uint32_t e0 = ex[0] | (ex[1] << 8) | (ex[2] << 16) | (ex[3] << 24);
            uint32_t e1 = ex[4] | (ex[5] << 8) | (ex[6] << 16) | (ex[7] << 24);
            patch(tile, t0, sv, e0, e1);
            if constexpr (Words::kPaged) {
                asm volatile("" : "+v"(table_flag));
                if (table_flag != 0) return;  // the same for every thread
            }
            for (uint32_t k = 0; k < 8 && i0 + k < n; k++) {
                const uint32_t x = ((k < 4 ? e0 : e1) >> (8 * (k & 3))) & 0xFFu;
                *words.at(i0 + k) = (uint16_t)recombine(sm[i0 + k], x);
            }
        }
    }
}

template <class Words>
hipError_t launch_decode_tiles(const uint8_t* src, uint64_t n, uint64_t e, const uint8_t* ws,
                               Words dst, int32_t* status, int /*num_cus*/, hipStream_t stream) {
    const TileIndexLayout l = tile_index_layout(n, Words::kBlocks);
    // (each block's index waves all write their flag)
    const uint64_t n_flags = Words::kBlocks ? l.max_flags : min_u64(index_groups(e), l.max_flags);
    // the one that writes the status, then the tiles' workgroups
    const dim3 grid((uint32_t)(min_u64(l.tiles, kMaxTileGroups) + 1), grid_blocks(dst));
    const uint64_t* idx = reinterpret_cast<const uint64_t*>(ws + l.idx_off);
    const uint32_t* flags = reinterpret_cast<const uint32_t*>(ws + l.flag_off);
    const uint32_t* slots = reinterpret_cast<const uint32_t*>(ws + l.slot_off);
    const bool aligned = ((kPrefixBytes + (n + 1) / 2) & 7) == 0;
    // (blocks pass e = 0 and take the variant for few records per tile: 2%
    // faster on KV blocks; escape-heavy blocks are the single-pass form's)
    const bool dense = e > l.tiles * kSlotRecords;
#define SZ_TILES(A, D)                                                                   \
    k_decode_tiles<A, Words, D><<<grid, kTileThreads, 0, stream>>>(                      \
        src, n, e, idx, flags, n_flags, slots, dst, status)
    if (aligned && !dense) SZ_TILES(true, false);
    else if (aligned) SZ_TILES(true, true);
    else if (!dense) SZ_TILES(false, false);
    else SZ_TILES(false, true);
#undef SZ_TILES
    return hipGetLastError();
}

// ------------------------------------------------------------------------
// Dense decode: the single pass again, for inputs with many escapes.  One
// workgroup per power-of-two range of words, walked in
// sub-ranges of kDecTile words.  For each sub-range the workgroup reads the
// escape records that fall in it straight from the escape stream (thread t
// takes records t, t + 512, ... after the last one consumed, and stops at
// the first whose position lies beyond the sub-range), writes each record's
// exponent into an LDS map with one entry per word, then rebuilds its words
// with the map's entries taking the place of the codebook's exponents.
// Thread t rebuilds the 8-word groups at t*8, t*8 + 4096, ... of the
// sub-range, so each wave's loads and stores cover consecutive bytes (wider
// per-thread runs measured slower on MI355X).  There are no LDS atomics and
// no record staging: two barriers per sub-range.

constexpr int kDenseThreads = 512;
constexpr int kDenseWaves = kDenseThreads / 64;
constexpr int kGroups = 4;                                 // 8-word groups per thread
constexpr uint32_t kGroupStride = 8 * kDenseThreads;       // words between a thread's groups
constexpr uint32_t kDenseTile = kGroups * kGroupStride;    // words per sub-range
constexpr uint32_t kMapEscaped = 0x100u;                   // map entry: 0x100 | exponent
constexpr uint32_t kDenseMaxLog2 = 16;                     // ranges of at most 2^16 words
constexpr uint32_t kDenseSubs = (1u << kDenseMaxLog2) / kDenseTile;  // sub-ranges per range
constexpr uint32_t kWaveRecords = 256;                     // records per wave and step
static_assert((1u << 14) % kDenseTile == 0, "ranges of at least 2^14 words hold whole sub-ranges");
static_assert(kDenseSubs + 1 <= kDenseWaves, "one wave per sub-range bound");
static_assert(kWaveRecords == 4 * 64, "four records per lane and step");

// Eight 16-bit map entries (one uint4) to the exponent bytes that replace
// e0 (elements 0..3) and e1 (elements 4..7) where an entry is set.
__device__ __forceinline__ void patch8(uint4 m, uint32_t& e0, uint32_t& e1) {
    if ((m.x | m.y | m.z | m.w) == 0) return;
    const uint32_t x0 = perm(m.y, m.x, 0x06040200u);   // exponent bytes, elements 0..3
    const uint32_t x1 = perm(m.w, m.z, 0x06040200u);   // elements 4..7
    const uint32_t f0 = perm(m.y, m.x, 0x07050301u);   // 1 where escaped, else 0
    const uint32_t f1 = perm(m.w, m.z, 0x07050301u);
    e0 = bitselect(f0 * 0xFFu, x0, e0);
    e1 = bitselect(f1 * 0xFFu, x1, e1);
}

// Codes (one dword) and sign|mantissa bytes (two dwords) of the 8 words
// from word w; the sign|mantissa stream is 8-byte aligned or not.
template <bool kAlignedSm>
__device__ __forceinline__ void load_group(const uint8_t* nib, const uint8_t* sm, uint64_t w,
                                           uint32_t& c, uint32_t& s0, uint32_t& s1) {
    c = *reinterpret_cast<const uint32_t*>(nib + w / 2);
    if (kAlignedSm) {
        const uint2 v = *reinterpret_cast<const uint2*>(sm + w);
        s0 = v.x;
        s1 = v.y;
    } else {
        s0 = load4_unaligned(sm + w);
        s1 = load4_unaligned(sm + w + 4);
    }
}

// The records [k0, k1) into the LDS map of the sub-range whose positions
// (in their segment) are place_lo .. place_hi - 1.  Wave w takes a
// contiguous slice of them, four consecutive records per lane and step:
// with kAlignedRec (the escape stream 16-byte aligned) one 16-byte load of
// positions and one 4-byte load of exponents for a whole group, else a
// load per record.  Every record must lie in valid_lo .. valid_hi - 1 and
// above its predecessor (the lane before's last record through a shuffle,
// the previous step's last lane, or for the slice's first record one more
// load); a record that fails sets *bad, and only records of the sub-range
// are placed.
template <bool kAlignedRec>
__device__ __forceinline__ void place_records(const EscapeReader& rd, uint64_t k0, uint64_t k1,
                                              uint32_t valid_lo, uint64_t valid_hi,
                                              uint32_t place_lo, uint64_t place_hi, uint16_t* map,
                                              int* bad) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t s0 = kAlignedRec ? (k0 & ~uint64_t{3}) : k0;
    // at least one step's worth per wave: with few records, the waves
    // without any go straight on to their codes
    const uint64_t spread = (k1 - s0 + 4 * kDenseWaves - 1) / (4 * kDenseWaves) * 4;
    const uint64_t per_wave = spread > kWaveRecords ? spread : kWaveRecords;
    const uint64_t w0 = s0 + (uint64_t)wave * per_wave;
    const uint64_t w1 = min_u64(w0 + per_wave, k1);
    if (w0 >= w1) return;  // the same for the whole wave
    // per-lane offsets are 32-bit, from the slice's first record (a slice
    // holds fewer than 2^14 records): records w0 + r
    const uint32_t count = (uint32_t)(w1 - w0);
    const uint32_t skip = k0 > w0 ? (uint32_t)(k0 - w0) : 0u;  // alignment, first slice only
    const bool carried = w0 > k0;  // the slice's first record has a predecessor here
    const uint8_t* pbase = rd.pos_lo + 4 * w0;
    const uint8_t* xbase = rd.exps + w0;
    // with kAlignedRec, buffer loads over the slice: a 32-bit offset per
    // lane from the slice's base in scalar registers, and reads past the
    // slice return 0
    const __amdgpu_buffer_rsrc_t rpos = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(pbase), (short)0, (int32_t)(4 * count), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rexp = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(xbase), (short)0, (int32_t)count, kBufferFlags);
    const uint32_t steps = (count + kWaveRecords - 1) / kWaveRecords;
    // the record before the slice (every slice but the first starts past k0)
    uint32_t carry = carried ? rd.low32(w0 - 1) : 0u;
    for (uint32_t i = 0; i < steps; i++) {
        const uint32_t r = i * kWaveRecords + 4 * (uint32_t)lane;
        uint32_t v[4], x;
        if (kAlignedRec && r + 4 <= count) {
            const auto p = __builtin_amdgcn_raw_buffer_load_b128(rpos, 4 * r, 0, 0);
            v[0] = p[0];
            v[1] = p[1];
            v[2] = p[2];
            v[3] = p[3];
            x = __builtin_amdgcn_raw_buffer_load_b32(rexp, r, 0, 0);
        } else if (kAlignedRec) {
            x = 0;
#pragma unroll
            for (int u = 0; u < 4; u++) {
                v[u] = __builtin_amdgcn_raw_buffer_load_b32(rpos, 4 * (r + u), 0, 0);
                x |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rexp, r + u, 0, 0) << (8 * u);
            }
        } else {
            x = 0;
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const bool in = r + u < count;
                v[u] = in ? rd.low32(w0 + r + u) : 0u;
                x |= (in ? (uint32_t)xbase[r + u] : 0u) << (8 * u);
            }
        }
        // every lane takes part in both shuffles, then picks
        const uint32_t up = __shfl_up(v[3], 1, 64);
        const uint32_t last = __shfl(v[3], 63, 64);
        const uint32_t before = lane == 0 ? carry : up;
        carry = last;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const uint32_t k = r + u;
            if (k < skip || k >= count) continue;
            const uint32_t lo = v[u];
            const uint32_t pred = u == 0 ? before : v[u - 1];
            const bool has_pred = k > skip || carried;
            if (lo < valid_lo || (uint64_t)lo >= valid_hi || (has_pred && !(lo > pred)))
                *bad = 1;
            else if (lo >= place_lo && (uint64_t)lo < place_hi)
                map[lo - place_lo] = (uint16_t)(kMapEscaped | ((x >> (8 * u)) & 0xFFu));
        }
    }
}

// One workgroup per range of at most 2^16 words, decoded in sub-ranges of
// 16384 words.  First the record interval of every sub-range, one 64-way
// search per wave, all at once: bound[j] = the first record at or above
// the sub-range's start.  Then per sub-range the thread's codes and
// sign|mantissa bytes are loaded, its records placed as 0x100 | exponent
// into a 16-bit-per-word LDS map while those loads are in flight, and,
// after a barrier, each thread rebuilds its 8-word groups with the map's
// exponents where set and clears the entries it read.  Neighbouring ranges
// compute the same bound for their shared boundary, so the intervals tile
// [0, e) when the first starts at 0, the last ends at e and none runs
// backwards; every record inside its sub-range and above its predecessor
// then means the whole stream is strictly ascending.
// Eight waves per SIMD (four workgroups per CU) need at most 64 VGPRs and
// the scalar-register cap.
template <bool kAlignedSm, bool kAlignedRec, class Words>
__global__ __launch_bounds__(kDenseThreads) SZ_EIGHT_WAVE_SGPR_CAP
__attribute__((amdgpu_waves_per_eu(8))) void k_decode_dense(
    const uint8_t* __restrict__ src, uint64_t src_bytes, uint64_t n, uint64_t e,
    uint32_t range_log2, Words out, int32_t* status) {
    __shared__ uint4 map4[kDenseTile / 8];   // kDenseTile 16-bit entries
    __shared__ uint64_t bound[kDenseSubs + 1];
    __shared__ uint64_t seg_table[16];
    __shared__ int bad;

    const int t = threadIdx.x;
    const int wave = t >> 6;
    uint16_t* map = reinterpret_cast<uint16_t*>(map4);
    if constexpr (Words::kBlocks) status += blockIdx.y;
    if (out.invalid()) {  // the same for every thread
        if (blockIdx.x == 0 && t == 0 && status)
            __hip_atomic_fetch_max(status, kStatusInvalid, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    if constexpr (Words::kBlocks) {
        // this block's container and its size, which gives E as
        // size = 176 + ceil(n/2) + n + 5E; a size that cannot be a container
        // of n words, or that runs past the block's pitch, is corrupt, and
        // nothing of the container is read
        src = byte_offset(src, block_pitch(out));
        src_bytes = out.sizes[blockIdx.y];
        const uint64_t fixed = container_bytes(n, 0);
        const uint64_t extra = src_bytes - fixed;
        e = extra / 5;
        if (src_bytes < fixed || src_bytes > out.pitch || extra % 5 != 0 || e > (15 * n) / 16) {
            if (blockIdx.x == 0 && t == 0)
                __hip_atomic_fetch_max(status, kStatusCorrupt, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
    const auto words = out.resolve();  // (after the address check)
    if (t == 0) bad = 0;
    if (blockIdx.x == 0 && t == 0 && !header_ok(src, src_bytes, n, e)) bad = 1;

    const uint4 cb = *reinterpret_cast<const uint4*>(src + kHeaderBytes);
    const uint8_t* nib = src + kPrefixBytes;
    const uint8_t* sm = nib + (n + 1) / 2;
    const uint64_t esc_off = kPrefixBytes + (n + 1) / 2 + n;
    EscapeReader rd;
    rd.pos_lo = src + esc_off;
    rd.exps = rd.pos_lo + 4 * e;
    rd.aligned = (esc_off & 3) == 0;
    rd.one_segment = n <= (1ull << 32);
    rd.seg_end = seg_table;
    if (t < 16) seg_table[t] = reinterpret_cast<const uint64_t*>(src + 32)[t];
    // every map entry starts clear; each thread clears the entries it reads
#pragma unroll
    for (int g = 0; g < kGroups; g++) map4[g * kDenseThreads + t] = make_uint4(0, 0, 0, 0);

    const uint64_t begin = min_u64((uint64_t)blockIdx.x << range_log2, n);
    const uint64_t end = min_u64(begin + (uint64_t{1} << range_log2), n);
    const uint32_t subs = (uint32_t)((end - begin + kDenseTile - 1) / kDenseTile);
    __syncthreads();  // seg_table, read by the searches
    // the range's records over the whole stream, then the sub-range
    // boundaries among those alone (fewer probes, on lines the placement
    // reads next)
    if (wave == 0 || (wave == 1 && subs > 0)) {
        const uint64_t b = wave_lower_bound(rd, 0, e, wave == 0 ? begin : end);
        if ((t & 63) == 0) bound[wave == 0 ? 0 : subs] = b;
    }
    __syncthreads();
    // a range with few records (one step of every wave) is read whole for
    // each of its sub-ranges, its second and later reads from the caches;
    // otherwise the sub-range boundaries are searched among its records
    const uint64_t k_lo = uniform64(bound[0]);
    const uint64_t k_hi = uniform64(bound[subs]);
    const bool few = k_hi <= k_lo + (uint64_t)kDenseWaves * kWaveRecords;
    if (!few && wave >= 1 && (uint32_t)wave < subs) {
        const uint64_t b = wave_lower_bound(rd, k_lo, k_hi, begin + (uint64_t)wave * kDenseTile);
        if ((t & 63) == 0) bound[wave] = b;
    }
    __syncthreads();
    if (t == 0) {
        if (blockIdx.x == 0 && bound[0] != 0) bad = 1;
        if (blockIdx.x == gridDim.x - 1 && bound[subs] != e) bad = 1;  // positions >= n
        if (k_hi < k_lo) bad = 1;
        if (!few)  // (the searches kept the inner bounds inside [k_lo, k_hi])
            for (uint32_t j = 0; j < subs; j++)
                if (bound[j + 1] < bound[j]) bad = 1;
    }

    for (uint32_t j = 0; j < subs; j++) {
        const uint64_t sub = begin + (uint64_t)j * kDenseTile;
        const uint64_t sub_end = min_u64(sub + kDenseTile, end);
        // the sub-range lies inside one 2^32-word segment, whose records are
        // [seg_lo, seg_hi): there a position is its stored low 32 bits
        // above the segment base
        const uint64_t k0 = few ? k_lo : uniform64(bound[j]);
        const uint64_t k1 = few ? k_hi : uniform64(bound[j + 1]);
        const uint32_t seg = (uint32_t)(sub >> 32);
        const uint64_t seg_lo = seg == 0 ? 0 : seg_table[seg - 1];
        const uint64_t seg_hi = seg_table[seg];
        const uint64_t base = (uint64_t)seg << 32;  // a range lies inside one segment
        if (k0 < seg_lo || k1 > seg_hi) {
            if (t == 0 && k1 > k0) bad = 1;
        } else if (k1 > k0) {
            place_records<kAlignedRec>(rd, k0, k1, (uint32_t)(few ? begin : sub),
                                       (few ? end : sub_end) - base, (uint32_t)sub,
                                       sub_end - base, map, &bad);
        }
        // this thread's codes and sign|mantissa bytes: loaded after the
        // records, so that the placement does not hold them in registers;
        // they arrive while the other waves finish placing
        const bool whole = sub + kDenseTile <= end;   // the same for every thread
        const uint64_t wt = sub + (uint64_t)t * 8;  // this thread's first word
        uint32_t c[kGroups], s[2 * kGroups];
        if constexpr (kAlignedSm) {
            // buffer loads over the sub-range's streams: 32-bit offsets per
            // lane from bases in scalar registers
            const uint32_t words = (uint32_t)(sub_end - sub);
            const __amdgpu_buffer_rsrc_t rnib = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(nib + sub / 2), (short)0, (int32_t)((words + 1) / 2),
                kBufferFlags);
            const __amdgpu_buffer_rsrc_t rsm = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(sm + sub), (short)0, (int32_t)words, kBufferFlags);
#pragma unroll
            for (int g = 0; g < kGroups; g++) {
                const uint32_t w = (uint32_t)t * 8 + (uint32_t)g * kGroupStride;  // from sub
                c[g] = s[2 * g] = s[2 * g + 1] = 0;
                if (whole || w + 8 <= words) {
                    c[g] = __builtin_amdgcn_raw_buffer_load_b32(rnib, w / 2, 0, 0);
                    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsm, w, 0, 0);
                    s[2 * g] = v[0];
                    s[2 * g + 1] = v[1];
                }
            }
        } else {
#pragma unroll
            for (int g = 0; g < kGroups; g++) {
                const uint64_t w = wt + (uint64_t)g * kGroupStride;
                c[g] = s[2 * g] = s[2 * g + 1] = 0;
                if (whole || w + 8 <= sub_end) load_group<kAlignedSm>(nib, sm, w, c[g], s[2 * g], s[2 * g + 1]);
            }
        }
        __syncthreads();

        // rebuild this thread's words, clearing the map entries as they are read
#pragma unroll
        for (int g = 0; g < kGroups; g++) {
            const uint64_t w = wt + (uint64_t)g * kGroupStride;
            uint4& slot = map4[g * kDenseThreads + t];
            if (whole || w + 8 <= sub_end) {
                const uint4 m = slot;
                slot = make_uint4(0, 0, 0, 0);
                uint32_t e0, e1;
                exponents8(c[g], cb, e0, e1);
                patch8(m, e0, e1);
                // a sub-range lies inside one page
                store_global(reinterpret_cast<uint4*>(words.at(sub) + (w - sub)),
                             words8(e0, e1, s[2 * g], s[2 * g + 1]));
            } else if (w < sub_end) {  // the input's last, partial group
                for (uint64_t i = w; i < sub_end; i++) {
                    const uint32_t code = (nib[i / 2] >> (4 * (i & 1))) & 0xFu;
                    const uint32_t m = map[(uint32_t)(i - sub)];
                    map[(uint32_t)(i - sub)] = 0;
                    const uint32_t ex = (m & kMapEscaped) ? (m & 0xFFu) : codebook_byte(cb, code);
                    *words.at(i) = (uint16_t)recombine(sm[i], ex);
                }
            }
        }
        __syncthreads();
    }
    __syncthreads();
    if (t == 0 && bad && status)
        __hip_atomic_fetch_max(status, kStatusCorrupt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class Words>
hipError_t launch_decode_dense(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                               Words dst, int32_t* status, hipStream_t stream) {
    uint32_t r = 14;
    // up to kMaxDecodeRanges workgroups as long as ranges stay at most
    // 2^kDenseMaxLog2 words (beyond, more workgroups): enough for several
    // waves of resident workgroups (a 10.7 GB input with 2048 ranges left
    // the last wave a quarter full: 16% slower); for blocks, over all their
    // words
    const uint64_t words = n * grid_blocks(dst);
    while (r < kDenseMaxLog2 && ((words + (1ull << r) - 1) >> r) > kMaxDecodeRanges) r++;
    uint64_t blocks = (n + (1ull << r) - 1) >> r;
    if (blocks == 0) blocks = 1;  // the header check still runs
    // (for blocks, the address check wrote every block's starting status)
    if (status && !Words::kBlocks) k_status_clear<<<1, 1, 0, stream>>>(status);
    // the sign|mantissa stream starts at 176 + ceil(n/2): 8-byte aligned
    // exactly when n is a multiple of 16; the escape stream, at
    // 176 + ceil(n/2) + n, 16-byte aligned when n is a multiple of 32
    const bool aligned_sm = ((kPrefixBytes + (n + 1) / 2) & 7) == 0;
    const bool aligned_rec = ((kPrefixBytes + (n + 1) / 2 + n) & 15) == 0;
    const dim3 grid((uint32_t)blocks, grid_blocks(dst));
    if (aligned_sm && aligned_rec)
        k_decode_dense<true, true, Words><<<grid, kDenseThreads, 0, stream>>>(
            src, src_bytes, n, e, r, dst, status);
    else if (aligned_sm)
        k_decode_dense<true, false, Words><<<grid, kDenseThreads, 0, stream>>>(
            src, src_bytes, n, e, r, dst, status);
    else
        k_decode_dense<false, false, Words><<<grid, kDenseThreads, 0, stream>>>(
            src, src_bytes, n, e, r, dst, status);
    return hipGetLastError();
}

#define SZ_DECODE_INSTANCES(W)                                                                  \
    template hipError_t launch_unpack<W>(const uint8_t*, uint64_t, uint64_t, uint64_t, W,       \
                                         int32_t*, int, hipStream_t);                           \
    template hipError_t launch_scatter<W>(const uint8_t*, uint64_t, uint64_t, W, int32_t*,      \
                                          hipStream_t);                                         \
    template hipError_t launch_decode_fused<W>(const uint8_t*, uint64_t, uint64_t, uint64_t, W, \
                                               int32_t*, hipStream_t);                          \
    template hipError_t launch_decode_dense<W>(const uint8_t*, uint64_t, uint64_t, uint64_t, W, \
                                               int32_t*, hipStream_t);                          \
    template hipError_t launch_decode_tiles<W>(const uint8_t*, uint64_t, uint64_t,              \
                                               const uint8_t*, W, int32_t*, int, hipStream_t);
SZ_DECODE_INSTANCES(FlatWords)
SZ_DECODE_INSTANCES(PagedWords)
#undef SZ_DECODE_INSTANCES
template hipError_t launch_decode_dense<BlockWords>(const uint8_t*, uint64_t, uint64_t, uint64_t,
                                                    BlockWords, int32_t*, hipStream_t);
template hipError_t launch_decode_tiles<BlockWords>(const uint8_t*, uint64_t, uint64_t,
                                                    const uint8_t*, BlockWords, int32_t*, int,
                                                    hipStream_t);

}  // namespace sz
