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

__device__ bool header_ok(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e) {
    if (*reinterpret_cast<const uint32_t*>(src + 0) != kMagic) return false;
    if (*reinterpret_cast<const uint16_t*>(src + 4) != kVersion) return false;
    if (*reinterpret_cast<const uint16_t*>(src + 6) != kElementBf16) return false;
    if (*reinterpret_cast<const uint64_t*>(src + 8) != n) return false;
    if (*reinterpret_cast<const uint64_t*>(src + 16) != e) return false;
    if (*reinterpret_cast<const uint64_t*>(src + 24) != src_bytes) return false;
    const uint64_t* seg_end = reinterpret_cast<const uint64_t*>(src + 32);
    const uint64_t segments_used = (n + 0xFFFFFFFFull) >> 32;
    uint64_t prev = 0;
    for (uint32_t s = 0; s < 16; s++) {
        const uint64_t v = seg_end[s];
        if (v < prev) return false;
        if ((uint64_t)s + 1 >= segments_used && v != e) return false;
        prev = v;
    }
    return true;
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

// First k in [0, e] whose position is >= target, for one wavefront: every
// step probes 64 evenly spaced records and keeps the bracket where the
// predicate turns true, so the interval shrinks on every step and the loop
// ends on any input (sorted input gives the exact lower bound).
__device__ uint64_t wave_lower_bound(const EscapeReader& r, uint64_t e, uint64_t target) {
    const uint64_t lane = threadIdx.x & 63;
    uint64_t lo = 0, hi = e;
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
        const uint64_t b = wave_lower_bound(rd, e, wave == 0 ? begin : end);
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
            *reinterpret_cast<uint4*>(out.at_wave(i0)) = words8(e0, e1, s0, s1);
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
// Tile decode: the single pass with the words handed out grid-stride.  A
// first kernel indexes the escape stream by 8192-word tile (the first record
// of every tile) and checks the header and the records' order; then a grid
// of two workgroups per CU walks the tiles b, b + gridDim.x, ..., so that
// the resident workgroups stream one region of memory together instead of
// one contiguous range each (on MI355X: 336-346 us against 375 us for the
// 1 GiB KV tensor).

constexpr int kIndexThreads = 256;
constexpr int kTileThreads = kTileWords / 8;    // 8 words per thread and tile
constexpr uint32_t kTileGroupsPerCu = 2;  // 16-wave workgroups: 8 waves per SIMD

// One workgroup per kIndexTiles consecutive tiles.  Record k is the first of
// the tiles after its predecessor's tile up to its own; the tiles after the
// block's last record get the block's end record.  Every record is checked
// against its predecessor and against the block's words, exactly as in the
// fused decode (neighbouring blocks find the same boundary record), and a
// fault leaves this block's flag set (entries of a faulty container may stay
// unwritten; the tile kernel clamps what it reads).
__global__ __launch_bounds__(kIndexThreads) void k_tile_index(const uint8_t* __restrict__ src,
                                                              uint64_t src_bytes, uint64_t n,
                                                              uint64_t e,
                                                              uint64_t* __restrict__ idx,
                                                              uint32_t* __restrict__ flags) {
    __shared__ uint64_t bounds[2];
    __shared__ uint64_t seg_table[16];
    __shared__ int bad;
    const int t = threadIdx.x;
    const int wave = t >> 6;
    if (t == 0) bad = 0;
    if (blockIdx.x == 0 && t == 0 && !header_ok(src, src_bytes, n, e)) bad = 1;
    const uint64_t esc_off = kPrefixBytes + (n + 1) / 2 + n;
    EscapeReader rd;
    rd.pos_lo = src + esc_off;
    rd.exps = rd.pos_lo + 4 * e;
    rd.aligned = (esc_off & 3) == 0;
    rd.one_segment = n <= (1ull << 32);
    rd.seg_end = seg_table;
    if (t < 16) seg_table[t] = reinterpret_cast<const uint64_t*>(src + 32)[t];
    __syncthreads();

    const uint64_t tiles = (n + kTileWords - 1) / kTileWords;
    const uint64_t t_begin = min_u64((uint64_t)blockIdx.x * kIndexTiles, tiles);
    const uint64_t t_end = min_u64(t_begin + kIndexTiles, tiles);
    const uint64_t nt = t_end - t_begin;  // tiles of this block, <= kIndexTiles
    const uint64_t begin = t_begin * kTileWords;
    const uint64_t end = min_u64(t_end * kTileWords, n);
    if (wave < 2) {
        const uint64_t b = wave_lower_bound(rd, e, wave == 0 ? begin : end);
        if ((t & 63) == 0) bounds[wave] = b;
    }
    __syncthreads();
    const uint64_t k_lo = uniform64(bounds[0]);
    const uint64_t k_hi = uniform64(bounds[1] > k_lo ? bounds[1] : k_lo);
    if (t == 0 && blockIdx.x == gridDim.x - 1) {
        if (bounds[1] != e) bad = 1;  // positions >= n
        idx[tiles] = k_hi;
    }

    // the block-local tile of a record inside the block's words, else nt
    auto local_tile = [&](uint64_t p) -> uint64_t {
        return p >= begin && p < end ? (p - begin) / kTileWords : nt;
    };
    for (uint64_t k = k_lo + t; k <= k_hi; k += kIndexThreads) {
        uint64_t cur = nt;  // k == k_hi: past the block's last tile
        if (k < k_hi) {
            const uint64_t p = rd.position(k);
            cur = local_tile(p);
            if (cur == nt || (k > 0 && !(p > rd.position(k - 1)))) bad = 1;
        }
        const uint64_t prev = k == k_lo ? 0 : local_tile(rd.position(k - 1)) + 1;
        for (uint64_t j = prev; j <= cur && j < nt; j++) idx[t_begin + j] = k;
    }
    __syncthreads();
    if (t == 0) flags[blockIdx.x] = bad ? 1u : 0u;
}

hipError_t launch_tile_index(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                             uint8_t* ws, hipStream_t stream) {
    const TileIndexLayout l = tile_index_layout(n);
    k_tile_index<<<(uint32_t)l.blocks, kIndexThreads, 0, stream>>>(
        src, src_bytes, n, e, reinterpret_cast<uint64_t*>(ws + l.idx_off),
        reinterpret_cast<uint32_t*>(ws + l.flag_off));
    return hipGetLastError();
}

// Workgroup 0 first turns the index blocks' flags into the status word
// (every index workgroup wrote its flag, so nothing needs clearing).  Per
// tile: the codes and sign|mantissa bytes are loaded, the tile's records
// (index entries clamped to [0, E]) mark an LDS exponent map and presence
// bits, and each thread patches and rebuilds its 8 words.
template <bool kAlignedSm, class Words>
__global__ __launch_bounds__(kTileThreads) SZ_EIGHT_WAVE_SGPR_CAP
__attribute__((amdgpu_waves_per_eu(8))) void k_decode_tiles(
    const uint8_t* __restrict__ src, uint64_t n, uint64_t e, const uint64_t* __restrict__ idx,
    const uint32_t* __restrict__ flags, uint32_t blocks, Words out, int32_t* status) {
    __shared__ uint8_t patch_exp[2][kTileWords];
    __shared__ uint32_t patch_bits[2][kTileWords / 32];
    __shared__ uint64_t seg_table[16];
    const int t = threadIdx.x;
    if (blockIdx.x == 0 && status) {
        uint32_t any = 0;
        for (uint32_t b = t; b < blocks; b += kTileThreads) any |= flags[b];
        any = __syncthreads_or(any);
        if (t == 0) *status = out.invalid() ? kStatusInvalid : (any ? kStatusCorrupt : 0);
    }
    if (out.invalid()) return;  // the same for every thread

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

    const uint64_t tiles = (n + kTileWords - 1) / kTileWords;
    const uint64_t whole = n / kTileWords;  // tiles with all kTileWords words
    const uint32_t* pos32 = reinterpret_cast<const uint32_t*>(rd.pos_lo);
    const bool fast_pos = rd.one_segment && rd.aligned;  // a position is its stored u32

    // the tile's escape records into the LDS map: entries clamped to [0, E]
    auto mark = [&](uint64_t tile, uint64_t t0, int parity) {
        const uint64_t ks = min_u64(uniform64(idx[tile]), e);
        const uint64_t ke = min_u64(uniform64(idx[tile + 1]), e);
        if (t < (int)(kTileWords / 32)) patch_bits[parity][t] = 0;
        __syncthreads();
        for (uint64_t q = ks + t; q < ke; q += kTileThreads) {
            const uint64_t d = (fast_pos ? (uint64_t)pos32[q] : rd.position(q)) - t0;
            if (d < kTileWords) {
                patch_exp[parity][d] = rd.exps[q];
                atomicOr(&patch_bits[parity][d >> 5], 1u << (d & 31));
            }
        }
        __syncthreads();
        return (patch_bits[parity][t >> 2] >> (8 * (t & 3))) & 0xFFu;  // this thread's 8 words
    };

    int parity = 0;
    // whole tiles: no per-word checks
    for (uint64_t tile = blockIdx.x; tile < whole; tile += gridDim.x, parity ^= 1) {
        const uint64_t t0 = tile * kTileWords;
        const uint64_t i0 = t0 + (uint64_t)t * 8;
        // a wave's words are 512 consecutive words: one page, whose address
        // (a page-table load for a paged tensor) is looked up before the
        // tile's loads so that its latency overlaps theirs
        uint16_t* words_out = nullptr;
        if constexpr (Words::kPaged) words_out = out.at_wave(i0);
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
        const uint32_t present = mark(tile, t0, parity);
        uint32_t e0, e1;
        exponents8(codes, cb, e0, e1);
        if (present) {
            const uint2 pe = *reinterpret_cast<const uint2*>(&patch_exp[parity][8 * t]);
            e0 = bitselect(bits_to_bytes(present), pe.x, e0);
            e1 = bitselect(bits_to_bytes(present >> 4), pe.y, e1);
        }
        // The tensor is larger than the caches (this form runs from 2^26
        // words), so its lines are written past them: none is left dirty for
        // the next kernel to write back (on MI355X the encode that follows a
        // 1 GiB decode ran 24 us faster, the decode itself 4 us slower).
        if constexpr (!Words::kPaged) words_out = out.at_wave(i0);
        store_streaming(reinterpret_cast<uint4*>(words_out), words8(e0, e1, s0, s1));
    }
    // the last, partial tile, by the workgroup whose turn it is
    if (whole < tiles && blockIdx.x == whole % gridDim.x) {
        const uint64_t t0 = whole * kTileWords;
        const uint32_t present = mark(whole, t0, parity);
        const uint64_t i0 = t0 + (uint64_t)t * 8;
        for (uint32_t k = 0; k < 8 && i0 + k < n; k++) {
            const uint64_t i = i0 + k;
            const uint32_t code = (nib[i / 2] >> (4 * (i & 1))) & 0xFu;
            const uint32_t ex = (present >> k) & 1u ? patch_exp[parity][8 * t + k]
                                                    : codebook_byte(cb, code);
            *out.at(i) = (uint16_t)recombine(sm[i], ex);
        }
    }
}

template <class Words>
hipError_t launch_decode_tiles(const uint8_t* src, uint64_t n, uint64_t e, const uint8_t* ws,
                               Words dst, int32_t* status, int num_cus, hipStream_t stream) {
    const TileIndexLayout l = tile_index_layout(n);
    uint64_t groups = (uint64_t)(num_cus > 0 ? num_cus : 256) * kTileGroupsPerCu;
    if (groups > l.tiles) groups = l.tiles;
    if (groups == 0) groups = 1;  // the status is still written
    const uint64_t* idx = reinterpret_cast<const uint64_t*>(ws + l.idx_off);
    const uint32_t* flags = reinterpret_cast<const uint32_t*>(ws + l.flag_off);
    const bool aligned = ((kPrefixBytes + (n + 1) / 2) & 7) == 0;
    if (aligned)
        k_decode_tiles<true, Words><<<(uint32_t)groups, kTileThreads, 0, stream>>>(
            src, n, e, idx, flags, (uint32_t)l.blocks, dst, status);
    else
        k_decode_tiles<false, Words><<<(uint32_t)groups, kTileThreads, 0, stream>>>(
            src, n, e, idx, flags, (uint32_t)l.blocks, dst, status);
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
constexpr int kGroups = 4;                                 // 8-word groups per thread
constexpr uint32_t kGroupStride = 8 * kDenseThreads;       // words between a thread's groups
constexpr uint32_t kDenseTile = kGroups * kGroupStride;    // words per sub-range
constexpr uint32_t kMapEscaped = 0x100u;                   // map entry: 0x100 | exponent
constexpr uint32_t kNoBreak = 0xFFFFFFFFu;
constexpr int kWalk = 2;                                   // records per thread and step
static_assert((1u << 14) % kDenseTile == 0, "ranges of at least 2^14 words hold whole sub-ranges");

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

// Eight waves per SIMD (four workgroups per CU) need at most 64 VGPRs and
// the scalar-register cap.
template <bool kAlignedSm, class Words>
__global__ __launch_bounds__(kDenseThreads) SZ_EIGHT_WAVE_SGPR_CAP
__attribute__((amdgpu_waves_per_eu(8))) void k_decode_dense(
    const uint8_t* __restrict__ src, uint64_t src_bytes, uint64_t n, uint64_t e,
    uint32_t range_log2, Words out, int32_t* status) {
    __shared__ uint4 map4[kDenseTile / 8];   // kDenseTile 16-bit entries
    __shared__ uint64_t bounds[2];
    __shared__ uint64_t seg_table[16];
    __shared__ uint32_t next_rel[2];
    __shared__ int bad;

    const int t = threadIdx.x;
    const int wave = t >> 6;
    uint16_t* map = reinterpret_cast<uint16_t*>(map4);
    if (out.invalid()) {  // the same for every thread
        if (blockIdx.x == 0 && t == 0 && status)
            __hip_atomic_fetch_max(status, kStatusInvalid, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    if (t == 0) {
        bad = 0;
        next_rel[0] = kNoBreak;
        next_rel[1] = kNoBreak;
    }
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
    __syncthreads();

    const uint64_t begin = min_u64((uint64_t)blockIdx.x << range_log2, n);
    const uint64_t end = min_u64(begin + (uint64_t{1} << range_log2), n);

    // escapes of this range: [k_lo, k_hi)
    if (wave < 2) {
        const uint64_t b = wave_lower_bound(rd, e, wave == 0 ? begin : end);
        if ((t & 63) == 0) bounds[wave] = b;
    }
    __syncthreads();
    const uint64_t k_lo = uniform64(bounds[0]);
    const uint64_t k_hi = uniform64(bounds[1] > k_lo ? bounds[1] : k_lo);
    if (t == 0 && blockIdx.x == gridDim.x - 1 && bounds[1] != e) bad = 1;  // positions >= n

    uint64_t k_cur = k_lo;   // first record not yet placed
    int parity = 0;
    for (uint64_t sub = begin; sub < end; sub += kDenseTile, parity ^= 1) {
        const uint64_t sub_end = min_u64(sub + kDenseTile, end);
        // place this sub-range's records; a record at or above sub_end ends
        // the thread's walk, and the lowest such index is where the next
        // sub-range starts.  A sub-range lies inside one 2^32-word segment,
        // whose records are [seg_lo, seg_hi): there a position is its stored
        // low 32 bits above the segment base.
        const uint32_t seg = (uint32_t)(sub >> 32);
        const uint64_t seg_lo = seg == 0 ? 0 : seg_table[seg - 1];
        const uint64_t seg_hi = seg_table[seg];
        const uint32_t lo_begin = (uint32_t)sub;
        const uint64_t lo_end = sub_end - ((uint64_t)seg << 32);  // at most 2^32
        // kWalk records per thread and step, their loads issued together
        uint32_t stop = kNoBreak;
        const uint64_t k_start = k_cur + t;
        for (uint64_t kb = k_start; kb < k_hi && stop == kNoBreak;
             kb += (uint64_t)kWalk * kDenseThreads) {
            uint32_t lo[kWalk], prev[kWalk], ex[kWalk];
#pragma unroll
            for (int u = 0; u < kWalk; u++) {
                const uint64_t k = kb + (uint64_t)u * kDenseThreads;
                const bool in = k < k_hi;
                lo[u] = in ? rd.low32(k) : 0u;
                prev[u] = in && k > 0 ? rd.low32(k - 1) : 0u;
                ex[u] = in ? rd.exps[k] : 0u;
            }
#pragma unroll
            for (int u = 0; u < kWalk; u++) {
                const uint64_t k = kb + (uint64_t)u * kDenseThreads;
                if (stop != kNoBreak || k >= k_hi) break;
                if (k >= seg_hi || lo[u] >= lo_end) {  // beyond this sub-range
                    stop = (uint32_t)min_u64(k - k_cur, kNoBreak - 1);
                    break;
                }
                // not below this sub-range, and strictly above the record
                // before (which, in an earlier segment, is below it anyway)
                if (k < seg_lo || lo[u] < lo_begin ||
                    (k > 0 && k - 1 >= seg_lo && !(lo[u] > prev[u]))) {
                    bad = 1;
                } else {
                    map[lo[u] - lo_begin] = (uint16_t)(kMapEscaped | ex[u]);
                }
            }
        }
        // this thread's codes and sign|mantissa bytes: loaded after the walk,
        // so that the walk does not hold them in registers; they arrive while
        // the other waves finish walking
        const bool whole = sub + kDenseTile <= end;   // the same for every thread
        const uint64_t wt = sub + (uint64_t)t * 8;  // this thread's first word
        uint32_t c[kGroups], s[2 * kGroups];
#pragma unroll
        for (int g = 0; g < kGroups; g++) {
            const uint64_t w = wt + (uint64_t)g * kGroupStride;
            c[g] = s[2 * g] = s[2 * g + 1] = 0;
            if (whole || w + 8 <= sub_end) load_group<kAlignedSm>(nib, sm, w, c[g], s[2 * g], s[2 * g + 1]);
        }

        if (stop != kNoBreak) atomicMin(&next_rel[parity], stop);
        __syncthreads();
        const uint32_t rel = next_rel[parity];
        k_cur = rel == kNoBreak ? k_hi : k_cur + rel;
        if (t == 0) next_rel[parity ^ 1] = kNoBreak;

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
                *reinterpret_cast<uint4*>(out.at(sub) + (w - sub)) =
                    words8(e0, e1, s[2 * g], s[2 * g + 1]);
            } else if (w < sub_end) {  // the input's last, partial group
                for (uint64_t i = w; i < sub_end; i++) {
                    const uint32_t code = (nib[i / 2] >> (4 * (i & 1))) & 0xFu;
                    const uint32_t m = map[(uint32_t)(i - sub)];
                    map[(uint32_t)(i - sub)] = 0;
                    const uint32_t ex = (m & kMapEscaped) ? (m & 0xFFu) : codebook_byte(cb, code);
                    *out.at(i) = (uint16_t)recombine(sm[i], ex);
                }
            }
        }
        __syncthreads();
    }
    // every record of the range must have been placed
    if (t == 0 && k_cur != k_hi) bad = 1;
    __syncthreads();
    if (t == 0 && bad && status)
        __hip_atomic_fetch_max(status, kStatusCorrupt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class Words>
hipError_t launch_decode_dense(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                               Words dst, int32_t* status, hipStream_t stream) {
    uint32_t r = 14;
    // at most kMaxDecodeRanges workgroups: enough for several waves of
    // resident workgroups (a 10.7 GB input with 2048 ranges left the last
    // wave a quarter full: 16% slower)
    while (r < 40 && ((n + (1ull << r) - 1) >> r) > kMaxDecodeRanges) r++;
    uint64_t blocks = (n + (1ull << r) - 1) >> r;
    if (blocks == 0) blocks = 1;  // the header check still runs
    if (status) k_status_clear<<<1, 1, 0, stream>>>(status);
    // the sign|mantissa stream starts at 176 + ceil(n/2): 8-byte aligned
    // exactly when n is a multiple of 16
    const bool aligned = ((kPrefixBytes + (n + 1) / 2) & 7) == 0;
    if (aligned)
        k_decode_dense<true, Words><<<(uint32_t)blocks, kDenseThreads, 0, stream>>>(
            src, src_bytes, n, e, r, dst, status);
    else
        k_decode_dense<false, Words><<<(uint32_t)blocks, kDenseThreads, 0, stream>>>(
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

}  // namespace sz
