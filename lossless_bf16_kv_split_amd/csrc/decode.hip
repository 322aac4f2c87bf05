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

// Eight words from one dword of codes (element 2j in the low nibble of byte
// j) and eight sign|mantissa bytes s0 (elements 0..3), s1 (4..7).  Per
// byte lane: high byte of the word = sign | exponent >> 1, low byte =
// (exponent & 1) << 7 | mantissa; then the two byte streams are interleaved.
__device__ __forceinline__ uint4 decode8(uint32_t codes, uint32_t s0, uint32_t s1, uint4 cb) {
    const uint32_t even = lookup4(codes & 0x0F0F0F0Fu, cb);         // elements 0,2,4,6
    const uint32_t odd = lookup4((codes >> 4) & 0x0F0F0F0Fu, cb);   // elements 1,3,5,7
    const uint32_t e0 = perm(odd, even, 0x05010400u);               // elements 0..3
    const uint32_t e1 = perm(odd, even, 0x07030602u);               // elements 4..7
    const uint32_t h0 = bitselect(0x80808080u, s0, e0 >> 1);
    const uint32_t l0 = bitselect(0x80808080u, e0 << 7, s0);
    const uint32_t h1 = bitselect(0x80808080u, s1, e1 >> 1);
    const uint32_t l1 = bitselect(0x80808080u, e1 << 7, s1);
    return make_uint4(perm(h0, l0, 0x05010400u), perm(h0, l0, 0x07030602u),
                      perm(h1, l1, 0x05010400u), perm(h1, l1, 0x07030602u));
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

template <bool kAlignedSm>
__global__ __launch_bounds__(kUnpackThreads) void k_unpack(const uint8_t* __restrict__ src,
                                                          uint64_t src_bytes, uint64_t n,
                                                          uint64_t e,
                                                          uint16_t* __restrict__ out,
                                                          int32_t* status) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && status)
        *status = header_ok(src, src_bytes, n, e) ? 0 : kStatusCorrupt;

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
        *reinterpret_cast<uint4*>(out + 8 * g) = decode8(codes, s0, s1, cb);
    }

    // the last n % 8 words
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = groups * 8 + threadIdx.x; i < n; i += kUnpackThreads) {
            const uint32_t code = (nib[i / 2] >> (4 * (i & 1))) & 0xFu;
            out[i] = (uint16_t)recombine(sm[i], codebook_byte(cb, code));
        }
    }
}

hipError_t launch_unpack(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                         uint16_t* dst, int32_t* status, int num_cus, hipStream_t stream) {
    const uint64_t groups = n / 8;
    uint64_t blocks = (groups + kUnpackThreads - 1) / kUnpackThreads;
    // four workgroups per CU: measured fastest for this read 1.5 / write 2
    // byte stream (more resident waves only add DRAM page conflicts)
    const uint64_t cap = (uint64_t)(num_cus > 0 ? num_cus : 256) * 4;
    if (blocks > cap) blocks = cap;
    if (blocks == 0) blocks = 1;  // header check and tail still run
    const bool aligned = ((kPrefixBytes + (n + 1) / 2) & 7) == 0;
    if (aligned)
        k_unpack<true><<<(uint32_t)blocks, kUnpackThreads, 0, stream>>>(src, src_bytes, n, e,
                                                                       dst, status);
    else
        k_unpack<false><<<(uint32_t)blocks, kUnpackThreads, 0, stream>>>(src, src_bytes, n, e,
                                                                        dst, status);
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

__global__ __launch_bounds__(kScatterThreads) void k_scatter(const uint8_t* __restrict__ src,
                                                            uint64_t n, uint64_t e,
                                                            uint16_t* __restrict__ out,
                                                            int32_t* status) {
    const uint64_t k = (uint64_t)blockIdx.x * kScatterThreads + threadIdx.x;
    if (k >= e) return;
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
    const uint32_t w = out[p];
    out[p] = (uint16_t)((w & 0x807Fu) | ((uint32_t)exps[k] << 7));
}

hipError_t launch_scatter(const uint8_t* src, uint64_t n, uint64_t e, uint16_t* dst,
                          int32_t* status, hipStream_t stream) {
    if (e == 0) return hipSuccess;
    const uint64_t blocks = (e + kScatterThreads - 1) / kScatterThreads;
    k_scatter<<<(uint32_t)blocks, kScatterThreads, 0, stream>>>(src, n, e, dst, status);
    return hipGetLastError();
}

}  // namespace sz
