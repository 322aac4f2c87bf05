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

// The 16-byte codebook held in registers as two 64-bit halves.
struct Codebook {
    uint64_t lo;  // codes 0..7
    uint64_t hi;  // codes 8..15
};

__device__ __forceinline__ Codebook load_codebook(const uint8_t* src) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + kHeaderBytes);
    return Codebook{(uint64_t)v.x | ((uint64_t)v.y << 32), (uint64_t)v.z | ((uint64_t)v.w << 32)};
}

// exponent of code c (0..15); the half is chosen with a mask rather than a
// branch or select so that the codebook stays in registers
__device__ __forceinline__ uint32_t codebook_exponent(Codebook cb, uint32_t c) {
    const uint64_t take_hi = 0ull - (uint64_t)((c >> 3) & 1u);
    const uint64_t half = cb.lo ^ ((cb.lo ^ cb.hi) & take_hi);
    return (uint32_t)(half >> (8 * (c & 7u))) & 0xFFu;
}

// sign in bit 7 and mantissa in bits 6..0 of sm, exponent between them
__device__ __forceinline__ uint32_t recombine(uint32_t sm, uint32_t e) {
    return ((sm & 0x80u) << 8) | (e << 7) | (sm & 0x7Fu);
}

// Two words from one nibble byte (low nibble = first word) and two
// sign|mantissa bytes (low byte = first word); returns them as one dword.
__device__ __forceinline__ uint32_t word_pair(uint32_t code_byte, uint32_t sm_pair,
                                              Codebook cb) {
    const uint32_t lo = recombine(sm_pair & 0xFFu, codebook_exponent(cb, code_byte & 0xFu));
    const uint32_t hi =
        recombine((sm_pair >> 8) & 0xFFu, codebook_exponent(cb, (code_byte >> 4) & 0xFu));
    return lo | (hi << 16);
}

__device__ __forceinline__ uint32_t load4_unaligned(const uint8_t* q) {
    return (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) |
           ((uint32_t)q[3] << 24);
}

__device__ __forceinline__ uint4 load16_unaligned(const uint8_t* q) {
    return make_uint4(load4_unaligned(q), load4_unaligned(q + 4), load4_unaligned(q + 8),
                      load4_unaligned(q + 12));
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

    const Codebook cb = load_codebook(src);
    const uint8_t* nib = src + kPrefixBytes;
    const uint8_t* sm = nib + (n + 1) / 2;

    const uint64_t groups = n / 16;  // 16 words per thread step
    const uint64_t stride = (uint64_t)gridDim.x * kUnpackThreads;
    for (uint64_t g = (uint64_t)blockIdx.x * kUnpackThreads + threadIdx.x; g < groups; g += stride) {
        const uint2 c = *reinterpret_cast<const uint2*>(nib + 8 * g);
        const uint4 s = kAlignedSm ? *reinterpret_cast<const uint4*>(sm + 16 * g)
                                   : load16_unaligned(sm + 16 * g);
        uint4* dst = reinterpret_cast<uint4*>(out + 16 * g);
        dst[0] = make_uint4(word_pair(c.x, s.x, cb), word_pair(c.x >> 8, s.x >> 16, cb),
                            word_pair(c.x >> 16, s.y, cb), word_pair(c.x >> 24, s.y >> 16, cb));
        dst[1] = make_uint4(word_pair(c.y, s.z, cb), word_pair(c.y >> 8, s.z >> 16, cb),
                            word_pair(c.y >> 16, s.w, cb), word_pair(c.y >> 24, s.w >> 16, cb));
    }

    // the last n % 16 words
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = groups * 16 + threadIdx.x; i < n; i += kUnpackThreads) {
            const uint32_t code = (nib[i / 2] >> (4 * (i & 1))) & 0xFu;
            out[i] = (uint16_t)recombine(sm[i], codebook_exponent(cb, code));
        }
    }
}

hipError_t launch_unpack(const uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t e,
                         uint16_t* dst, int32_t* status, int num_cus, hipStream_t stream) {
    const uint64_t groups = n / 16;
    uint64_t blocks = (groups + kUnpackThreads - 1) / kUnpackThreads;
    const uint64_t cap = (uint64_t)(num_cus > 0 ? num_cus : 256) * 8;
    if (blocks > cap) blocks = cap;
    if (blocks == 0) blocks = 1;  // header check and tail still run
    const bool aligned = ((kPrefixBytes + (n + 1) / 2) & 15) == 0;
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
    const uint8_t* sm = src + kPrefixBytes + (n + 1) / 2;
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
    out[p] = (uint16_t)recombine(sm[p], exps[k]);
}

hipError_t launch_scatter(const uint8_t* src, uint64_t n, uint64_t e, uint16_t* dst,
                          int32_t* status, hipStream_t stream) {
    if (e == 0) return hipSuccess;
    const uint64_t blocks = (e + kScatterThreads - 1) / kScatterThreads;
    k_scatter<<<(uint32_t)blocks, kScatterThreads, 0, stream>>>(src, n, e, dst, status);
    return hipGetLastError();
}

}  // namespace sz
