/*
 * szref.c -- CPU oracle for the SplitZip BF16 container (test infrastructure
 * only; see szref.h for the format and for who may use this file).
 *
 * Plain C99, one thread, integer arithmetic only.  Every step is written in
 * the order the SplitZip explainer gives it, without blocking or fusion, so
 * that it can be checked against the pages by eye:
 *   encode: split fields -> exponent histogram -> top-16 codebook ->
 *           per element: 4-bit code (two per byte), sign|mantissa byte,
 *           escape record for exponents outside the codebook -> header;
 *   decode: check header -> per element: code -> exponent, recombine with
 *           sign|mantissa -> overwrite every escaped slot.
 */
#include "szref.h"

#include <stdlib.h>
#include <string.h>

#define HEADER_BYTES 160u
#define CODEBOOK_BYTES 16u
#define PREFIX_BYTES (HEADER_BYTES + CODEBOOK_BYTES)
#define MAGIC 0x564B5A53u
#define VERSION 1u
#define ELEMENT_BF16 1u
#define MAX_ELEMENTS (1ull << 36)
#define SEGMENTS 16u

/* ---- little-endian field access (reading: the container is little-endian) */

static void put_u16(uint8_t *p, uint16_t v) {
    p[0] = (uint8_t)(v & 0xFF);
    p[1] = (uint8_t)(v >> 8);
}
static void put_u32(uint8_t *p, uint32_t v) {
    for (int i = 0; i < 4; i++) p[i] = (uint8_t)((v >> (8 * i)) & 0xFF);
}
static void put_u64(uint8_t *p, uint64_t v) {
    for (int i = 0; i < 8; i++) p[i] = (uint8_t)((v >> (8 * i)) & 0xFF);
}
static uint16_t get_u16(const uint8_t *p) {
    return (uint16_t)(p[0] | (p[1] << 8));
}
static uint32_t get_u32(const uint8_t *p) {
    uint32_t v = 0;
    for (int i = 3; i >= 0; i--) v = (v << 8) | p[i];
    return v;
}
static uint64_t get_u64(const uint8_t *p) {
    uint64_t v = 0;
    for (int i = 7; i >= 0; i--) v = (v << 8) | p[i];
    return v;
}

/* ---- the three fields of a BF16 word (explainer section "1. La structure
 * de la Note": sign, mantissa, exponent).  BF16 = 1 sign bit (15),
 * 8 exponent bits (14..7), 7 mantissa bits (6..0). */

static unsigned bf16_sign(uint16_t w) { return (w >> 15) & 1u; }
static unsigned bf16_exponent(uint16_t w) { return (w >> 7) & 0xFFu; }
static unsigned bf16_mantissa(uint16_t w) { return w & 0x7Fu; }

/* Reading: the sign|mantissa byte keeps the sign in bit 7 and the mantissa
 * in bits 6..0, i.e. the word with its exponent field removed. */
static uint8_t sign_mantissa_byte(uint16_t w) {
    return (uint8_t)((bf16_sign(w) << 7) | bf16_mantissa(w));
}

/* Decoding bullet of section "4. Pourquoi est-ce rapide ?": put the
 * exponent back between sign and mantissa. */
static uint16_t recombine(uint8_t sm, unsigned exponent) {
    unsigned sign = (sm >> 7) & 1u;
    unsigned mantissa = sm & 0x7Fu;
    return (uint16_t)((sign << 15) | (exponent << 7) | mantissa);
}

/* ---- sizes ---------------------------------------------------------------- */

uint64_t szref_container_size(uint64_t n, uint64_t e) {
    uint64_t nibble_bytes = (n + 1) / 2; /* two 4-bit codes per byte */
    uint64_t sm_bytes = n;               /* one sign|mantissa byte each */
    uint64_t escape_bytes = 5 * e;       /* u32 position + u8 exponent */
    return PREFIX_BYTES + nibble_bytes + sm_bytes + escape_bytes;
}

/* The 16 largest of 256 counts that sum to n hold at least 16n/256 = n/16
 * of the elements, so at most n - ceil(n/16) = floor(15n/16) escape. */
uint64_t szref_max_compressed_size(uint64_t n) {
    if (n > MAX_ELEMENTS) return 0;
    return szref_container_size(n, (15 * n) / 16);
}

/* ---- step 1: exponent histogram (section "2. La decouverte secrete":
 * the exponents repeat, so count them) ------------------------------------ */

void szref_exponent_histogram(const uint16_t *words, uint64_t n, uint64_t hist[256]) {
    for (int x = 0; x < 256; x++) hist[x] = 0;
    for (uint64_t i = 0; i < n; i++) hist[bf16_exponent(words[i])] += 1;
}

/* ---- step 2: the top-16 list (section "3. La strategie SplitZip",
 * shortcut bullet).  Reading: all 256 exponent values are ranked, most
 * frequent first, equal counts broken toward the smaller exponent, and the
 * code of an exponent is its rank.  Absent exponents rank after present
 * ones, so with fewer than 16 distinct exponents the remaining slots hold
 * the smallest absent values. */

static int ranks_before(const uint64_t hist[256], unsigned a, unsigned b) {
    if (hist[a] != hist[b]) return hist[a] > hist[b];
    return a < b;
}

void szref_select_codebook(const uint64_t hist[256], uint8_t codebook[16]) {
    unsigned order[256];
    for (unsigned x = 0; x < 256; x++) order[x] = x;
    /* insertion sort of the 256 exponent values by the ranking above */
    for (unsigned i = 1; i < 256; i++) {
        unsigned v = order[i];
        unsigned j = i;
        while (j > 0 && ranks_before(hist, v, order[j - 1])) {
            order[j] = order[j - 1];
            j--;
        }
        order[j] = v;
    }
    for (unsigned c = 0; c < 16; c++) codebook[c] = (uint8_t)order[c];
}

/* ---- escape positions above 2^32 (reading: positions are stored as u32;
 * a 16-entry table in the header tells which 2^32-element segment each
 * escape falls in) ----------------------------------------------------- */

void szref_segment_table(const uint64_t *positions, uint64_t n_escapes,
                         uint64_t seg_end[16]) {
    uint64_t per_segment[SEGMENTS];
    for (unsigned s = 0; s < SEGMENTS; s++) per_segment[s] = 0;
    for (uint64_t k = 0; k < n_escapes; k++) per_segment[positions[k] >> 32] += 1;
    uint64_t running = 0;
    for (unsigned s = 0; s < SEGMENTS; s++) {
        running += per_segment[s];
        seg_end[s] = running;
    }
}

uint64_t szref_escape_position(const uint64_t seg_end[16], uint64_t k, uint32_t pos_lo) {
    uint64_t segment = 0;
    for (unsigned s = 0; s < SEGMENTS; s++)
        if (seg_end[s] <= k) segment += 1;
    return (segment << 32) | (uint64_t)pos_lo;
}

/* ---- encode ------------------------------------------------------------- */

int szref_encode(const uint16_t *words, uint64_t n, uint8_t *dst, uint64_t cap,
                 uint64_t *out_bytes) {
    if (n > MAX_ELEMENTS) return SZREF_ERR_TOO_LARGE;
    if (dst == NULL || (n > 0 && words == NULL)) return SZREF_ERR_INVALID_ARGUMENT;

    /* exponent histogram and top-16 codebook */
    uint64_t hist[256];
    uint8_t codebook[16];
    szref_exponent_histogram(words, n, hist);
    szref_select_codebook(hist, codebook);

    /* code of every exponent value; -1 = not in the codebook (escape) */
    int code_of[256];
    for (int x = 0; x < 256; x++) code_of[x] = -1;
    for (int c = 0; c < 16; c++) code_of[codebook[c]] = c;

    /* escapes = elements whose exponent is outside the codebook */
    uint64_t e = 0;
    for (int x = 0; x < 256; x++)
        if (code_of[x] < 0) e += hist[x];

    uint64_t total = szref_container_size(n, e);
    if (cap < total) return SZREF_ERR_CAPACITY;

    uint8_t *nibbles = dst + PREFIX_BYTES;
    uint8_t *sm = nibbles + (n + 1) / 2;
    uint8_t *pos_lo = sm + n;
    uint8_t *exps = pos_lo + 4 * e;
    uint64_t *positions = NULL;
    if (e > 0) {
        positions = (uint64_t *)malloc(e * sizeof(uint64_t));
        if (positions == NULL) return SZREF_ERR_INVALID_ARGUMENT;
    }

    /* reading: an odd element count leaves the last high nibble at 0 */
    if (n % 2 == 1) nibbles[n / 2] = 0;

    uint64_t k = 0;
    for (uint64_t i = 0; i < n; i++) {
        uint16_t w = words[i];
        unsigned x = bf16_exponent(w);
        /* reading: an escaped element writes code 0; its slot is fixed up
         * by the escape stream on decode */
        unsigned code = code_of[x] >= 0 ? (unsigned)code_of[x] : 0u;
        if (i % 2 == 0)
            nibbles[i / 2] = (uint8_t)code;
        else
            nibbles[i / 2] = (uint8_t)(nibbles[i / 2] | (code << 4));
        sm[i] = sign_mantissa_byte(w);
        if (code_of[x] < 0) {
            positions[k] = i;
            put_u32(pos_lo + 4 * k, (uint32_t)(i & 0xFFFFFFFFull));
            exps[k] = (uint8_t)x;
            k += 1;
        }
    }

    uint64_t seg_end[SEGMENTS];
    szref_segment_table(positions, e, seg_end);
    free(positions);

    put_u32(dst + 0, MAGIC);
    put_u16(dst + 4, VERSION);
    put_u16(dst + 6, ELEMENT_BF16);
    put_u64(dst + 8, n);
    put_u64(dst + 16, e);
    put_u64(dst + 24, total);
    for (unsigned s = 0; s < SEGMENTS; s++) put_u64(dst + 32 + 8 * s, seg_end[s]);
    for (unsigned c = 0; c < 16; c++) dst[HEADER_BYTES + c] = codebook[c];

    if (out_bytes != NULL) *out_bytes = total;
    return SZREF_OK;
}

/* ---- decode ------------------------------------------------------------- */

int szref_decode(const uint8_t *src, uint64_t src_bytes, uint16_t *words, uint64_t n) {
    if (n > MAX_ELEMENTS) return SZREF_ERR_TOO_LARGE;
    if (src == NULL || (n > 0 && words == NULL)) return SZREF_ERR_INVALID_ARGUMENT;

    /* header checks */
    if (src_bytes < PREFIX_BYTES) return SZREF_ERR_CORRUPT;
    if (get_u32(src + 0) != MAGIC) return SZREF_ERR_CORRUPT;
    if (get_u16(src + 4) != VERSION) return SZREF_ERR_CORRUPT;
    if (get_u16(src + 6) != ELEMENT_BF16) return SZREF_ERR_CORRUPT;
    if (get_u64(src + 8) != n) return SZREF_ERR_CORRUPT;
    uint64_t e = get_u64(src + 16);
    if (e > n) return SZREF_ERR_CORRUPT;
    uint64_t total = get_u64(src + 24);
    if (total != src_bytes || total != szref_container_size(n, e)) return SZREF_ERR_CORRUPT;

    uint64_t seg_end[SEGMENTS];
    for (unsigned s = 0; s < SEGMENTS; s++) seg_end[s] = get_u64(src + 32 + 8 * s);
    /* segments are counted cumulatively, and no escape may lie in a
     * segment at or past the one holding element n-1 */
    uint64_t segments_used = (n + 0xFFFFFFFFull) >> 32; /* ceil(n / 2^32) */
    for (unsigned s = 0; s < SEGMENTS; s++) {
        if (s > 0 && seg_end[s] < seg_end[s - 1]) return SZREF_ERR_CORRUPT;
        if ((uint64_t)s + 1 >= segments_used && seg_end[s] != e) return SZREF_ERR_CORRUPT;
    }

    const uint8_t *codebook = src + HEADER_BYTES;
    const uint8_t *nibbles = src + PREFIX_BYTES;
    const uint8_t *sm = nibbles + (n + 1) / 2;
    const uint8_t *pos_lo = sm + n;
    const uint8_t *exps = pos_lo + 4 * e;

    /* every element: code -> exponent -> word */
    for (uint64_t i = 0; i < n; i++) {
        unsigned byte = nibbles[i / 2];
        unsigned code = (i % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
        words[i] = recombine(sm[i], codebook[code]);
    }

    /* every escape: overwrite its slot with the stored exponent */
    uint64_t previous = 0;
    for (uint64_t k = 0; k < e; k++) {
        uint64_t p = szref_escape_position(seg_end, k, get_u32(pos_lo + 4 * k));
        if (p >= n) return SZREF_ERR_CORRUPT;
        if (k > 0 && p <= previous) return SZREF_ERR_CORRUPT;
        words[p] = recombine(sm[p], exps[k]);
        previous = p;
    }
    return SZREF_OK;
}
