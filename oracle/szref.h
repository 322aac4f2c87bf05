/*
 * szref.h -- CPU oracle for the SplitZip BF16 container.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, single-threaded
 * reference that the GPU codec is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product library never links, loads or calls it, and it shares no code,
 * header, table or constant with the product.
 *
 * What it computes follows the SplitZip explainers (gist.science, arXiv
 * 2605.01708, French and Japanese pages, same title "SplitZip: Ultra Fast
 * Lossless KV Compression for Disaggregated LLM Serving"):
 *   - a BF16 word is split into sign, exponent and mantissa
 *     (section "1. La structure de la Note");
 *   - the 16 most frequent exponents form a codebook, each gets a fixed
 *     4-bit code, and two codes share one byte
 *     (section "3. La strategie SplitZip", bullets on the shortcut and the
 *     packing);
 *   - every other exponent is kept as a (position, exponent) escape record
 *     (same section, bullet on the list of rare values);
 *   - decode looks each code up, recombines it with sign and mantissa and
 *     then overwrites the escaped slots (section "4. Pourquoi est-ce
 *     rapide ?", decoding bullet);
 *   - the round trip is bit-exact (section "Les Resultats").
 * Where the pages leave a choice open (byte layout, tie-breaks, header),
 * this file takes the readings listed in the design notes; each function
 * below names the ones it relies on.
 *
 * Container, little-endian, no padding:
 *   off 0    u32  magic 0x564B5A53 ("SZKV")
 *   off 4    u16  version 1
 *   off 6    u16  element type 1 (bf16)
 *   off 8    u64  N, number of elements
 *   off 16   u64  E, number of escapes
 *   off 24   u64  total container bytes = 176 + ceil(N/2) + N + 5E
 *   off 32   u64  seg_end[16]: escapes whose position is < (s+1) * 2^32
 *   off 160  u8   codebook[16], code c -> exponent
 *   off 176  u8   nibbles[ceil(N/2)]: element 2j low nibble, 2j+1 high
 *   then     u8   sm[N]: sign in bit 7, mantissa in bits 6..0
 *   then     u32  pos_lo[E]: escape position mod 2^32, ascending positions
 *   then     u8   exp[E]: exponent of each escape
 */
#ifndef SZREF_H
#define SZREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SZREF_OK = 0,
    SZREF_ERR_INVALID_ARGUMENT = 1,
    SZREF_ERR_CAPACITY = 2,
    SZREF_ERR_TOO_LARGE = 3,
    SZREF_ERR_CORRUPT = 4
};

/* Largest container any input of n elements can need (E <= floor(15n/16)),
 * or 0 when n exceeds 2^36 elements. */
uint64_t szref_max_compressed_size(uint64_t n);

/* Exact container size for n elements and e escapes. */
uint64_t szref_container_size(uint64_t n, uint64_t e);

/* hist[x] = number of words whose 8-bit exponent field equals x. */
void szref_exponent_histogram(const uint16_t *words, uint64_t n, uint64_t hist[256]);

/* The 16 exponents that come first when all 256 exponent values are
 * ordered by count (descending), ties by exponent value (ascending);
 * codebook[c] is the c-th of them. */
void szref_select_codebook(const uint64_t hist[256], uint8_t codebook[16]);

/* seg_end[s] = number of the given (strictly ascending) escape positions
 * that are below (s+1) * 2^32. */
void szref_segment_table(const uint64_t *positions, uint64_t n_escapes,
                         uint64_t seg_end[16]);

/* Full position of escape k given its stored low 32 bits and seg_end. */
uint64_t szref_escape_position(const uint64_t seg_end[16], uint64_t k,
                               uint32_t pos_lo);

/* Encode n BF16 words into dst (capacity cap bytes).  On success returns
 * SZREF_OK and stores the container size in *out_bytes. */
int szref_encode(const uint16_t *words, uint64_t n, uint8_t *dst, uint64_t cap,
                 uint64_t *out_bytes);

/* Decode a container of src_bytes bytes into n BF16 words.  Returns
 * SZREF_ERR_CORRUPT when the container fails any structural check. */
int szref_decode(const uint8_t *src, uint64_t src_bytes, uint16_t *words, uint64_t n);

#ifdef __cplusplus
}
#endif

#endif /* SZREF_H */
