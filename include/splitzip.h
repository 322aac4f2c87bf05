/*
 * splitzip.h -- C ABI of the MI355X (gfx950) SplitZip BF16 KV-cache codec.
 *
 * The method is the one the SplitZip explainers describe ("SplitZip: Ultra
 * Fast Lossless KV Compression for Disaggregated LLM Serving", gist.science
 * pages for arXiv 2605.01708, French and Japanese): every BF16 word is split
 * into sign, exponent and mantissa (section "1. La structure de la Note");
 * the 16 most frequent exponents of the tensor get fixed 4-bit codes, two
 * codes per byte, and every other exponent is written as a (position,
 * exponent) escape record (section "3. La strategie SplitZip"); decoding
 * looks the codes up, recombines them with sign and mantissa and overwrites
 * the escaped slots (section "4. Pourquoi est-ce rapide ?"); the round trip
 * is bit-exact (section "Les Resultats").
 *
 * Container produced by sz_encode (little-endian, no padding):
 *   off 0    u32  magic 0x564B5A53 (bytes 'S' 'Z' 'K' 'V')
 *   off 4    u16  version 1
 *   off 6    u16  element type 1 (bf16)
 *   off 8    u64  N, number of elements
 *   off 16   u64  E, number of escapes
 *   off 24   u64  total bytes = 176 + ceil(N/2) + N + 5E
 *   off 32   u64  seg_end[16]: number of escapes whose position is below
 *                 (s+1) * 2^32 (escape positions are stored modulo 2^32)
 *   off 160  u8   codebook[16]: code c -> exponent; codes are ranks by count
 *                 (descending), equal counts ordered by exponent (ascending)
 *   off 176  u8   nibbles[ceil(N/2)]: element 2j in the low nibble of byte j,
 *                 element 2j+1 in the high nibble; escaped elements hold 0
 *   +        u8   sm[N]: sign in bit 7, mantissa in bits 6..0
 *   +        u32  pos_lo[E]: escape positions mod 2^32, strictly ascending
 *   +        u8   exp[E]: the exponent of each escape
 *
 * Conventions for every call below:
 *   - Pointers named d_* are device pointers (hipMalloc or a PyTorch CUDA
 *     tensor) owned by the caller; the library keeps none of them after the
 *     stream work completes.  BF16 and container pointers must be 16-byte
 *     aligned; workspaces 256-byte aligned.
 *   - Calls are asynchronous on `stream` and never synchronise the host,
 *     except the two sz_ship_* calls, which return when their data is in
 *     place.  The return value reports errors found on the host before
 *     anything is launched (nothing is launched then), or SZ_ERR_HIP for a
 *     failed launch or allocation.  Results are valid once the stream work
 *     is done.
 *   - Calls on different streams may run concurrently if they use different
 *     buffers.
 */
#ifndef SPLITZIP_H
#define SPLITZIP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SZ_HEADER_BYTES 160u
#define SZ_CODEBOOK_BYTES 16u
#define SZ_PREFIX_BYTES 176u
#define SZ_MAX_ELEMENTS (1ull << 36)

typedef enum {
    SZ_OK = 0,
    SZ_ERR_INVALID_ARGUMENT = 1, /* NULL or misaligned pointer, overlap, bad workspace */
    SZ_ERR_CAPACITY = 2,         /* destination smaller than sz_max_compressed_size(n) */
    SZ_ERR_TOO_LARGE = 3,        /* n > SZ_MAX_ELEMENTS */
    SZ_ERR_CORRUPT = 4,          /* container inconsistent with n or with itself */
    SZ_ERR_HIP = 5               /* a HIP launch or allocation failed */
} sz_status;

/* Upper bound of the container size for n elements: 176 + ceil(n/2) + n +
 * 5*floor(15n/16).  SplitZip explainer section "3. La strategie SplitZip":
 * every exponent gets a fixed 4-bit code stored two per byte (ceil(n/2)
 * bytes), every word keeps its sign and mantissa (n bytes), and an exponent
 * outside the 16-entry list costs one (position, exponent) note (5 bytes
 * here); the 16 most frequent of 256 exponents always cover at least n/16
 * elements, so at most floor(15n/16) words need a note.  Returns 0 when
 * n > SZ_MAX_ELEMENTS.  Host-only, touches no device. */
uint64_t sz_max_compressed_size(uint64_t n_elements);

/* Bytes of device workspace the staged encode calls need for n elements
 * (at most about 4.3 MB).  Host-only. */
uint64_t sz_workspace_size(uint64_t n_elements);

/* Compress n BF16 words at d_src into the container format above at d_dst.
 * SplitZip explainer section "3. La strategie SplitZip" (top-16 exponent
 * codebook, 4-bit codes two per byte, escape records for the rest).
 *   d_src             n little-endian BF16 words (any bit patterns)
 *   d_dst             container buffer, dst_capacity bytes; must be at least
 *                     sz_max_compressed_size(n) (else SZ_ERR_CAPACITY).  The
 *                     container is its first `total bytes`; any byte below
 *                     sz_max_compressed_size(n) may be written (see below),
 *                     none at or past it
 *   d_compressed_size optional device u64 that receives the container size
 *                     (the same value is stored at container offset 24)
 * From 2^26 elements on (sz_encode_single_read(n) says 1) the input is read
 * once when a sample of it predicts the codebook: the bytes of d_dst past the
 * container, up to sz_max_compressed_size(n), then serve as scratch and are
 * left unspecified.  The container is the same either way.
 * Allocates its workspace (sz_workspace_size(n)) from a library-owned,
 * stream-ordered device memory pool and returns it on the same stream.
 * While `stream` is being captured into a graph, returns
 * SZ_ERR_INVALID_ARGUMENT and launches nothing: the staged calls below, with
 * a workspace the caller owns, are the capturable form. */
sz_status sz_encode(const void *d_src, uint64_t n_elements, void *d_dst,
                    uint64_t dst_capacity, uint64_t *d_compressed_size,
                    hipStream_t stream);

/* For callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * sz_encode with the same arguments, passes and container, but its
 * workspace is a fixed array of SZ_NOALLOC_WORKSPACE_BYTES in the library's
 * device memory, one per GPU, loaded with the library and held until the
 * process ends.  The call allocates nothing (no hipMalloc, no pool, no
 * hipFree) and may be captured into a graph.  Every call on one GPU uses
 * that GPU's array: calls that can overlap on one GPU (other streams, or
 * several replays of graphs in flight at once) race and give unspecified
 * containers, so callers serialise them.  No pass needs the array to hold
 * anything at its start (each pass writes what the next one reads).
 * SZ_ERR_TOO_LARGE when n's workspace (sz_workspace_size(n)) exceeds the
 * array; with this library's chunk plan no n up to SZ_MAX_ELEMENTS does. */
#define SZ_NOALLOC_WORKSPACE_BYTES (4608ull * 1024ull)
sz_status sz_encode_noalloc(const void *d_src, uint64_t n_elements, void *d_dst,
                            uint64_t dst_capacity, uint64_t *d_compressed_size,
                            hipStream_t stream);

/* Decompress a container of src_bytes bytes into n BF16 words at d_dst,
 * bit-exactly.  SplitZip explainer section "4. Pourquoi est-ce rapide ?"
 * (code -> exponent lookup, recombination with sign and mantissa, escaped
 * slots overwritten).  The form depends on the size and escape density:
 * from 2^26 words with at most one escape in 128, one pass over grid-stride
 * tiles (sz_decode_index, then sz_decode_tiles, with a workspace from a
 * library-owned stream-ordered pool); below 2^26 words with at most one
 * escape in 256, the two passes sz_decode_unpack and sz_decode_scatter;
 * otherwise, and whenever the stream is being captured into a graph, one
 * pass with a per-word exponent map (sz_decode_dense).  Same result every
 * way.
 *   src_bytes   must equal the container's total size: the host derives E
 *               from it, so no device read is needed before launching
 *   d_status    optional device i32: SZ_OK, or SZ_ERR_CORRUPT when the
 *               header or an escape position fails a check on the device
 *               (d_dst content is then unspecified, but no write ever leaves
 *               d_dst[0..n))
 * Host-side SZ_ERR_CORRUPT: src_bytes < 176 + ceil(n/2) + n, or the rest is
 * not a multiple of 5 bytes, or implies more than floor(15n/16) escapes. */
sz_status sz_decode(const void *d_src, uint64_t src_bytes, void *d_dst,
                    uint64_t n_elements, int32_t *d_status, hipStream_t stream);

/* ---- staged form: the same kernels, one call per pass ------------------
 * sz_encode = sz_encode_histogram; sz_encode_codebook; sz_encode_pack on one
 * stream with one workspace of at least sz_workspace_size(n) bytes that the
 * caller owns and does not touch in between.  sz_decode_unpack followed by
 * sz_decode_scatter gives the same words and status as sz_decode.
 * Out-of-order use cannot write outside the caller's buffers, but yields an
 * unspecified result. */

/* Pass 1, exponent histogram (explainer section "2. La decouverte
 * secrete": the exponents are highly repetitive): one 256-bin count per
 * fixed-size chunk of the input, into the workspace. */
sz_status sz_encode_histogram(const void *d_src, uint64_t n_elements,
                              void *d_workspace, uint64_t workspace_bytes,
                              hipStream_t stream);

/* Pass 2, top-16 selection (section "3. La strategie SplitZip", shortcut
 * bullet): merges the chunk counts, ranks the 256 exponents, writes the
 * header and codebook to d_dst, the escape offset of every chunk to the
 * workspace and the container size to *d_compressed_size (optional). */
sz_status sz_encode_codebook(uint64_t n_elements, void *d_workspace,
                             uint64_t workspace_bytes, void *d_dst,
                             uint64_t dst_capacity, uint64_t *d_compressed_size,
                             hipStream_t stream);

/* Pass 3, packing (same section, packing and rare-value bullets): 4-bit
 * codes two per byte, sign|mantissa bytes, and the escape records of each
 * chunk written to their final slots in ascending position order. */
sz_status sz_encode_pack(const void *d_src, uint64_t n_elements,
                         const void *d_workspace, uint64_t workspace_bytes,
                         void *d_dst, uint64_t dst_capacity, hipStream_t stream);

/* Passes 2 and 3 in one launch, after sz_encode_histogram, for
 * 1 <= n_elements <= 2^21 (at most 128 chunks of the plan; otherwise
 * SZ_ERR_INVALID_ARGUMENT): every pack workgroup sums and ranks the chunk
 * counts itself (the selection of section "3. La strategie SplitZip") and
 * works out its chunk's first escape slot, so no codebook pass runs between
 * the two launches.  Writes the same container as sz_encode_codebook then
 * sz_encode_pack, and the container size to *d_compressed_size (optional);
 * sz_encode takes this form for such n.  Same arguments and checks as
 * sz_encode_pack. */
sz_status sz_encode_pack_ranked(const void *d_src, uint64_t n_elements,
                                const void *d_workspace, uint64_t workspace_bytes,
                                void *d_dst, uint64_t dst_capacity,
                                uint64_t *d_compressed_size, hipStream_t stream);

/* ---- staged form of the single-read encode (n >= 2^20) -----------------
 * sz_encode_sample; sz_encode_first_pass; sz_encode_finish on one stream,
 * one workspace, gives the container of sz_encode.  Not part of the pages'
 * method: a way to read the input once.  A fixed sample (512 blocks of 2048
 * words spread evenly over the input) gives a provisional codebook by the
 * same ranking rule; the first pass packs every chunk with it while it
 * takes the exact counts; the finish pass ranks the exact codebook, then
 * keeps what the first pass wrote when the exact codebook equals the
 * provisional one, rewrites the 4-bit codes when it holds the same 16
 * exponents in another order, and packs again (a second read) otherwise,
 * or when a chunk held more than 1/16 escapes, or when the sample predicted
 * more than one escape in 32.  The workspace may hold any bytes before the
 * first call: every call gives the same container (the first call on a
 * workspace in an unknown state may take the slower finish).
 * These calls return SZ_ERR_INVALID_ARGUMENT for n < 2^20 (besides the
 * checks of the two-read calls); the first pass and the finish use the bytes
 * of d_dst past the container, up to sz_max_compressed_size(n), as scratch. */

/* 1 when sz_encode takes the single-read passes for n elements (n >= 2^26),
 * else 0.  Host-only. */
int sz_encode_single_read(uint64_t n_elements);

/* The sample's exponent counts, then the provisional codebook and whether
 * the first pass packs, into the workspace. */
sz_status sz_encode_sample(const void *d_src, uint64_t n_elements, void *d_workspace,
                           uint64_t workspace_bytes, hipStream_t stream);

/* The first pass: the exact per-chunk exponent counts to the workspace (laid
 * out for sz_encode_finish, not for sz_encode_codebook) and, when the sample
 * predicts few escapes, the nibble and sign|mantissa streams plus each
 * chunk's escape records (to the scratch area). */
sz_status sz_encode_first_pass(const void *d_src, uint64_t n_elements,
                               void *d_workspace, uint64_t workspace_bytes,
                               void *d_dst, uint64_t dst_capacity, hipStream_t stream);

/* The exact codebook (the selection of section "3. La strategie SplitZip",
 * as sz_encode_codebook takes it), the header, and the container size to
 * *d_compressed_size (optional); then escape records to their final slots,
 * codes rewritten, or the input packed again, as described above. */
sz_status sz_encode_finish(const void *d_src, uint64_t n_elements,
                           void *d_workspace, uint64_t workspace_bytes,
                           void *d_dst, uint64_t dst_capacity,
                           uint64_t *d_compressed_size, hipStream_t stream);

/* Decode pass 1: header check (sets *d_status to SZ_OK or SZ_ERR_CORRUPT)
 * and every word rebuilt from its code and its sign|mantissa byte. */
sz_status sz_decode_unpack(const void *d_src, uint64_t src_bytes, void *d_dst,
                           uint64_t n_elements, int32_t *d_status,
                           hipStream_t stream);

/* Decode pass 2: every escape record overwrites the exponent field of the
 * word pass 1 wrote at its position; a position >= n or not above the
 * previous one raises *d_status to SZ_ERR_CORRUPT and is skipped.  Launches
 * nothing when E = 0. */
sz_status sz_decode_scatter(const void *d_src, uint64_t src_bytes, void *d_dst,
                            uint64_t n_elements, int32_t *d_status,
                            hipStream_t stream);

/* Decode in a single pass whatever the escape density: each workgroup
 * finds its range's escape records by a 64-way search over the sorted
 * positions, stages them in LDS and overwrites the escaped exponents before
 * the words are stored (explainer section "4. Pourquoi est-ce rapide ?").
 * Same arguments, result and status as sz_decode. */
sz_status sz_decode_fused(const void *d_src, uint64_t src_bytes, void *d_dst,
                          uint64_t n_elements, int32_t *d_status, hipStream_t stream);

/* Decode in a single pass, laid out for many escapes: each workgroup walks
 * its range in sub-ranges of 16384 words, reads the escape records of each
 * sub-range straight from the escape stream into a per-word LDS map, and
 * rebuilds the words with the mapped exponents in place of the codebook's
 * (explainer section "4. Pourquoi est-ce rapide ?").  Same arguments,
 * result and status as sz_decode, which picks this form above one escape
 * in 128 words, for small tensors above one in 256, and whenever it cannot
 * allocate. */
sz_status sz_decode_dense(const void *d_src, uint64_t src_bytes, void *d_dst,
                          uint64_t n_elements, int32_t *d_status, hipStream_t stream);

/* Decode in a single pass, one short-lived workgroup per 2048-word tile, in
 * two calls over a caller workspace of sz_decode_workspace_size(n) bytes
 * (256-byte aligned, not overlapping the container or the output; about
 * 72 bytes per tile plus 4 bytes per 64 possible escapes, at most 4 MiB of
 * those).  sz_decode_index
 * records, for every tile, the first escape record at or after the tile's
 * start and the tile's first records (each of its waves takes a run of 64
 * records and fills the tile entries up to its last record: no search), and
 * checks the header and that
 * the records ascend below n; sz_decode_tiles then rebuilds every tile's
 * words with its records' exponents in place of the codebook's (explainer
 * section "4. Pourquoi est-ce rapide ?").  sz_decode_tiles writes
 * *d_status (optional): SZ_OK, or SZ_ERR_CORRUPT when the index call found
 * a fault (the output content is then unspecified, but no write leaves
 * d_dst[0..n)); it only reads the workspace, so it may run again on the
 * same index.  The index call also copies each tile's records (up to 15)
 * into a 64-byte slot of the tile, which the tile call reads together with
 * the tile's codes; a tile with more records reads them from the escape
 * stream.  Together they give the result and status of sz_decode, which
 * takes this form, with a workspace from its pool, from 2^26 words with up
 * to one escape in 128. */
uint64_t sz_decode_workspace_size(uint64_t n_elements);
sz_status sz_decode_index(const void *d_src, uint64_t src_bytes, uint64_t n_elements,
                          void *d_workspace, uint64_t workspace_bytes, hipStream_t stream);
sz_status sz_decode_tiles(const void *d_src, uint64_t src_bytes, const void *d_workspace,
                          uint64_t workspace_bytes, void *d_dst, uint64_t n_elements,
                          int32_t *d_status, hipStream_t stream);

/* ---- paged tensors -----------------------------------------------------
 * Serving stacks keep KV caches in fixed-size pages (the explainers'
 * serving setting, section "Les Resultats").  These calls take such a
 * tensor as it lies: n words spread over pages of page_elems words, page i
 * at the device address d_pages[i] (d_pages is a device array of
 * pointers), so that the tensor is the concatenation of the pages in table
 * order (the last page may be partly used).  The container is exactly the
 * one sz_encode gives for that concatenation, so any decode call reads it,
 * and sz_decode_pages decodes any container into pages.  One launch per
 * pass for the whole tensor, whatever the number of pages.
 *   page_elems  a power of two, at least 16384
 *   n_pages     entries in d_pages; only the first ceil(n / page_elems)
 *               are read, each must be non-NULL and 16-byte aligned
 * The table's addresses are checked on the device: a NULL or misaligned
 * one makes the call touch no page and report SZ_ERR_INVALID_ARGUMENT in
 * *d_status (the container is then not valid).  Pages must not overlap
 * each other or the container.  The library allocates a small flag from
 * its stream-ordered pool (and, for encode, sz_encode's workspace), so
 * while `stream` is being captured into a graph both calls return
 * SZ_ERR_INVALID_ARGUMENT and launch nothing. */

/* sz_encode_pages: sz_encode of the paged tensor; *d_status (optional
 * device i32) receives SZ_OK or SZ_ERR_INVALID_ARGUMENT. */
sz_status sz_encode_pages(const void *const *d_pages, uint64_t n_pages, uint64_t page_elems,
                          uint64_t n_elements, void *d_dst, uint64_t dst_capacity,
                          uint64_t *d_compressed_size, int32_t *d_status, hipStream_t stream);

/* sz_decode_pages: sz_decode into the paged tensor (same forms, same
 * checks and status; SZ_ERR_INVALID_ARGUMENT in *d_status for a bad
 * page table). */
sz_status sz_decode_pages(const void *d_src, uint64_t src_bytes, void *const *d_pages,
                          uint64_t n_pages, uint64_t page_elems, uint64_t n_elements,
                          int32_t *d_status, hipStream_t stream);

/* ---- per-layer blocks, one container each -----------------------------
 * A serving stack holds a model's KV cache as one block per layer (the
 * explainers' serving setting, section "Les Resultats"), and each block may
 * travel on its own.  These calls take n_blocks blocks of block_elems words
 * each, block b at the device address d_blocks[b] (a device array of
 * pointers, each non-NULL and 16-byte aligned), and give block b its own
 * container, exactly the one sz_encode gives for that block alone, so that
 * sz_decode reads it too.  One launch per pass for all blocks.
 *   containers  block b's container starts at the container buffer plus
 *               b * pitch bytes (the buffer spans n_blocks * pitch bytes)
 *   d_sizes     device array of n_blocks u64: block b's container size
 *   n_blocks    1 .. 65535
 * Block addresses are checked on the device: a NULL or misaligned one
 * makes the calls touch none of that block's memory and report
 * SZ_ERR_INVALID_ARGUMENT as the block's status; the other blocks are
 * unaffected.  Blocks must not overlap one another or the containers.
 * Neither call allocates, so both may be captured into a graph.
 *
 * sz_blocks_workspace_size: bytes of device workspace sz_encode_blocks
 * needs: for each block, the per-chunk counts and escape bases of a chunk
 * plan made for all the blocks' words together (at most about 4.3 MB a
 * block, much less for small blocks), at 256-byte strides, then a flag
 * word per block; 0 for block_elems > SZ_MAX_ELEMENTS or a block count
 * outside 1 .. 65535.  Host-only. */
uint64_t sz_blocks_workspace_size(uint64_t block_elems, uint64_t n_blocks);

/* sz_encode_blocks: sz_encode of every block, each pass one launch for
 * all blocks, after an address check.  The passes are the ones sz_encode
 * takes for as many words as all blocks hold: from 2^26 words in total,
 * with blocks of at least 2^20 words, the single-read passes (sample,
 * first pass, finish), else the two-read ones (counts, codebook, pack).
 *   d_dst      container buffer, 16-byte aligned; dst_pitch a multiple of
 *              16 and at least sz_max_compressed_size(block_elems), else
 *              SZ_ERR_CAPACITY.  In the single-read form the bytes of a
 *              block's pitch past its container, up to
 *              sz_max_compressed_size(block_elems), serve as scratch and are
 *              left unspecified; no byte past that is written.
 *   d_sizes    written: each block's container size (0 for a block whose
 *              address failed the check)
 *   d_workspace, workspace_bytes   256-byte aligned, at least
 *              sz_blocks_workspace_size(block_elems, n_blocks); it may hold
 *              any bytes when the call starts
 *   d_status   optional device array of n_blocks i32: SZ_OK or
 *              SZ_ERR_INVALID_ARGUMENT per block */
sz_status sz_encode_blocks(const void *const *d_blocks, uint64_t n_blocks, uint64_t block_elems,
                           void *d_dst, uint64_t dst_pitch, uint64_t *d_sizes,
                           void *d_workspace, uint64_t workspace_bytes, int32_t *d_status,
                           hipStream_t stream);

/* sz_blocks_decode_workspace_size: bytes of device workspace that give
 * sz_decode_blocks its tile form (per block: a tile index, a fault flag
 * per 16384 words (64 to 4096 of them) and the tiles' record slots, at
 * 256-byte strides; about 1/30 of the block's words in bytes); 0 for bad
 * arguments as above.  Host-only. */
uint64_t sz_blocks_decode_workspace_size(uint64_t block_elems, uint64_t n_blocks);

/* sz_decode_blocks: the reverse, block b's container read from d_src +
 * b * src_pitch, d_sizes[b] bytes, and its words written to d_blocks[b],
 * with the checks of sz_decode.  A size that is no container of
 * block_elems words, or exceeds src_pitch, counts as corrupt: nothing
 * outside the block's pitch is read, and its words are then unspecified.
 * With d_workspace NULL, one pass per range of each block
 * (sz_decode_dense's form, the one for escape-heavy data); with a
 * workspace of at least sz_blocks_decode_workspace_size(block_elems,
 * n_blocks) bytes (256-byte aligned, any content), a tile index of every
 * block, then its tiles (sz_decode_index / sz_decode_tiles' form, the
 * faster one for KV data, and much the slower one at many escapes per
 * 2048 words).  Both forms are one launch per pass for all blocks.
 *   src_pitch  a multiple of 16, at least 176 + ceil(n/2) + n for
 *              n = block_elems
 *   d_status   required device array of n_blocks i32: SZ_OK, SZ_ERR_CORRUPT
 *              or SZ_ERR_INVALID_ARGUMENT per block */
sz_status sz_decode_blocks(const void *d_src, uint64_t src_pitch, const uint64_t *d_sizes,
                           uint64_t n_blocks, uint64_t block_elems, void *const *d_blocks,
                           void *d_workspace, uint64_t workspace_bytes, int32_t *d_status,
                           hipStream_t stream);

/* ---- compressed transfer to and from host memory ----------------------
 * The explainers present the codec as a way to shrink the KV transfer
 * between prefill and decode servers (introduction and "Les Resultats").
 * These calls wrap it around the transfer one GPU has, the PCIe copy to and
 * from host memory: the n words are cut into chunks of chunk_elems words
 * (the last one shorter), each chunk becomes an ordinary container with its
 * own codebook, and the codec runs on `stream` while earlier chunks'
 * containers are copied on a second stream, through three device staging
 * buffers.  Every call blocks the host until the transfer is complete.
 * Host buffers should be pinned (hipHostMalloc, or a PyTorch tensor with
 * pin_memory=True) for the copies to overlap.
 *
 * A transfer context (sz_ship_context_create) holds the copy stream, the
 * staging buffers and the events for one chunk size on the device current
 * when it is made; the _ctx calls use it and allocate nothing, except that
 * the first decode on a context enlarges its staging buffers to hold a
 * group of chunks (at least 2^24 words' worth, at most 128 MiB a buffer;
 * a decode moves small chunks a group at a time), and a decode with more
 * chunks than any before it grows the per-chunk status array.  A context
 * serves one transfer at a time.  The one-shot calls sz_ship_to_host /
 * sz_ship_from_host make a context, use it and release it.
 *
 * sz_ship_to_host: encode d_src[0..n) chunk by chunk into h_dst.
 *   chunk_elems  > 0, a multiple of 8 (keeps every chunk 16-byte aligned)
 *   h_dst        host buffer of h_capacity bytes; chunk c's container is at
 *                h_dst + h_offsets[c], h_offsets[c+1] - h_offsets[c] bytes
 *   h_offsets    host array of ceil(n / chunk_elems) + 1 entries, written
 * SZ_ERR_CAPACITY when the containers do not fit in h_capacity (found only
 * once a chunk's size is known: h_offsets is then valid up to the chunks
 * shipped before it).  SZ_ERR_INVALID_ARGUMENT for a bad chunk size, NULL
 * or misaligned pointers. */
sz_status sz_ship_to_host(const void *d_src, uint64_t n_elements, uint64_t chunk_elems,
                          void *h_dst, uint64_t h_capacity, uint64_t *h_offsets,
                          hipStream_t stream);

/* sz_ship_from_host: the reverse; h_src and h_offsets as sz_ship_to_host
 * wrote them, the words land in d_dst[0..n).  Returns SZ_ERR_CORRUPT (and
 * writes it to the optional device word *d_status, else SZ_OK there) when
 * an offset is out of order or a chunk's size cannot be a container of its
 * length (checked on the host before anything is copied), or when a chunk
 * fails a device-side check. */
sz_status sz_ship_from_host(const void *h_src, const uint64_t *h_offsets, uint64_t n_elements,
                            uint64_t chunk_elems, void *d_dst, int32_t *d_status,
                            hipStream_t stream);

/* A transfer context for chunks of chunk_elems words (> 0, a multiple of
 * 8) on the current device, to *ctx.  SZ_ERR_INVALID_ARGUMENT for a bad
 * chunk size or NULL ctx, SZ_ERR_HIP when an allocation fails (nothing is
 * then left allocated). */
typedef struct sz_ship_context sz_ship_context;
sz_status sz_ship_context_create(uint64_t chunk_elems, sz_ship_context **ctx);

/* Releases a context (NULL is ignored) after its copies have drained. */
void sz_ship_context_destroy(sz_ship_context *ctx);

/* sz_ship_to_host / sz_ship_from_host over a context, with its chunk size;
 * SZ_ERR_INVALID_ARGUMENT also when the context was made on another device. */
sz_status sz_ship_to_host_ctx(sz_ship_context *ctx, const void *d_src, uint64_t n_elements,
                              void *h_dst, uint64_t h_capacity, uint64_t *h_offsets,
                              hipStream_t stream);
sz_status sz_ship_from_host_ctx(sz_ship_context *ctx, const void *h_src,
                                const uint64_t *h_offsets, uint64_t n_elements, void *d_dst,
                                int32_t *d_status, hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char *sz_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPLITZIP_H */
