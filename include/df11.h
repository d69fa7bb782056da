/*
 * df11.h -- C-ABI of libdf11: DFloat11 (DF11) block encoding on the host and
 * block decoding on an AMD Instinct MI355X (gfx950).
 *
 * What the library computes (from the pages on DFloat11):
 *  - hada.io summary of the DFloat11 paper, section "Le format DFloat11": only
 *    the 8-bit exponent of each BF16 weight is entropy coded, with a Huffman
 *    code built from the exponent distribution; the codes are bit-packed into
 *    an EncodedExponent byte array and the sign and 7-bit mantissa are kept
 *    verbatim in a PackedSignMantissa byte array.
 *  - same page, section "Noyau GPU en deux etapes et metadonnees
 *    auxiliaires": each GPU thread owns 8 consecutive bytes (64 bits) of the
 *    encoded exponents and decodes the codes that start in them; a 5-bit gap
 *    per thread gives the offset of its first code; output positions are
 *    stored only once per group of threads; the kernel counts in a first
 *    phase, prefix-sums the counts, decodes again in a second phase into an
 *    on-chip buffer and writes it out coalesced.
 *  - same page, section "Decompression par bloc transformer": all matrices of
 *    one transformer block are decoded together in one launch.
 *  - chatpaper.ai abstract of the DFloat11 paper: the decoded weights are
 *    bit-for-bit identical to the original BF16 weights.
 *
 * Format version 1 (readings of points the pages leave open):
 *  - A block is the concatenation of its matrices (row-major, in the order
 *    given), with one codebook for the whole block.
 *  - Code lengths: Huffman with ties broken by (weight, creation order), where
 *    leaves are ordered by (count, exponent) and precede merged nodes; if a
 *    code would exceed 32 bits the lengths come from package-merge with cap 32
 *    (a leaf precedes a package of equal weight).  A one-symbol alphabet gets
 *    length 1.
 *  - Canonical codewords: symbols in (length, exponent) order, first code 0,
 *    next = (prev + 1) << (length step).
 *  - Stream bit j is bit (7 - j % 8) of byte j / 8 (MSB first).
 *  - sign_mant[i] = (sign << 7) | mantissa.
 *  - Window w = stream bits [64w, 64w + 64).  gap[w] = first code start at or
 *    after 64w, minus 64w; total_bits - 64w when none (only possible in the
 *    last window).  Always in [0, 31].  Packed as 5-bit fields, MSB first,
 *    field w at bits [5w, 5w + 5).
 *  - Unit u = windows [64u, 64u + 64) (one 64-lane wavefront).
 *    unit_pos[u] = number of codes starting before bit 4096u, for
 *    u < n_units, and unit_pos[n_units] = n_total.
 *  - Section sizes: stream 512 * n_units + 16 bytes, sign_mant
 *    round_up(n_total, 16) bytes, gaps 40 * n_units + 8 bytes, unit_pos
 *    n_units + 1 entries; all padding is zero.
 *
 * Threading: encoder calls are re-entrant.  Decode calls are stream ordered;
 * concurrent decodes into distinct outputs are safe.
 */
#ifndef DF11_H
#define DF11_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DF11_FORMAT_VERSION 1u
#define DF11_WINDOW_BITS 64u        /* 8 bytes of encoded exponents per thread */
#define DF11_UNIT_WINDOWS 64u       /* windows per stored output position */
#define DF11_MAX_CODE_LEN 32u
#define DF11_MAX_UNIT_WEIGHTS 4096u /* 64 windows x at most 64 code starts */

typedef int32_t df11_status;
#define DF11_OK 0
#define DF11_E_INVALID_ARG (-1)      /* null pointer, bad size or alignment */
#define DF11_E_NOMEM (-2)            /* host allocation failed (memory, threads or a lock) */
#define DF11_E_FORMAT (-3)           /* sections are inconsistent */
#define DF11_E_BUFFER_TOO_SMALL (-4) /* caller buffer shorter than needed */
#define DF11_E_UNSUPPORTED (-5)      /* version or feature not supported */
#define DF11_E_HIP (-6)              /* the HIP runtime reported an error */

/* A host view of raw BF16 bit patterns (caller-owned, read only). */
typedef struct df11_bf16_view {
    const uint16_t *data;
    uint64_t numel;
} df11_bf16_view;

/* An encoded block: one library-owned host allocation (the "blob") holding
 * every section at a 256-byte aligned offset.  Opaque. */
typedef struct df11_encoded df11_encoded;

/* Host views into an encoded blob, valid until df11_encoded_free.  Every
 * off_* field is the byte offset of that section inside the blob, so a device
 * copy of the whole blob can be addressed with the same offsets. */
typedef struct df11_sections {
    uint32_t version;
    uint32_t n_mats;
    uint32_t n_symbols;             /* exponents with a nonzero count */
    uint32_t max_code_len;          /* longest codeword, bits */
    uint32_t n_tables;              /* 256-entry decode tables (root first) */
    uint32_t reserved;
    uint64_t n_total;               /* weights in the block */
    uint64_t total_bits;            /* stream bits: the codewords (and filler, aligned units) */
    uint64_t n_windows;             /* ceil(total_bits / 64) */
    uint64_t n_units;               /* ceil(n_windows / 64) */
    uint64_t max_unit_count;        /* max over u of unit_pos[u+1] - unit_pos[u] */
    const uint8_t *code_len;        /* [256]; 0 = exponent absent */
    const uint64_t *mat_offset;     /* [n_mats + 1] element offsets */
    const uint8_t *stream;          /* EncodedExponent */
    uint64_t stream_bytes;
    const uint8_t *sign_mant;       /* PackedSignMantissa */
    uint64_t sign_mant_bytes;
    const uint8_t *gaps;            /* 5-bit gap fields */
    uint64_t gaps_bytes;
    const uint64_t *unit_pos;       /* [n_units + 1] */
    const uint8_t *tables;          /* decode tables built from code_len */
    uint64_t tables_bytes;
    const uint8_t *blob;
    uint64_t blob_bytes;
    uint64_t off_code_len, off_mat_offset, off_stream, off_sign_mant, off_gaps, off_unit_pos,
        off_tables;
    double exp_entropy_bits;        /* Shannon entropy of the exponents, bits/weight */
    double mean_code_len_bits;      /* codeword bits / n_total (filler excluded) */
    /* Optional per-window code counts (blobs encoded with
     * DF11_ENCODE_WINDOW_COUNTS, else counts = NULL, counts_bytes = 0): byte w
     * is the number of codes that start in window w, i.e. in bits
     * [64w + gap_w, min(64w + 64, total_bits)); 0..64.  Padded with zeros to
     * 64 * n_units bytes. */
    const uint8_t *counts;
    uint64_t counts_bytes;
    uint64_t off_counts;
    /* Aligned-units layout (blobs encoded with DF11_ENCODE_ALIGNED_UNITS, else
     * unit_end = NULL, unit_end_bytes = 0): unit_end[u] = where the codes of
     * unit u end, in bits from the unit's first bit (1..4096); the bits after
     * it up to the next unit are zero filler.  total_bits then counts the
     * stream's bits including the filler. */
    const uint16_t *unit_end;
    uint64_t unit_end_bytes;
    uint64_t off_unit_end;
} df11_sections;

/* Encodes the concatenation of n_mats BF16 matrices with one shared codebook
 * (hada.io summary of the DFloat11 paper: section "Le format DFloat11" for
 * the exponent histogram, the Huffman code, EncodedExponent and
 * PackedSignMantissa; section "Noyau GPU en deux etapes et metadonnees
 * auxiliaires" for the per-window gaps and stored output positions; section
 * "Decompression par bloc transformer" for one codebook per block).
 * mats: host views, caller-owned, read only.  n_threads: host threads to use
 * (0 = all CPUs the process may run on).  *out receives a new blob that the
 * caller releases with df11_encoded_free.  n_mats may be 0 and views may be
 * empty (an empty block is valid).  Errors: DF11_E_INVALID_ARG (null
 * pointers), DF11_E_NOMEM. */
df11_status df11_encode_block(const df11_bf16_view *mats, uint32_t n_mats, uint32_t n_threads,
                              df11_encoded **out);

/* Encoder options (bit flags). */
#define DF11_ENCODE_WINDOW_COUNTS 1u  /* also store the per-window code counts */
#define DF11_ENCODE_ALIGNED_UNITS 2u  /* lay codes out so that units start on 32-weight boundaries */

/* df11_encode_block with options; neither is part of the pages' format.
 * DF11_ENCODE_WINDOW_COUNTS adds a section: the number of codes starting in
 * each 64-bit window.  It costs one byte per window (about 1.3 % more bytes
 * per decode at 2.7 bits per exponent) and lets DF11_VARIANT_COUNTS skip the
 * counting pass.  DF11_ENCODE_ALIGNED_UNITS takes the codes in groups of 32
 * weights and starts a group at the next unit (4,096 stream bits) when one of
 * its codes would otherwise start in a later unit than its first, leaving the
 * rest of the unit as zero filler (about 1 % more stream bits, 0.1 % more
 * bytes per decode).  Every unit then begins at a weight that is a multiple of
 * 32, so the decode's writes of neighbouring units meet on 64-byte
 * boundaries; it adds the unit_end section (2 bytes per unit).  Any decode
 * variant reads both layouts.  Unknown flags: DF11_E_INVALID_ARG; otherwise
 * as df11_encode_block. */
df11_status df11_encode_block_ex(const df11_bf16_view *mats, uint32_t n_mats, uint32_t n_threads,
                                 uint32_t flags, df11_encoded **out);

/* Fills *out with views into enc.  Errors: DF11_E_INVALID_ARG. */
df11_status df11_encoded_sections(const df11_encoded *enc, df11_sections *out);

/* Releases a blob from df11_encode_block (NULL is ignored). */
void df11_encoded_free(df11_encoded *enc);

/* Host-side structural check of the sections (sizes, code lengths form a
 * prefix code of at most 32 bits, gaps within [0, 31] and consistent with
 * total_bits, unit_pos non-decreasing from 0 to n_total, max_unit_count,
 * decode tables equal to the ones built from code_len, and when present, per
 * window counts of at most 64 that sum over each unit to its unit_pos
 * difference; for the aligned-units layout, unit positions that are multiples
 * of 32, unit ends within their units, zero filler and gaps consistent with
 * the unit ends).  It does not decode the stream.  The arrays must hold what
 * the fields say: stream_bytes, sign_mant_bytes, gaps_bytes, counts_bytes and
 * unit_end_bytes bytes, n_units + 1 unit positions, tables_bytes of tables;
 * n_total and total_bits are bounded (at most 2^48 weights, at most 32 bits
 * per weight, 64 with filler) before any size is derived from them.  Returns
 * DF11_OK or DF11_E_FORMAT / DF11_E_INVALID_ARG (DF11_E_NOMEM if host memory
 * runs out). */
df11_status df11_validate(const df11_sections *s);

/* Decode tables for the GPU kernel, derived from the 256 code lengths: a
 * hierarchy of 256-entry tables indexed by 8 stream bits each (the pages'
 * compact LUTs, section "Decodage fonde sur des LUT hierarchiques"), with
 * 32-bit entries, followed by a 1024-entry count table and a 2048-entry emit
 * table that resolve several codes per lookup (20 KiB).  df11_tables_size
 * reports the bytes needed and the number of hierarchical tables;
 * df11_build_tables writes them to dst (host memory, dst_bytes at least that
 * size).  Errors: DF11_E_INVALID_ARG, DF11_E_FORMAT (lengths do
 * not form a prefix code of at most 32 bits), DF11_E_BUFFER_TOO_SMALL,
 * DF11_E_NOMEM. */
df11_status df11_tables_size(const uint8_t code_len[256], uint64_t *bytes, uint32_t *n_tables);
df11_status df11_build_tables(const uint8_t code_len[256], void *dst, uint64_t dst_bytes);

/* Device-side description of one encoded block.  Every pointer is device
 * memory owned by the caller (for example torch tensors), 16-byte aligned,
 * and must stay valid until the decode has run on its stream. */
typedef struct df11_device_block {
    const void *tables;
    uint64_t tables_bytes;
    const uint8_t *stream;
    uint64_t stream_bytes;
    const uint8_t *sign_mant;
    uint64_t sign_mant_bytes;
    const uint8_t *gaps;
    uint64_t gaps_bytes;
    const uint64_t *unit_pos;
    uint64_t n_total, total_bits, n_windows, n_units, max_unit_count;
    uint32_t version;
    uint32_t n_tables;
    const uint8_t *counts;          /* per-window counts, 64 * n_units bytes, or NULL */
    const uint16_t *unit_end;       /* aligned-units layout: n_units entries, or NULL */
} df11_device_block;

/* Fills *out for a device copy of a whole blob starting at device_blob. */
df11_status df11_device_block_from_blob(const df11_sections *s, const void *device_blob,
                                        df11_device_block *out);

/* Decodes the block into out_bf16[0 .. n_total) (device memory, 16-byte
 * aligned, out_capacity elements): the two-phase kernel of the hada.io
 * summary of the DFloat11 paper, section "Noyau GPU en deux etapes et
 * metadonnees auxiliaires" (count, prefix sum, decode into an on-chip buffer,
 * coalesced write), with the compact hierarchical tables of section
 * "Decodage fonde sur des LUT hierarchiques" in LDS, over every matrix of a
 * transformer block at once (section "Decompression par bloc transformer").
 * The result is the original BF16 bits (chatpaper.ai abstract of the paper:
 * bit-for-bit identical output).  One kernel launch on the HIP stream
 * `hip_stream` (a hipStream_t; NULL = the null stream); the call does not
 * synchronize and allocates nothing.  Exactly n_total elements are written;
 * nothing else is touched.  Argument, capacity, alignment and version errors
 * are reported synchronously (DF11_E_INVALID_ARG, DF11_E_BUFFER_TOO_SMALL,
 * DF11_E_UNSUPPORTED); so are sizes that no encoder produces (more than 2^48
 * weights, fewer than 1 or more than 32 bits per weight, 64 with the aligned
 * layout's filler: DF11_E_INVALID_ARG).  A launch failure returns DF11_E_HIP.  Corrupted
 * section contents are not detected on the device, but every store stays in
 * [0, n_total) and every loop is bounded.  n_total = 0 is a no-op. */
df11_status df11_decode_block(const df11_device_block *blk, uint16_t *out_bf16,
                              uint64_t out_capacity, void *hip_stream);

/* Kernel variants (the output never depends on the choice):
 *  DF11_VARIANT_SINGLE: one code per table lookup in both phases, 8-bit
 *    indexed hierarchical tables only (the pages' kernel design);
 *  DF11_VARIANT_MULTI: phase 1 takes every code that ends in the next 10 bits
 *    per lookup (count table), phase 2 up to four codes in the next 11 bits
 *    (emit table); longer codes go through the hierarchical tables.  The
 *    default.
 *  DF11_VARIANT_COUNTS: DF11_VARIANT_MULTI with the counting pass replaced by
 *    the stored per-window counts; needs blk->counts (a blob encoded with
 *    DF11_ENCODE_WINDOW_COUNTS), else DF11_E_INVALID_ARG.  Not the pages'
 *    format: a variant that trades one byte per window for the first pass.
 * The multi-code kernels check the count and emit tables when they load them;
 * a workgroup that finds an entry no table builder writes decodes with the
 * hierarchical tables alone (as DF11_VARIANT_SINGLE), so the output is still
 * complete, and exact when the hierarchical tables are intact. */
#define DF11_VARIANT_SINGLE 1u
#define DF11_VARIANT_MULTI 2u
#define DF11_VARIANT_COUNTS 3u

/* Launch geometry for df11_decode_block_ex (0 = automatic). */
typedef struct df11_launch {
    uint32_t waves_per_group;  /* 64-lane waves per workgroup: 1, 2, 4, 8 or 16 */
    uint32_t max_groups;       /* cap on the grid size */
    uint32_t variant;          /* DF11_VARIANT_*, 0 = DF11_VARIANT_MULTI */
    uint32_t oversubscribe;    /* workgroups launched per resident workgroup slot
                                  (1 = persistent grid); 0 = automatic: about
                                  four units per wave, at least one workgroup
                                  per resident slot */
} df11_launch;

/* df11_decode_block with an explicit launch geometry; the output does not
 * depend on it. */
df11_status df11_decode_block_ex(const df11_device_block *blk, uint16_t *out_bf16,
                                 uint64_t out_capacity, void *hip_stream,
                                 const df11_launch *launch);

/* ---- Bandwidth references (measurement aids) -----------------------------
 * Streaming kernels that move the HBM bytes of one df11_decode_block launch
 * of blk (or one direction of them), without decoding, so that the decode's
 * rate can be set against what the same traffic reaches on the same GPU.
 * The decode reads
 * the compressed sections once and writes the block once, coalesced (hada.io
 * summary of the DFloat11 paper, section "Noyau GPU en deux etapes et
 * metadonnees auxiliaires").  The first two write out_bf16[i] = the block's
 * weight i with its exponent field zero (sign and mantissa from sign_mant),
 * for i in [0, n_total), and nothing else.
 *  DF11_REFERENCE_SKELETON: the decode's own HBM accesses unit by unit (one
 *    64-lane wave per unit of 64 windows: window words with their halo, gap
 *    bytes and the unit's positions one unit ahead, 8-byte sign/mantissa
 *    loads, 16-byte non-temporal stores of whole 64-byte sectors, 2-byte
 *    stores of sectors shared with the neighbouring units), with the
 *    decode's workgroup size and grid rule.
 *  DF11_REFERENCE_STREAM: the same byte counts moved in whole tiles of 4,096
 *    weights per wave (no unit boundaries, no shared sectors).
 *  DF11_REFERENCE_WRITES: the stream reference's stores alone: out_bf16[i] =
 *    0 for i in [0, n_total), no section read.
 *  DF11_REFERENCE_READS: the stream reference's loads alone: the sections
 *    read, out_bf16 left as it was.
 * Same arguments, checks, errors and stream semantics as df11_decode_block_ex
 * (launch: waves_per_group, max_groups and oversubscribe are used; variant is
 * ignored; NULL = automatic).  Blocks with stored window counts or the
 * aligned-units layout: DF11_E_UNSUPPORTED; an unknown kind:
 * DF11_E_INVALID_ARG. */
#define DF11_REFERENCE_SKELETON 1u
#define DF11_REFERENCE_STREAM 2u
#define DF11_REFERENCE_WRITES 3u
#define DF11_REFERENCE_READS 4u

df11_status df11_bandwidth_reference(const df11_device_block *blk, uint16_t *out_bf16, uint64_t out_capacity,
                                     uint32_t kind, void *hip_stream, const df11_launch *launch);

/* ---- GPU-side encoder ---------------------------------------------------
 * The step before the decode, for a block whose BF16 weights are already in
 * device memory: the exponent histogram is taken on the device, the host
 * turns its 256 counts into code lengths (the same rule as
 * df11_encode_block), and the device computes every code's bit offset by a
 * prefix sum and packs all sections.  The sections are byte for byte those of
 * df11_encode_block on the same weights (hada.io summary of the DFloat11
 * paper, sections "Le format DFloat11" and "Noyau GPU en deux etapes et
 * metadonnees auxiliaires").  All calls are stream-ordered on hip_stream
 * (NULL = the null stream), never synchronize and allocate nothing. */

/* Bytes of the per-chunk histograms of n weights: 256 uint16 counts for each
 * chunk of 4,096 weights (the last chunk may be shorter). */
uint64_t df11_gpu_chunk_hist_bytes(uint64_t n);

/* hist[0..256) (device, uint64) := histogram of the exponents of x[0..n)
 * (device, BF16 bit patterns, 16-byte aligned); and, when chunk_hist is not
 * NULL, chunk_hist (device, df11_gpu_chunk_hist_bytes(n) bytes, 16-byte
 * aligned) := for every chunk of 4,096 weights its 256 exponent counts.
 * df11_gpu_encode takes the chunk counts, so that it does not read the
 * weights a second time to size each chunk's codes.  Errors:
 * DF11_E_INVALID_ARG, DF11_E_HIP (launch failure). */
df11_status df11_gpu_histogram(const uint16_t *x, uint64_t n, uint64_t *hist, uint16_t *chunk_hist,
                               void *hip_stream);

/* What the GPU encoder will produce for a histogram, and the buffers it needs
 * (bytes, caller-allocated device memory). */
typedef struct df11_gpu_plan {
    uint8_t code_len[256];          /* code length per exponent, 0 = absent */
    uint32_t n_symbols, max_code_len, n_tables, flags;
    uint64_t n_total, total_bits, n_windows, n_units;
    uint64_t stream_bytes;          /* 512 * n_units + 16 */
    uint64_t sign_mant_bytes;       /* n_total rounded up to 16 */
    uint64_t gaps_bytes;            /* 40 * n_units + 8 */
    uint64_t unit_pos_bytes;        /* 8 * (n_units + 1) */
    uint64_t counts_bytes;          /* 64 * n_units with DF11_ENCODE_WINDOW_COUNTS, else 0 */
    uint64_t tables_bytes;          /* df11_build_tables output for code_len */
    uint64_t workspace_bytes;       /* device scratch for df11_gpu_encode */
} df11_gpu_plan;

/* Host: the plan for a histogram (host copy of df11_gpu_histogram's result)
 * and encoder flags (DF11_ENCODE_WINDOW_COUNTS or 0; the aligned-units layout
 * is made by the host encoder only).  Errors: DF11_E_INVALID_ARG (unknown or
 * unsupported flags, or more than 2^48 weights in the histogram),
 * DF11_E_FORMAT. */
df11_status df11_gpu_plan_build(const uint64_t hist[256], uint32_t flags, df11_gpu_plan *plan);

/* Encodes x[0..plan->n_total) (device) into the caller's device buffers, sized
 * as in the plan: stream (16-byte aligned), sign_mant (16-byte aligned), gaps,
 * unit_pos (8-byte aligned), counts (NULL unless plan->flags has
 * DF11_ENCODE_WINDOW_COUNTS) and workspace (plan->workspace_bytes, 16-byte
 * aligned, contents are scratch).  x and chunk_hist must be the weights and
 * the per-chunk counts df11_gpu_histogram took the plan's histogram from.
 * The decode tables are built on the host with
 * df11_build_tables(plan->code_len).  Errors: DF11_E_INVALID_ARG (null or
 * misaligned pointers, flags that do not match, a plan whose sizes do not
 * follow from n_total and total_bits or that has more than 2^48 weights),
 * DF11_E_HIP. */
df11_status df11_gpu_encode(const df11_gpu_plan *plan, const uint16_t *x, const uint16_t *chunk_hist,
                            uint8_t *stream, uint8_t *sign_mant, uint8_t *gaps, uint64_t *unit_pos,
                            uint8_t *counts, void *workspace, void *hip_stream);

/* df11_gpu_encode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without `workspace`, and the same output.  The
 * workspace is a device array inside the library, one per GPU, of
 * DF11_NOALLOC_WORKSPACE_BYTES (48 MiB: at 2.7 bits per exponent code,
 * enough for about 1.1 G weights without window counts, 130 M with them),
 * held from the first call on a GPU until the process ends.  No call allocates or frees device memory.
 * Plans that need more workspace: DF11_E_BUFFER_TOO_SMALL, before anything
 * is launched.  Every call on one GPU uses that GPU's array: calls whose work
 * overlaps on one GPU (different streams, or host threads without ordering
 * between their streams) race and must not be made; stream-ordered calls are
 * safe.  Nothing needs clearing between calls (every workspace word is written
 * before it is read).  Otherwise as df11_gpu_encode (DF11_E_HIP also when
 * the array's address cannot be found). */
#define DF11_NOALLOC_WORKSPACE_BYTES (48ull << 20)

df11_status df11_gpu_encode_noalloc(const df11_gpu_plan *plan, const uint16_t *x, const uint16_t *chunk_hist,
                                    uint8_t *stream, uint8_t *sign_mant, uint8_t *gaps, uint64_t *unit_pos,
                                    uint8_t *counts, void *hip_stream);

/* Text for a status code (static storage). */
const char *df11_status_str(df11_status s);

/* The last HIP error code recorded by a failing decode call in this thread
 * (0 if none), and the HIP runtime's name for a HIP error code. */
int32_t df11_last_hip_error(void);
const char *df11_hip_error_name(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* DF11_H */
