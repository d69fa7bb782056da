/*
 * df11_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of the DFloat11 (DF11)
 * exponent coding: the encoder that produces the compressed sections and a
 * bit-serial Huffman decoder that walks the code tree one bit at a time.
 * It exists to check the GPU path and the library encoder.  Only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark may load it.
 * It shares no code, header, table or helper with the product library.
 *
 * Sources (web pages on DFloat11; cited by page and section):
 *   [SUM]  hada.io French summary of the DFloat11 paper
 *          ("DFloat11 : compression sans perte pour l'inference GPU ..."),
 *          sections "La marge de compression restante dans l'exposant BFloat16",
 *          "Le format DFloat11", "Decompression adaptee a l'inference GPU",
 *          "Noyau GPU en deux etapes et metadonnees auxiliaires".
 *   [ABS]  chatpaper.ai abstract of "70% Size, 100% Accuracy: Lossless LLM
 *          Compression ... via Dynamic-Length Float" (losslessness claim).
 *
 * Readings where the pages leave a step open (each one is listed, with its
 * reason, in the design notes of the repository):
 *   R1  Huffman ties: leaves ordered by (count, exponent) get sequence numbers
 *       0..n-1, merged nodes get n, n+1, ... in creation order; every merge takes
 *       the two live nodes with the smallest (weight, sequence) key.
 *   R2  Codes longer than 32 bits: lengths are recomputed by package-merge with
 *       cap 32; on equal weights a leaf precedes a package.
 *   R3  Canonical code: symbols sorted by (length, exponent), first code 0,
 *       next = (prev + 1) << (len_next - len_prev).
 *   R4  EncodedExponent is MSB-first: stream bit j is bit (7 - j%8) of byte j/8.
 *   R5  PackedSignMantissa byte = (sign << 7) | mantissa.
 *   R6  Windows of 64 bits (8 bytes per thread); gap[w] = (first code start
 *       >= 64w, or total_bits if none) - 64w.
 *   R7  Gaps packed as 5-bit fields, MSB-first, field w at bits [5w, 5w+5).
 *   R8  Output positions per unit of 64 windows: unit_pos[u] = number of codes
 *       starting before bit 4096u; unit_pos[n_units] = N.
 *   R9  Section sizes: stream 512*n_units + 16 bytes, sign/mantissa
 *       round_up(N, 16) bytes, gaps 40*n_units + 8 bytes, all zero padded.
 *   R10 A one-symbol alphabet gets length 1 (codeword "0").
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_NOMEM (-2)
#define ORC_ERR_DATA (-3)

#define ORC_CAP 32

/* ---- BF16 field split ([SUM] "La marge de compression ...": 1 sign bit,
 *      8 exponent bits, 7 mantissa bits) -------------------------------- */
static unsigned orc_exponent_of(uint16_t x) { return (x >> 7) & 0xFFu; }
static unsigned orc_sign_of(uint16_t x) { return (x >> 15) & 1u; }
static unsigned orc_mantissa_of(uint16_t x) { return x & 0x7Fu; }

/* Exponent histogram over the whole block ([SUM] "Le format DFloat11": the
 * Huffman tree is built from the distribution of the exponents). */
void orc_histogram(const uint16_t *x, uint64_t n, uint64_t counts[256])
{
    for (int e = 0; e < 256; ++e) counts[e] = 0;
    for (uint64_t i = 0; i < n; ++i) counts[orc_exponent_of(x[i])] += 1;
}

/* Symbols with a nonzero count, ordered by (count ascending, exponent
 * ascending).  Plain selection, n <= 256. Returns how many. */
static int orc_sorted_symbols(const uint64_t counts[256], int sym[256])
{
    int n = 0;
    for (int e = 0; e < 256; ++e)
        if (counts[e] > 0) sym[n++] = e;
    for (int a = 0; a < n; ++a) {
        int best = a;
        for (int b = a + 1; b < n; ++b) {
            int sb = sym[b], sk = sym[best];
            if (counts[sb] < counts[sk] || (counts[sb] == counts[sk] && sb < sk)) best = b;
        }
        int t = sym[a]; sym[a] = sym[best]; sym[best] = t;
    }
    return n;
}

/* Huffman code lengths, reading R1.  Node k < n is the k-th leaf in
 * (count, exponent) order; merged nodes are appended.  Each merge scans all
 * live nodes for the two smallest (weight, node index) keys. */
static void orc_huffman_lengths(const uint64_t counts[256], uint32_t len[256])
{
    int sym[256];
    int n = orc_sorted_symbols(counts, sym);
    for (int e = 0; e < 256; ++e) len[e] = 0;
    if (n == 0) return;
    if (n == 1) { len[sym[0]] = 1; return; }          /* R10 */

    uint64_t weight[512];
    int parent[512], live[512];
    int total = n;
    for (int k = 0; k < n; ++k) { weight[k] = counts[sym[k]]; parent[k] = -1; live[k] = 1; }
    for (int merge = 0; merge < n - 1; ++merge) {
        int pick[2];
        for (int p = 0; p < 2; ++p) {
            int best = -1;
            for (int k = 0; k < total; ++k) {
                if (!live[k]) continue;
                if (best < 0 || weight[k] < weight[best]) best = k;   /* ties keep the lower index */
            }
            live[best] = 0;
            pick[p] = best;
        }
        weight[total] = weight[pick[0]] + weight[pick[1]];
        parent[total] = -1;
        live[total] = 1;
        parent[pick[0]] = total;
        parent[pick[1]] = total;
        total += 1;
    }
    for (int k = 0; k < n; ++k) {
        uint32_t depth = 0;
        for (int v = k; parent[v] >= 0; v = parent[v]) depth += 1;
        len[sym[k]] = depth;
    }
}

/* Package-merge (Larmore & Hirschberg) with a length cap, reading R2.
 * Every list item carries the number of times each leaf occurs inside it;
 * the lengths are the occurrence counts summed over the first 2n-2 items of
 * the last list.  Returns ORC_OK or an error. */
static int orc_package_merge(const uint64_t counts[256], uint32_t cap, uint32_t len[256])
{
    int sym[256];
    int n = orc_sorted_symbols(counts, sym);
    for (int e = 0; e < 256; ++e) len[e] = 0;
    if (n == 0) return ORC_OK;
    if (n == 1) { len[sym[0]] = 1; return ORC_OK; }
    if (cap < 1 || cap > 63 || ((uint64_t)1 << cap) < (uint64_t)n) return ORC_ERR_ARG;

    int max_items = 2 * n;
    uint64_t *w_cur = malloc(sizeof(uint64_t) * max_items);
    uint64_t *w_nxt = malloc(sizeof(uint64_t) * max_items);
    uint16_t *c_cur = malloc(sizeof(uint16_t) * (size_t)max_items * n);
    uint16_t *c_nxt = malloc(sizeof(uint16_t) * (size_t)max_items * n);
    if (!w_cur || !w_nxt || !c_cur || !c_nxt) {
        free(w_cur); free(w_nxt); free(c_cur); free(c_nxt);
        return ORC_ERR_NOMEM;
    }

    /* deepest list: the leaves alone */
    int m = n;
    memset(c_cur, 0, sizeof(uint16_t) * (size_t)max_items * n);
    for (int k = 0; k < n; ++k) { w_cur[k] = counts[sym[k]]; c_cur[(size_t)k * n + k] = 1; }

    for (uint32_t level = cap; level >= 2; --level) {
        /* packages: consecutive pairs of the current list */
        int n_pkg = m / 2;
        /* merge leaves with packages; a leaf goes first on equal weight */
        int li = 0, pi = 0, out = 0;
        memset(c_nxt, 0, sizeof(uint16_t) * (size_t)max_items * n);
        while (li < n || pi < n_pkg) {
            int take_leaf;
            if (li >= n) take_leaf = 0;
            else if (pi >= n_pkg) take_leaf = 1;
            else {
                uint64_t pw = w_cur[2 * pi] + w_cur[2 * pi + 1];
                take_leaf = counts[sym[li]] <= pw;
            }
            if (take_leaf) {
                w_nxt[out] = counts[sym[li]];
                c_nxt[(size_t)out * n + li] = 1;
                li += 1;
            } else {
                w_nxt[out] = w_cur[2 * pi] + w_cur[2 * pi + 1];
                for (int k = 0; k < n; ++k)
                    c_nxt[(size_t)out * n + k] =
                        (uint16_t)(c_cur[(size_t)(2 * pi) * n + k] + c_cur[(size_t)(2 * pi + 1) * n + k]);
                pi += 1;
            }
            out += 1;
        }
        m = out;
        uint64_t *tw = w_cur; w_cur = w_nxt; w_nxt = tw;
        uint16_t *tc = c_cur; c_cur = c_nxt; c_nxt = tc;
    }
    /* cap == 1 never reaches here with n >= 2 except n == 2 (list = leaves). */
    int take = 2 * n - 2;
    if (take > m) { free(w_cur); free(w_nxt); free(c_cur); free(c_nxt); return ORC_ERR_ARG; }
    for (int k = 0; k < n; ++k) {
        uint32_t l = 0;
        for (int it = 0; it < take; ++it) l += c_cur[(size_t)it * n + k];
        len[sym[k]] = l;
    }
    free(w_cur); free(w_nxt); free(c_cur); free(c_nxt);
    return ORC_OK;
}

/* Code lengths with a cap: Huffman (R1); if its longest code exceeds the cap,
 * package-merge (R2).  Returns the longest length, or a negative error. */
int orc_code_lengths_capped(const uint64_t counts[256], uint32_t cap, uint32_t len[256])
{
    orc_huffman_lengths(counts, len);
    uint32_t mx = 0;
    for (int e = 0; e < 256; ++e) if (len[e] > mx) mx = len[e];
    if (mx > cap) {
        int rc = orc_package_merge(counts, cap, len);
        if (rc != ORC_OK) return rc;
        mx = 0;
        for (int e = 0; e < 256; ++e) if (len[e] > mx) mx = len[e];
    }
    return (int)mx;
}

int orc_code_lengths(const uint64_t counts[256], uint32_t len[256])
{
    return orc_code_lengths_capped(counts, ORC_CAP, len);
}

/* Exposed for the tests of reading R2 at small caps. */
int orc_package_merge_lengths(const uint64_t counts[256], uint32_t cap, uint32_t len[256])
{
    return orc_package_merge(counts, cap, len);
}

/* Canonical codewords, reading R3.  code[e] holds len[e] bits, right aligned. */
void orc_canonical_codes(const uint32_t len[256], uint64_t code[256])
{
    int order[256], n = 0;
    for (int e = 0; e < 256; ++e) { code[e] = 0; if (len[e] > 0) order[n++] = e; }
    for (int a = 0; a < n; ++a) {                        /* sort by (length, exponent) */
        int best = a;
        for (int b = a + 1; b < n; ++b) {
            int eb = order[b], ek = order[best];
            if (len[eb] < len[ek] || (len[eb] == len[ek] && eb < ek)) best = b;
        }
        int t = order[a]; order[a] = order[best]; order[best] = t;
    }
    uint64_t c = 0;
    for (int k = 0; k < n; ++k) {
        if (k > 0) c = (c + 1) << (len[order[k]] - len[order[k - 1]]);
        code[order[k]] = c;
    }
}

/* ---- section sizes (reading R9) ---------------------------------------- */
typedef struct {
    uint64_t n, total_bits, n_windows, n_units;
    uint64_t stream_bytes, sm_bytes, gaps_bytes, unit_pos_entries;
} orc_sizes;

static void orc_sizes_for(uint64_t n, uint64_t total_bits, orc_sizes *s)
{
    s->n = n;
    s->total_bits = total_bits;
    s->n_windows = (total_bits + 63) / 64;
    s->n_units = (s->n_windows + 63) / 64;
    s->stream_bytes = 512 * s->n_units + 16;
    s->sm_bytes = (n + 15) / 16 * 16;
    s->gaps_bytes = 40 * s->n_units + 8;
    s->unit_pos_entries = s->n_units + 1;
}

/* First pass of the encoder: histogram, lengths, codes and the section sizes.
 * out_sizes = {n, total_bits, n_windows, n_units, stream_bytes, sm_bytes,
 *              gaps_bytes, unit_pos_entries}.  Returns max length or < 0. */
int orc_plan(const uint16_t *x, uint64_t n, uint32_t len[256], uint64_t out_sizes[8])
{
    uint64_t counts[256];
    orc_histogram(x, n, counts);
    int mx = orc_code_lengths(counts, len);
    if (mx < 0) return mx;
    uint64_t total_bits = 0;
    for (int e = 0; e < 256; ++e) total_bits += counts[e] * (uint64_t)len[e];
    orc_sizes s;
    orc_sizes_for(n, total_bits, &s);
    out_sizes[0] = s.n; out_sizes[1] = s.total_bits; out_sizes[2] = s.n_windows;
    out_sizes[3] = s.n_units; out_sizes[4] = s.stream_bytes; out_sizes[5] = s.sm_bytes;
    out_sizes[6] = s.gaps_bytes; out_sizes[7] = s.unit_pos_entries;
    return mx;
}

static void orc_put_bit(uint8_t *buf, uint64_t bitpos, unsigned bit)
{
    if (bit) buf[bitpos >> 3] |= (uint8_t)(0x80u >> (bitpos & 7));
}

static unsigned orc_get_bit(const uint8_t *buf, uint64_t bitpos)
{
    return (buf[bitpos >> 3] >> (7 - (bitpos & 7))) & 1u;
}

/* Encoder, second pass.  Buffers are caller-owned and sized by orc_plan.
 * Appends each exponent's codeword one bit at a time (R4), writes the
 * sign/mantissa byte (R5), and records the gaps (R6, R7) and unit positions
 * (R8) while walking the code start positions in order. */
int orc_encode(const uint16_t *x, uint64_t n, const uint32_t len[256],
               uint8_t *stream, uint64_t stream_bytes,
               uint8_t *sm, uint64_t sm_bytes,
               uint8_t *gaps, uint64_t gaps_bytes,
               uint64_t *unit_pos, uint64_t unit_pos_entries,
               uint64_t *total_bits_out)
{
    uint64_t code[256];
    orc_canonical_codes(len, code);
    uint64_t total_bits = 0;
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t l = len[orc_exponent_of(x[i])];
        if (l == 0) return ORC_ERR_ARG;
        total_bits += l;
    }
    orc_sizes s;
    orc_sizes_for(n, total_bits, &s);
    if (stream_bytes != s.stream_bytes || sm_bytes != s.sm_bytes || gaps_bytes != s.gaps_bytes ||
        unit_pos_entries != s.unit_pos_entries)
        return ORC_ERR_ARG;
    memset(stream, 0, stream_bytes);
    memset(sm, 0, sm_bytes);
    memset(gaps, 0, gaps_bytes);

    uint32_t *gap_value = malloc(sizeof(uint32_t) * (s.n_windows ? s.n_windows : 1));
    if (!gap_value) return ORC_ERR_NOMEM;

    uint64_t bitpos = 0, next_window = 0, next_unit = 0;
    for (uint64_t i = 0; i < n; ++i) {
        /* code i starts at bitpos: it is the first start at or after 64w for
         * every window w not yet given a gap with 64w <= bitpos */
        while (next_window < s.n_windows && 64 * next_window <= bitpos) {
            gap_value[next_window] = (uint32_t)(bitpos - 64 * next_window);
            next_window += 1;
        }
        while (next_unit < s.n_units && 4096 * next_unit <= bitpos) {
            unit_pos[next_unit] = i;
            next_unit += 1;
        }
        unsigned e = orc_exponent_of(x[i]);
        uint32_t l = len[e];
        for (uint32_t b = l; b-- > 0;) {
            orc_put_bit(stream, bitpos, (unsigned)((code[e] >> b) & 1u));
            bitpos += 1;
        }
        sm[i] = (uint8_t)((orc_sign_of(x[i]) << 7) | orc_mantissa_of(x[i]));
    }
    while (next_window < s.n_windows) {       /* no code starts in it (R6) */
        gap_value[next_window] = (uint32_t)(total_bits - 64 * next_window);
        next_window += 1;
    }
    while (next_unit < s.n_units) { unit_pos[next_unit] = n; next_unit += 1; }
    unit_pos[s.n_units] = n;

    for (uint64_t w = 0; w < s.n_windows; ++w) {
        if (gap_value[w] > 31) { free(gap_value); return ORC_ERR_DATA; }
        for (int b = 4; b >= 0; --b)
            orc_put_bit(gaps, 5 * w + (uint64_t)(4 - b), (gap_value[w] >> b) & 1u);
    }
    free(gap_value);
    *total_bits_out = total_bits;
    return ORC_OK;
}

/* ---- bit-serial decoder ([SUM] "Decompression adaptee a l'inference GPU":
 *      the classic decoder walks the Huffman tree one bit at a time) ------- */
typedef struct { int child[2]; int symbol; } orc_node;

/* Builds the binary code tree from the canonical codes.  Returns the node
 * count (>= 1) or a negative error; nodes must hold 2*256 entries. */
static int orc_build_tree(const uint32_t len[256], orc_node *nodes)
{
    uint64_t code[256];
    orc_canonical_codes(len, code);
    int count = 1;
    nodes[0].child[0] = nodes[0].child[1] = -1;
    nodes[0].symbol = -1;
    for (int e = 0; e < 256; ++e) {
        if (len[e] == 0) continue;
        if (len[e] > 63) return ORC_ERR_ARG;
        int v = 0;
        for (uint32_t b = len[e]; b-- > 0;) {
            if (nodes[v].symbol >= 0) return ORC_ERR_DATA;      /* not prefix free */
            int bit = (int)((code[e] >> b) & 1u);
            if (nodes[v].child[bit] < 0) {
                if (count >= 512) return ORC_ERR_DATA;
                nodes[count].child[0] = nodes[count].child[1] = -1;
                nodes[count].symbol = -1;
                nodes[v].child[bit] = count++;
            }
            v = nodes[v].child[bit];
        }
        if (nodes[v].symbol >= 0 || nodes[v].child[0] >= 0 || nodes[v].child[1] >= 0)
            return ORC_ERR_DATA;
        nodes[v].symbol = e;
    }
    return count;
}

/* Decodes `count` codes starting at stream bit `bit0`, rebuilding BF16 values
 * from the exponent and the sign/mantissa bytes sm[first .. first+count). */
static int orc_walk(const orc_node *nodes, const uint8_t *stream, uint64_t stream_bits,
                    uint64_t bit0, const uint8_t *sm, uint64_t first, uint64_t count,
                    uint16_t *out)
{
    uint64_t bitpos = bit0;
    for (uint64_t i = first; i < first + count; ++i) {
        int v = 0;
        while (nodes[v].symbol < 0) {
            if (bitpos >= stream_bits) return ORC_ERR_DATA;
            v = nodes[v].child[orc_get_bit(stream, bitpos)];
            bitpos += 1;
            if (v < 0) return ORC_ERR_DATA;
        }
        unsigned e = (unsigned)nodes[v].symbol;
        unsigned s = sm[i];
        out[i] = (uint16_t)(((s >> 7) << 15) | (e << 7) | (s & 0x7Fu));
    }
    return ORC_OK;
}

/* Whole-stream decode from bit 0, exactly n codes. */
int orc_decode(const uint32_t len[256], const uint8_t *stream, uint64_t stream_bytes,
               const uint8_t *sm, uint64_t n, uint16_t *out)
{
    orc_node nodes[512];
    int rc = orc_build_tree(len, nodes);
    if (rc < 0) return rc;
    if (n == 0) return ORC_OK;
    return orc_walk(nodes, stream, 8 * stream_bytes, 0, sm, 0, n, out);
}

/* Decode of units [u_begin, u_end) on their own: unit u starts at stream bit
 * 4096u + gap[64u] and holds unit_pos[u+1] - unit_pos[u] codes whose outputs
 * start at unit_pos[u] ([SUM] "Noyau GPU en deux etapes ...": the gaps fix
 * where a thread's first code starts, the stored positions fix where its
 * outputs go). */
static uint32_t orc_gap_field(const uint8_t *gaps, uint64_t w)
{
    uint32_t g = 0;
    for (int b = 0; b < 5; ++b) g = (g << 1) | orc_get_bit(gaps, 5 * w + (uint64_t)b);
    return g;
}

int orc_decode_units(const uint32_t len[256], const uint8_t *stream, uint64_t stream_bytes,
                     const uint8_t *sm, const uint8_t *gaps, const uint64_t *unit_pos,
                     uint64_t u_begin, uint64_t u_end, uint16_t *out)
{
    orc_node nodes[512];
    int rc = orc_build_tree(len, nodes);
    if (rc < 0) return rc;
    for (uint64_t u = u_begin; u < u_end; ++u) {
        uint64_t first = unit_pos[u], last = unit_pos[u + 1];
        if (last < first) return ORC_ERR_DATA;
        uint64_t bit0 = 4096 * u + orc_gap_field(gaps, 64 * u);
        rc = orc_walk(nodes, stream, 8 * stream_bytes, bit0, sm, first, last - first, out);
        if (rc != ORC_OK) return rc;
    }
    return ORC_OK;
}

/* Several threads, each decoding a contiguous range of units. */
typedef struct {
    const uint32_t *len; const uint8_t *stream; uint64_t stream_bytes;
    const uint8_t *sm; const uint8_t *gaps; const uint64_t *unit_pos;
    uint64_t u_begin, u_end; uint16_t *out; int rc;
} orc_job;

static void *orc_job_run(void *arg)
{
    orc_job *j = (orc_job *)arg;
    j->rc = orc_decode_units(j->len, j->stream, j->stream_bytes, j->sm, j->gaps, j->unit_pos,
                             j->u_begin, j->u_end, j->out);
    return NULL;
}

int orc_decode_units_threads(const uint32_t len[256], const uint8_t *stream, uint64_t stream_bytes,
                             const uint8_t *sm, const uint8_t *gaps, const uint64_t *unit_pos,
                             uint64_t u_begin, uint64_t u_end, uint16_t *out, int threads)
{
    if (threads < 1) return ORC_ERR_ARG;
    if (threads > 256) threads = 256;
    pthread_t tid[256];
    orc_job jobs[256];
    uint64_t span = u_end > u_begin ? u_end - u_begin : 0;
    int started = 0;
    for (int t = 0; t < threads; ++t) {
        orc_job *j = &jobs[t];
        j->len = len; j->stream = stream; j->stream_bytes = stream_bytes; j->sm = sm;
        j->gaps = gaps; j->unit_pos = unit_pos; j->out = out; j->rc = ORC_OK;
        j->u_begin = u_begin + span * (uint64_t)t / (uint64_t)threads;
        j->u_end = u_begin + span * (uint64_t)(t + 1) / (uint64_t)threads;
        if (pthread_create(&tid[t], NULL, orc_job_run, j) != 0) { j->rc = ORC_ERR_NOMEM; break; }
        started += 1;
    }
    int rc = ORC_OK;
    for (int t = 0; t < started; ++t) {
        pthread_join(tid[t], NULL);
        if (jobs[t].rc != ORC_OK) rc = jobs[t].rc;
    }
    if (started < threads) rc = ORC_ERR_NOMEM;
    return rc;
}
