// Internal declarations shared by the host-side translation units of libdf11.
#pragma once

#include <cstdint>
#include <new>

#include "df11.h"

// Decode-table entry layout (32 bits), used by the table builder and the
// kernel:
//   leaf    : bit 31 = 0; bits 30..23 = exponent (so bits 31..16 hold
//             exponent << 7, the exponent field of a BF16 value);
//             bits 12..8 = code length - 1; bits 4..0 = (32 - length) & 31.
//   pointer : bit 31 = 1; bits 30..16 = index of the 256-entry sub-table
//             indexed by the next 8 stream bits; the length fields read as 8.
namespace df11i {

// Runs the body of a C entry point so that no C++ exception crosses the C
// ABI: a failed host allocation, or a thread or lock the system could not
// provide, becomes DF11_E_NOMEM.
template <class F>
df11_status guarded(F &&body) noexcept {
    try {
        return body();
    } catch (const std::bad_alloc &) {
        return DF11_E_NOMEM;
    } catch (...) {
        return DF11_E_NOMEM;
    }
}

constexpr uint32_t kPointerFlag = 0x80000000u;

constexpr uint32_t leaf_entry(uint32_t exponent, uint32_t length) {
    return (exponent << 23) | ((length - 1u) << 8) | ((32u - length) & 31u);
}
constexpr uint32_t pointer_entry(uint32_t table) {
    return kPointerFlag | (table << 16) | (7u << 8) | 24u;
}
// Filler for entries no codeword reaches (only with a one-symbol alphabet or
// corrupt lengths): a 1-bit leaf of exponent 0, so a decoder always advances.
constexpr uint32_t kFillerEntry = leaf_entry(0, 1);

// Multi-code tables, placed after the hierarchical ones (all derived from the
// same canonical code):
//   count table, indexed by the next kCountBits stream bits, 32-bit entries:
//     bits 29..20 = start mask (bit 20+j set when a code starts at offset j and
//     ends inside the index bits), bits 15..8 = number of those codes, bits
//     7..0 = t, the bits they take (also the amount of a 64-bit shift, which
//     reads only bits 5..0).  When the first code is longer than kCountBits
//     the entry is kCountEscape: no codes, t = 128 (a shift by 0, and a step
//     large enough that a decoder's remaining-bits count turns negative).
//   emit table, indexed by the next kEmitBits bits, 64-bit entries holding
//     four 16-bit slots, slot k = (exponent_k << 7) | field_k, for the first
//     n = min(4, complete codes) codes.  An exponent shifted into its BF16
//     position leaves bits 6..0 free, which carry: field_0 = t, the bits of
//     the n codes (also the amount of a 64-bit shift, which reads only bits
//     5..0 of the entry), field_1 = n.  When the first code is longer than
//     kEmitBits the entry has t = 0 and field_1 = kEmitEscape (64), a step
//     that shifts by nothing and is too long for any lane's remaining count.
//     Slots past n are 0.  The whole entry can be written to a staging
//     buffer as is: a reader takes only bits 14..7 of a slot.
constexpr uint32_t kCountBits = 10;
constexpr uint32_t kCountEscape = 128;
constexpr uint32_t kEmitBits = 11;
constexpr uint32_t kEmitCodes = 4;
constexpr uint32_t kEmitEscape = 64;
constexpr uint32_t kCountEntries = 1u << kCountBits;
constexpr uint32_t kEmitEntries = 1u << kEmitBits;
constexpr uint64_t kMultiTableBytes = uint64_t{kCountEntries} * 4 + uint64_t{kEmitEntries} * 8;
constexpr uint64_t tables_bytes_for(uint32_t n_hier) { return uint64_t{n_hier} * 1024 + kMultiTableBytes; }

// Builds the decode tables for the 256 code lengths into dst (32-bit words:
// the hierarchical tables, then the count and emit tables), or only counts
// the hierarchical tables when dst is null.  Returns DF11_OK, DF11_E_FORMAT
// or DF11_E_BUFFER_TOO_SMALL.
df11_status build_tables(const uint8_t code_len[256], uint32_t *dst, uint64_t dst_words,
                         uint32_t *n_tables);

// Canonical codewords for the lengths (right aligned).  Returns false if the
// lengths exceed 32 bits or overflow the code space.
bool canonical_codes(const uint8_t code_len[256], uint32_t code[256]);

// Number of host threads to use for a request (0 = all CPUs available).
uint32_t thread_count(uint32_t requested);

// Code lengths for an exponent histogram: the deterministic Huffman code,
// length-limited to DF11_MAX_CODE_LEN by package-merge when needed (the rule
// of df11_encode_block); also the longest code, the symbols present and the
// stream length in bits.
df11_status code_lengths_for(const uint64_t cnt[256], uint8_t code_len[256], uint32_t *max_len,
                             uint32_t *n_symbols, uint64_t *total_bits);

// Host checks of a device block and its output before a launch: version,
// pointers, capacity, 16-byte alignment, sizes that no encoder produces
// (more than 2^48 weights, fewer than 1 or more than 32 bits per weight, 64
// with the aligned layout's filler), section sizes against n_total and
// total_bits.  n_total = 0 passes with only the version checked.
df11_status check_device_block(const df11_device_block *b, const uint16_t *out, uint64_t cap);

// The HIP error code of the last failing launch in this thread, for every
// entry point that launches kernels (reported by df11_last_hip_error).
extern thread_local int32_t last_hip_error;

}  // namespace df11i

struct df11_encoded {
    uint8_t *blob;
    uint64_t blob_bytes;
    df11_sections sec;
};
