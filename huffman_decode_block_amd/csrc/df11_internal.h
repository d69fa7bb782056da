// Internal declarations shared by the host-side translation units of libdf11.
#pragma once

#include <cstdint>

#include "df11.h"

// Decode-table entry layout (32 bits), used by the table builder and the
// kernel:
//   leaf    : bit 31 = 0; bits 30..23 = exponent (so bits 31..16 hold
//             exponent << 7, the exponent field of a BF16 value);
//             bits 12..8 = code length - 1; bits 4..0 = (32 - length) & 31.
//   pointer : bit 31 = 1; bits 30..16 = index of the 256-entry sub-table
//             indexed by the next 8 stream bits; the length fields read as 8.
namespace df11i {

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

// Builds the decode tables for the 256 code lengths into dst (entries), or
// only counts them when dst is null.  Returns DF11_OK, DF11_E_FORMAT or
// DF11_E_BUFFER_TOO_SMALL.
df11_status build_tables(const uint8_t code_len[256], uint32_t *dst, uint64_t dst_entries,
                         uint32_t *n_tables);

// Canonical codewords for the lengths (right aligned).  Returns false if the
// lengths exceed 32 bits or overflow the code space.
bool canonical_codes(const uint8_t code_len[256], uint32_t code[256]);

// Number of host threads to use for a request (0 = all CPUs available).
uint32_t thread_count(uint32_t requested);

}  // namespace df11i

struct df11_encoded {
    uint8_t *blob;
    uint64_t blob_bytes;
    df11_sections sec;
};
