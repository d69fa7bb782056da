// Decode tables for the GPU kernel, derived from the code lengths.
//
// The pages (hada.io summary of the DFloat11 paper, section "Decodage fonde
// sur des LUT hierarchiques") split the Huffman tree into disjoint subtrees of
// height 8, one 256-entry table each, some entries of which refer to a
// lower-level table.  Here every entry is 32 bits wide (layout in
// df11_internal.h): the pointer flag needs no reserved exponent values, a leaf
// entry carries the exponent already shifted into its BF16 position plus the
// code length in the two forms the kernel consumes, so one LDS read per code
// gives everything.
#include <algorithm>
#include <vector>

#include "df11_internal.h"

namespace df11i {

bool canonical_codes(const uint8_t code_len[256], uint32_t code[256]) {
    // counts per length, then the first code of each length
    uint64_t per_len[DF11_MAX_CODE_LEN + 1] = {0};
    for (int e = 0; e < 256; ++e) {
        if (code_len[e] > DF11_MAX_CODE_LEN) return false;
        if (code_len[e]) per_len[code_len[e]] += 1;
    }
    uint64_t first[DF11_MAX_CODE_LEN + 2] = {0};
    uint64_t c = 0;
    for (uint32_t l = 1; l <= DF11_MAX_CODE_LEN; ++l) {
        c = (c + per_len[l - 1]) << 1;
        first[l] = c;
    }
    // within one length, codes follow the exponent order
    for (int e = 0; e < 256; ++e) {
        code[e] = 0;
        uint32_t l = code_len[e];
        if (!l) continue;
        uint64_t v = first[l]++;
        if (v >> l) return false;  // code space exhausted (Kraft sum > 1)
        code[e] = static_cast<uint32_t>(v);
    }
    return true;
}

namespace {

// One code from a left-aligned 32-bit window, through the hierarchical tables.
uint32_t walk(const std::vector<uint32_t> &t, uint32_t window) {
    uint32_t e = t[window >> 24];
    for (int lvl = 1; lvl < 4 && (e & kPointerFlag); ++lvl)
        e = t[((e >> 16) & 0x7FFFu) * 256 + ((window >> (24 - 8 * lvl)) & 0xFFu)];
    return e;
}

uint32_t entry_length(uint32_t e) { return ((e >> 8) & 31u) + 1; }

}  // namespace

df11_status build_tables(const uint8_t code_len[256], uint32_t *dst, uint64_t dst_words,
                         uint32_t *n_tables) {
    uint32_t code[256];
    if (!canonical_codes(code_len, code)) return DF11_E_FORMAT;
    constexpr uint32_t kUnset = 0xFFFFFFFFu;
    std::vector<uint32_t> t(256, kUnset);
    // place symbols in (length, exponent) order so parents exist before leaves
    std::vector<int> order;
    for (int e = 0; e < 256; ++e)
        if (code_len[e]) order.push_back(e);
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return code_len[a] < code_len[b]; });
    for (int e : order) {
        const uint32_t len = code_len[e];
        const uint32_t c = code[e];
        uint32_t table = 0, used = 0;  // bits resolved by the tables above
        while (len - used > 8) {
            const uint32_t idx = (c >> (len - used - 8)) & 0xFFu;
            uint32_t &slot = t[table * 256 + idx];
            if (slot == kUnset) {
                const uint32_t fresh = static_cast<uint32_t>(t.size() / 256);
                if (fresh > 0x7FFFu) return DF11_E_FORMAT;
                slot = pointer_entry(fresh);
                t.resize(t.size() + 256, kUnset);
                table = fresh;
            } else if (slot & kPointerFlag) {
                table = (slot >> 16) & 0x7FFFu;
            } else {
                return DF11_E_FORMAT;  // a shorter code is a prefix of this one
            }
            used += 8;
        }
        const uint32_t rest = len - used;  // 1..8 bits inside this table
        const uint32_t base = (c & ((1u << rest) - 1u)) << (8 - rest);
        for (uint32_t k = 0; k < (1u << (8 - rest)); ++k) {
            uint32_t &slot = t[table * 256 + base + k];
            if (slot != kUnset) return DF11_E_FORMAT;
            slot = leaf_entry(static_cast<uint32_t>(e), len);
        }
    }
    for (auto &v : t)
        if (v == kUnset) v = kFillerEntry;
    const uint32_t nt = static_cast<uint32_t>(t.size() / 256);
    if (n_tables) *n_tables = nt;
    if (!dst) return DF11_OK;
    if (dst_words < tables_bytes_for(nt) / 4) return DF11_E_BUFFER_TOO_SMALL;
    std::copy(t.begin(), t.end(), dst);

    // count table: every code that starts and ends inside the index bits
    uint32_t *count = dst + t.size();
    for (uint32_t p = 0; p < kCountEntries; ++p) {
        uint32_t pos = 0, mask = 0, n = 0;
        while (pos < kCountBits) {
            const uint32_t window = (p << (32 - kCountBits)) << pos;
            const uint32_t l = entry_length(walk(t, window));
            if (l > kCountBits - pos) break;
            mask |= 1u << pos;
            pos += l;
            n += 1;
        }
        count[p] = pos ? (mask << 20) | (n << 8) | pos : kCountEscape;
    }
    // emit table: up to four codes that end inside the index bits
    uint32_t *emit = count + kCountEntries;
    for (uint32_t p = 0; p < kEmitEntries; ++p) {
        uint32_t pos = 0, n = 0, slot[kEmitCodes] = {0, 0, 0, 0};
        while (n < kEmitCodes && pos < kEmitBits) {
            const uint32_t window = (p << (32 - kEmitBits)) << pos;
            const uint32_t e = walk(t, window);
            const uint32_t l = entry_length(e);
            if (l > kEmitBits - pos) break;
            slot[n] = e >> 16;  // exponent << 7
            pos += l;
            n += 1;
        }
        if (n) {
            slot[0] |= pos;
            slot[1] |= n;
        } else {
            slot[1] = kEmitEscape;
        }
        emit[2 * p] = slot[0] | (slot[1] << 16);
        emit[2 * p + 1] = slot[2] | (slot[3] << 16);
    }
    return DF11_OK;
}

}  // namespace df11i

extern "C" df11_status df11_tables_size(const uint8_t code_len[256], uint64_t *bytes,
                                        uint32_t *n_tables) {
    if (!code_len || !bytes) return DF11_E_INVALID_ARG;
    return df11i::guarded([&] {
        uint32_t nt = 0;
        const df11_status rc = df11i::build_tables(code_len, nullptr, 0, &nt);
        if (rc != DF11_OK) return rc;
        *bytes = df11i::tables_bytes_for(nt);
        if (n_tables) *n_tables = nt;
        return DF11_OK;
    });
}

extern "C" df11_status df11_build_tables(const uint8_t code_len[256], void *dst,
                                         uint64_t dst_bytes) {
    if (!code_len || !dst) return DF11_E_INVALID_ARG;
    return df11i::guarded([&] {
        return df11i::build_tables(code_len, static_cast<uint32_t *>(dst), dst_bytes / sizeof(uint32_t), nullptr);
    });
}
