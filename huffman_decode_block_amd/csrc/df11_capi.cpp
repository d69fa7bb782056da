// Host-only parts of the C-ABI: status text, structural validation of the
// sections, and device-block construction from a device copy of a blob.
#include <algorithm>
#include <cstring>
#include <vector>

#include "df11_internal.h"

extern "C" const char *df11_status_str(df11_status s) {
    switch (s) {
        case DF11_OK: return "ok";
        case DF11_E_INVALID_ARG: return "invalid argument";
        case DF11_E_NOMEM: return "out of host memory";
        case DF11_E_FORMAT: return "inconsistent DF11 sections";
        case DF11_E_BUFFER_TOO_SMALL: return "buffer too small";
        case DF11_E_UNSUPPORTED: return "unsupported version or feature";
        case DF11_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

namespace {

// No block holds more weights (2^48, 512 TB of BF16); below it no size the
// validator computes from n_total or total_bits can overflow 64 bits.
constexpr uint64_t kMaxWeights = uint64_t{1} << 48;

uint32_t gap_field(const uint8_t *gaps, uint64_t w) {
    const uint64_t bit = 5 * w;
    const uint32_t two = (uint32_t{gaps[bit >> 3]} << 8) | gaps[(bit >> 3) + 1];
    return (two >> (11 - (bit & 7))) & 31u;
}

}  // namespace

namespace {

df11_status validate(const df11_sections *s) {
    if (!s) return DF11_E_INVALID_ARG;
    if (s->version != DF11_FORMAT_VERSION) return DF11_E_UNSUPPORTED;
    if (!s->code_len || !s->stream || !s->gaps || !s->unit_pos || !s->tables) return DF11_E_INVALID_ARG;
    if (s->n_total && !s->sign_mant) return DF11_E_INVALID_ARG;
    // bounds first, so that no size computed below can wrap around
    if (s->n_total > kMaxWeights) return DF11_E_FORMAT;
    const bool aligned = s->unit_end_bytes != 0;
    // filler (aligned units) adds at most the rest of a unit to the codes
    if (s->total_bits < s->n_total ||
        s->total_bits > (aligned ? 2u : 1u) * uint64_t{DF11_MAX_CODE_LEN} * s->n_total)
        return DF11_E_FORMAT;
    const uint64_t nw = (s->total_bits + 63) / 64, nu = (nw + 63) / 64;
    if (s->n_windows != nw || s->n_units != nu) return DF11_E_FORMAT;
    if (s->stream_bytes < 512 * nu + 16 || s->gaps_bytes < 40 * nu + 8 ||
        s->sign_mant_bytes < (s->n_total + 15) / 16 * 16)
        return DF11_E_FORMAT;
    // code lengths: a prefix code of at most 32 bits; tables match them
    uint32_t code[256];
    if (!df11i::canonical_codes(s->code_len, code)) return DF11_E_FORMAT;
    uint32_t mx = 0, ns = 0;
    for (int e = 0; e < 256; ++e) {
        mx = std::max<uint32_t>(mx, s->code_len[e]);
        ns += s->code_len[e] ? 1u : 0u;
    }
    if (s->n_total && ns == 0) return DF11_E_FORMAT;
    uint32_t nt = 0;
    if (df11i::build_tables(s->code_len, nullptr, 0, &nt) != DF11_OK) return DF11_E_FORMAT;
    if (s->n_tables != nt || s->tables_bytes != df11i::tables_bytes_for(nt)) return DF11_E_FORMAT;
    std::vector<uint32_t> t(df11i::tables_bytes_for(nt) / 4);
    df11i::build_tables(s->code_len, t.data(), t.size(), nullptr);
    if (std::memcmp(t.data(), s->tables, s->tables_bytes) != 0) return DF11_E_FORMAT;
    // unit positions
    if (s->unit_pos[0] != 0 || s->unit_pos[nu] != s->n_total) return DF11_E_FORMAT;
    uint64_t mu = 0;
    for (uint64_t u = 0; u < nu; ++u) {
        if (s->unit_pos[u + 1] < s->unit_pos[u]) return DF11_E_FORMAT;
        const uint64_t d = s->unit_pos[u + 1] - s->unit_pos[u];
        if (d > DF11_MAX_UNIT_WEIGHTS) return DF11_E_FORMAT;
        mu = std::max(mu, d);
    }
    if (mu != s->max_unit_count) return DF11_E_FORMAT;
    // aligned units: unit ends within their units (the last one at the
    // stream's end), units beginning on multiples of 32 weights, zero filler
    if (aligned) {
        if (!s->unit_end || s->unit_end_bytes < 2 * nu) return DF11_E_FORMAT;
        for (uint64_t u = 0; u < nu; ++u) {
            const uint64_t ue = s->unit_end[u];
            if (ue < 1 || ue > 4096 || s->unit_pos[u] % 32 != 0) return DF11_E_FORMAT;
            if (u + 1 == nu ? 4096 * u + ue != s->total_bits : false) return DF11_E_FORMAT;
            if (u + 1 < nu)
                for (uint64_t b = 4096 * u + ue; b < 4096 * (u + 1); ++b)
                    if ((s->stream[b >> 3] >> (7 - (b & 7))) & 1u) return DF11_E_FORMAT;
        }
    }
    // gaps: the first code of a window starts inside it, or is the end of the
    // codes of its unit (aligned units: a window wholly past it has gap 0)
    for (uint64_t w = 0; w < nw; ++w) {
        const uint64_t g = gap_field(s->gaps, w), start = 64 * w + g;
        const uint64_t end = aligned ? 4096 * (w / 64) + s->unit_end[w / 64] : s->total_bits;
        if (aligned && 64 * w >= end) {
            if (g != 0) return DF11_E_FORMAT;
            continue;
        }
        if (start > end) return DF11_E_FORMAT;
        if (!aligned && start == end && w + 1 != nw) return DF11_E_FORMAT;
    }
    // optional per-window counts: at most 64 each, summing to each unit's count
    if (s->counts_bytes) {
        if (!s->counts || s->counts_bytes < 64 * nu) return DF11_E_FORMAT;
        for (uint64_t u = 0; u < nu; ++u) {
            uint64_t sum = 0;
            for (uint64_t w = 64 * u; w < 64 * u + 64; ++w) {
                const uint64_t c = s->counts[w];
                if (c > 64 || (w >= nw && c != 0)) return DF11_E_FORMAT;
                sum += c;
            }
            if (sum != s->unit_pos[u + 1] - s->unit_pos[u]) return DF11_E_FORMAT;
        }
    }
    return DF11_OK;
}

}  // namespace

extern "C" df11_status df11_validate(const df11_sections *s) {
    return df11i::guarded([&] { return validate(s); });
}

extern "C" df11_status df11_device_block_from_blob(const df11_sections *s, const void *device_blob,
                                                   df11_device_block *out) {
    if (!s || !device_blob || !out) return DF11_E_INVALID_ARG;
    const uint8_t *b = static_cast<const uint8_t *>(device_blob);
    df11_device_block d{};
    d.tables = b + s->off_tables;
    d.tables_bytes = s->tables_bytes;
    d.stream = b + s->off_stream;
    d.stream_bytes = s->stream_bytes;
    d.sign_mant = b + s->off_sign_mant;
    d.sign_mant_bytes = s->sign_mant_bytes;
    d.gaps = b + s->off_gaps;
    d.gaps_bytes = s->gaps_bytes;
    d.unit_pos = reinterpret_cast<const uint64_t *>(b + s->off_unit_pos);
    d.n_total = s->n_total;
    d.total_bits = s->total_bits;
    d.n_windows = s->n_windows;
    d.n_units = s->n_units;
    d.max_unit_count = s->max_unit_count;
    d.version = s->version;
    d.n_tables = s->n_tables;
    d.counts = s->counts_bytes ? b + s->off_counts : nullptr;
    d.unit_end = s->unit_end_bytes ? reinterpret_cast<const uint16_t *>(b + s->off_unit_end) : nullptr;
    *out = d;
    return DF11_OK;
}
