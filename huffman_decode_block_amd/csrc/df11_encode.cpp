// Host-side DF11 block encoder (multithreaded C++17).
//
// Follows the hada.io summary of the DFloat11 paper: section "La marge de
// compression restante dans l'exposant BFloat16" (1 sign, 8 exponent and 7
// mantissa bits; the exponent carries little information), section "Le format
// DFloat11" (Huffman code from the exponent histogram, codes bit-packed into
// EncodedExponent, sign and mantissa verbatim in PackedSignMantissa), and
// section "Noyau GPU en deux etapes et metadonnees auxiliaires" (8-byte
// thread windows, a 5-bit gap per window, output positions stored once per
// group of windows).  The format choices the pages leave open are stated in
// include/df11.h.
#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <sched.h>
#include <thread>
#include <exception>
#include <memory>
#include <vector>

#include "df11_internal.h"

namespace {

using df11i::thread_count;

// Runs fn(t) for t in [0, n) on up to n threads.  An exception in any of
// them, or in starting a thread, is rethrown here once every thread that
// started has been joined: none escapes a thread or leaves one running.
void run_parallel(uint32_t n, const std::function<void(uint32_t)> &fn) {
    if (n <= 1) {
        if (n == 1) fn(0);
        return;
    }
    std::vector<std::exception_ptr> err(n);
    auto body = [&](uint32_t t) {
        try {
            fn(t);
        } catch (...) {
            err[t] = std::current_exception();
        }
    };
    std::vector<std::thread> pool;
    pool.reserve(n - 1);
    std::exception_ptr start_err;
    try {
        for (uint32_t t = 1; t < n; ++t) pool.emplace_back(body, t);
    } catch (...) {
        start_err = std::current_exception();
    }
    if (!start_err) body(0);
    for (auto &th : pool) th.join();
    if (start_err) std::rethrow_exception(start_err);
    for (auto &e : err)
        if (e) std::rethrow_exception(e);
}

// The block as one logical array over the caller's matrices.
struct Source {
    const df11_bf16_view *mats;
    std::vector<uint64_t> off;  // n_mats + 1 prefix offsets

    template <class F>
    void visit(uint64_t b, uint64_t e, F &&f) const {
        if (b >= e) return;
        size_t s = std::upper_bound(off.begin(), off.end(), b) - off.begin() - 1;
        uint64_t i = b;
        while (i < e) {
            while (off[s + 1] <= i) ++s;
            const uint16_t *p = mats[s].data;
            const uint64_t o = off[s];
            const uint64_t stop = std::min(e, off[s + 1]);
            for (; i < stop; ++i) f(i, p[i - o]);
        }
    }
    uint16_t at(uint64_t i) const {
        size_t s = std::upper_bound(off.begin(), off.end(), i) - off.begin() - 1;
        while (off[s + 1] <= i) ++s;
        return mats[s].data[i - off[s]];
    }
};

inline uint32_t exponent_of(uint16_t x) { return (x >> 7) & 0xFFu; }

// Huffman code lengths with the two-queue method: leaves sorted by
// (count, exponent) in one queue, merged nodes in creation order in the
// other (their weights never decrease); on equal weight the leaf goes first.
// Returns the longest length.
uint32_t huffman_lengths(const uint64_t cnt[256], uint32_t len[256]) {
    std::vector<int> sym;
    for (int e = 0; e < 256; ++e) {
        len[e] = 0;
        if (cnt[e]) sym.push_back(e);
    }
    std::sort(sym.begin(), sym.end(),
              [&](int a, int b) { return cnt[a] != cnt[b] ? cnt[a] < cnt[b] : a < b; });
    const int n = static_cast<int>(sym.size());
    if (n == 0) return 0;
    if (n == 1) {
        len[sym[0]] = 1;
        return 1;
    }
    std::vector<uint64_t> w(2 * n - 1);
    std::vector<int> parent(2 * n - 1, -1);
    for (int k = 0; k < n; ++k) w[k] = cnt[sym[k]];
    int leaf = 0, inner = n, next = n;
    for (int m = 0; m < n - 1; ++m) {
        int pick[2];
        for (int &p : pick) {
            const bool take_leaf = leaf < n && (inner >= next || w[leaf] <= w[inner]);
            p = take_leaf ? leaf++ : inner++;
        }
        w[next] = w[pick[0]] + w[pick[1]];
        parent[pick[0]] = parent[pick[1]] = next;
        ++next;
    }
    std::vector<uint32_t> depth(2 * n - 1, 0);
    uint32_t mx = 0;
    for (int v = 2 * n - 3; v >= 0; --v) {
        depth[v] = depth[parent[v]] + 1;
        if (v < n) {
            len[sym[v]] = depth[v];
            mx = std::max(mx, depth[v]);
        }
    }
    return mx;
}

// Length-limited lengths by package-merge, computed as counts: the lists of
// every level are built bottom-up as (weight, is-leaf) sequences, then the
// selection of the first 2n-2 items of the top list is pushed down, level by
// level, as "the first a_d leaves plus the first p_d packages".  A leaf of
// sorted index k gets the number of levels with k < a_d.  On equal weight a
// leaf precedes a package.
bool package_merge_lengths(const uint64_t cnt[256], uint32_t cap, uint32_t len[256]) {
    std::vector<int> sym;
    for (int e = 0; e < 256; ++e) {
        len[e] = 0;
        if (cnt[e]) sym.push_back(e);
    }
    std::sort(sym.begin(), sym.end(),
              [&](int a, int b) { return cnt[a] != cnt[b] ? cnt[a] < cnt[b] : a < b; });
    const size_t n = sym.size();
    if (n == 0) return true;
    if (n == 1) {
        len[sym[0]] = 1;
        return true;
    }
    if (cap < 1 || cap > 62 || (uint64_t{1} << cap) < n) return false;
    std::vector<uint64_t> lw(n);
    for (size_t k = 0; k < n; ++k) lw[k] = cnt[sym[k]];
    std::vector<std::vector<uint64_t>> wt(cap + 1);
    std::vector<std::vector<uint8_t>> is_leaf(cap + 1);
    wt[cap] = lw;
    is_leaf[cap].assign(n, 1);
    for (uint32_t d = cap - 1; d >= 1; --d) {
        const auto &below = wt[d + 1];
        const size_t npk = below.size() / 2;
        auto &W = wt[d];
        auto &L = is_leaf[d];
        W.reserve(n + npk);
        size_t i = 0, j = 0;
        while (i < n || j < npk) {
            const uint64_t pw = j < npk ? below[2 * j] + below[2 * j + 1] : 0;
            if (j >= npk || (i < n && lw[i] <= pw)) {
                W.push_back(lw[i++]);
                L.push_back(1);
            } else {
                W.push_back(pw);
                L.push_back(0);
                ++j;
            }
        }
        if (d == 1) break;
    }
    std::vector<size_t> leaves_at(cap + 1, 0);
    size_t m = 2 * n - 2;
    for (uint32_t d = 1; d <= cap; ++d) {
        if (m > wt[d].size()) return false;
        size_t a = 0;
        for (size_t k = 0; k < m; ++k) a += is_leaf[d][k];
        leaves_at[d] = a;
        m = 2 * (m - a);
    }
    if (m != 0) return false;
    for (size_t k = 0; k < n; ++k) {
        uint32_t l = 0;
        for (uint32_t d = 1; d <= cap; ++d) l += (k < leaves_at[d]) ? 1u : 0u;
        len[sym[k]] = l;
    }
    return true;
}

inline uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

}  // namespace

namespace df11i {

uint32_t thread_count(uint32_t requested) {
    if (requested) return requested;
    cpu_set_t set;
    CPU_ZERO(&set);
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int c = CPU_COUNT(&set);
        if (c > 0) return static_cast<uint32_t>(c);
    }
    unsigned h = std::thread::hardware_concurrency();
    return h ? h : 1u;
}

df11_status code_lengths_for(const uint64_t cnt[256], uint8_t code_len[256], uint32_t *max_len,
                             uint32_t *n_symbols, uint64_t *total_bits) {
    uint32_t len32[256];
    uint32_t ml = huffman_lengths(cnt, len32);
    if (ml > DF11_MAX_CODE_LEN) {
        if (!package_merge_lengths(cnt, DF11_MAX_CODE_LEN, len32)) return DF11_E_FORMAT;
        ml = 0;
        for (int e = 0; e < 256; ++e) ml = std::max(ml, len32[e]);
    }
    uint32_t ns = 0;
    uint64_t tb = 0;
    for (int e = 0; e < 256; ++e) {
        code_len[e] = static_cast<uint8_t>(len32[e]);
        ns += cnt[e] ? 1u : 0u;
        tb += cnt[e] * len32[e];
    }
    *max_len = ml;
    *n_symbols = ns;
    *total_bits = tb;
    return DF11_OK;
}

}  // namespace df11i

extern "C" df11_status df11_encode_block(const df11_bf16_view *mats, uint32_t n_mats,
                                         uint32_t n_threads, df11_encoded **out) {
    return df11_encode_block_ex(mats, n_mats, n_threads, 0u, out);
}

namespace {

df11_status encode_block(const df11_bf16_view *mats, uint32_t n_mats, uint32_t n_threads, uint32_t flags,
                         df11_encoded **out) {
    if (!out || (n_mats && !mats) || (flags & ~(DF11_ENCODE_WINDOW_COUNTS | DF11_ENCODE_ALIGNED_UNITS)))
        return DF11_E_INVALID_ARG;
    const bool with_counts = (flags & DF11_ENCODE_WINDOW_COUNTS) != 0;
    const bool aligned = (flags & DF11_ENCODE_ALIGNED_UNITS) != 0;
    *out = nullptr;
    Source src{mats, std::vector<uint64_t>(n_mats + 1, 0)};
    for (uint32_t m = 0; m < n_mats; ++m) {
        if (mats[m].numel && !mats[m].data) return DF11_E_INVALID_ARG;
        src.off[m + 1] = src.off[m] + mats[m].numel;
    }
    const uint64_t N = src.off[n_mats];
    const uint32_t T = std::max<uint32_t>(
        1, std::min<uint64_t>(thread_count(n_threads), std::max<uint64_t>(1, N >> 20)));

    // ---- exponent histogram
    std::vector<std::array<uint64_t, 256>> part(T);
    run_parallel(T, [&](uint32_t t) {
        auto &h = part[t];
        h.fill(0);
        src.visit(N * t / T, N * (t + 1) / T, [&](uint64_t, uint16_t x) { h[exponent_of(x)]++; });
    });
    uint64_t cnt[256] = {0};
    for (auto &h : part)
        for (int e = 0; e < 256; ++e) cnt[e] += h[e];

    // ---- code lengths and canonical codes
    uint8_t code_len[256];
    uint32_t max_len = 0, n_symbols = 0;
    uint64_t total_bits = 0;
    if (df11i::code_lengths_for(cnt, code_len, &max_len, &n_symbols, &total_bits) != DF11_OK)
        return DF11_E_FORMAT;
    uint32_t len32[256];
    for (int e = 0; e < 256; ++e) len32[e] = code_len[e];
    uint32_t code[256];
    if (!df11i::canonical_codes(code_len, code)) return DF11_E_FORMAT;
    uint32_t n_tables = 0;
    if (df11i::build_tables(code_len, nullptr, 0, &n_tables) != DF11_OK) return DF11_E_FORMAT;

    const uint64_t code_bits = total_bits;  // the codewords alone

    // ---- aligned-units layout: where each group of 32 codes starts.  Group
    // bit counts in parallel, then one pass in order: a group whose last code
    // would start in a later unit than its first goes to the next unit, the
    // rest of the current unit being filler.  Chunks of the packing below
    // then begin on group boundaries at these positions.
    constexpr uint64_t kGroup = 32, kUnitBits = 4096;
    std::vector<uint64_t> gstart;  // per group: first bit (aligned layout only)
    std::vector<uint16_t> uend;    // per unit: end of its codes from its first bit
    if (aligned && N) {
        const uint64_t n_groups = (N + kGroup - 1) / kGroup;
        std::vector<uint32_t> gbits(n_groups), glast(n_groups);  // bits, offset of the last start
        run_parallel(T, [&](uint32_t t) {
            for (uint64_t g = n_groups * t / T; g < n_groups * (t + 1) / T; ++g) {
                uint32_t b = 0, last = 0;
                src.visit(g * kGroup, std::min(N, (g + 1) * kGroup), [&](uint64_t, uint16_t x) {
                    last = b;
                    b += len32[exponent_of(x)];
                });
                gbits[g] = b;
                glast[g] = last;
            }
        });
        gstart.resize(n_groups);
        std::vector<std::pair<uint64_t, uint64_t>> filler;  // (unit, end of its codes), in order
        uint64_t pos = 0;
        for (uint64_t g = 0; g < n_groups; ++g) {
            const uint64_t u = pos / kUnitBits;
            if (pos + glast[g] >= (u + 1) * kUnitBits) {
                filler.emplace_back(u, pos);
                pos = (u + 1) * kUnitBits;
            }
            gstart[g] = pos;
            pos += gbits[g];
        }
        total_bits = pos;
        const uint64_t nu = ((total_bits + 63) / 64 + 63) / 64;
        uend.assign(nu, static_cast<uint16_t>(kUnitBits));
        for (const auto &f : filler) uend[f.first] = static_cast<uint16_t>(f.second - f.first * kUnitBits);
        if (nu) uend[nu - 1] = static_cast<uint16_t>(total_bits - (nu - 1) * kUnitBits);
    }

    // ---- sizes and blob layout (256-byte aligned sections)
    const uint64_t n_windows = (total_bits + 63) / 64;
    const uint64_t n_units = (n_windows + 63) / 64;
    df11_sections s{};
    s.version = DF11_FORMAT_VERSION;
    s.n_mats = n_mats;
    s.n_symbols = n_symbols;
    s.max_code_len = max_len;
    s.n_tables = n_tables;
    s.n_total = N;
    s.total_bits = total_bits;
    s.n_windows = n_windows;
    s.n_units = n_units;
    s.stream_bytes = 512 * n_units + 16;
    s.sign_mant_bytes = round_up(N, 16);
    s.gaps_bytes = 40 * n_units + 8;
    s.tables_bytes = df11i::tables_bytes_for(n_tables);
    uint64_t off = 256;  // reserved header
    auto place = [&](uint64_t bytes) {
        const uint64_t at = off;
        off = round_up(off + bytes, 256);
        return at;
    };
    s.off_code_len = place(256);
    s.off_mat_offset = place(8 * (uint64_t{n_mats} + 1));
    s.off_tables = place(s.tables_bytes);
    s.off_stream = place(s.stream_bytes);
    s.off_sign_mant = place(s.sign_mant_bytes);
    s.off_gaps = place(s.gaps_bytes);
    s.off_unit_pos = place(8 * (n_units + 1));
    s.counts_bytes = with_counts ? 64 * n_units : 0;
    s.off_counts = with_counts ? place(s.counts_bytes) : 0;
    s.unit_end_bytes = aligned ? 2 * n_units : 0;
    s.off_unit_end = aligned ? place(s.unit_end_bytes) : 0;
    s.blob_bytes = off;

    void *mem = nullptr;
    if (posix_memalign(&mem, 4096, round_up(s.blob_bytes, 4096)) != 0 || !mem) return DF11_E_NOMEM;
    uint8_t *blob = static_cast<uint8_t *>(mem);
    auto *enc = new (std::nothrow) df11_encoded{blob, s.blob_bytes, s};
    if (!enc) {
        free(mem);
        return DF11_E_NOMEM;
    }
    // freed on every way out but success, exceptions included
    std::unique_ptr<df11_encoded, void (*)(df11_encoded *)> owner(enc, &df11_encoded_free);
    std::memset(blob, 0, s.off_stream);  // header, code_len, mat_offset, tables
    std::memcpy(blob, "DF11", 4);
    std::memcpy(blob + s.off_code_len, code_len, 256);
    std::memcpy(blob + s.off_mat_offset, src.off.data(), 8 * (uint64_t{n_mats} + 1));
    df11i::build_tables(code_len, reinterpret_cast<uint32_t *>(blob + s.off_tables),
                        s.tables_bytes / 4, nullptr);

    uint8_t *stream = blob + s.off_stream;
    uint8_t *sm = blob + s.off_sign_mant;
    uint8_t *gaps = blob + s.off_gaps;
    uint64_t *unit_pos = reinterpret_cast<uint64_t *>(blob + s.off_unit_pos);
    uint64_t *words = reinterpret_cast<uint64_t *>(stream);  // stream as 64-bit words, bit 63 first
    const uint64_t n_words = s.stream_bytes / 8;
    std::vector<uint8_t> gap8(n_windows, 0xFF);
    constexpr uint64_t kNoStart = ~uint64_t{0};
    std::vector<uint64_t> wfirst(with_counts ? n_windows : 0, kNoStart);  // first element starting in w

    // zero the stream, the tails of the other sections; unit_pos starts at N
    run_parallel(T, [&](uint32_t t) {
        std::memset(stream + s.stream_bytes * t / T, 0,
                    s.stream_bytes * (t + 1) / T - s.stream_bytes * t / T);
        for (uint64_t u = (n_units + 1) * t / T; u < (n_units + 1) * (t + 1) / T; ++u) unit_pos[u] = N;
    });
    std::memset(sm + N, 0, s.sign_mant_bytes - N);
    std::memset(gaps, 0, s.gaps_bytes);
    std::memset(blob + s.off_sign_mant + s.sign_mant_bytes, 0,
                s.off_gaps - s.off_sign_mant - s.sign_mant_bytes);

    // ---- chunked packing: bit offset of each chunk, then each chunk packs its
    // codes; words shared with a neighbouring chunk are merged atomically.
    // Chunk boundaries fall on group boundaries in the aligned layout.
    const uint64_t n_chunks = N ? std::min<uint64_t>(aligned ? (N + kGroup - 1) / kGroup : N, uint64_t{T} * 8) : 0;
    auto chunk_begin = [&](uint64_t c) {
        if (!aligned) return N * c / n_chunks;
        const uint64_t n_groups = (N + kGroup - 1) / kGroup;
        return std::min(N, n_groups * c / n_chunks * kGroup);
    };
    std::vector<uint64_t> chunk_bits(n_chunks + 1, 0);
    if (aligned) {
        for (uint64_t c = 0; c < n_chunks; ++c) chunk_bits[c] = gstart[chunk_begin(c) / kGroup];
    } else {
        run_parallel(T, [&](uint32_t t) {
            for (uint64_t c = t; c < n_chunks; c += T) {
                uint64_t b = 0;
                src.visit(chunk_begin(c), chunk_begin(c + 1), [&](uint64_t, uint16_t x) { b += len32[exponent_of(x)]; });
                chunk_bits[c + 1] = b;
            }
        });
        for (uint64_t c = 0; c < n_chunks; ++c) chunk_bits[c + 1] += chunk_bits[c];
    }

    run_parallel(T, [&](uint32_t t) {
        for (uint64_t c = t; c < n_chunks; c += T) {
            const uint64_t i0 = chunk_begin(c), i1 = chunk_begin(c + 1);
            const uint64_t bit0 = chunk_bits[c];
            uint64_t bit = bit0;
            // the previous code's start (for the first-start rules); none for the block's first
            uint64_t prev_start = 0;
            if (i0) {
                const uint64_t lp = len32[exponent_of(src.at(i0 - 1))];
                prev_start = aligned ? gstart[(i0 - 1) / kGroup] : bit0 - lp;
                if (aligned)  // the previous group's last code: its start from the group's
                    src.visit((i0 - 1) / kGroup * kGroup, i0 - 1,
                              [&](uint64_t, uint16_t x) { prev_start += len32[exponent_of(x)]; });
            }
            uint64_t acc = 0;
            uint32_t fill = static_cast<uint32_t>(bit0 & 63);
            uint64_t word = bit0 >> 6;
            auto flush = [&](bool last) {
                if (word * 64 < bit0 || last)
                    __atomic_fetch_or(&words[word], acc, __ATOMIC_RELAXED);
                else
                    words[word] = acc;
            };
            src.visit(i0, i1, [&](uint64_t i, uint16_t x) {
                const uint32_t e = exponent_of(x);
                const uint32_t l = len32[e];
                if (aligned && i % kGroup == 0 && gstart[i / kGroup] != bit) {  // a filler before this group
                    if (fill) flush(true);
                    bit = gstart[i / kGroup];
                    acc = 0;
                    fill = static_cast<uint32_t>(bit & 63);
                    word = bit >> 6;
                }
                // first code start in its window / unit?
                const uint64_t w = bit >> 6;
                if (i == 0 || (prev_start >> 6) < w) {
                    gap8[w] = static_cast<uint8_t>(bit - 64 * w);
                    if (with_counts) wfirst[w] = i;
                }
                const uint64_t u = bit >> 12;
                if (i == 0 || (prev_start >> 12) < u) unit_pos[u] = i;
                sm[i] = static_cast<uint8_t>(((x >> 8) & 0x80u) | (x & 0x7Fu));
                const uint64_t cw = code[e];
                if (fill + l < 64) {
                    acc |= cw << (64 - fill - l);
                    fill += l;
                } else {
                    const uint32_t r = 64 - fill;  // bits that still fit, 1..32
                    acc |= (l > r) ? (cw >> (l - r)) : cw;
                    flush(false);
                    ++word;
                    const uint32_t spill = l - r;
                    acc = spill ? (cw << (64 - spill)) : 0;
                    fill = spill;
                }
                prev_start = bit;
                bit += l;
            });
            if (fill) flush(true);
        }
    });

    // words -> MSB-first bytes
    run_parallel(T, [&](uint32_t t) {
        for (uint64_t k = n_words * t / T; k < n_words * (t + 1) / T; ++k)
            words[k] = __builtin_bswap64(words[k]);
    });

    // ---- gaps of windows where no code starts: the end of the unit's codes
    // minus the window's first bit when it comes later (the last window of
    // the stream, or one that a filler begins in), else 0 (a window of filler)
    for (uint64_t w = 0; w < n_windows; ++w) {
        if (gap8[w] == 0xFF) {
            const uint64_t u = w / 64;
            const uint64_t end = aligned ? u * kUnitBits + uend[u] : total_bits;
            if (!aligned && w + 1 != n_windows) {
                return DF11_E_FORMAT;
            }
            const uint64_t g = end > 64 * w ? end - 64 * w : 0;
            if (g > 31) {
                return DF11_E_FORMAT;
            }
            gap8[w] = static_cast<uint8_t>(g);
        } else if (aligned) {  // a start at or after the end of the unit's codes (only in filler: none)
            const uint64_t u = w / 64;
            const uint64_t end = u * kUnitBits + uend[u];
            if (64 * w + gap8[w] >= end && 64 * w < end) {
                return DF11_E_FORMAT;
            }
        }
    }
    const uint64_t n_groups = (n_windows + 7) / 8;  // 8 fields = 5 bytes
    run_parallel(T, [&](uint32_t t) {
        for (uint64_t g = n_groups * t / T; g < n_groups * (t + 1) / T; ++g) {
            uint64_t v = 0;
            for (uint64_t j = 0; j < 8; ++j) {
                const uint64_t w = 8 * g + j;
                v = (v << 5) | (w < n_windows ? gap8[w] : 0u);
            }
            for (int b = 0; b < 5; ++b) gaps[5 * g + b] = static_cast<uint8_t>(v >> (32 - 8 * b));
        }
    });
    unit_pos[n_units] = N;
    if (with_counts) {  // codes starting in window w: up to the next window's first
        uint8_t *counts = blob + s.off_counts;
        std::memset(counts, 0, s.counts_bytes);
        uint64_t next = N;
        for (uint64_t w = n_windows; w-- > 0;) {
            if (wfirst[w] == kNoStart) continue;  // only the last window may have none
            const uint64_t c = next - wfirst[w];
            if (c > 64) {
                return DF11_E_FORMAT;
            }
            counts[w] = static_cast<uint8_t>(c);
            next = wfirst[w];
        }
    }
    if (aligned && n_units) std::memcpy(blob + s.off_unit_end, uend.data(), 2 * n_units);
    uint64_t mu = 0;
    for (uint64_t u = 0; u < n_units; ++u) mu = std::max(mu, unit_pos[u + 1] - unit_pos[u]);
    enc->sec.max_unit_count = mu;

    // ---- statistics
    double h = 0.0;
    for (int e = 0; e < 256; ++e) {
        if (!cnt[e]) continue;
        const double p = static_cast<double>(cnt[e]) / static_cast<double>(N);
        h -= p * std::log2(p);
    }
    enc->sec.exp_entropy_bits = h;
    enc->sec.mean_code_len_bits = N ? static_cast<double>(code_bits) / static_cast<double>(N) : 0.0;
    *out = owner.release();
    return DF11_OK;
}

}  // namespace

extern "C" df11_status df11_encode_block_ex(const df11_bf16_view *mats, uint32_t n_mats,
                                            uint32_t n_threads, uint32_t flags, df11_encoded **out) {
    if (out) *out = nullptr;
    return df11i::guarded([&] { return encode_block(mats, n_mats, n_threads, flags, out); });
}

extern "C" df11_status df11_encoded_sections(const df11_encoded *enc, df11_sections *out) {
    if (!enc || !out) return DF11_E_INVALID_ARG;
    *out = enc->sec;
    const uint8_t *b = enc->blob;
    out->blob = b;
    out->blob_bytes = enc->blob_bytes;
    out->code_len = b + out->off_code_len;
    out->mat_offset = reinterpret_cast<const uint64_t *>(b + out->off_mat_offset);
    out->stream = b + out->off_stream;
    out->sign_mant = b + out->off_sign_mant;
    out->gaps = b + out->off_gaps;
    out->unit_pos = reinterpret_cast<const uint64_t *>(b + out->off_unit_pos);
    out->tables = b + out->off_tables;
    out->counts = out->counts_bytes ? b + out->off_counts : nullptr;
    out->unit_end = out->unit_end_bytes ? reinterpret_cast<const uint16_t *>(b + out->off_unit_end) : nullptr;
    return DF11_OK;
}

extern "C" void df11_encoded_free(df11_encoded *enc) {
    if (!enc) return;
    free(enc->blob);
    delete enc;
}
