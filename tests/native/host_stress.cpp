// Host-only stress of the library's host code (encoder, section views, validator,
// table builder), built by tests/test_host_sanitizers.py with g++ under
// AddressSanitizer + UBSan and under ThreadSanitizer.  Random blocks of every
// layout and thread count must encode and validate; corrupted copies of their
// sections must make the validator return (OK or an error), never read out of
// bounds.  Exit status 0 = no problem found (sanitizer reports abort the run).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <cmath>
#include <random>
#include <vector>
#include "df11.h"

static std::mt19937_64 rng(12345);
static uint16_t bf16_of(float f) { uint32_t u; memcpy(&u, &f, 4); u += 0x7FFF + ((u >> 16) & 1); return (uint16_t)(u >> 16); }

static std::vector<uint16_t> make(int fam, size_t n) {
    std::vector<uint16_t> x(n);
    std::normal_distribution<float> nd(0.f, 0.02f);
    std::uniform_int_distribution<uint32_t> ud(0, 65535);
    for (size_t i = 0; i < n; ++i) {
        switch (fam) {
            case 0: x[i] = bf16_of(nd(rng)); break;
            case 1: x[i] = (uint16_t)ud(rng); break;                       // any pattern
            case 2: x[i] = 0; break;                                         // one symbol
            case 3: x[i] = (ud(rng) % 50) ? 0 : bf16_of(nd(rng)); break;    // sparse
            case 4: x[i] = (uint16_t)((ud(rng) % 2) ? 0x3F80 : 0x0001); break;  // two symbols
            default: { // fibonacci-like skew: exponent e with weight ~ 2^-e
                uint32_t e = 1; while (e < 254 && (ud(rng) & 1)) ++e;
                x[i] = (uint16_t)((e << 7) | (ud(rng) & 0x807F));
            }
        }
    }
    return x;
}

struct Owned {  // mutable copies of the sections
    std::vector<uint8_t> code_len, stream, sm, gaps, tables, counts;
    std::vector<uint64_t> unit_pos;
    std::vector<uint16_t> unit_end;
};

int main(int argc, char **argv) {
    int iters = argc > 1 ? atoi(argv[1]) : 200;
    long bad = 0, corrupt_ok = 0, corrupt_rej = 0;
    const uint32_t flag_set[4] = {0, DF11_ENCODE_WINDOW_COUNTS, DF11_ENCODE_ALIGNED_UNITS,
                                  DF11_ENCODE_WINDOW_COUNTS | DF11_ENCODE_ALIGNED_UNITS};
    for (int it = 0; it < iters; ++it) {
        const int fam = it % 6;
        size_t n = (it % 7 == 0) ? (size_t)(rng() % 4) : (size_t)(rng() % (it % 5 == 0 ? 2000000 : 20000));
        std::vector<uint16_t> x = make(fam, n);
        uint32_t nm = 1 + rng() % 5;
        std::vector<df11_bf16_view> views;
        size_t at = 0;
        for (uint32_t m = 0; m < nm; ++m) {
            size_t len = m + 1 == nm ? n - at : (n - at) / 2;
            views.push_back({x.data() + at, (uint64_t)len});
            at += len;
        }
        const uint32_t flags = flag_set[it % 4];
        const uint32_t threads = (uint32_t)(rng() % 9);
        df11_encoded *enc = nullptr;
        df11_status st = df11_encode_block_ex(views.data(), nm, threads, flags, &enc);
        if (st != DF11_OK) { printf("encode failed it=%d st=%d n=%zu\n", it, st, n); ++bad; continue; }
        df11_sections s;
        if (df11_encoded_sections(enc, &s) != DF11_OK) { printf("sections failed\n"); ++bad; }
        if (df11_validate(&s) != DF11_OK) { printf("validate rejected a fresh blob it=%d n=%zu flags=%u\n", it, n, flags); ++bad; }
        uint64_t tb = 0; uint32_t nt = 0;
        if (df11_tables_size(s.code_len, &tb, &nt) != DF11_OK || tb != s.tables_bytes || nt != s.n_tables) { printf("tables_size mismatch\n"); ++bad; }
        std::vector<uint8_t> tcopy(tb);
        if (tb && df11_build_tables(s.code_len, tcopy.data(), tb) != DF11_OK) { printf("build_tables failed\n"); ++bad; }
        if (tb && memcmp(tcopy.data(), s.tables, tb) != 0) { printf("tables differ\n"); ++bad; }
        if (tb && df11_build_tables(s.code_len, tcopy.data(), tb - 1) == DF11_OK) { printf("short table buffer accepted\n"); ++bad; }
        // corrupted copies: validate must return, never read out of bounds
        for (int k = 0; k < 40; ++k) {
            Owned o;
            o.code_len.assign(s.code_len, s.code_len + 256);
            o.stream.assign(s.stream, s.stream + s.stream_bytes);
            o.sm.assign(s.sign_mant, s.sign_mant + s.sign_mant_bytes);
            o.gaps.assign(s.gaps, s.gaps + s.gaps_bytes);
            o.unit_pos.assign(s.unit_pos, s.unit_pos + s.n_units + 1);
            o.tables.assign(s.tables, s.tables + s.tables_bytes);
            if (s.counts_bytes) o.counts.assign(s.counts, s.counts + s.counts_bytes);
            if (s.unit_end_bytes) o.unit_end.assign(s.unit_end, s.unit_end + s.unit_end_bytes / 2);
            df11_sections c = s;
            c.code_len = o.code_len.data(); c.stream = o.stream.data(); c.sign_mant = o.sm.data();
            c.gaps = o.gaps.data(); c.unit_pos = o.unit_pos.data(); c.tables = o.tables.data();
            c.counts = s.counts_bytes ? o.counts.data() : nullptr;
            c.unit_end = s.unit_end_bytes ? o.unit_end.data() : nullptr;
            const uint64_t r = rng();
            switch (k % 10) {
                case 0: o.code_len[r % 256] = (uint8_t)(rng() % 40); break;
                case 1: if (!o.stream.empty()) o.stream[r % o.stream.size()] ^= (uint8_t)(1 + rng() % 255); break;
                case 2: if (!o.gaps.empty()) o.gaps[r % o.gaps.size()] ^= (uint8_t)(1 + rng() % 255); break;
                case 3: o.unit_pos[r % o.unit_pos.size()] += (rng() % 3) - 1 + (rng() % 2 ? 0 : (uint64_t)rng()); break;
                case 4: if (!o.tables.empty()) o.tables[r % o.tables.size()] ^= (uint8_t)(1 + rng() % 255); break;
                case 5: if (!o.counts.empty()) o.counts[r % o.counts.size()] = (uint8_t)rng(); else c.counts_bytes = 64; break;
                case 6: if (!o.unit_end.empty()) o.unit_end[r % o.unit_end.size()] = (uint16_t)rng(); break;
                case 7: c.total_bits += (int64_t)(rng() % 129) - 64; break;
                case 8: c.n_total += (int64_t)(rng() % 5) - 2; break;
                default: c.max_unit_count = rng() % 3000; break;
            }
            // a blob that claims more than the copies hold is a caller error, not a validate bug
            if (c.counts_bytes > o.counts.size()) c.counts_bytes = o.counts.size();
            const df11_status v = df11_validate(&c);
            (v == DF11_OK ? corrupt_ok : corrupt_rej) += 1;
        }
        df11_encoded_free(enc);
    }
    // random code length arrays for the table builder
    for (int it = 0; it < 20000; ++it) {
        uint8_t cl[256] = {0};
        const int ns = 1 + rng() % 256;
        for (int i = 0; i < ns; ++i) cl[rng() % 256] = (uint8_t)(rng() % 34);
        uint64_t tb = 0; uint32_t nt = 0;
        if (df11_tables_size(cl, &tb, &nt) == DF11_OK) {
            std::vector<uint8_t> t(tb);
            if (df11_build_tables(cl, t.data(), tb) != DF11_OK) { printf("build after size failed\n"); ++bad; }
        }
    }
    printf("done: %d blocks, %ld problems, corrupted copies accepted %ld rejected %ld\n", iters, bad, corrupt_ok, corrupt_rej);
    return bad ? 1 : 0;
}
