// DF11 block decode for gfx950 (CDNA4), HIP.
//
// What is computed follows the hada.io summary of the DFloat11 paper:
//   section "Decodage fonde sur des LUT hierarchiques": codes are decoded by
//     256-entry tables indexed by 8 stream bits, chained for codes longer
//     than 8 bits, resident in on-chip memory;
//   section "Noyau GPU en deux etapes et metadonnees auxiliaires": a thread
//     owns 8 bytes (64 bits) of the encoded exponents and decodes the codes
//     starting there, beginning at its 5-bit gap; phase 1 only counts, a
//     prefix sum of the counts plus the stored position gives each thread's
//     output index, phase 2 decodes again into an on-chip buffer that is then
//     written to HBM with coalesced stores;
//   section "Decompression par bloc transformer": one launch decodes every
//     matrix of a transformer block.
//
// Mapping to CDNA4: one 64-lane wavefront decodes one unit of 64 windows, so
// the prefix sum is a wave-level scan (DPP) and the stored position is per
// unit.  Waves of a workgroup share the decode tables in LDS and each owns a
// private LDS staging area, so no workgroup barrier is needed after the tables
// are loaded; the grid walks groups of units with a stride (several
// workgroups per resident slot).  Unit inputs and outputs go through buffer
// resources (base and size in scalar registers, 32-bit lane offsets).
//
// Two ways to take codes from the stream, same output:
//   one code per lookup through the hierarchical tables (the pages' design);
//   multi-code: phase 1 counts every code that ends in the next 10 bits with
//   one lookup (count table), phase 2 takes up to four codes per lookup of
//   the next 11 bits (emit table); longer codes fall back to the hierarchical
//   tables.  A variant reads stored per-window counts instead of phase 1.
// Staging holds each exponent already shifted into place (exponent << 7) as a
// 16-bit slot; the multi-code phase 2 writes a table entry's four slots with
// four 2-byte LDS stores (one 8-byte store at a 2-byte aligned address would
// stall the LDS pipe).
// The merge with the sign/mantissa bytes is one byte permute and one bitfield
// insert per pair of weights, and the output goes out as 16-byte
// non-temporal stores (16-bit stores only at the two ends of a unit).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "df11_internal.h"
#include "df11_wave.h"

namespace {

constexpr uint32_t kLdsTableMax = 32;     // sub-tables beyond this stay in global memory
constexpr uint64_t kUnitsPerWave = 4;     // units each wave walks in the automatic grid (about)
constexpr uint64_t kMaxWeights = uint64_t{1} << 48;  // no block holds more (512 TB of BF16)

struct KParams {
    const uint32_t *tables;
    const uint8_t *stream;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint64_t *unit_pos;
    const uint8_t *counts;  // per-window code counts (the counting-free variant only)
    const uint16_t *unit_end;  // per unit, where its codes end (aligned-units layout), or null
    uint16_t *out;
    uint64_t n_total, total_bits, n_windows, n_units;
    uint32_t last_unit_bits;  // stream bits in the last unit (1..4096)
    uint32_t n_tables;
    uint32_t stage_elems;  // 16-bit staging elements per wave, multiple of 8
    uint32_t out_phase;    // (address of out / 2) mod 32: where 64-byte sectors start
    uint32_t unit_queue;   // 1: a workgroup's waves take its units in turn from an LDS counter
};

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sub-table walk for codes longer than 8 bits: up to three more levels, each
// indexed by the next 8 bits of the 32-bit look-ahead `h`.
template <bool kDeepGlobal>
__device__ __forceinline__ uint32_t deep_lookup(const uint32_t *lut, const uint32_t *gtab,
                                                          uint32_t n_tables, uint32_t e, uint32_t h) {
#pragma unroll
    for (int lvl = 1; lvl < 4; ++lvl) {
        uint32_t t = (e >> 16) & 0x7FFFu;
        t = t < n_tables ? t : n_tables - 1;
        const uint32_t idx = (t << 8) | ((h >> (24 - 8 * lvl)) & 0xFFu);
        e = kDeepGlobal ? gtab[idx] : lut[idx];
        if (static_cast<int32_t>(e) >= 0) break;
    }
    return e;
}

template <bool kDeepGlobal>
__device__ __forceinline__ uint32_t lookup(const uint32_t *lut, const uint32_t *gtab, uint32_t n_tables,
                                           uint32_t h) {
    uint32_t e = lut[h >> 24];
    if (__builtin_expect(static_cast<int32_t>(e) < 0, 0)) e = deep_lookup<kDeepGlobal>(lut, gtab, n_tables, e, h);
    return e;
}

// 96-bit shift register (h:l:r, h = next 32 stream bits) positioned `g` bits
// (0..31) into the window words w0:w1:w2.
__device__ __forceinline__ void start_at(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t g, uint32_t &h,
                                         uint32_t &l, uint32_t &r) {
    const uint64_t a = ((static_cast<uint64_t>(w0) << 32) | w1) << g;
    const uint64_t b = ((static_cast<uint64_t>(w1) << 32) | w2) << g;
    h = static_cast<uint32_t>(a >> 32);
    l = static_cast<uint32_t>(b >> 32);
    r = static_cast<uint32_t>(b);
}

// Consume one code: a leaf entry's low 5 bits hold (32 - length) & 31, which
// is exactly the alignbit amount for a left shift by `length` (1..32).
__device__ __forceinline__ void consume(uint32_t e, uint32_t &h, uint32_t &l, uint32_t &r) {
    h = __builtin_amdgcn_alignbit(h, l, e);
    l = __builtin_amdgcn_alignbit(l, r, e);
    r = __builtin_amdgcn_alignbit(r, 0u, e);
}

// Two BF16 values from two staged (exponent << 7) halves and the sign/mantissa
// bytes selected by `sel`: the byte permute puts each sm byte in both bytes
// of its 16-bit slot, so bit 15 = sign and bits 6..0 = mantissa.
__device__ __forceinline__ uint32_t merge2(uint32_t staged, uint32_t sm4, uint32_t sel) {
    const uint32_t dup = __builtin_amdgcn_perm(sm4, sm4, sel);
    return (dup & 0x807F807Fu) | (staged & 0x7F807F80u);
}

// One code through the hierarchical tables, consumed; returns its entry.
template <bool kDeepGlobal>
__device__ __forceinline__ uint32_t single_step(const uint32_t *lut, const KParams &p, uint32_t &h,
                                                uint32_t &l, uint32_t &r) {
    const uint32_t e = lookup<kDeepGlobal>(lut, p.tables, p.n_tables, h);
    consume(e, h, l, r);
    return e;
}

__device__ __forceinline__ int entry_length(uint32_t e) { return static_cast<int>((e >> 8) & 31u) + 1; }

// Phase 1, one code per lookup: count the codes that start in [pos, end).
template <bool kDeepGlobal>
__device__ __forceinline__ uint32_t count_single(const uint32_t *lut, const KParams &p, uint32_t h,
                                                 uint32_t l, uint32_t r, int pos, int end) {
    uint32_t cnt = 0;
    while (pos < end) {
        pos += entry_length(single_step<kDeepGlobal>(lut, p, h, l, r));
        ++cnt;
    }
    return cnt;
}

// Phase 1 with the count table: `S` holds the window from the current code
// start, followed by zeros instead of the 4-byte halo: only the last code
// that starts inside the window can reach past it, and as the code is prefix
// free, its zero-padded decode is longer than the window bits it covers, so
// the next start it implies lies past the end and is not counted.
//
// While more than 10 window bits remain, every code of an entry starts
// inside the window and the entry's count is taken whole (two steps per loop
// test while more than 20 remain); the last steps count only the starts
// before the end, from the entry's start mask.  An escape entry (first code
// longer than the index) shifts by 0 and subtracts 128 from `rem`, which ends
// both loops without a test in the loop body; the code is then taken from
// the hierarchical tables and the loops resume.
template <bool kDeepGlobal>
__device__ __forceinline__ uint32_t count_multi(const uint32_t *lut, const uint32_t *ct, const KParams &p,
                                                uint64_t S, int rem) {
    uint32_t cnt = 0;
    auto full = [&]() {
        const uint32_t e = ct[static_cast<uint32_t>(S >> (64 - df11i::kCountBits))];
        cnt += (e >> 8) & 0xFFu;
        S <<= (e & 63u);
        rem -= static_cast<int>(e & 0xFFu);
    };
    while (true) {
        while (rem > 2 * static_cast<int>(df11i::kCountBits)) {
            full();
            full();
        }
        if (rem > static_cast<int>(df11i::kCountBits)) full();
        while (rem > 0) {
            const uint32_t e = ct[static_cast<uint32_t>(S >> (64 - df11i::kCountBits))];
            cnt += __popc(__builtin_amdgcn_ubfe(e, 20u, static_cast<uint32_t>(rem)));
            S <<= (e & 63u);
            rem -= static_cast<int>(e & 0xFFu);
        }
        // rem is now in (-10, 0] when done, or lowered by 128 per escape
        const int fix = (64 - rem) & ~127;
        if (__builtin_expect(fix == 0, 1)) break;
        rem += fix;
        const int len = entry_length(lookup<kDeepGlobal>(lut, p.tables, p.n_tables, static_cast<uint32_t>(S >> 32)));
        S <<= len;
        rem -= len;
        ++cnt;
    }
    return cnt;
}

// Phase 2, one code per lookup: stage n values starting at dst.
template <bool kDeepGlobal>
__device__ __forceinline__ void emit_single(const uint32_t *lut, const KParams &p, uint32_t h, uint32_t l,
                                            uint32_t r, uint16_t *dst, uint32_t n) {
    for (uint32_t j = 0; j < n; ++j) dst[j] = static_cast<uint16_t>(single_step<kDeepGlobal>(lut, p, h, l, r) >> 16);
}

// Phase 2 with the emit table keeps the 96-bit look-ahead h:l:r as two
// 64-bit pairs, A = h:l and B = l:r: shifting both left by t and copying
// B's high half into A's low half advances by t bits for any t in 0..32, so
// an entry's t (its low bits) is applied as it is, and t = 0 is a no-op.
struct Look96 {
    uint64_t A, B;
    __device__ __forceinline__ uint32_t h() const { return static_cast<uint32_t>(A >> 32); }
    __device__ __forceinline__ void shift(uint32_t t) {
        A <<= (t & 63u);
        B <<= (t & 63u);
        A = (A & 0xFFFFFFFF00000000ull) | (B >> 32);
    }
};

// Up to four codes per lookup.  Each step writes the entry's four 16-bit
// slots at the lane's next slot q with two LDS stores: slot 0 as a 2-byte
// store, then one dword pair at the first 4-byte boundary at or after q,
// which holds slots 0..3 when q is even and slots 1..3 plus one spare slot
// when q is odd.  The slots past the entry's n codes (and the spare) are
// rewritten by the lane's next step, so only the lane's own range is ever
// written and the staging needs no clearing; this needs q + 4 inside the
// range, so full steps run while at least five slots are left.  (A single
// 8-byte store at a 2-byte aligned address would stall the LDS pipe, and four
// 2-byte stores cost twice the LDS issue of these two.)  Slots carry control
// fields in bits 6..0, below the exponent, which the merge never reads.  An
// escape entry (first code longer than the index) shifts by 0 and moves the
// lane's cursor 64 slots on, which ends the loop with no test in its body;
// the lane then undoes that, takes the code from the hierarchical tables and
// goes back in (the slots the escape entry wrote lie inside the lane's range
// and are rewritten).  The last one to four codes are written one slot at a
// time, only as many as the lane owns.
typedef __attribute__((address_space(3))) volatile uint16_t lds_u16;
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef __attribute__((address_space(3))) u32x2_a4 lds_pair;

__device__ __forceinline__ lds_u16 *lds_slot(uint32_t b) { return reinterpret_cast<lds_u16 *>(b); }

template <bool kDeepGlobal>
__device__ __forceinline__ void emit_multi(const uint32_t *lut, const uint2 *et, const KParams &p, Look96 s,
                                           uint16_t *stage, uint32_t first, uint32_t n) {
    // the staging is LDS: the low 32 bits of its generic address are the LDS address
    uint32_t b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stage)) + 2u * first;
    const uint32_t bend = b + 2u * n;  // past the lane's last slot
    const uint32_t bfull = bend - 2u * (df11i::kEmitCodes + 1u);  // last start with five own slots (LDS addresses are far above 10)
    auto entry = [&]() { return *reinterpret_cast<const uint64_t *>(et + (s.h() >> (32 - df11i::kEmitBits))); };
    auto escape_step = [&]() {
        const uint32_t e = lookup<kDeepGlobal>(lut, p.tables, p.n_tables, s.h());
        *lds_slot(b) = static_cast<uint16_t>(e >> 16);  // a leaf entry's bits 30..16 are exponent << 7
        b += 2u;
        s.shift(static_cast<uint32_t>(entry_length(e)));
    };
    while (true) {
        // An escape advances b by 64 slots, past bend (a lane has at most 53
        // codes left when it meets a code longer than the index), which ends
        // the loop; it is then undone.  Each step's table read is issued
        // last and waited for at the top of the next step.
        uint64_t ev = entry();
        asm volatile("" ::"v"(ev));  // keeps that order (else the read moves to the loop head)
        while (b <= bfull) {
            const uint32_t lo = static_cast<uint32_t>(ev), hi = static_cast<uint32_t>(ev >> 32);
            s.shift(lo);
            *lds_slot(b) = static_cast<uint16_t>(lo);
            const uint32_t odd = b & 2u;  // q odd: the pair starts one slot on
            const uint32_t sh = odd << 3;
            u32x2_a4 pair;
            pair.x = __builtin_amdgcn_alignbit(hi, lo, sh);
            pair.y = hi >> sh;
            *reinterpret_cast<lds_pair *>(b + odd) = pair;
            // n slots, or 64 for an escape; the field is kept opaque so that
            // the advance is one bitfield extract and one shift-add
            uint32_t nslots = __builtin_amdgcn_ubfe(lo, 16u, 7u);
            asm("" : "+v"(nslots));
            b = nslots * 2u + b;
            ev = entry();  // past the last step: read, not used
        }
        if (__builtin_expect(b <= bend, 1)) break;
        b -= 2u * df11i::kEmitEscape;
        escape_step();
    }
    while (b < bend) {  // the last one to four codes
        const uint64_t ev = entry();
        const uint32_t lo = static_cast<uint32_t>(ev);
        const uint32_t m = (lo >> 16) & 127u;
        if (__builtin_expect(m == df11i::kEmitEscape, 0)) {
            escape_step();
            continue;
        }
        const uint32_t left = (bend - b) >> 1;  // 1..4
        const uint32_t k = m < left ? m : left;
        lds_u16 *w = lds_slot(b);
        w[0] = static_cast<uint16_t>(lo);
        if (k > 1) w[1] = static_cast<uint16_t>(lo >> 16);
        if (k > 2) w[2] = static_cast<uint16_t>(ev >> 32);
        if (k > 3) w[3] = static_cast<uint16_t>(ev >> 48);
        b += 2u * k;
        s.shift(lo);  // past the lane's last code the state is not used
    }
}

// The count and emit tables have a fixed size, so they live in static LDS
// (their offsets fold into the ds_read immediate); only the multi-code
// kernels reference them, so only those allocate them.
__shared__ __align__(16) uint32_t s_count_table[df11i::kCountEntries];
__shared__ __align__(16) uint2 s_emit_table[df11i::kEmitEntries];
// one word per wave: whether that wave found a bad multi-code table entry
constexpr uint32_t kMaxWaves = 16;
__shared__ __align__(16) uint32_t s_wave_bad[kMaxWaves];
constexpr uint32_t kMultiStaticBytes = static_cast<uint32_t>(df11i::kMultiTableBytes) + 4u * kMaxWaves;

using df11w::kNonTemporal;
using df11w::kOff;
using df11w::rsrc;
using df11w::Rsrc;
using df11w::v2u;
using df11w::v4u;

__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, uint32_t k) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), k);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), k);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Everything a unit needs from HBM before decoding: the lane's window words
// (8 bytes + 4-byte halo), its two gap bytes (assembled only when used: any
// computation on a load result makes the wave wait for it) and the unit's
// output range.  Loaded one unit ahead so the latency overlaps the previous
// unit.  Straight-line code: the compiler can then count the loads in flight
// exactly and wait only for the ones it needs.
struct UnitInputs {
    uint32_t w0, w1, w2, g0, g1;
    uint32_t c;    // the window's stored code count (counting-free variant)
    uint32_t ue;   // where the unit's codes end (aligned-units layout; 0 otherwise)
    uint64_t pos;  // unit_pos[u] in even lanes, unit_pos[u + 1] in odd lanes
};

template <bool kCounts>
__device__ __forceinline__ void load_unit(const KParams &p, uint64_t u, uint32_t lane, UnitInputs &in) {
    const Rsrc st = rsrc(p.stream + 512 * u, 528);  // the unit's 64 windows + 16-byte guard
    const v2u a = __builtin_amdgcn_raw_buffer_load_b64(st, 8 * lane, 0, 0);
    in.w0 = a.x;
    in.w1 = a.y;
    in.w2 = __builtin_amdgcn_raw_buffer_load_b32(st, 8 * lane + 8, 0, 0);
    const Rsrc gp = rsrc(p.gaps + 40 * u, 48);
    in.g0 = __builtin_amdgcn_raw_buffer_load_b8(gp, (5 * lane) >> 3, 0, 0);
    in.g1 = __builtin_amdgcn_raw_buffer_load_b8(gp, ((5 * lane) >> 3) + 1, 0, 0);
    const Rsrc up = rsrc(p.unit_pos + u, 16);
    const v2u q = __builtin_amdgcn_raw_buffer_load_b64(up, 8 * (lane & 1), 0, 0);
    in.pos = (static_cast<uint64_t>(q.y) << 32) | q.x;
    in.c = kCounts ? __builtin_amdgcn_raw_buffer_load_b8(rsrc(p.counts + 64 * u, 64), lane, 0, 0) : 0u;
    // a range of 0 bytes (reads 0) when the block has no unit ends
    const Rsrc ur = p.unit_end ? rsrc(p.unit_end + u, 2) : rsrc(p.unit_pos, 0);
    in.ue = __builtin_amdgcn_raw_buffer_load_b16(ur, 0, 0, 0);
}

constexpr uint32_t kChunksPerPass = 64;  // 8-output chunks, one per lane
constexpr int kPrefetchChunks = 4;        // passes whose sign/mantissa bytes are loaded early

template <bool kDeepGlobal, bool kMulti, bool kCounts>
__device__ __forceinline__ void decode_unit(const KParams &p, const uint32_t *lut, const uint32_t *ct,
                                            const uint2 *et, uint16_t *stage, uint32_t lane, uint64_t u,
                                            const UnitInputs &in, const UnitInputs &next) {
    // output range of the unit (uniform): staged element k is output base + k
    const uint64_t q1 = lane_u64(in.pos, 1), q0 = lane_u64(in.pos, 0);
    const uint64_t P1 = q1 < p.n_total ? q1 : p.n_total;
    const uint64_t P0 = q0 < P1 ? q0 : P1;
    const uint64_t base = P0 & ~uint64_t{7};
    const uint64_t span64 = P1 - base;
    const uint32_t span = span64 < p.stage_elems ? static_cast<uint32_t>(span64) : p.stage_elems;
    const uint32_t lead = static_cast<uint32_t>(P0 - base);  // staged slots before P0
    const uint32_t chunks = (span + 7) / 8;
    const Rsrc smr = rsrc(p.sm + base, 8 * chunks);

    // Outputs in the 64-byte sectors (32 weights) that the unit shares with
    // its neighbours go out element by element through the cache, where the
    // two units' parts of a sector meet: lanes 0..31 take the head sector's
    // staged elements [lead, e1), lanes 32..63 the tail sector's [e2, span).
    // Chunks [full_lo, full_hi) fill whole sectors and go out as 16-byte
    // non-temporal stores.  Sector boundaries fall where the address of
    // out[base + k] is a multiple of 64 bytes (out is 16-byte aligned and
    // base a multiple of 8, so b32 is a multiple of 8).
    const uint32_t b32 = (p.out_phase + static_cast<uint32_t>(base)) & 31u;
    const uint32_t hs = ((b32 + lead + 31u) & ~31u) - b32;  // first whole sector
    const uint32_t ts = b32 + span >= 32u ? ((b32 + span) & ~31u) - b32 : 0u;  // end of the last one
    const uint32_t e1 = hs < span ? hs : span;
    const uint32_t e2 = ts > e1 ? ts : e1;
    const uint32_t full_lo = e1 / 8;
    const uint32_t full_hi = e2 / 8;
    const uint32_t ek = lane < 32 ? lead + lane : e2 + (lane - 32u);
    const bool edge = ek < (lane < 32 ? e1 : span);

    // sign/mantissa bytes of the unit, requested before decoding starts
    // (chunks past the unit read as 0); read once, so non-temporal
    uint2 smv[kPrefetchChunks];
    const bool pass3 = chunks > 3 * kChunksPerPass;  // uniform
#pragma unroll
    for (int k = 0; k < kPrefetchChunks; ++k) {
        if (k == 3 && !pass3) {
            smv[k] = make_uint2(0u, 0u);
            continue;
        }
        const v2u t = __builtin_amdgcn_raw_buffer_load_b64(smr, 8 * (lane + kChunksPerPass * k), 0, kNonTemporal);
        smv[k] = make_uint2(t.x, t.y);
    }
    const uint32_t esm = __builtin_amdgcn_raw_buffer_load_b8(smr, edge ? ek : kOff, 0, 0);

    // ---- this lane's window: gap and end (bits of the stream left in it)
    const uint32_t ulim = p.unit_end ? __builtin_amdgcn_readfirstlane(in.ue)
                                     : u == p.n_units - 1 ? p.last_unit_bits : 4096u;
    const int end = min(max(static_cast<int>(ulim) - 64 * static_cast<int>(lane), 0), 64);
    const uint32_t gap2 = (in.g0 << 8) | in.g1;  // big-endian 16 bits
    const uint32_t gap = (gap2 >> (11u - ((5 * lane) & 7))) & 31u;
    const uint32_t w0 = __builtin_bswap32(in.w0), w1 = __builtin_bswap32(in.w1), w2 = __builtin_bswap32(in.w2);

    // ---- phase 1: count the codes that start in [gap, end)
    uint32_t cnt;
    uint32_t h, l, r;
    Look96 look;
    if constexpr (kMulti) {
        // A = h:l and B = l:r, the window words from the gap on (A's low half
        // is B's high half: it carries the halo bits that enter l)
        look.B = ((static_cast<uint64_t>(w1) << 32) | w2) << gap;
        const uint64_t a = ((static_cast<uint64_t>(w0) << 32) | w1) << gap;
        look.A = (a & 0xFFFFFFFF00000000ull) | (look.B >> 32);
        if constexpr (kCounts)
            cnt = in.c;  // stored with the block: the counting pass is skipped
        else
            cnt = count_multi<kDeepGlobal>(lut, ct, p, look.A, end - static_cast<int>(gap));
    } else {
        start_at(w0, w1, w2, gap, h, l, r);
        cnt = count_single<kDeepGlobal>(lut, p, h, l, r, static_cast<int>(gap), end);
    }

    // ---- wave prefix sum of the counts
    const uint32_t excl = df11w::wave_inclusive_scan(cnt) - cnt;

    // ---- phase 2: decode again, stage (exponent << 7) at the output slot
    const uint32_t first = lead + excl;
    // never past this wave's staging (both ways write only the lane's own slots)
    const uint32_t room = first < p.stage_elems ? p.stage_elems - first : 0u;
    const uint32_t n2 = cnt < room ? cnt : room;
    if constexpr (kMulti)
        emit_multi<kDeepGlobal>(lut, et, p, look, stage, first, n2);
    else
        emit_single<kDeepGlobal>(lut, p, h, l, r, stage + first, n2);
    wave_sync();

    // ---- merge with sign/mantissa and store.  All of the unit's outputs are
    // computed before its first store: vmcnt is in order, so a wait for a load
    // issued before a store would also wait for that store.
    auto merge_chunk = [&](uint32_t c, uint2 sm) {
        const uint4 ev = *reinterpret_cast<const uint4 *>(stage + 8 * c);
        v4u o;
        o.x = merge2(ev.x, sm.x, 0x01010000u);
        o.y = merge2(ev.y, sm.x, 0x03030202u);
        o.z = merge2(ev.z, sm.y, 0x01010000u);
        o.w = merge2(ev.w, sm.y, 0x03030202u);
        return o;
    };
    const Rsrc outr = rsrc(p.out + base, 16 * full_hi);  // full chunks only
    // the output is written once and not read back here: non-temporal
    auto put_chunk = [&](uint32_t c, const v4u &o) {
        __builtin_amdgcn_raw_buffer_store_b128(o, outr, c >= full_lo ? 16 * c : kOff, 0, kNonTemporal);
    };
    v4u outv[kPrefetchChunks];
#pragma unroll
    for (int k = 0; k < 3; ++k) outv[k] = merge_chunk(lane + kChunksPerPass * k, smv[k]);
    if (pass3) outv[3] = merge_chunk(lane + kChunksPerPass * 3, smv[3]);
    // the edge element: bit 15 = sign, bits 6..0 = mantissa from its sm byte
    const uint32_t st = stage[edge ? ek : 0];
    const uint32_t eo = __builtin_amdgcn_perm(esm, esm, 0x0c0c0000u);  // sm byte in both bytes
    const uint32_t eout = (eo & 0x807Fu) | (st & 0x7F80u);
    // The next unit's inputs were requested before this unit's sign/mantissa
    // loads, so they have arrived; taking them here keeps the copy into the
    // current set (after the stores) from waiting on the stores.
    asm volatile("" ::"v"(next.w0), "v"(next.w1), "v"(next.w2), "v"(next.g0), "v"(next.g1), "v"(next.pos),
                 "v"(next.c), "v"(next.ue), "v"(eout));
#pragma unroll
    for (int k = 0; k < 3; ++k) put_chunk(lane + kChunksPerPass * k, outv[k]);
    if (pass3) put_chunk(lane + kChunksPerPass * 3, outv[3]);
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(eout), rsrc(p.out + base, 2 * span),
                                          edge ? 2 * ek : kOff, 0, 0);
    if (chunks > kChunksPerPass * kPrefetchChunks) {  // units above 2,048 outputs (uniform)
        for (uint32_t c = lane + kChunksPerPass * kPrefetchChunks; c < chunks; c += kChunksPerPass) {
            const v2u t = __builtin_amdgcn_raw_buffer_load_b64(smr, 8 * c, 0, kNonTemporal);
            put_chunk(c, merge_chunk(c, make_uint2(t.x, t.y)));
        }
    }
    wave_sync();  // the staging is rewritten by the next unit
}

// Register budget: 8 waves per SIMD (64 VGPRs), the most a CU can hold;
// the rare kernels that walk sub-tables in global memory get 4 (no spills).
template <bool kDeepGlobal>
struct WavesPerEU {
    static constexpr int value = kDeepGlobal ? 4 : 8;
};

// The unit loop of one wave: decode unit u, then further units of its
// workgroup.  A workgroup's units are group0 + r + j * stride for r below its
// wave count and j = 0, 1, ...: position j * waves + r in the workgroup's
// order.  Without the queue wave r takes positions r, r + waves, ...; with it
// each wave takes its first position statically and then the workgroup's next
// position from an LDS counter when it starts its next unit, so that the
// workgroup's waves finish together: the workgroup holds its LDS and wave
// slots until its last wave is done, and units take different times.
// `cur` holds unit u's inputs, already requested.
template <bool kDeepGlobal, bool kMulti, bool kCounts>
__device__ __forceinline__ void unit_loop(const KParams &p, const uint32_t *lut, uint16_t *stage, uint32_t lane,
                                          uint64_t u, uint64_t stride, UnitInputs cur, uint32_t *next_pos,
                                          uint64_t group0, uint32_t wmask, uint32_t wshift) {
    const uint64_t last = p.n_units - 1;
    // Wait for the first unit's inputs here: the loop head then sees them
    // complete on both of its entries, and needs no wait that would also
    // drain the previous unit's stores (vmcnt counts loads and stores in
    // issue order).
    asm volatile("" ::"v"(cur.w0), "v"(cur.w1), "v"(cur.w2), "v"(cur.g0), "v"(cur.g1), "v"(cur.pos), "v"(cur.c),
                 "v"(cur.ue));
    while (true) {
        // the next unit's inputs (a repeat of the last unit at the end, so the
        // loads are unconditional)
        // Values derived from the lane index are computed again for every
        // unit rather than held in registers through it: that leaves phase 2
        // enough registers for eight waves per SIMD without spills.
        asm volatile("" : "+v"(lane));
        uint64_t un;
        if (p.unit_queue) {  // uniform
            uint32_t k = 0;
            if (lane == 0) k = atomicAdd(next_pos, 1u);
            k = __builtin_amdgcn_readfirstlane(k);
            // positions past the workgroup's last unit map past the block's
            // last unit, and so do all later ones: every wave leaves the loop
            un = uniform_u64(group0 + (k & wmask) + uint64_t{k >> wshift} * stride);
        } else {
            un = uniform_u64(u + stride);
        }
        UnitInputs nxt;
        load_unit<kCounts>(p, un < last ? un : last, lane, nxt);
        decode_unit<kDeepGlobal, kMulti, kCounts>(p, lut, s_count_table, s_emit_table, stage, lane, u, cur, nxt);
        if (un >= p.n_units) break;
        cur = nxt;  // waits for the next unit's inputs, requested a whole unit ago
        u = un;
    }
}

template <bool kDeepGlobal, bool kMulti, bool kCounts>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(WavesPerEU<kDeepGlobal>::value)))
df11_decode_kernel(KParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    // dynamic LDS: hierarchical tables, then one staging area per wave
    const uint32_t lds_tables = kDeepGlobal ? 1u : p.n_tables;
    uint32_t *lut = reinterpret_cast<uint32_t *>(lds);

    const uint32_t lane = threadIdx.x & 63u;
    // wave index and wave count are uniform: keep unit indices in scalar registers
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t waves = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    const uint64_t u = uniform_u64(uint64_t{blockIdx.x} * waves + wave);
    const uint64_t last = p.n_units - 1;  // the host launches only for blocks with weights
    // The first unit's inputs are requested before the tables are copied, so
    // that the two memory latencies overlap (a wave with no unit loads the
    // last one and leaves after the workgroup barrier).
    UnitInputs cur;
    load_unit<kCounts>(p, u < last ? u : last, lane, cur);
    // The tables go to LDS in one pass.  Every thread requests its first two
    // 16-byte pieces in straight-line code, right after the unit's inputs and
    // before it waits for anything, so the two memory latencies overlap (a
    // loop here would wait for every earlier load at its head); more pieces
    // per thread (small workgroups, many sub-tables) go in a loop after that.
    // The multi-code tables are checked in registers on the way: every count
    // entry advances (1..10 bits) or is the escape, every emit entry takes
    // 1..4 codes or is the escape, so the loops over them end whatever the
    // stream holds.  When any entry breaks this, the workgroup decodes with
    // the hierarchical tables alone (one code per lookup).  Each wave leaves
    // its verdict in its own LDS word, read by all after the one barrier.
    //
    // The same barrier publishes the workgroup's next unit position, for
    // waves that take its units in turn (positions below `waves` are the
    // waves' first units).
    __shared__ uint32_t s_next_pos;
    if (threadIdx.x == 0) s_next_pos = waves;
    bool bad = false;
    {
        const uint32_t n_hier = lds_tables * 64u;  // 16-byte pieces
        constexpr uint32_t kCountPieces = df11i::kCountEntries / 4u, kEmitPieces = df11i::kEmitEntries / 2u;
        const uint32_t n_all = n_hier + (kMulti ? kCountPieces + kEmitPieces : 0u);
        // piece i < n_hier is hierarchical piece i; the multi-code tables
        // follow all n_tables hierarchical tables in the blob
        const uint32_t skip = (p.n_tables - lds_tables) * 64u;
        const uint4 *src = reinterpret_cast<const uint4 *>(p.tables);
        auto fetch = [&](uint32_t i) { return src[i + (i < n_hier ? 0u : skip)]; };
        auto place = [&](uint32_t i, const uint4 &v) {
            if (i < n_hier) {
                reinterpret_cast<uint4 *>(lut)[i] = v;
            } else if constexpr (kMulti) {
                const uint32_t j = i - n_hier;
                if (j < kCountPieces) {
                    reinterpret_cast<uint4 *>(s_count_table)[j] = v;
                    const uint32_t ce[4] = {v.x, v.y, v.z, v.w};
                    for (const uint32_t e : ce) {
                        const uint32_t t = e & 0xFFu;
                        bad |= !((t >= 1u && t <= df11i::kCountBits) || e == df11i::kCountEscape);
                    }
                } else {
                    reinterpret_cast<uint4 *>(s_emit_table)[j - kCountPieces] = v;
                    const uint32_t el[2] = {v.x, v.z};  // low words of the two entries
                    for (const uint32_t lo : el) {
                        const uint32_t m = (lo >> 16) & 127u;
                        bad |= !((m >= 1u && m <= df11i::kEmitCodes) || m == df11i::kEmitEscape);
                    }
                }
            }
        };
        const uint32_t nthr = blockDim.x;
        const uint32_t i0 = threadIdx.x, i1 = i0 + nthr;
        const uint4 v0 = fetch(min(i0, n_all - 1u));  // clamped: always a piece of the tables
        const uint4 v1 = fetch(min(i1, n_all - 1u));
        if (i0 < n_all) place(i0, v0);
        if (i1 < n_all) place(i1, v1);
        for (uint32_t i = i1 + nthr; i < n_all; i += nthr) place(i, fetch(i));
        if constexpr (kMulti) {
            const uint64_t any = __builtin_amdgcn_ballot_w64(bad);
            if (lane == 0) s_wave_bad[wave] = any != 0 ? 1u : 0u;
        }
        __syncthreads();
        if constexpr (kMulti) {
            uint32_t f = 0;
            for (uint32_t w = 0; w < waves; ++w) f |= s_wave_bad[w];
            bad = f != 0;
        }
    }

    uint16_t *stage = reinterpret_cast<uint16_t *>(lds + lds_tables * 1024u) + wave * p.stage_elems;
    const uint64_t stride = uniform_u64(uint64_t{gridDim.x} * waves);
    const uint64_t group0 = uniform_u64(uint64_t{blockIdx.x} * waves);
    const uint32_t wshift = __builtin_amdgcn_readfirstlane(31u - __clz(waves));  // waves is a power of two
    if (u >= p.n_units) return;  // uniform across the wave
    if constexpr (kMulti) {
        if (__builtin_expect(bad, 0)) {  // uniform across the workgroup
            unit_loop<kDeepGlobal, false, false>(p, lut, stage, lane, u, stride, cur, &s_next_pos, group0, waves - 1u,
                                                 wshift);
            return;
        }
    }
    unit_loop<kDeepGlobal, kMulti, kCounts>(p, lut, stage, lane, u, stride, cur, &s_next_pos, group0, waves - 1u,
                                            wshift);
}

// ------------------------------------------------------------------ host side

struct DeviceInfo {
    int cus = 0;
    int lds_per_group = 0;
};

std::mutex g_mu;
DeviceInfo g_dev[64];

int device_attr(hipDeviceAttribute_t a, int dev, int fallback) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, a, dev) != hipSuccess) {
        (void)hipGetLastError();  // our own failed query: do not leave it to the caller
        return fallback;
    }
    return v > 0 ? v : fallback;
}

DeviceInfo device_info(int dev) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (dev < 0 || dev >= 64) return DeviceInfo{256, 65536};
    if (!g_dev[dev].cus) {
        g_dev[dev].cus = device_attr(hipDeviceAttributeMultiprocessorCount, dev, 256);
        g_dev[dev].lds_per_group = device_attr(hipDeviceAttributeMaxSharedMemoryPerBlock, dev, 65536);
    }
    return g_dev[dev];
}

int occupancy(const void *fn, uint32_t waves, uint32_t lds_bytes) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, static_cast<int>(64 * waves), lds_bytes) !=
        hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    return per_cu > 0 ? per_cu : 0;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

thread_local int32_t df11i::last_hip_error = 0;

df11_status df11i::check_device_block(const df11_device_block *b, const uint16_t *out, uint64_t cap) {
    if (!b) return DF11_E_INVALID_ARG;
    if (b->version != DF11_FORMAT_VERSION) return DF11_E_UNSUPPORTED;
    if (b->n_total == 0) return DF11_OK;
    if (!out || !b->tables || !b->stream || !b->sign_mant || !b->gaps || !b->unit_pos)
        return DF11_E_INVALID_ARG;
    if (cap < b->n_total) return DF11_E_BUFFER_TOO_SMALL;
    // bounds first, so that no size computed below can wrap around: each code
    // takes 1..32 bits (up to twice that with the aligned layout's filler)
    if (b->n_total > kMaxWeights || b->total_bits < b->n_total ||
        b->total_bits > (b->unit_end ? 2u : 1u) * uint64_t{DF11_MAX_CODE_LEN} * b->n_total)
        return DF11_E_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(b->stream, 16) || !aligned(b->sign_mant, 16) ||
        !aligned(b->unit_pos, 8) || !aligned(b->tables, 16) || !aligned(b->unit_end, 2))
        return DF11_E_INVALID_ARG;
    const uint64_t nw = (b->total_bits + 63) / 64, nu = (nw + 63) / 64;
    if (b->n_windows != nw || b->n_units != nu) return DF11_E_INVALID_ARG;
    if (b->stream_bytes < 512 * nu + 16 || b->gaps_bytes < 40 * nu + 8 ||
        b->sign_mant_bytes < (b->n_total + 15) / 16 * 16)
        return DF11_E_INVALID_ARG;
    if (b->n_tables < 1 || b->tables_bytes < uint64_t{b->n_tables} * 1024) return DF11_E_INVALID_ARG;
    if (b->max_unit_count > DF11_MAX_UNIT_WEIGHTS) return DF11_E_INVALID_ARG;
    return DF11_OK;
}

extern "C" int32_t df11_last_hip_error(void) { return df11i::last_hip_error; }

extern "C" const char *df11_hip_error_name(int32_t code) {
    return hipGetErrorName(static_cast<hipError_t>(code));
}

namespace {

df11_status decode_block(const df11_device_block *blk, uint16_t *out_bf16, uint64_t out_capacity, void *hip_stream,
                         const df11_launch *launch) {
    df11_status rc = df11i::check_device_block(blk, out_bf16, out_capacity);
    if (rc != DF11_OK || blk->n_total == 0) return rc;
    const uint32_t variant = (launch && launch->variant) ? launch->variant : DF11_VARIANT_MULTI;
    if (variant != DF11_VARIANT_SINGLE && variant != DF11_VARIANT_MULTI && variant != DF11_VARIANT_COUNTS)
        return DF11_E_INVALID_ARG;
    const bool counts = variant == DF11_VARIANT_COUNTS;
    const bool multi = variant == DF11_VARIANT_MULTI || counts;
    if (counts && !blk->counts) return DF11_E_INVALID_ARG;
    if (multi && blk->tables_bytes < df11i::tables_bytes_for(blk->n_tables)) return DF11_E_INVALID_ARG;
    const uint32_t asked = launch ? launch->waves_per_group : 0u;
    if (asked != 0 && asked != 1 && asked != 2 && asked != 4 && asked != 8 && asked != 16)
        return DF11_E_INVALID_ARG;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        dev = 0;
    }
    const DeviceInfo info = device_info(dev);
    const bool deep_global = blk->n_tables > kLdsTableMax;
    const void *fn;
    if (counts)
        fn = deep_global ? reinterpret_cast<const void *>(&df11_decode_kernel<true, true, true>)
                         : reinterpret_cast<const void *>(&df11_decode_kernel<false, true, true>);
    else if (multi)
        fn = deep_global ? reinterpret_cast<const void *>(&df11_decode_kernel<true, true, false>)
                         : reinterpret_cast<const void *>(&df11_decode_kernel<false, true, false>);
    else
        fn = deep_global ? reinterpret_cast<const void *>(&df11_decode_kernel<true, false, false>)
                         : reinterpret_cast<const void *>(&df11_decode_kernel<false, false, false>);

    // LDS per workgroup: static (count and emit tables) + hierarchical tables
    // + one staging area per wave; it bounds how many waves are resident.
    const uint32_t lds_tables = deep_global ? 1u : blk->n_tables;
    const uint32_t fixed_static = (multi ? kMultiStaticBytes : 0u) + 16u;  // + the unit position counter
    // staging: the unit's outputs after up to 7 slots of lead, rounded to
    // 8-output chunks
    const uint32_t stage_elems = static_cast<uint32_t>((blk->max_unit_count + 7 + 7) / 8 * 8);
    // The merge reads whole passes of 64 chunks (up to staged slot 2,047),
    // also past the end of a small unit's staging; the values read there are
    // never stored, and this pad keeps the last wave's such reads inside the
    // workgroup's LDS.
    const uint32_t pad = stage_elems * 2u < 4096u ? 4096u - stage_elems * 2u : 0u;
    auto lds_for = [&](uint32_t w) { return lds_tables * 1024u + w * stage_elems * 2u + pad; };
    uint32_t waves = 0, per_cu = 0;
    for (uint32_t w = 16; w >= 1; w >>= 1) {  // the geometry with the most resident waves
        if (asked && w != asked) continue;
        if (fixed_static + lds_for(w) > static_cast<uint32_t>(info.lds_per_group)) continue;
        const uint32_t occ = static_cast<uint32_t>(occupancy(fn, w, lds_for(w)));
        if (occ && (!waves || occ * w > per_cu * waves)) {
            waves = w;
            per_cu = occ;
        }
    }
    if (!waves) return DF11_E_UNSUPPORTED;
    const uint32_t lds_bytes = lds_for(waves);

    KParams p;
    p.tables = static_cast<const uint32_t *>(blk->tables);
    p.stream = blk->stream;
    p.sm = blk->sign_mant;
    p.gaps = blk->gaps;
    p.unit_pos = blk->unit_pos;
    p.counts = blk->counts;
    p.unit_end = blk->unit_end;
    p.out = out_bf16;
    p.n_total = blk->n_total;
    p.total_bits = blk->total_bits;
    p.n_windows = blk->n_windows;
    p.n_units = blk->n_units;
    p.last_unit_bits = static_cast<uint32_t>(blk->total_bits - 4096 * (blk->n_units - 1));
    p.n_tables = blk->n_tables;
    p.stage_elems = stage_elems;
    p.out_phase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(out_bf16) >> 1) & 31u;

    // The automatic grid gives each wave about four units to walk, whatever
    // the block's size (one persistent wave of workgroups streams worse, and so
    // do short-lived waves that each pay the table load and the first unit's
    // latency for one unit), but never fewer workgroups than resident slots.
    const uint64_t groups = (blk->n_units + waves - 1) / waves;
    const uint64_t resident = uint64_t(info.cus) * uint64_t(per_cu);
    uint64_t grid;
    if (launch && launch->oversubscribe)
        grid = std::min<uint64_t>(groups, resident * launch->oversubscribe);
    else
        grid = std::min<uint64_t>(groups, std::max<uint64_t>(resident, (groups + kUnitsPerWave - 1) / kUnitsPerWave));
    if (launch && launch->max_groups) grid = std::min<uint64_t>(grid, launch->max_groups);
    grid = std::max<uint64_t>(grid, 1);
    // Units taken in turn within a workgroup pay an LDS round trip before each
    // next unit's loads: a gain of about 1 % when the waves have two units or
    // more on average, a loss of about 1 % when most have one.
    p.unit_queue = grid * waves * 2 <= blk->n_units ? 1u : 0u;

    // hipLaunchKernel reports the status of this launch only (hipGetLastError
    // would also return errors left behind by earlier runtime calls).
    void *args[] = {&p};
    const hipError_t err = hipLaunchKernel(fn, dim3(static_cast<uint32_t>(grid)), dim3(64 * waves), args,
                                           lds_bytes, static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) {
        df11i::last_hip_error = static_cast<int32_t>(err);
        return DF11_E_HIP;
    }
    return DF11_OK;
}

}  // namespace

extern "C" df11_status df11_decode_block_ex(const df11_device_block *blk, uint16_t *out_bf16,
                                            uint64_t out_capacity, void *hip_stream,
                                            const df11_launch *launch) {
    return df11i::guarded([&] { return decode_block(blk, out_bf16, out_capacity, hip_stream, launch); });
}

extern "C" df11_status df11_decode_block(const df11_device_block *blk, uint16_t *out_bf16,
                                         uint64_t out_capacity, void *hip_stream) {
    return df11_decode_block_ex(blk, out_bf16, out_capacity, hip_stream, nullptr);
}
