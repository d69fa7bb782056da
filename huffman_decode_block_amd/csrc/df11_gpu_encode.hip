// DF11 block encoder on the GPU (gfx950): the step before the decode.
//
// What is produced follows the hada.io summary of the DFloat11 paper,
// section "Le format DFloat11" (exponent-only Huffman code, EncodedExponent
// bit-packed, PackedSignMantissa verbatim) and section "Noyau GPU en deux
// etapes et metadonnees auxiliaires" (64-bit windows with a 5-bit gap to
// their first code, stored output positions).  The code lengths come from the
// host (the block's 256 exponent counts, taken here on the device); the
// device computes every code's bit offset with a prefix sum and packs all
// sections, byte for byte as the host encoder does.
//
// Passes (one stream, in order):
//   hist    (df11_gpu_histogram) per chunk of 4,096 weights its 256 exponent
//           counts, and their sum over the block
//   bits    bits per chunk from its counts and the code lengths (the weights
//           are not read again), and their exclusive prefix within each
//           segment of 256 chunks
//   top     exclusive prefix of the segment totals (one workgroup)
//   bounds  zeroes the stream words that two neighbouring chunks share and
//           the padding past what later passes write (stream, gaps, counts,
//           sign/mantissa); presets unit_pos and the first-start records for
//           the last unit and window, the only ones where no code may start
//   pack    persistent waves, one chunk per wave at a time: sign/mantissa
//           bytes; each lane shifts the codes of its 64 consecutive weights
//           into a register and writes the finished words into the wave's
//           LDS frame (its start from a wave scan of the lanes' bits), which
//           goes to HBM with global atomic OR only on the two words shared
//           with the neighbouring chunks; the lane whose code is the first to
//           start in a window writes that window's records (gap, unit
//           position, first weight)
//   finish  5-bit gap fields (8 windows per 5 bytes) and window counts
// The aligned-units layout is produced by the host encoder only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "df11_internal.h"
#include "df11_wave.h"

namespace {

constexpr uint32_t kThreads = 256;
constexpr uint64_t kMaxWeights = uint64_t{1} << 48;  // no block holds more (512 TB of BF16)
constexpr uint32_t kPerThread = 16;                   // weights per thread in hist
constexpr uint32_t kChunk = kThreads * kPerThread;    // 4,096 weights per chunk
constexpr uint32_t kSegChunks = kThreads;             // chunks per segment of the two-level scan
constexpr uint32_t kScanThreads = 1024;
constexpr uint32_t kBitsThreads = 1024;               // bits: threads per workgroup (one segment)

struct EncParams {
    const uint16_t *x;
    const uint16_t *chunk_hist;  // per chunk, 256 exponent counts
    uint8_t *stream, *sm, *gaps, *counts;
    uint64_t *unit_pos;
    uint32_t *chunk_pre;  // per chunk: its segment's bits before it
    uint64_t *seg_sum;    // per segment: its bits
    uint64_t *seg_off;    // per segment: the bits before it (one more entry: the total)
    uint8_t *gap8;
    uint64_t *wfirst;
    uint64_t n, total_bits, n_windows, n_units, n_chunks, n_segs;
    uint64_t stream_bytes, sm_bytes, gaps_bytes, counts_bytes;
    uint32_t code[256];
    uint8_t len[256];
};

__device__ __forceinline__ uint32_t exponent_of(uint32_t x) { return (x >> 7) & 0xFFu; }

// Workgroup barrier that orders LDS accesses only: global loads and stores in
// flight are not waited for (the passes never read back, within a pass, what
// another wave wrote to global memory).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- histogram
__global__ void __launch_bounds__(256) hist_zero(uint64_t *hist) {
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
}

constexpr uint32_t kWindow = 8;        // exponents counted in lane-private counters
constexpr uint32_t kWindowBelow = 5;   // the window starts this many exponents below the last chunk's mode
constexpr uint32_t kNoWindow = 0x100;  // a window base that no exponent reaches (before the first mode)
constexpr uint32_t kHistWaves = 4;                       // waves per workgroup
constexpr uint32_t kHistThreads = 64 * kHistWaves;
constexpr uint32_t kHistRound = 1024;                    // weights a wave counts per round (16 per lane)
constexpr uint32_t kHistRounds = kChunk / kHistRound;    // rounds per chunk
constexpr uint32_t kHistAhead = 2;                       // rounds requested ahead (register sets)
constexpr uint32_t kHistGroupsPerCU = 3;                 // workgroups per CU at most
static_assert(kHistRounds % kHistAhead == 0, "a register set must hold the same round of every chunk");

// The lane's 16 weights of round r of chunk c as two 16-byte loads; each of
// the wave's two loads reads one contiguous 1 KB piece (zeros past the
// block's end, through a buffer range that stops there; a chunk past the last
// reads as zeros).  Non-temporal: the input is streamed once per pass and is
// larger than the caches, so that it does not displace other lines.
__device__ __forceinline__ void hist_load(const uint16_t *x, uint64_t n, uint64_t c, uint32_t r, uint32_t lane,
                                          df11w::v4u &a, df11w::v4u &b) {
    const uint64_t first = c * kChunk + uint64_t{r} * kHistRound;
    const uint64_t left = first < n ? n - first : 0;
    const df11w::Rsrc rs =
        df11w::rsrc(x + (left ? first : 0), static_cast<uint32_t>(2 * (left < kHistRound ? left : kHistRound)));
    a = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, 0, df11w::kNonTemporal);
    b = __builtin_amdgcn_raw_buffer_load_b128(rs, 1024 + 16 * lane, 0, df11w::kNonTemporal);
}

// Largest value over the 64 lanes, in every lane (DPP row shifts and row
// broadcasts, then lane 63's value).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    uint32_t m = x;
    m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, m, 0x111, 0xF, 0xF, true)));  // row_shr:1
    m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, m, 0x112, 0xF, 0xF, true)));  // row_shr:2
    m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, m, 0x114, 0xF, 0xF, true)));  // row_shr:4
    m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, m, 0x118, 0xF, 0xF, true)));  // row_shr:8
    m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, m, 0x142, 0xA, 0xF, false))); // row_bcast:15
    m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, m, 0x143, 0xC, 0xF, false))); // row_bcast:31
    return __builtin_amdgcn_readlane(m, 63);
}

// Orders one wave's LDS accesses across its lanes (no other wave reads them).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The window's first exponent for a mode (the most frequent exponent so far).
__device__ __forceinline__ uint32_t window_base(uint32_t mode) {
    return __builtin_amdgcn_readfirstlane(min(mode > kWindowBelow ? mode - kWindowBelow : 0u, 256u - kWindow));
}

// Most frequent of the lane's four bins 4 lane .. 4 lane + 3 over the wave
// (ties: the larger exponent).
__device__ __forceinline__ uint32_t wave_mode(const uint32_t cnt[4], uint32_t lane) {
    uint32_t m = 0;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) m = max(m, (cnt[k] << 8) | (4 * lane + k));
    return wave_max(m) & 0xFFu;
}

// One round: each of the lane's 16 exponents goes to its own counter when it
// falls in the window, else to the wave's bins.
__device__ __forceinline__ void hist_count(const df11w::v4u &a, const df11w::v4u &b, uint32_t base, uint32_t *wc,
                                           uint32_t *bins) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t e = exponent_of(w[k / 2] >> (16 * (k & 1)));
        const uint32_t d = e - base;
        if (d < kWindow)
            atomicAdd(wc + 64 * d, 1u);  // this lane's own counter
        else
            atomicAdd(bins + e, 1u);
    }
}

// The end of a chunk's count: lane l takes bins 4l .. 4l + 3 of the wave
// (clearing them), stores them as the chunk's counts (through a buffer range,
// none without chunk_hist, so that the store is not behind a branch) and adds
// them to its totals.
__device__ __forceinline__ void hist_chunk_out(uint32_t *bins, uint16_t *chunk_hist, uint64_t c, uint32_t lane,
                                               uint64_t total[4], uint32_t cnt[4]) {
    wave_lds_fence();
    const uint4 v = *reinterpret_cast<const uint4 *>(bins + 4 * lane);
    *reinterpret_cast<uint4 *>(bins + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    cnt[0] = v.x, cnt[1] = v.y, cnt[2] = v.z, cnt[3] = v.w;
    const df11w::Rsrc ch = df11w::rsrc(chunk_hist ? chunk_hist + c * 256 : nullptr, chunk_hist ? 512u : 0u);
    __builtin_amdgcn_raw_buffer_store_b64(df11w::v2u{cnt[0] | (cnt[1] << 16), cnt[2] | (cnt[3] << 16)}, ch, 8 * lane,
                                          0, 0);
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) total[k] += cnt[k];
}

__global__ void __launch_bounds__(kHistThreads) hist_kernel(const uint16_t *x, uint64_t n, uint64_t *hist,
                                                        uint16_t *chunk_hist) {
    // Each wave counts whole chunks on its own, with no workgroup barrier
    // until the end.  Weight exponents cluster on a few values, and
    // same-address LDS atomics are serialised, so a window of 8 exponents,
    // from 5 below the wave's last mode, is counted in lane-private LDS
    // counters (counter d of lane l at word 64 d + l: no two lanes share a
    // bank or an address) and only exponents outside it go to the wave's 256
    // bins.  After a chunk the wave adds its window counters over its lanes
    // (DPP) into the bins, and lane l reads, clears and stores bins
    // 4l .. 4l + 3 as the chunk's counts, adds them to its running totals and
    // offers them to the choice of the next window.  A wave's first window
    // comes from the bins of its first round.  A chunk is counted in 4 rounds
    // of 1,024 weights, each requested two rounds ahead.  The block's last
    // chunk, when not whole, is counted weight by weight after the loop (a
    // buffer load that ends past the range does not return its first part).
    // At the end the workgroup adds its waves' totals in LDS and then into
    // the block's histogram.
    __shared__ __align__(16) uint32_t win[kHistWaves][kWindow * 64];
    __shared__ __align__(16) uint32_t bins_all[kHistWaves][256];
    __shared__ unsigned long long tot[256];
    const uint32_t t = threadIdx.x, lane = t & 63u;
    // uniform per wave, so that the buffer resources built from it stay in
    // scalar registers
    const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
    uint32_t *wc = &win[wave][lane];
    uint32_t *bins = bins_all[wave];
#pragma unroll
    for (uint32_t d = 0; d < kWindow; ++d) wc[64 * d] = 0;
    *reinterpret_cast<uint4 *>(bins + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    for (uint32_t i = t; i < 256; i += kHistThreads) tot[i] = 0;
    __syncthreads();

    const uint64_t n_full = n / kChunk;  // whole chunks
    const uint64_t stride = uint64_t{gridDim.x} * kHistWaves;
    uint64_t total[4] = {0, 0, 0, 0};
    uint32_t cnt[4];
    uint32_t base = kNoWindow;  // uniform
    uint64_t c = uint64_t{blockIdx.x} * kHistWaves + wave;
    // round r of a chunk is counted from register set r mod kHistAhead, which
    // is then refilled with the round kHistAhead rounds later (of this chunk
    // or the next one)
    df11w::v4u a[kHistAhead], b[kHistAhead];
#pragma unroll
    for (uint32_t k = 0; k < kHistAhead; ++k) {
        // in this order, as in the loop: a wait for one round then leaves the
        // later ones in flight on both paths into the loop
        hist_load(x, n, c, k, lane, a[k], b[k]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (; c < n_full; c += stride) {
#pragma unroll
        for (uint32_t r = 0; r < kHistRounds; ++r) {
            const uint32_t k = r % kHistAhead, rn = r + kHistAhead;
            hist_count(a[k], b[k], base, wc, bins);
            hist_load(x, n, rn < kHistRounds ? c : c + stride, rn % kHistRounds, lane, a[k], b[k]);
            if (r == 0 && base == kNoWindow) {  // uniform: the wave's first window, from its first round
                wave_lds_fence();
                const uint4 v = *reinterpret_cast<const uint4 *>(bins + 4 * lane);
                const uint32_t first[4] = {v.x, v.y, v.z, v.w};
                base = window_base(wave_mode(first, lane));
            }
        }

        // the window counters, summed over the lanes two at a time (at most
        // 64 per lane and 4,096 per chunk: 16-bit halves), into the bins
#pragma unroll
        for (uint32_t j = 0; j < kWindow / 2; ++j) {
            const uint32_t pair = wc[64 * (2 * j)] | (wc[64 * (2 * j + 1)] << 16);
            wc[64 * (2 * j)] = 0;
            wc[64 * (2 * j + 1)] = 0;
            const uint32_t sum = __builtin_amdgcn_readlane(df11w::wave_inclusive_scan(pair), 63);
            if (lane == 0) {
                atomicAdd(bins + base + 2 * j, sum & 0xFFFFu);
                atomicAdd(bins + base + 2 * j + 1, sum >> 16);
            }
        }
        hist_chunk_out(bins, chunk_hist, c, lane, total, cnt);
        base = window_base(wave_mode(cnt, lane));
    }
    if (c == n_full && n_full * kChunk < n) {  // uniform: this wave's sequence holds the last, partial chunk
        for (uint64_t i = n_full * kChunk + lane; i < n; i += 64) atomicAdd(bins + exponent_of(x[i]), 1u);
        hist_chunk_out(bins, chunk_hist, c, lane, total, cnt);
    }
    // the waves' totals, then one global atomic per nonzero bin
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k)
        if (total[k]) atomicAdd(&tot[4 * lane + k], static_cast<unsigned long long>(total[k]));
    __syncthreads();
    for (uint32_t i = t; i < 256; i += kHistThreads)
        if (tot[i]) atomicAdd(reinterpret_cast<unsigned long long *>(hist + i), tot[i]);
}

// ---------------------------------------------------------------- padding
__device__ __forceinline__ void fill_padding(const EncParams &p, uint64_t tid, uint64_t step) {
    // Only what no later pass writes: pack stores every stream word up to the
    // one holding the last code bit, finish every gap byte of the 5-byte groups
    // and every window count, so only the padding past them is zeroed here.
    for (uint64_t i = p.total_bits / 32 * 4 + tid; i < p.stream_bytes; i += step) p.stream[i] = 0;
    for (uint64_t i = (p.n_windows + 7) / 8 * 5 + tid; i < p.gaps_bytes; i += step) p.gaps[i] = 0;
    for (uint64_t i = p.n + tid; i < p.sm_bytes; i += step) p.sm[i] = 0;
    if (p.counts)
        for (uint64_t i = p.n_windows + tid; i < p.counts_bytes; i += step) p.counts[i] = 0;
    // a code starts in every window but possibly the last (its gap then ends
    // at total_bits), so only the last unit can lack a first code start
    if (tid == 0) {
        p.unit_pos[p.n_units] = p.n;
        if (p.n_units) p.unit_pos[p.n_units - 1] = p.n;
    }
    if (tid == 0 && p.n_windows) {
        p.gap8[p.n_windows - 1] = static_cast<uint8_t>(p.total_bits - 64 * (p.n_windows - 1));
        if (p.counts) {
            p.wfirst[p.n_windows - 1] = p.n;
            p.wfirst[p.n_windows] = p.n;
        }
    }
}

// Whether chunk c holds kChunk weights (all but possibly the block's last).
__device__ __forceinline__ bool chunk_is_full(const EncParams &p, uint64_t c) { return (c + 1) * kChunk <= p.n; }

// Block-wide exclusive sum of one value per thread (kWaves waves): a scan
// inside each wave, then each wave adds the totals of the waves before it;
// also the block total.  `wsum` holds kWaves values.
template <uint32_t kWaves>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t *wsum, uint32_t &total) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t incl = df11w::wave_inclusive_scan(v);
    if (lane == 63) wsum[wave] = incl;
    lds_barrier();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (uint32_t k = 0; k < kWaves; ++k) {
        const uint32_t w = wsum[k];
        before += k < wave ? w : 0u;
        total += w;
    }
    return before + incl - v;
}

// ---------------------------------------------------------------- chunk bits
// One thread per chunk: its bits are the sum over exponents of count x code
// length; then the exclusive prefix within the segment (one workgroup).
__global__ void __launch_bounds__(kBitsThreads) bits_kernel(EncParams p) {
    // The bits of each chunk of this segment from its 256 counts: 8 lanes per
    // chunk, each reading 32 counts (64 contiguous bytes, so that a wave reads
    // 8 chunks' counts in one piece), summed over the 8 lanes with DPP; then
    // the block scan of the segment's 256 chunk totals.  16 waves per
    // segment, so that a chunk's counts are requested by two threads' loops at
    // most and enough reads are in flight (a segment per 4 waves left most CUs
    // with one or no workgroup).
    __shared__ uint32_t len[256];
    __shared__ uint32_t cbits[kSegChunks];
    __shared__ uint32_t wsum[kBitsThreads / 64];
    const uint32_t t = threadIdx.x;
    if (t < 256) len[t] = p.len[t];
    __syncthreads();
    const uint32_t sub = t & 7u;  // this lane's eighth of a chunk's counts
    const uint64_t seg0 = uint64_t{blockIdx.x} * kSegChunks;
    for (uint32_t k = t >> 3; k < kSegChunks; k += kBitsThreads / 8) {
        const uint64_t c = seg0 + k;
        uint32_t bits = 0;
        if (c < p.n_chunks) {
            const uint4 *h = reinterpret_cast<const uint4 *>(p.chunk_hist + c * 256 + 32 * sub);
#pragma unroll
            for (uint32_t j = 0; j < 4; ++j) {  // exponents 32 sub + 8j .. 32 sub + 8j + 7
                const uint4 v = h[j];
                const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (uint32_t m = 0; m < 4; ++m) {
                    const uint32_t e = 32 * sub + 8 * j + 2 * m;
                    bits += (q[m] & 0xFFFFu) * len[e] + (q[m] >> 16) * len[e + 1];
                }
            }
        }
        // sum over the chunk's 8 lanes: quad xor 1, quad xor 2, then half-row mirror
        bits += __builtin_amdgcn_update_dpp(0u, bits, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
        bits += __builtin_amdgcn_update_dpp(0u, bits, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
        bits += __builtin_amdgcn_update_dpp(0u, bits, 0x141, 0xF, 0xF, false);  // row_half_mirror
        if (sub == 0) cbits[k] = bits;
    }
    __syncthreads();
    const uint64_t c = seg0 + t;
    uint32_t seg_bits;
    const uint32_t pre = block_exclusive_sum<kBitsThreads / 64>(t < kSegChunks ? cbits[t] : 0u, wsum, seg_bits);
    if (t < kSegChunks && c < p.n_chunks) p.chunk_pre[c] = pre;
    if (t == 0) p.seg_sum[blockIdx.x] = seg_bits;
}

// ---------------------------------------------------------------- top scan
__global__ void __launch_bounds__(kScanThreads) top_kernel(EncParams p) {
    // Each thread sums a contiguous run of segment totals, one block scan of
    // the 1,024 run sums, then each thread writes its run's offsets.
    __shared__ uint64_t part[kScanThreads];
    const uint32_t t = threadIdx.x;
    const uint64_t per = (p.n_segs + kScanThreads - 1) / kScanThreads;
    const uint64_t b = std::min<uint64_t>(t * per, p.n_segs), e = std::min<uint64_t>(b + per, p.n_segs);
    uint64_t s = 0;
    for (uint64_t k = b; k < e; ++k) s += p.seg_sum[k];
    part[t] = s;
    __syncthreads();
    for (uint32_t d = 1; d < kScanThreads; d <<= 1) {  // Hillis-Steele, 64-bit
        const uint64_t add = t >= d ? part[t - d] : 0u;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    uint64_t run = part[t] - s;
    for (uint64_t k = b; k < e; ++k) {
        p.seg_off[k] = run;
        run += p.seg_sum[k];
    }
    if (t == kScanThreads - 1) p.seg_off[p.n_segs] = part[t];
}

// Before pack, with every chunk's first bit known: the stream word where
// chunk c starts is shared with the previous chunk when that one ends inside
// it (both OR their bits into it), so it is zeroed; and the padding and
// presets of fill_padding.
__global__ void __launch_bounds__(kThreads) bounds_kernel(EncParams p) {
    const uint64_t tid = uint64_t{blockIdx.x} * blockDim.x + threadIdx.x;
    const uint64_t step = uint64_t{gridDim.x} * blockDim.x;
    for (uint64_t c = 1 + tid; c < p.n_chunks; c += step) {
        const uint64_t cb = p.seg_off[c / kSegChunks] + p.chunk_pre[c];
        if (cb & 31u) reinterpret_cast<uint32_t *>(p.stream)[cb >> 5] = 0;
    }
    fill_padding(p, tid, step);
}

// ---------------------------------------------------------------- pack
// Persistent waves, each packing one 4,096-weight chunk at a time with no
// workgroup barrier: lane l takes weights 64 l .. 64 l + 63 of the chunk,
// whose codes form one run of at least 64 bits, so that a 32-bit word is
// shared by two neighbouring lanes at most.
// The lane shifts its codes one after the other into a 64-bit register and
// writes the last finished word into the wave's LDS frame after each code;
// its first word, which the lane before also reaches into, is completed by
// that lane's OR of its last partial word once the wave's runs are written.
// Every weight's exponent is staged in LDS first (the chunk is read in
// coalesced 16-byte pieces), so that each lane can take its 64 in order.
// A window's record (gap, first weight, unit position) is written by the lane
// whose code is the first to start in the window.  Chunks whose bits would
// not fit the frame, and the block's last chunk when not whole, are packed
// with global atomic ORs of each code instead.  A chunk's weights are
// requested when the wave starts on it: holding the next chunk's 32 registers
// through the packing loop would cost waves per SIMD (or spills).  Six waves
// per SIMD (80 registers) leave room to request the table entries of the
// next four weights before the current four are packed.
constexpr uint32_t kRunWaves = 4;                                // waves per workgroup
constexpr uint32_t kRunThreads = 64 * kRunWaves;
constexpr uint32_t kRunPer = kChunk / 64;                        // weights per lane (64)
constexpr uint32_t kRunStageWords = 64 * (kRunPer + 4) / 4;      // 1,088: 68 bytes of exponents per lane
constexpr uint32_t kRunFrameWords = kRunStageWords - 64;         // then one spare word per lane
constexpr uint32_t kRunFrameBits = 32 * (kRunFrameWords - 1);    // a chunk fits when its head and bits do
constexpr uint32_t kRunGapSlots = (kRunFrameBits + 63) / 64 / 4 * 4 + 4;  // windows of a frame, bytes
static_assert(kRunGapSlots * 64 >= kRunFrameBits + 63, "every window of a frame has a gap slot");

// What a wave requests for a chunk: its 512 pieces of 8 weights (piece
// lane + 64 k in w[k]; zeros for a chunk that is not whole), its first bit
// (segment offset + prefix) and the 4-byte word whose high half is the
// previous chunk's last weight.
struct RunInputs {
    df11w::v4u w[8];
    uint32_t seg_lo, seg_hi, pre, xw;
};

__device__ __forceinline__ void run_load(const EncParams &p, uint64_t c, uint32_t lane, RunInputs &in) {
    const df11w::v2u so = __builtin_amdgcn_raw_buffer_load_b64(df11w::rsrc(p.seg_off + c / kSegChunks, 8), 0, 0, 0);
    in.seg_lo = so.x;
    in.seg_hi = so.y;
    in.pre = __builtin_amdgcn_raw_buffer_load_b32(df11w::rsrc(p.chunk_pre + c, 4), 0, 0, 0);
    // (chunk 0: any readable word, not used)
    const uint32_t *wl = c ? reinterpret_cast<const uint32_t *>(p.x + c * kChunk - 2) : p.chunk_pre;
    in.xw = __builtin_amdgcn_raw_buffer_load_b32(df11w::rsrc(wl, 4), 0, 0, 0);
    const bool full = chunk_is_full(p, c);
    const df11w::Rsrc r = df11w::rsrc(p.x + (full ? c * kChunk : 0), full ? 2 * kChunk : 0u);
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k)
        in.w[k] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (lane + 64 * k), 0, df11w::kNonTemporal);
}

// The chunk's sign/mantissa bytes to HBM and its exponents into the staging:
// exponent i of the chunk at byte i + 4 (i / 64), so that lane l reads its
// 64 as 16 words at word 17 l + j (no two lanes in one bank).
__device__ __forceinline__ void run_stage(const EncParams &p, uint64_t c, uint32_t lane, const RunInputs &in,
                                          bool full, uint32_t *stage) {
    // Addresses are a per-lane base plus a constant per piece, so that no
    // per-piece address is kept in a register across chunks.  The block's
    // last chunk, when not whole, is read and written element by element
    // through buffer ranges that end at the block's end.
    const uint32_t left = full ? kChunk : static_cast<uint32_t>(p.n - c * kChunk);
    const df11w::Rsrc smr = df11w::rsrc(p.sm + c * kChunk, left);
    const df11w::Rsrc xr = df11w::rsrc(p.x + c * kChunk, 2 * left);
    uint32_t *st = stage + 2 * lane + (lane >> 3);
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
        const uint32_t w0 = 8 * lane + 512 * k;  // weights w0 .. w0 + 7 of the chunk: piece lane + 64 k
        uint32_t a[4] = {in.w[k].x, in.w[k].y, in.w[k].z, in.w[k].w};
        if (!full) {
#pragma unroll
            for (uint32_t h = 0; h < 4; ++h)
                a[h] = __builtin_amdgcn_raw_buffer_load_b16(xr, 2 * (w0 + 2 * h), 0, 0) |
                       (static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(xr, 2 * (w0 + 2 * h + 1), 0, 0))
                        << 16);
        }
        uint32_t smw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t x0 = a[2 * h], x1 = a[2 * h + 1];
            const uint32_t s0 = ((x0 >> 8) & 0x00800080u) | (x0 & 0x007F007Fu);  // two sm bytes in 16-bit halves
            const uint32_t s1 = ((x1 >> 8) & 0x00800080u) | (x1 & 0x007F007Fu);
            smw[h] = __builtin_amdgcn_perm(s1, s0, 0x06040200u);
        }
        if (full) {  // written once and not read here: non-temporal
            __builtin_amdgcn_raw_buffer_store_b64(df11w::v2u{smw[0], smw[1]}, smr, w0, 0, df11w::kNonTemporal);
        } else {
#pragma unroll
            for (uint32_t h = 0; h < 8; ++h)
                __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(smw[h / 4] >> (8 * (h & 3))), smr, w0 + h, 0,
                                                     0);
        }
        // piece lane + 64 k's exponents at word 2 pc + pc / 8 = (2 lane + lane / 8) + 136 k
        st[136 * k] = __builtin_amdgcn_perm(a[1] >> 7, a[0] >> 7, 0x06040200u);      // weights 0..3
        st[136 * k + 1] = __builtin_amdgcn_perm(a[3] >> 7, a[2] >> 7, 0x06040200u);  // and 4..7
    }
}

// The packing loop of a chunk that fits the frame (see run_pack_kernel):
// the lane's codes into the frame and its window records; returns the shift
// register and the frame bit after the lane's last code.
template <bool kCounts>
__device__ __forceinline__ void run_lane_codes(const EncParams &p, const uint32_t ex[16], const uint2 *ent,
                                               uint32_t *stage, uint8_t *gst, uint32_t lane, uint32_t pos0, int32_t nwb,
                                               uint64_t wbase, uint64_t first0, uint64_t &acc_out, uint32_t &pos_out) {
    uint64_t acc = 0;
    uint32_t pos = pos0;
    const uint32_t hw4 = 4 * (pos0 >> 5) + 4;
    // Window records: nw is the frame window after the one where the code
    // before started.  A code opens window pos / 64 when that is nw (it
    // cannot start later: the code before is at most 32 bits), and its gap is
    // then pos mod 64; codes that open none write their gap to the lane's
    // spare word past the frame.  A lane's run spans fewer than 64 windows,
    // so it opens at most one unit: uw, the first unit window from nw on,
    // taken at weight uj.
    uint32_t nw = static_cast<uint32_t>(nwb) >> 6;
    const uint32_t uw = nw + ((64u - ((static_cast<uint32_t>(wbase) + nw) & 63u)) & 63u);
    uint32_t uj = kRunPer;  // none
    uint8_t *const spare = reinterpret_cast<uint8_t *>(stage + kRunFrameWords + lane);
    const uint32_t first_lo = static_cast<uint32_t>(first0), first_hi = static_cast<uint32_t>(first0 >> 32);
    // the frame's windows of wfirst, up to the last one of the block
    const uint64_t wleft = kCounts && p.n_windows > wbase ? p.n_windows - wbase : 0;
    const df11w::Rsrc wfr = df11w::rsrc(kCounts ? p.wfirst + wbase : nullptr,
                                        static_cast<uint32_t>(8 * (wleft < kRunGapSlots ? wleft : kRunGapSlots)));
    // table entries requested a group of four weights ahead (LDS latency)
    uint2 ceq[2][4];
#pragma unroll
    for (uint32_t b = 0; b < 4; ++b) ceq[0][b] = ent[(ex[0] >> (8 * b)) & 0xFFu];
#pragma unroll
    for (uint32_t j = 0; j < kRunPer; ++j) {
        if ((j & 3) == 0 && j + 4 < kRunPer) {
#pragma unroll
            for (uint32_t b = 0; b < 4; ++b) ceq[((j / 4) + 1) & 1][b] = ent[(ex[j / 4 + 1] >> (8 * b)) & 0xFFu];
        }
        const uint2 ce = ceq[(j / 4) & 1][j & 3];
        const uint32_t pw = pos >> 6;
        const bool opens = pw >= nw;
        *(opens ? gst + pw : spare) = static_cast<uint8_t>(pos & 63u);
        uj = opens && pw == uw ? j : uj;
        if (kCounts)  // the window's first weight (first0 is a multiple of 64)
            __builtin_amdgcn_raw_buffer_store_b64(df11w::v2u{first_lo | j, first_hi}, wfr, opens ? 8 * pw : df11w::kOff,
                                                  0, 0);
        nw += opens ? 1u : 0u;
        acc = (acc << ce.y) | ce.x;
        pos += ce.y;
        // the last finished word (before the lane's first word is finished:
        // that word, rewritten once it is)
        const uint32_t a4 = max((pos >> 3) & ~3u, hw4) - 4;
        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(stage) + a4) =
            static_cast<uint32_t>(acc >> (pos & 31u));
        if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
    if (uj < kRunPer) {
        const uint64_t w = wbase + uw;
        if (w < p.n_windows) p.unit_pos[w >> 6] = first0 + uj;
    }
    acc_out = acc;
    pos_out = pos;
}

template <bool kCounts>  // with the window records of the stored window counts
__global__ void __launch_bounds__(kRunThreads) __attribute__((amdgpu_waves_per_eu(6))) run_pack_kernel(EncParams p) {
    __shared__ uint2 ent[256];  // per exponent: code, length
    __shared__ uint8_t lentab[256];
    __shared__ __align__(16) uint32_t stage_all[kRunWaves][kRunStageWords];
    __shared__ __align__(16) uint32_t gap_all[kRunWaves][kRunGapSlots / 4];
    const uint32_t t = threadIdx.x, lane = t & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
    uint32_t *stage = stage_all[wave];
    uint8_t *gst = reinterpret_cast<uint8_t *>(gap_all[wave]);  // per window of the frame: its gap, or 0xFF
    if (t < 256) {
        ent[t] = make_uint2(p.code[t], p.len[t]);
        lentab[t] = p.len[t];
    }
    for (uint32_t k = lane; k < kRunGapSlots / 4; k += 64) gap_all[wave][k] = 0xFFFFFFFFu;
    __syncthreads();
    const uint64_t stride = uint64_t{gridDim.x} * kRunWaves;
    uint64_t c = uint64_t{blockIdx.x} * kRunWaves + wave;
    if (c >= p.n_chunks) return;  // uniform per wave; no barrier follows
    while (true) {
        RunInputs cur;
        run_load(p, c, lane, cur);
        const bool full = chunk_is_full(p, c);  // uniform
        wave_lds_fence();  // the previous chunk's frame has been read out
        run_stage(p, c, lane, cur, full, stage);
        // readfirstlane returns a signed int: each half is taken as uint32_t
        // before it is widened
        const uint32_t seg_lo = __builtin_amdgcn_readfirstlane(cur.seg_lo);
        const uint32_t seg_hi = __builtin_amdgcn_readfirstlane(cur.seg_hi);
        const uint32_t chunk_pre = __builtin_amdgcn_readfirstlane(cur.pre);
        const uint32_t xw = __builtin_amdgcn_readfirstlane(cur.xw);
        const uint64_t cb = ((static_cast<uint64_t>(seg_hi) << 32) | seg_lo) + chunk_pre;  // the chunk's first bit
        const uint64_t cn = c + stride;
        wave_lds_fence();

        // the lane's 64 exponents (weight 64 lane + 4 j + b in byte b of ex[j])
        uint32_t ex[16];
#pragma unroll
        for (uint32_t j = 0; j < 16; ++j) ex[j] = stage[17 * lane + j];
        const uint64_t first0 = c * kChunk + uint64_t{kRunPer} * lane;  // the lane's first weight
        const uint32_t m = full ? kRunPer
                                : (first0 < p.n ? static_cast<uint32_t>(p.n - first0 < kRunPer ? p.n - first0 : kRunPer)
                                                : 0u);
        uint32_t sum = 0, lastlen = 0;
        if (full) {  // uniform
#pragma unroll
            for (uint32_t j = 0; j < kRunPer; ++j) {
                const uint32_t l = lentab[(ex[j / 4] >> (8 * (j & 3))) & 0xFFu];
                sum += l;
                if (j == kRunPer - 1) lastlen = l;
                if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);  // few lookups in flight: registers
            }
        } else {
            for (uint32_t j = 0; j < m; ++j) sum += lentab[reinterpret_cast<const uint8_t *>(stage)[68 * lane + j]];
            lastlen = lentab[reinterpret_cast<const uint8_t *>(stage)[68 * lane + kRunPer - 1]];
        }
        // the exponents are taken apart again in the packing loop rather
        // than kept from here (64 more registers)
#pragma unroll
        for (uint32_t j = 0; j < 16; ++j) asm volatile("" : "+v"(ex[j]));
        const uint32_t incl = df11w::wave_inclusive_scan(sum);
        const uint32_t chunk_bits = __builtin_amdgcn_readlane(incl, 63);
        const uint32_t head = static_cast<uint32_t>(cb & 63u);
        const uint64_t wbase = cb >> 6;  // the frame's first window
        // the code before the lane's first one: the previous lane's last, or
        // the previous chunk's last weight (none before the block's first)
        const uint32_t up = __shfl_up(lastlen, 1);
        const uint32_t prevlen = lane ? up : (c ? static_cast<uint32_t>(lentab[exponent_of(xw >> 16)]) : 64u);
        const uint32_t pos0 = head + incl - sum;  // frame bit of the lane's first code
        // the first window boundary at or after the previous code's start: a
        // code starting there or later opens a window
        int32_t nwb = ((static_cast<int32_t>(pos0) - static_cast<int32_t>(prevlen)) >> 6) * 64 + 64;
        const uint32_t k0 = head >> 5;
        const uint32_t nwords = (head + chunk_bits + 31) >> 5;
        const bool head_shared = (cb & 31u) != 0;
        const bool tail_shared = ((cb + chunk_bits) & 31u) != 0;
        uint32_t *out = reinterpret_cast<uint32_t *>(p.stream) + 2 * wbase;
        const uint64_t room = p.stream_bytes / 4 > 2 * wbase ? p.stream_bytes / 4 - 2 * wbase : 0;

        if (full && head + chunk_bits <= kRunFrameBits) {  // uniform
            uint64_t acc;
            uint32_t pos;
            run_lane_codes<kCounts>(p, ex, ent, stage, gst, lane, pos0, nwb, wbase, first0, acc, pos);
            // the lane's last partial word is the next lane's first word
            // (ORed into it) or the chunk's last word (stored)
            const uint32_t r = pos & 31u;
            const uint32_t tailw = static_cast<uint32_t>(acc << (32u - r));
            wave_lds_fence();
            if (r) {
                if (lane < 63)
                    atomicOr(&stage[pos >> 5], tailw);
                else
                    stage[pos >> 5] = tailw;
            }
            wave_lds_fence();

            // out to HBM as big-endian words; the first and last words are
            // shared with the neighbouring chunks when the chunk does not
            // start or end on a word boundary
            for (uint32_t k = k0 + lane; k < nwords; k += 64) {
                const uint32_t v = __builtin_bswap32(stage[k]);
                if (k >= room) continue;
                if ((k == k0 && head_shared) || (k == nwords - 1 && tail_shared))
                    atomicOr(out + k, v);
                else
                    out[k] = v;
            }
            const uint32_t nwin = (head + chunk_bits + 63) >> 6;
            for (uint32_t j = lane; j < nwin; j += 64) {
                const uint8_t g = gst[j];
                gst[j] = 0xFF;
                if (g != 0xFF && wbase + j < p.n_windows) p.gap8[wbase + j] = g;
            }
        } else {
            // Each code ORed into the stream in HBM.  The chunk's words that
            // no neighbouring chunk shares are zeroed first (the shared ones
            // were zeroed before this pass).
            const uint32_t z0 = k0 + (head_shared ? 1u : 0u), z1 = nwords - (tail_shared ? 1u : 0u);
            for (uint32_t k = z0 + lane; k < z1; k += 64)
                if (k < room) out[k] = 0;
            __threadfence();
            uint32_t pos = pos0;
            const uint8_t *lane_exp = reinterpret_cast<const uint8_t *>(stage) + 68 * lane;  // still staged
            for (uint32_t j = 0; j < m; ++j) {
                const uint2 ce = ent[lane_exp[j]];
                if (static_cast<int32_t>(pos) >= nwb) {
                    const uint32_t wr = static_cast<uint32_t>(nwb) >> 6;
                    const uint64_t w = wbase + wr;
                    if (w < p.n_windows) {
                        p.gap8[w] = static_cast<uint8_t>(pos - static_cast<uint32_t>(nwb));
                        if ((w & 63u) == 0) p.unit_pos[w >> 6] = first0 + j;
                        if (p.wfirst) p.wfirst[w] = first0 + j;
                    }
                    nwb += 64;
                }
                const uint32_t wi = pos >> 5, sh = pos & 31u;
                const uint64_t v = static_cast<uint64_t>(ce.x) << (64u - sh - ce.y);
                if (wi < room) atomicOr(out + wi, __builtin_bswap32(static_cast<uint32_t>(v >> 32)));
                if (static_cast<uint32_t>(v) && wi + 1 < room)
                    atomicOr(out + wi + 1, __builtin_bswap32(static_cast<uint32_t>(v)));
                pos += ce.y;
            }
        }
        if (cn >= p.n_chunks) break;  // uniform
        c = cn;
    }
}

// ---------------------------------------------------------------- finish
__global__ void __launch_bounds__(kThreads) finish_kernel(EncParams p) {
    const uint64_t tid = uint64_t{blockIdx.x} * blockDim.x + threadIdx.x;
    const uint64_t step = uint64_t{gridDim.x} * blockDim.x;
    // 5-bit gap fields, 8 windows per 5 bytes (big-endian), 32 windows per
    // thread: the gap bytes read as four 8-byte words, the 20 field bytes
    // written as five 4-byte words (byte by byte at the end of the section or
    // when the section is not 4-byte aligned).
    const uint64_t groups = (p.n_windows + 7) / 8;
    const uint64_t quads = (groups + 3) / 4;
    const bool words = (reinterpret_cast<uintptr_t>(p.gaps) & 3u) == 0;
    for (uint64_t q = tid; q < quads; q += step) {
        const uint64_t w0 = 32 * q;
        uint64_t g[4] = {0, 0, 0, 0};  // window w0 + 8i + j in byte j of g[i]
        if (w0 + 32 <= p.n_windows) {
            const uint64_t *src = reinterpret_cast<const uint64_t *>(p.gap8 + w0);
#pragma unroll
            for (int i = 0; i < 4; ++i) g[i] = src[i];
        } else {
            for (uint32_t j = 0; j < 32 && w0 + j < p.n_windows; ++j)
                g[j / 8] |= static_cast<uint64_t>(p.gap8[w0 + j]) << (8 * (j % 8));
        }
        uint64_t v[4];  // each group's 40 field bits
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[i] = (v[i] << 5) | ((g[i] >> (8 * j)) & 31u);
        }
        const uint32_t wd[5] = {  // the 160 field bits as big-endian words
            static_cast<uint32_t>(v[0] >> 8),
            static_cast<uint32_t>((v[0] << 24) | (v[1] >> 16)),
            static_cast<uint32_t>((v[1] << 16) | (v[2] >> 24)),
            static_cast<uint32_t>((v[2] << 8) | (v[3] >> 32)),
            static_cast<uint32_t>(v[3])};
        const uint64_t b0 = 20 * q;
        if (words && b0 + 20 <= p.gaps_bytes) {
            uint32_t *dst = reinterpret_cast<uint32_t *>(p.gaps + b0);
#pragma unroll
            for (int k = 0; k < 5; ++k) dst[k] = __builtin_bswap32(wd[k]);
        } else {
            for (uint32_t k = 0; k < 20 && b0 + k < p.gaps_bytes; ++k)
                p.gaps[b0 + k] = static_cast<uint8_t>(wd[k / 4] >> (24 - 8 * (k % 4)));
        }
    }
    if (p.counts)
        for (uint64_t w = tid; w < p.n_windows; w += step)
            p.counts[w] = static_cast<uint8_t>(p.wfirst[w + 1] - p.wfirst[w]);
}

uint64_t align256(uint64_t v) { return (v + 255) / 256 * 256; }

struct Workspace {
    uint64_t pre, seg_sum, seg_off, gap8, wfirst, bytes;
};

Workspace workspace_layout(uint64_t n, uint64_t n_windows, bool counts) {
    Workspace w{};
    const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
    const uint64_t n_segs = (n_chunks + kSegChunks - 1) / kSegChunks;
    w.pre = 0;
    w.seg_sum = align256(4 * n_chunks);
    w.seg_off = w.seg_sum + align256(8 * n_segs);
    w.gap8 = w.seg_off + align256(8 * (n_segs + 1));
    w.wfirst = w.gap8 + align256(n_windows);
    w.bytes = w.wfirst + (counts ? align256(8 * (n_windows + 1)) : 0);
    return w;
}

uint64_t chunk_hist_bytes(uint64_t n) { return (n + kChunk - 1) / kChunk * 256 * sizeof(uint16_t); }

// Workspace of df11_gpu_encode_noalloc: one file-scope device array per GPU
// (it lives as long as the process), for callers that cannot allocate.  In
// host code its name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns for the current device, taken once per device.
constexpr uint64_t kScratchBytes = DF11_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The current device's address of `scratch`, or null (the HIP error is then
// recorded).
void *scratch_address() {
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess || dev < 0 || dev >= 64) {
        df11i::last_hip_error = static_cast<int32_t>(err != hipSuccess ? err : hipErrorInvalidDevice);
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !ptr) {
            df11i::last_hip_error = static_cast<int32_t>(err != hipSuccess ? err : hipErrorInvalidSymbol);
            return nullptr;
        }
        addr[dev] = ptr;
    }
    return addr[dev];
}

bool aligned(const void *ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

// hipLaunchKernel reports the status of this launch only (hipGetLastError
// would also return errors left behind by earlier runtime calls).
template <class... A>
hipError_t launch(void (*kernel)(A...), uint32_t grid, uint32_t block, hipStream_t st, A... args) {
    void *argv[] = {static_cast<void *>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3(grid), dim3(block), argv, 0, st);
}

// Compute units of the current device (taken once per device; a failed query
// falls back to 256 and clears only its own error).
uint32_t cu_count() {
    static std::mutex mu;
    static uint32_t cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        dev = 0;
    }
    std::lock_guard<std::mutex> lk(mu);
    if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
        (void)hipGetLastError();
        cus = 256;
    }
    if (dev >= 0 && dev < 64) cached[dev] = static_cast<uint32_t>(cus);
    return static_cast<uint32_t>(cus);
}

// Workgroups for the persistent pack pass: as many as can be resident on
// the device (taken once per device; a failed query falls back to a fixed
// count and clears only its own error).
uint32_t run_groups() {
    const uint32_t cus = cu_count();
    static std::mutex mu;
    static uint32_t cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        dev = 0;
    }
    std::lock_guard<std::mutex> lk(mu);
    if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&run_pack_kernel<false>),
                                                     static_cast<int>(kRunThreads), 0) != hipSuccess ||
        per_cu < 1) {
        (void)hipGetLastError();
        per_cu = 6;
    }
    const uint32_t g = cus * static_cast<uint32_t>(per_cu);
    if (dev >= 0 && dev < 64) cached[dev] = g;
    return g;
}

uint32_t grid_for(uint64_t items, uint32_t cap) {
    const uint64_t g = (items + kThreads - 1) / kThreads;
    return static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>(g, cap)));
}

}  // namespace

extern "C" uint64_t df11_gpu_chunk_hist_bytes(uint64_t n) { return chunk_hist_bytes(n); }

extern "C" df11_status df11_gpu_histogram(const uint16_t *x, uint64_t n, uint64_t *hist, uint16_t *chunk_hist,
                                          void *hip_stream) {
    if (!hist || (n && !x) || !aligned(x, 16) || !aligned(hist, 8) || !aligned(chunk_hist, 16))
        return DF11_E_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    hipError_t err = launch(hist_zero, 1, 256, st, hist);
    const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
    if (err == hipSuccess && n)
        err = launch(hist_kernel,
                     static_cast<uint32_t>(std::min<uint64_t>((n_chunks + kHistWaves - 1) / kHistWaves,
                                                              uint64_t{kHistGroupsPerCU} * cu_count())),
                     kHistThreads, st, x, n,
                     hist, chunk_hist);
    if (err != hipSuccess) {
        df11i::last_hip_error = static_cast<int32_t>(err);
        return DF11_E_HIP;
    }
    return DF11_OK;
}

namespace {

df11_status plan_build(const uint64_t hist[256], uint32_t flags, df11_gpu_plan *plan) {
    if (!hist || !plan || (flags & ~DF11_ENCODE_WINDOW_COUNTS)) return DF11_E_INVALID_ARG;
    df11_gpu_plan q{};
    uint64_t n = 0;
    for (int e = 0; e < 256; ++e) {
        // a histogram of more weights than any block holds: refused before the
        // sums below can wrap around
        if (hist[e] > kMaxWeights || n + hist[e] > kMaxWeights) return DF11_E_INVALID_ARG;
        n += hist[e];
    }
    if (df11i::code_lengths_for(hist, q.code_len, &q.max_code_len, &q.n_symbols, &q.total_bits) != DF11_OK)
        return DF11_E_FORMAT;
    if (df11i::build_tables(q.code_len, nullptr, 0, &q.n_tables) != DF11_OK) return DF11_E_FORMAT;
    q.flags = flags;
    q.n_total = n;
    q.n_windows = (q.total_bits + 63) / 64;
    q.n_units = (q.n_windows + 63) / 64;
    q.stream_bytes = 512 * q.n_units + 16;
    q.sign_mant_bytes = (n + 15) / 16 * 16;
    q.gaps_bytes = 40 * q.n_units + 8;
    q.unit_pos_bytes = 8 * (q.n_units + 1);
    q.counts_bytes = (flags & DF11_ENCODE_WINDOW_COUNTS) ? 64 * q.n_units : 0;
    q.tables_bytes = df11i::tables_bytes_for(q.n_tables);
    q.workspace_bytes = workspace_layout(n, q.n_windows, (flags & DF11_ENCODE_WINDOW_COUNTS) != 0).bytes;
    *plan = q;
    return DF11_OK;
}

df11_status gpu_encode(const df11_gpu_plan *plan, const uint16_t *x, const uint16_t *chunk_hist, uint8_t *stream,
                       uint8_t *sign_mant, uint8_t *gaps, uint64_t *unit_pos, uint8_t *counts, void *workspace,
                       void *hip_stream) {
    if (!plan || !stream || !sign_mant || !gaps || !unit_pos || !workspace) return DF11_E_INVALID_ARG;
    const bool with_counts = (plan->flags & DF11_ENCODE_WINDOW_COUNTS) != 0;
    if (with_counts != (counts != nullptr) || (plan->n_total && (!x || !chunk_hist))) return DF11_E_INVALID_ARG;
    if (plan->n_total > kMaxWeights) return DF11_E_INVALID_ARG;  // no size below can then wrap around
    if (!aligned(x, 16) || !aligned(chunk_hist, 16) || !aligned(stream, 16) || !aligned(sign_mant, 16) ||
        !aligned(unit_pos, 8) || !aligned(workspace, 16))
        return DF11_E_INVALID_ARG;
    // the plan must be self-consistent (sizes follow from n_total and total_bits)
    const uint64_t nw = (plan->total_bits + 63) / 64, nu = (nw + 63) / 64;
    if (plan->n_windows != nw || plan->n_units != nu || plan->stream_bytes != 512 * nu + 16 ||
        plan->gaps_bytes != 40 * nu + 8 || plan->sign_mant_bytes != (plan->n_total + 15) / 16 * 16 ||
        plan->counts_bytes != (with_counts ? 64 * nu : 0) ||
        plan->total_bits > uint64_t{DF11_MAX_CODE_LEN} * plan->n_total)
        return DF11_E_INVALID_ARG;
    uint32_t code32[256];
    if (!df11i::canonical_codes(plan->code_len, code32)) return DF11_E_FORMAT;

    const Workspace ws = workspace_layout(plan->n_total, nw, with_counts);
    uint8_t *wsb = static_cast<uint8_t *>(workspace);
    EncParams p;
    std::memset(&p, 0, sizeof(p));
    p.x = x;
    p.chunk_hist = chunk_hist;
    p.stream = stream;
    p.sm = sign_mant;
    p.gaps = gaps;
    p.counts = counts;
    p.unit_pos = unit_pos;
    p.chunk_pre = reinterpret_cast<uint32_t *>(wsb + ws.pre);
    p.seg_sum = reinterpret_cast<uint64_t *>(wsb + ws.seg_sum);
    p.seg_off = reinterpret_cast<uint64_t *>(wsb + ws.seg_off);
    p.gap8 = wsb + ws.gap8;
    p.wfirst = with_counts ? reinterpret_cast<uint64_t *>(wsb + ws.wfirst) : nullptr;
    p.n = plan->n_total;
    p.total_bits = plan->total_bits;
    p.n_windows = nw;
    p.n_units = nu;
    p.n_chunks = (plan->n_total + kChunk - 1) / kChunk;
    p.n_segs = (p.n_chunks + kSegChunks - 1) / kSegChunks;
    p.stream_bytes = plan->stream_bytes;
    p.sm_bytes = plan->sign_mant_bytes;
    p.gaps_bytes = plan->gaps_bytes;
    p.counts_bytes = plan->counts_bytes;
    for (int e = 0; e < 256; ++e) {
        p.code[e] = code32[e];
        p.len[e] = plan->code_len[e];
    }
    if (p.n_chunks > 0xFFFFFFFFull) return DF11_E_UNSUPPORTED;  // one workgroup per chunk

    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const uint32_t chunks = static_cast<uint32_t>(p.n_chunks);
    hipError_t err = hipSuccess;
    if (chunks) err = launch(bits_kernel, static_cast<uint32_t>(p.n_segs), kBitsThreads, st, p);
    if (err == hipSuccess && chunks) err = launch(top_kernel, 1, kScanThreads, st, p);
    if (err == hipSuccess) err = launch(bounds_kernel, grid_for(p.n_chunks, 1u << 20), kThreads, st, p);
    if (err == hipSuccess && chunks) {
        // a few workgroups per resident slot: enough to fill the GPU, each
        // taking many chunks so that the next chunk's loads overlap the current
        const uint32_t groups =
            static_cast<uint32_t>(std::min<uint64_t>((chunks + kRunWaves - 1) / kRunWaves, run_groups()));
        err = with_counts ? launch(run_pack_kernel<true>, groups, kRunThreads, st, p)
                          : launch(run_pack_kernel<false>, groups, kRunThreads, st, p);
    }
    if (err == hipSuccess && nw)
        err = launch(finish_kernel, grid_for(with_counts ? nw : nw / 32 + 1, 4096), kThreads, st, p);
    if (err != hipSuccess) {
        df11i::last_hip_error = static_cast<int32_t>(err);
        return DF11_E_HIP;
    }
    return DF11_OK;
}

}  // namespace

extern "C" df11_status df11_gpu_plan_build(const uint64_t hist[256], uint32_t flags, df11_gpu_plan *plan) {
    return df11i::guarded([&] { return plan_build(hist, flags, plan); });
}

extern "C" df11_status df11_gpu_encode_noalloc(const df11_gpu_plan *plan, const uint16_t *x,
                                               const uint16_t *chunk_hist, uint8_t *stream, uint8_t *sign_mant,
                                               uint8_t *gaps, uint64_t *unit_pos, uint8_t *counts,
                                               void *hip_stream) {
    return df11i::guarded([&]() -> df11_status {
        if (!plan) return DF11_E_INVALID_ARG;
        if (plan->n_total > kMaxWeights || plan->total_bits > uint64_t{DF11_MAX_CODE_LEN} * plan->n_total)
            return DF11_E_INVALID_ARG;
        // the workspace this plan needs, from its own sizes (not from its
        // workspace_bytes field), against the array's size
        const bool with_counts = (plan->flags & DF11_ENCODE_WINDOW_COUNTS) != 0;
        const uint64_t nw = (plan->total_bits + 63) / 64;
        if (workspace_layout(plan->n_total, nw, with_counts).bytes > kScratchBytes) return DF11_E_BUFFER_TOO_SMALL;
        void *ws = scratch_address();
        if (!ws) return DF11_E_HIP;
        return gpu_encode(plan, x, chunk_hist, stream, sign_mant, gaps, unit_pos, counts, ws, hip_stream);
    });
}

extern "C" df11_status df11_gpu_encode(const df11_gpu_plan *plan, const uint16_t *x, const uint16_t *chunk_hist,
                                       uint8_t *stream, uint8_t *sign_mant, uint8_t *gaps, uint64_t *unit_pos,
                                       uint8_t *counts, void *workspace, void *hip_stream) {
    return df11i::guarded([&] {
        return gpu_encode(plan, x, chunk_hist, stream, sign_mant, gaps, unit_pos, counts, workspace, hip_stream);
    });
}
