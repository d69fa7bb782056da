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
//   fill    defaults: zeroed stream, gaps, counts and padding; unit_pos and
//           the first-start records preset for units/windows where no code
//           starts (only possible at the end of the stream)
//   bits    bits per chunk from its counts and the code lengths (the weights
//           are not read again), and their exclusive prefix within each
//           segment of 256 chunks
//   top     exclusive prefix of the segment totals (one workgroup)
//   pack    persistent, per chunk: each weight's bit offset (block scan),
//           its sign/mantissa byte, its code and its start ORed into an LDS
//           bit buffer and an LDS start bitmap; the buffer is written out
//           (global atomic OR only on the two words shared with the
//           neighbouring chunks) and the bitmap gives the first code start of
//           every window (gap) and unit (position) in the chunk
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
constexpr uint32_t kPackThreads = 512;                // pack: threads per workgroup
constexpr uint32_t kPackPer = kChunk / kPackThreads;  // pack: weights per thread (8)
constexpr uint32_t kScanThreads = 1024;

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

constexpr uint32_t kHistCopies = 16;  // sub-histograms per workgroup, one per lane & 15
constexpr uint32_t kHistStride = 257; // padded rows: copies of one exponent fall in different banks

// Thread t's 16 weights of chunk c as two 16-byte loads (zeros past the
// block's end, through a buffer range that stops there).
__device__ __forceinline__ void hist_load(const uint16_t *x, uint64_t n, uint64_t c, uint32_t t, df11w::v4u &a,
                                          df11w::v4u &b) {
    const uint64_t first = c * kChunk;
    const uint64_t left = first < n ? n - first : 0;
    const df11w::Rsrc r = df11w::rsrc(x + (first < n ? first : 0), static_cast<uint32_t>(2 * (left < kChunk ? left : kChunk)));
    a = __builtin_amdgcn_raw_buffer_load_b128(r, 32 * t, 0, 0);
    b = __builtin_amdgcn_raw_buffer_load_b128(r, 32 * t + 16, 0, 0);
}

__global__ void __launch_bounds__(kThreads) hist_kernel(const uint16_t *x, uint64_t n, uint64_t *hist,
                                                        uint16_t *chunk_hist) {
    // A block's values cluster on a few exponents: same-address LDS atomics
    // are serialised, so lanes spread over 16 copies of the histogram.
    // Thread t owns exponent t: after each chunk it adds up and clears the
    // copies of its bin, records the chunk's count and keeps a running total.
    // Each chunk's weights are requested a chunk ahead; the barriers order LDS
    // only, so the chunk's count store is not waited for.
    __shared__ uint32_t h[kHistCopies * kHistStride];
    const uint32_t t = threadIdx.x;
    uint32_t *mine = h + (t & (kHistCopies - 1)) * kHistStride;
    for (uint32_t i = t; i < kHistCopies * kHistStride; i += blockDim.x) h[i] = 0;
    __syncthreads();
    const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
    uint64_t total = 0;
    uint64_t c = blockIdx.x;
    df11w::v4u a, b;
    hist_load(x, n, c, t, a, b);
    for (; c < n_chunks; c += gridDim.x) {
        df11w::v4u na, nb;
        hist_load(x, n, c + gridDim.x, t, na, nb);
        const uint64_t i0 = c * kChunk + uint64_t{t} * kPerThread;
        if (i0 + kPerThread <= n) {
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                atomicAdd(&mine[exponent_of(w[k])], 1u);
                atomicAdd(&mine[exponent_of(w[k] >> 16)], 1u);
            }
        } else {
            for (uint64_t i = i0; i < n && i < i0 + kPerThread; ++i) atomicAdd(&mine[exponent_of(x[i])], 1u);
        }
        lds_barrier();
        uint32_t cnt = 0;
#pragma unroll
        for (uint32_t k = 0; k < kHistCopies; ++k) {
            cnt += h[k * kHistStride + t];
            h[k * kHistStride + t] = 0;
        }
        if (chunk_hist) chunk_hist[c * 256 + t] = static_cast<uint16_t>(cnt);  // at most 4,096
        total += cnt;
        lds_barrier();
        a = na;
        b = nb;
    }
    if (total) atomicAdd(reinterpret_cast<unsigned long long *>(hist + t), static_cast<unsigned long long>(total));
}

// ---------------------------------------------------------------- fill
__global__ void __launch_bounds__(kThreads) fill_kernel(EncParams p) {
    const uint64_t tid = uint64_t{blockIdx.x} * blockDim.x + threadIdx.x;
    const uint64_t step = uint64_t{gridDim.x} * blockDim.x;
    for (uint64_t i = tid; i < p.stream_bytes / 16; i += step)
        reinterpret_cast<uint4 *>(p.stream)[i] = make_uint4(0u, 0u, 0u, 0u);
    for (uint64_t i = tid; i < p.gaps_bytes; i += step) p.gaps[i] = 0;
    for (uint64_t i = tid; i <= p.n_units; i += step) p.unit_pos[i] = p.n;
    for (uint64_t i = p.n + tid; i < p.sm_bytes; i += step) p.sm[i] = 0;
    if (p.counts)
        for (uint64_t i = tid; i < p.counts_bytes; i += step) p.counts[i] = 0;
    if (tid == 0 && p.n_windows) {
        // the last window may hold no code start: its gap ends at total_bits
        p.gap8[p.n_windows - 1] = static_cast<uint8_t>(p.total_bits - 64 * (p.n_windows - 1));
        if (p.counts) {
            p.wfirst[p.n_windows - 1] = p.n;
            p.wfirst[p.n_windows] = p.n;
        }
    }
}

// Weights of pack thread t of chunk c, eight as four packed words (two
// weights each, the first in the low half).  load_full requests them for a
// whole chunk (a chunk that is not whole reads as zeros, through a buffer
// range of 0 bytes) and does not use them, so that the loads stay in flight;
// load_partial reads the block's last, partial chunk element by element.
__device__ __forceinline__ bool chunk_is_full(const EncParams &p, uint64_t c) { return (c + 1) * kChunk <= p.n; }

__device__ __forceinline__ void load_full(const EncParams &p, uint64_t c, uint32_t t, uint32_t w[4]) {
    const bool full = chunk_is_full(p, c);
    const df11w::Rsrc r = df11w::rsrc(p.x + (full ? c * kChunk : 0), full ? 2 * kChunk : 0u);
    const df11w::v4u a = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * t, 0, 0);
    w[0] = a.x, w[1] = a.y, w[2] = a.z, w[3] = a.w;
}

__device__ __forceinline__ void load_partial(const EncParams &p, uint64_t c, uint32_t t, uint32_t m,
                                             uint32_t w[4]) {
    const uint64_t i0 = c * kChunk + uint64_t{t} * kPackPer;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        const uint32_t lo = 2 * k < m ? p.x[i0 + 2 * k] : 0u;
        const uint32_t hi = 2 * k + 1 < m ? p.x[i0 + 2 * k + 1] : 0u;
        w[k] = lo | (hi << 16);
    }
}

// Weights of chunk c that pack thread t takes (0..8).
__device__ __forceinline__ uint32_t weights_of(const EncParams &p, uint64_t c, uint32_t t) {
    const uint64_t i0 = c * kChunk + uint64_t{t} * kPackPer;
    return i0 >= p.n ? 0u : static_cast<uint32_t>(p.n - i0 < kPackPer ? p.n - i0 : kPackPer);
}

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
__global__ void __launch_bounds__(kThreads) bits_kernel(EncParams p) {
    __shared__ uint32_t len[256];
    __shared__ uint32_t wsum[kThreads / 64];
    const uint32_t t = threadIdx.x;
    len[t] = p.len[t];
    __syncthreads();
    const uint64_t c = uint64_t{blockIdx.x} * kSegChunks + t;
    uint32_t bits = 0;
    if (c < p.n_chunks) {
        const uint4 *h = reinterpret_cast<const uint4 *>(p.chunk_hist + c * 256);
#pragma unroll 8
        for (uint32_t j = 0; j < 32; ++j) {  // exponents 8j .. 8j + 7
            const uint4 v = h[j];
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k)
                bits += (q[k] & 0xFFFFu) * len[8 * j + 2 * k] + (q[k] >> 16) * len[8 * j + 2 * k + 1];
        }
    }
    uint32_t seg_bits;
    const uint32_t pre = block_exclusive_sum<kThreads / 64>(bits, wsum, seg_bits);
    if (c < p.n_chunks) p.chunk_pre[c] = pre;
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

// ---------------------------------------------------------------- pack
// Persistent: each workgroup takes chunks c, c + grid, ... and requests the
// next chunk's weights before packing the current one.  Per chunk, thread t
// takes weights 8t .. 8t + 7: their codes form one run of bits that starts
// at the chunk's offset plus the block prefix of the threads' run lengths.
//
// LDS frame: bit positions count from the start of the 64-bit window that
// holds the chunk's first code, so a 32-bit word index serves the code
// buffer and the code-start bitmap alike, and windows are word pairs.
//
// First-start records come from the bitmap: a window's gap is the position of
// its first set bit, the first weight of the window is the chunk's first
// weight plus the starts before it (prefix of popcounts), and a window that
// opens a unit (64 windows) gives that unit's position.  A window belongs to
// the chunk that holds its first start: the chunk's first window is left to
// the previous chunk when that one's last code starts in it.
// 32-bit words of a chunk's frame: at most 63 + 32 x 4,096 bits, the word after
// the last one a code reaches, whole windows; a multiple of 4
constexpr uint32_t kFrameWords = kChunk + 4;
constexpr uint32_t kWinPerThread = (kFrameWords / 2 + kPackThreads - 1) / kPackThreads;

__device__ __forceinline__ uint32_t clz64(uint64_t v) { return v ? static_cast<uint32_t>(__clzll(v)) : 64u; }

// What the loop requests for the next chunk while packing the current one.
// The loaded values are not combined here: any use makes the wave wait.
// The per-chunk values are the same for every lane but go through vector
// loads: a scalar load shares its wait counter with the LDS operations, so
// the chunk's first LDS wait would also wait for the next chunk's values.
struct ChunkInputs {
    uint32_t w[4];            // the thread's eight weights, packed
    uint32_t seg_lo, seg_hi;  // the chunk's first bit is seg_off + pre
    uint32_t pre;
    uint32_t xw;              // high half: the previous chunk's last weight (chunk 0: not used)
};

__device__ __forceinline__ void load_inputs(const EncParams &p, uint64_t c, uint32_t t, ChunkInputs &in) {
    const uint64_t cc = c < p.n_chunks ? c : 0;  // past the end: chunk 0 again, not used
    const df11w::v2u so = __builtin_amdgcn_raw_buffer_load_b64(df11w::rsrc(p.seg_off + cc / kSegChunks, 8), 0, 0, 0);
    in.seg_lo = so.x;
    in.seg_hi = so.y;
    in.pre = __builtin_amdgcn_raw_buffer_load_b32(df11w::rsrc(p.chunk_pre + cc, 4), 0, 0, 0);
    // the 4-byte word whose high half is the previous chunk's last weight
    // (chunk 0: any readable word, not used)
    const uint32_t *wl = cc ? reinterpret_cast<const uint32_t *>(p.x + cc * kChunk - 2) : p.chunk_pre;
    in.xw = __builtin_amdgcn_raw_buffer_load_b32(df11w::rsrc(wl, 4), 0, 0, 0);
    load_full(p, c, t, in.w);
}

// Packs chunk c.  Its stores of the code words and window records come after
// `next` is taken (its loads were requested before this chunk's work, so
// they have arrived): vmcnt counts loads and stores in issue order, and a wait
// for the next chunk's loads after these stores would also wait for them.
template <bool kWhole>
__device__ __forceinline__ void pack_chunk(const EncParams &p, uint64_t c, const ChunkInputs &in,
                                           const ChunkInputs &next, const uint2 *ent, uint32_t *bits,
                                           uint32_t *starts, uint32_t *wsum, uint32_t *wsum2) {
    const uint32_t t = threadIdx.x;
    const uint64_t i0 = c * kChunk + uint64_t{t} * kPackPer;
    const uint32_t m = kWhole ? kPackPer : weights_of(p, c, t);
    const uint32_t *wc = in.w;
    // readfirstlane returns a signed int: each half is taken as uint32_t before
    // it is widened (a sign-extended low half would corrupt offsets past 2^31 bits)
    const uint32_t seg_lo = __builtin_amdgcn_readfirstlane(in.seg_lo);
    const uint32_t seg_hi = __builtin_amdgcn_readfirstlane(in.seg_hi);
    const uint32_t chunk_pre = __builtin_amdgcn_readfirstlane(in.pre);
    const uint64_t cb = ((static_cast<uint64_t>(seg_hi) << 32) | seg_lo) + chunk_pre;
    const uint32_t len_last = ent[exponent_of(in.xw >> 16)].y;

    // sign/mantissa bytes, (sign << 7) | mantissa, two weights per word
    uint32_t smw[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t a = wc[2 * k], b = wc[2 * k + 1];
        const uint32_t sa = ((a >> 8) & 0x00800080u) | (a & 0x007F007Fu);  // two sm bytes in 16-bit halves
        const uint32_t sb = ((b >> 8) & 0x00800080u) | (b & 0x007F007Fu);
        smw[k] = __builtin_amdgcn_perm(sb, sa, 0x06040200u);
    }
    if (kWhole || m == kPackPer) {
        reinterpret_cast<uint2 *>(p.sm + i0)[0] = make_uint2(smw[0], smw[1]);
    } else {
        for (uint32_t k = 0; k < m; ++k) p.sm[i0 + k] = static_cast<uint8_t>(smw[k / 4] >> (8 * (k & 3)));
    }

    // codes and lengths of the thread's weights (length 0 past the end)
    uint32_t code[kPackPer], len[kPackPer];
    uint32_t sum = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPackPer; ++k) {
        const uint2 e = ent[exponent_of(wc[k / 2] >> (16 * (k & 1)))];
        code[k] = (kWhole || k < m) ? e.x : 0u;
        len[k] = (kWhole || k < m) ? e.y : 0u;
        sum += len[k];
    }

    // this thread's first bit in the frame
    uint32_t chunk_bits;
    const uint32_t pre = block_exclusive_sum<kPackThreads / 64>(sum, wsum, chunk_bits);
    const uint32_t head = static_cast<uint32_t>(cb & 63u);

    // Each code is ORed into the code buffer at its own position (one 64-bit
    // shift, two 32-bit ORs: the word it starts in and the next) and its
    // start into the bitmap, so that no thread waits on another's words.
    uint32_t pos = head + pre;
#pragma unroll
    for (uint32_t k = 0; k < kPackPer; ++k) {
        const uint32_t l = len[k];
        const uint32_t wi = pos >> 5, sh = pos & 31u;
        const uint64_t v = static_cast<uint64_t>(code[k]) << ((64u - sh - l) & 63u);
        atomicOr(&bits[wi], static_cast<uint32_t>(v >> 32));
        atomicOr(&bits[wi + 1], static_cast<uint32_t>(v));
        if (kWhole || k < m) atomicOr(&starts[wi], 0x80000000u >> sh);
        pos += l;
    }
    lds_barrier();
    asm volatile("" ::"v"(next.w[0]), "v"(next.w[1]), "v"(next.w[2]), "v"(next.w[3]), "v"(next.seg_lo),
                 "v"(next.seg_hi), "v"(next.pre), "v"(next.xw));

    // out to HBM as big-endian words, clearing the buffer for the next chunk;
    // the first and last words are shared with the neighbouring chunks when
    // the chunk does not start or end on a word boundary
    const uint32_t k0 = head >> 5;
    const uint32_t nwords = (head + chunk_bits + 31u) >> 5;
    const bool head_shared = (cb & 31u) != 0;
    const bool tail_shared = ((cb + chunk_bits) & 31u) != 0;
    uint32_t *out = reinterpret_cast<uint32_t *>(p.stream) + 2 * (cb >> 6);
    const uint64_t room = p.stream_bytes / 4 > 2 * (cb >> 6) ? p.stream_bytes / 4 - 2 * (cb >> 6) : 0;
    for (uint32_t k = k0 + t; k < nwords; k += kPackThreads) {
        const uint32_t v = __builtin_bswap32(bits[k]);
        bits[k] = 0;
        if (k >= room) continue;
        if ((k == k0 && head_shared) || (k == nwords - 1 && tail_shared))
            atomicOr(out + k, v);
        else
            out[k] = v;
    }

    // window records: thread t takes windows t*q .. t*q + q - 1 of the
    // chunk's nwin, counts the starts in each, and the block scan of the
    // counts gives every window the starts before it
    const uint64_t wbase = cb >> 6;
    const uint32_t nwin = (head + chunk_bits + 63u) >> 6;
    const uint32_t q = (nwin + kPackThreads - 1) / kPackThreads;
    const uint32_t jb = t * q;
    uint64_t wv[kWinPerThread];
    uint32_t cnt = 0;
#pragma unroll
    for (uint32_t i = 0; i < kWinPerThread; ++i) {
        const uint32_t j = jb + i;
        wv[i] = 0;
        if (i < q && j < nwin) {
            wv[i] = (static_cast<uint64_t>(starts[2 * j]) << 32) | starts[2 * j + 1];
            starts[2 * j] = 0;
            starts[2 * j + 1] = 0;
            cnt += static_cast<uint32_t>(__popcll(wv[i]));
        }
    }
    uint32_t total;
    uint32_t before = block_exclusive_sum<kPackThreads / 64>(cnt, wsum2, total);
    const bool prev_has_start = c > 0 && head >= len_last;  // the previous chunk's last code starts in window 0
#pragma unroll
    for (uint32_t i = 0; i < kWinPerThread; ++i) {
        const uint32_t j = jb + i;
        const uint64_t w = wbase + j;
        if (wv[i] && (j > 0 || !prev_has_start) && w < p.n_windows) {
            const uint64_t first = c * kChunk + before;  // the window's first weight
            p.gap8[w] = static_cast<uint8_t>(clz64(wv[i]));
            if (p.wfirst) p.wfirst[w] = first;
            if ((w & 63u) == 0) p.unit_pos[w >> 6] = first;
        }
        before += static_cast<uint32_t>(__popcll(wv[i]));
    }
}

__global__ void __launch_bounds__(kPackThreads) pack_kernel(EncParams p) {
    __shared__ uint2 ent[256];  // per exponent: code, length
    __shared__ __align__(16) uint32_t bits[kFrameWords];
    __shared__ __align__(16) uint32_t starts[kFrameWords];
    __shared__ uint32_t wsum[kPackThreads / 64], wsum2[kPackThreads / 64];
    const uint32_t t = threadIdx.x;
    uint64_t c = blockIdx.x;
    if (c >= p.n_chunks) return;  // uniform
    if (t < 256) ent[t] = make_uint2(p.code[t], p.len[t]);
    for (uint32_t k = t; k < kFrameWords / 4; k += blockDim.x) {
        reinterpret_cast<uint4 *>(bits)[k] = make_uint4(0u, 0u, 0u, 0u);
        reinterpret_cast<uint4 *>(starts)[k] = make_uint4(0u, 0u, 0u, 0u);
    }
    ChunkInputs cur;
    load_inputs(p, c, t, cur);
    // the first chunk's inputs before the loop: its head then sees them
    // complete, with no wait that would also drain the stores
    asm volatile("" ::"v"(cur.w[0]), "v"(cur.w[1]), "v"(cur.w[2]), "v"(cur.w[3]), "v"(cur.seg_lo),
                 "v"(cur.seg_hi), "v"(cur.pre), "v"(cur.xw));
    lds_barrier();

    while (true) {
        // the next chunk's inputs, requested a whole chunk ahead
        const uint64_t cn = c + gridDim.x;
        ChunkInputs nxt;
        load_inputs(p, cn, t, nxt);
        if (chunk_is_full(p, c)) {  // uniform
            pack_chunk<true>(p, c, cur, nxt, ent, bits, starts, wsum, wsum2);
        } else {  // the block's last chunk
            load_partial(p, c, t, weights_of(p, c, t), cur.w);
            pack_chunk<false>(p, c, cur, nxt, ent, bits, starts, wsum, wsum2);
        }
        if (cn >= p.n_chunks) break;  // uniform
        c = cn;
        cur = nxt;  // arrived: taken before this chunk's stores
    }
}

// ---------------------------------------------------------------- finish
__global__ void __launch_bounds__(kThreads) finish_kernel(EncParams p) {
    const uint64_t tid = uint64_t{blockIdx.x} * blockDim.x + threadIdx.x;
    const uint64_t step = uint64_t{gridDim.x} * blockDim.x;
    const uint64_t groups = (p.n_windows + 7) / 8;
    for (uint64_t g = tid; g < groups; g += step) {
        uint64_t v = 0;
        for (uint32_t j = 0; j < 8; ++j) {
            const uint64_t w = 8 * g + j;
            v = (v << 5) | (w < p.n_windows ? (p.gap8[w] & 31u) : 0u);
        }
        for (uint32_t k = 0; k < 5; ++k) p.gaps[5 * g + k] = static_cast<uint8_t>(v >> (32 - 8 * k));
    }
    if (p.counts)
        for (uint64_t w = tid; w < p.n_windows; w += step)
            p.counts[w] = static_cast<uint8_t>(p.wfirst[w + 1] - p.wfirst[w]);
}

thread_local int32_t g_last_hip_error = 0;

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

bool aligned(const void *ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

// hipLaunchKernel reports the status of this launch only (hipGetLastError
// would also return errors left behind by earlier runtime calls).
template <class... A>
hipError_t launch(void (*kernel)(A...), uint32_t grid, uint32_t block, hipStream_t st, A... args) {
    void *argv[] = {static_cast<void *>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3(grid), dim3(block), argv, 0, st);
}

// Workgroups for the persistent pack pass: as many as can be resident on
// the device (taken once per device; a failed query falls back to a fixed
// count and clears only its own error).
uint32_t pack_groups() {
    static std::mutex mu;
    static uint32_t cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        dev = 0;
    }
    std::lock_guard<std::mutex> lk(mu);
    if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
        (void)hipGetLastError();
        cus = 256;
    }
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&pack_kernel),
                                                     static_cast<int>(kPackThreads), 0) != hipSuccess ||
        per_cu < 1) {
        (void)hipGetLastError();
        per_cu = 4;
    }
    const uint32_t g = static_cast<uint32_t>(cus) * static_cast<uint32_t>(per_cu);
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
        err = launch(hist_kernel, static_cast<uint32_t>(std::min<uint64_t>(n_chunks, 2048)), kThreads, st, x, n,
                     hist, chunk_hist);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int32_t>(err);
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
    hipError_t err = launch(fill_kernel, grid_for(std::max(plan->stream_bytes / 16, nu + 1), 4096), kThreads, st, p);
    if (err == hipSuccess && chunks)
        err = launch(bits_kernel, static_cast<uint32_t>(p.n_segs), kThreads, st, p);
    if (err == hipSuccess && chunks) err = launch(top_kernel, 1, kScanThreads, st, p);
    if (err == hipSuccess && chunks) {
        // a few workgroups per resident slot: enough to fill the GPU, each
        // taking many chunks so that the next chunk's loads overlap the current
        err = launch(pack_kernel, std::min<uint32_t>(chunks, pack_groups()), kPackThreads, st, p);
    }
    if (err == hipSuccess && nw) err = launch(finish_kernel, grid_for(nw / 8 + 1, 4096), kThreads, st, p);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int32_t>(err);
        return DF11_E_HIP;
    }
    return DF11_OK;
}

}  // namespace

extern "C" df11_status df11_gpu_plan_build(const uint64_t hist[256], uint32_t flags, df11_gpu_plan *plan) {
    return df11i::guarded([&] { return plan_build(hist, flags, plan); });
}

extern "C" df11_status df11_gpu_encode(const df11_gpu_plan *plan, const uint16_t *x, const uint16_t *chunk_hist,
                                       uint8_t *stream, uint8_t *sign_mant, uint8_t *gaps, uint64_t *unit_pos,
                                       uint8_t *counts, void *workspace, void *hip_stream) {
    return df11i::guarded([&] {
        return gpu_encode(plan, x, chunk_hist, stream, sign_mant, gaps, unit_pos, counts, workspace, hip_stream);
    });
}
