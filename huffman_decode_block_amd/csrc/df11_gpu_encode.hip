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
//   pack    per chunk: each weight's bit offset (block scan), its
//           sign/mantissa byte, its code ORed into an LDS bit buffer that is
//           then written out (global atomic OR only on the two words shared
//           with the neighbouring chunks), and the first code start of every
//           window (gap) and unit (position) it contains
//   finish  5-bit gap fields (8 windows per 5 bytes) and window counts
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "df11_internal.h"
#include "df11_wave.h"

namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kPerThread = 16;                   // weights per thread in hist/pack
constexpr uint32_t kChunk = kThreads * kPerThread;    // 4,096 weights per chunk
constexpr uint32_t kBitWords = kChunk * 32 / 32 + 2;  // LDS words for a chunk's codes
constexpr uint32_t kSegChunks = kThreads;             // chunks per segment of the two-level scan
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

__global__ void __launch_bounds__(kThreads) hist_kernel(const uint16_t *x, uint64_t n, uint64_t *hist,
                                                        uint16_t *chunk_hist) {
    // A block's values cluster on a few exponents: same-address LDS atomics
    // are serialised, so lanes spread over 16 copies of the histogram.
    // Thread t owns exponent t: after each chunk it adds up and clears the
    // copies of its bin, records the chunk's count and keeps a running total.
    __shared__ uint32_t h[kHistCopies * kHistStride];
    const uint32_t t = threadIdx.x;
    uint32_t *mine = h + (t & (kHistCopies - 1)) * kHistStride;
    for (uint32_t i = t; i < kHistCopies * kHistStride; i += blockDim.x) h[i] = 0;
    __syncthreads();
    const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
    uint64_t total = 0;
    for (uint64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const uint64_t i0 = c * kChunk + uint64_t{t} * kPerThread;
        if (i0 + kPerThread <= n) {
            const uint4 a = reinterpret_cast<const uint4 *>(x + i0)[0];
            const uint4 b = reinterpret_cast<const uint4 *>(x + i0)[1];
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                atomicAdd(&mine[exponent_of(w[k])], 1u);
                atomicAdd(&mine[exponent_of(w[k] >> 16)], 1u);
            }
        } else {
            for (uint64_t i = i0; i < n && i < i0 + kPerThread; ++i) atomicAdd(&mine[exponent_of(x[i])], 1u);
        }
        __syncthreads();
        uint32_t cnt = 0;
#pragma unroll
        for (uint32_t k = 0; k < kHistCopies; ++k) {
            cnt += h[k * kHistStride + t];
            h[k * kHistStride + t] = 0;
        }
        if (chunk_hist) chunk_hist[c * 256 + t] = static_cast<uint16_t>(cnt);  // at most 4,096
        total += cnt;
        __syncthreads();
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

// Weights of thread t of chunk c, sixteen as eight packed words (two weights
// each, the first in the low half).  load_full requests them for a whole
// chunk (a chunk that is not whole reads as zeros, through a buffer range of
// 0 bytes) and does not use them, so that the loads stay in flight;
// load_partial reads the block's last, partial chunk element by element.
__device__ __forceinline__ bool chunk_is_full(const EncParams &p, uint64_t c) { return (c + 1) * kChunk <= p.n; }

__device__ __forceinline__ void load_full(const EncParams &p, uint64_t c, uint32_t t, uint32_t w[8]) {
    const bool full = chunk_is_full(p, c);
    const df11w::Rsrc r = df11w::rsrc(p.x + (full ? c * kChunk : 0), full ? 2 * kChunk : 0u);
    const df11w::v4u a = __builtin_amdgcn_raw_buffer_load_b128(r, 32 * t, 0, 0);
    const df11w::v4u b = __builtin_amdgcn_raw_buffer_load_b128(r, 32 * t + 16, 0, 0);
    w[0] = a.x, w[1] = a.y, w[2] = a.z, w[3] = a.w, w[4] = b.x, w[5] = b.y, w[6] = b.z, w[7] = b.w;
}

__device__ __forceinline__ void load_partial(const EncParams &p, uint64_t c, uint32_t t, uint32_t m,
                                             uint32_t w[8]) {
    const uint64_t i0 = c * kChunk + uint64_t{t} * kPerThread;
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
        const uint32_t lo = 2 * k < m ? p.x[i0 + 2 * k] : 0u;
        const uint32_t hi = 2 * k + 1 < m ? p.x[i0 + 2 * k + 1] : 0u;
        w[k] = lo | (hi << 16);
    }
}

// Weights of chunk c that thread t takes (0..16).
__device__ __forceinline__ uint32_t weights_of(const EncParams &p, uint64_t c, uint32_t t) {
    const uint64_t i0 = c * kChunk + uint64_t{t} * kPerThread;
    return i0 >= p.n ? 0u : static_cast<uint32_t>(p.n - i0 < kPerThread ? p.n - i0 : kPerThread);
}

// Block-wide exclusive sum of one value per thread (256 threads = 4 waves):
// a scan inside each wave, then each wave adds the totals of the waves before
// it; also the block total.  `wsum` holds 4 values.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t *wsum, uint32_t &total) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t incl = df11w::wave_inclusive_scan(v);
    if (lane == 63) wsum[wave] = incl;
    lds_barrier();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (uint32_t k = 0; k < kThreads / 64; ++k) {
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
    const uint32_t pre = block_exclusive_sum(bits, wsum, seg_bits);
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
// takes weights 16t .. 16t + 15: their codes form one run of bits that starts
// at the chunk's offset plus the block prefix of the threads' run lengths.
//
// First-start records (the gap of every window, the first weight of every
// unit, and with window counts the first weight of every window): a code is
// the first to start in its window when the code before it started in an
// earlier window.  Each thread decides this for its codes 1..15 and, at the
// end of its run, for the code that follows it (the next thread's or next
// chunk's first), which it knows to start where its own run ends; the
// block's very first code is the first of window 0 and unit 0.
constexpr uint32_t kChunkWindows = kChunk * 32 / 64 + 2;  // windows a chunk's records can fall in
constexpr uint8_t kNoStart = 0xFF;                          // a window without a record here

__global__ void __launch_bounds__(kThreads) pack_kernel(EncParams p) {
    __shared__ uint2 ent[256];  // per exponent: code, length
    __shared__ __align__(16) uint32_t bits[kBitWords + 2];
    __shared__ uint32_t wsum[kThreads / 64];
    // window records of the chunk, from its first code's window on: the gap,
    // and the first weight's offset from the chunk's first weight
    __shared__ uint8_t gap_l[kChunkWindows];
    __shared__ uint16_t wfirst_l[kChunkWindows];
    const uint32_t t = threadIdx.x;
    uint64_t c = blockIdx.x;
    if (c >= p.n_chunks) return;  // uniform
    ent[t] = make_uint2(p.code[t], p.len[t]);
    for (uint32_t k = t; k < (kBitWords + 2) / 4; k += blockDim.x)
        reinterpret_cast<uint4 *>(bits)[k] = make_uint4(0u, 0u, 0u, 0u);
    for (uint32_t k = t; k < kChunkWindows; k += blockDim.x) gap_l[k] = kNoStart;
    uint32_t wc[8];
    load_full(p, c, t, wc);
    lds_barrier();
    if (c == 0 && t == 0) {  // the block's first code starts at bit 0
        p.gap8[0] = 0;
        if (p.wfirst) p.wfirst[0] = 0;
        p.unit_pos[0] = 0;
    }

    while (true) {
        const uint64_t cb = p.seg_off[c / kSegChunks] + p.chunk_pre[c];
        // the next chunk's weights, requested a whole chunk ahead
        const uint64_t cn = c + gridDim.x;
        uint32_t wn[8];
        load_full(p, cn, t, wn);
        const uint64_t i0 = c * kChunk + uint64_t{t} * kPerThread;
        const uint32_t m = weights_of(p, c, t);
        if (!chunk_is_full(p, c)) load_partial(p, c, t, m, wc);  // the block's last chunk (uniform)

        // sign/mantissa bytes, (sign << 7) | mantissa, two weights per word
        if (m == kPerThread) {
            uint32_t v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t a = wc[2 * k], b = wc[2 * k + 1];
                const uint32_t sa = ((a >> 8) & 0x00800080u) | (a & 0x007F007Fu);  // two sm bytes in 16-bit halves
                const uint32_t sb = ((b >> 8) & 0x00800080u) | (b & 0x007F007Fu);
                v[k] = __builtin_amdgcn_perm(sb, sa, 0x06040200u);
            }
            reinterpret_cast<uint4 *>(p.sm + i0)[0] = make_uint4(v[0], v[1], v[2], v[3]);
        } else {
            for (uint32_t k = 0; k < m; ++k) {
                const uint32_t x = (wc[k / 2] >> (16 * (k & 1))) & 0xFFFFu;
                p.sm[i0 + k] = static_cast<uint8_t>(((x >> 8) & 0x80u) | (x & 0x7Fu));
            }
        }

        // codes and lengths of the thread's weights (length 0 past the end)
        uint32_t code[kPerThread], len[kPerThread];
        uint32_t sum = 0;
#pragma unroll
        for (uint32_t k = 0; k < kPerThread; ++k) {
            const uint2 e = ent[exponent_of(wc[k / 2] >> (16 * (k & 1)))];
            code[k] = k < m ? e.x : 0u;
            len[k] = k < m ? e.y : 0u;
            sum += len[k];
        }

        // this thread's first bit: chunk offset + block prefix of the run lengths
        uint32_t chunk_bits;
        const uint32_t pre = block_exclusive_sum(sum, wsum, chunk_bits);
        const uint64_t b0 = cb + pre;
        const uint32_t lb = static_cast<uint32_t>(cb & 31u) + pre;  // bit index in the LDS buffer

        // Each code is ORed into the LDS bit buffer at its own position (one
        // 64-bit shift, two 32-bit ORs: the word it starts in and the next),
        // so that no thread waits on another's words and no branch is taken
        // per code.  Lengths past the block's end are 0, their codes 0.
        //
        // First-start rules in 32-bit arithmetic: a code's start is kept as
        // b0's offset in its window plus 64 plus the lengths before it (at
        // most 512 bits on): the window index changes exactly when the bits
        // from 6 up differ from the previous code's start.  Unit starts are
        // window starts; the unit rule is checked only for those.
        const uint64_t lim64 = p.total_bits > b0 ? p.total_bits - b0 : 0;
        const uint32_t lim = lim64 < 0xFFFFFFFFull ? static_cast<uint32_t>(lim64) : 0xFFFFFFFFu;
        const uint32_t rw = static_cast<uint32_t>(b0 & 63u) + 64u;
        const uint32_t ru = static_cast<uint32_t>(b0 & 4095u) + 4096u;
        const uint64_t w0 = (b0 >> 6) - 1, u0 = (b0 >> 12) - 1;  // window/unit index of a biased 0
        const uint64_t wbase = cb >> 6;  // the chunk's first window
        const uint32_t wl0 = static_cast<uint32_t>(w0 - wbase);  // w0 + x is window wbase + wl0 + x
        auto record = [&](uint32_t cw, uint32_t cwp, uint32_t j) {  // code c * 4096 + j starts at biased cw
            const uint32_t o = cw - rw;
            if (((cw ^ cwp) >= 64u) && o < lim) {  // the first code to start in its window
                const uint32_t wl = wl0 + (cw >> 6);
                gap_l[wl] = static_cast<uint8_t>(cw & 63u);
                wfirst_l[wl] = static_cast<uint16_t>(j);
                const uint32_t cu = ru + o, pu = ru + (cwp - rw);
                if ((cu >> 12) != (pu >> 12)) p.unit_pos[u0 + (cu >> 12)] = c * kChunk + j;  // and in its unit
            }
        };
        // Code k's rule runs at step k (k >= 1); the code after the run is
        // decided at step m when the run is short (the block's end: steps past
        // it see equal starts and record nothing), else after the last step.
        uint32_t pos = lb;    // LDS bit position of code k
        uint32_t cw = rw;     // biased start of code k
        uint32_t cwp = rw;    // biased start of code k - 1
#pragma unroll
        for (uint32_t k = 0; k < kPerThread; ++k) {
            const uint32_t l = len[k];
            if (k > 0) record(cw, cwp, t * kPerThread + k);
            const uint64_t v = static_cast<uint64_t>(code[k]) << ((64u - (pos & 31u) - l) & 63u);
            atomicOr(&bits[pos >> 5], static_cast<uint32_t>(v >> 32));
            atomicOr(&bits[(pos >> 5) + 1], static_cast<uint32_t>(v));
            cwp = cw;
            cw += l;
            pos += l;
        }
        if (m == kPerThread) record(cw, cwp, t * kPerThread + kPerThread);  // the code after the run
        lds_barrier();

        // out to HBM as big-endian words, clearing the buffer for the next
        // chunk; the first and last words are shared with the neighbouring
        // chunks when the chunk is not word-aligned there
        const uint32_t head = static_cast<uint32_t>(cb & 31u);
        const uint32_t nwords = (head + chunk_bits + 31u) >> 5;
        const bool tail_shared = ((cb + chunk_bits) & 31u) != 0;
        uint32_t *out = reinterpret_cast<uint32_t *>(p.stream) + (cb >> 5);
        const uint64_t room = p.stream_bytes / 4 > (cb >> 5) ? p.stream_bytes / 4 - (cb >> 5) : 0;
        for (uint32_t k = t; k < nwords; k += blockDim.x) {
            const uint32_t v = __builtin_bswap32(bits[k]);
            bits[k] = 0;
            if (k >= room) continue;
            if ((k == 0 && head) || (k == nwords - 1 && tail_shared))
                atomicOr(out + k, v);
            else
                out[k] = v;
        }
        // the window records, from the chunk's first window to the window of
        // the next chunk's first code (clearing them for the next chunk)
        const uint32_t nwin = static_cast<uint32_t>(((cb + chunk_bits) >> 6) - wbase) + 1;
        for (uint32_t k = t; k < nwin; k += blockDim.x) {
            const uint32_t g = gap_l[k];
            if (g == kNoStart) continue;
            gap_l[k] = kNoStart;
            if (wbase + k >= p.n_windows) continue;
            p.gap8[wbase + k] = static_cast<uint8_t>(g);
            if (p.wfirst) p.wfirst[wbase + k] = c * kChunk + wfirst_l[k];
        }
        if (cn >= p.n_chunks) break;  // uniform
        c = cn;
#pragma unroll
        for (int k = 0; k < 8; ++k) wc[k] = wn[k];
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
                                                     static_cast<int>(kThreads), 0) != hipSuccess ||
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

extern "C" df11_status df11_gpu_plan_build(const uint64_t hist[256], uint32_t flags, df11_gpu_plan *plan) {
    if (!hist || !plan || (flags & ~DF11_ENCODE_WINDOW_COUNTS)) return DF11_E_INVALID_ARG;
    df11_gpu_plan q{};
    uint64_t n = 0;
    for (int e = 0; e < 256; ++e) n += hist[e];
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

extern "C" df11_status df11_gpu_encode(const df11_gpu_plan *plan, const uint16_t *x, const uint16_t *chunk_hist,
                                       uint8_t *stream, uint8_t *sign_mant, uint8_t *gaps, uint64_t *unit_pos,
                                       uint8_t *counts, void *workspace, void *hip_stream) {
    if (!plan || !stream || !sign_mant || !gaps || !unit_pos || !workspace) return DF11_E_INVALID_ARG;
    const bool with_counts = (plan->flags & DF11_ENCODE_WINDOW_COUNTS) != 0;
    if (with_counts != (counts != nullptr) || (plan->n_total && (!x || !chunk_hist))) return DF11_E_INVALID_ARG;
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
        err = launch(pack_kernel, std::min<uint32_t>(chunks, pack_groups()), kThreads, st, p);
    }
    if (err == hipSuccess && nw) err = launch(finish_kernel, grid_for(nw / 8 + 1, 4096), kThreads, st, p);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int32_t>(err);
        return DF11_E_HIP;
    }
    return DF11_OK;
}
