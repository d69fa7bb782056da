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
//   fill    defaults: zeroed stream, gaps, counts and padding; unit_pos and
//           the first-start records preset for units/windows where no code
//           starts (only possible at the end of the stream)
//   sums    bits per chunk of 4,096 weights
//   scan    exclusive prefix of the chunk sums (one workgroup)
//   pack    per chunk: each weight's bit offset (block scan), its
//           sign/mantissa byte, its code ORed into an LDS bit buffer that is
//           then written out (global atomic OR only on the two words shared
//           with the neighbouring chunks), and the first code start of every
//           window (gap) and unit (position) it contains
//   finish  5-bit gap fields (8 windows per 5 bytes) and window counts
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "df11_internal.h"

namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kPerThread = 16;                   // weights per thread in sums/pack
constexpr uint32_t kChunk = kThreads * kPerThread;    // 4,096 weights per chunk
constexpr uint32_t kBitWords = kChunk * 32 / 32 + 2;  // LDS words for a chunk's codes
constexpr uint32_t kScanThreads = 1024;

struct EncParams {
    const uint16_t *x;
    uint8_t *stream, *sm, *gaps, *counts;
    uint64_t *unit_pos;
    uint32_t *chunk_sums;
    uint64_t *chunk_off;
    uint8_t *gap8;
    uint64_t *wfirst;
    uint64_t n, total_bits, n_windows, n_units, n_chunks;
    uint64_t stream_bytes, sm_bytes, gaps_bytes, counts_bytes;
    uint32_t code[256];
    uint8_t len[256];
};

__device__ __forceinline__ uint32_t exponent_of(uint32_t x) { return (x >> 7) & 0xFFu; }

// ---------------------------------------------------------------- histogram
__global__ void __launch_bounds__(256) hist_zero(uint64_t *hist) {
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
}

constexpr uint32_t kHistCopies = 16;  // sub-histograms per workgroup, one per lane & 15
constexpr uint32_t kHistStride = 257; // padded rows: copies of one exponent fall in different banks

__global__ void __launch_bounds__(kThreads) hist_kernel(const uint16_t *x, uint64_t n, uint64_t *hist) {
    // A block's values cluster on a few exponents: same-address LDS atomics
    // are serialised, so lanes spread over 16 copies of the histogram.
    __shared__ uint32_t h[kHistCopies * kHistStride];
    uint32_t *mine = h + (threadIdx.x & (kHistCopies - 1)) * kHistStride;
    for (uint32_t i = threadIdx.x; i < kHistCopies * kHistStride; i += blockDim.x) h[i] = 0;
    __syncthreads();
    const uint64_t n8 = n / 8;
    const uint64_t step = uint64_t{gridDim.x} * blockDim.x;
    for (uint64_t g = uint64_t{blockIdx.x} * blockDim.x + threadIdx.x; g < n8; g += step) {
        const uint4 v = reinterpret_cast<const uint4 *>(x)[g];
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            atomicAdd(&mine[exponent_of(q[k])], 1u);
            atomicAdd(&mine[exponent_of(q[k] >> 16)], 1u);
        }
    }
    if (blockIdx.x == 0)
        for (uint64_t i = 8 * n8 + threadIdx.x; i < n; i += blockDim.x) atomicAdd(&mine[exponent_of(x[i])], 1u);
    __syncthreads();
    for (uint32_t e = threadIdx.x; e < 256; e += blockDim.x) {
        uint32_t c = 0;
        for (uint32_t k = 0; k < kHistCopies; ++k) c += h[k * kHistStride + e];
        if (c) atomicAdd(reinterpret_cast<unsigned long long *>(hist + e), static_cast<unsigned long long>(c));
    }
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

// Sixteen weights of thread t of chunk c (fewer at the end of the block).
__device__ __forceinline__ uint32_t load16(const EncParams &p, uint64_t i0, uint32_t xs[kPerThread]) {
    const uint32_t m = i0 >= p.n ? 0u : static_cast<uint32_t>(p.n - i0 < kPerThread ? p.n - i0 : kPerThread);
    if (m == kPerThread) {
        const uint4 a = reinterpret_cast<const uint4 *>(p.x + i0)[0];
        const uint4 b = reinterpret_cast<const uint4 *>(p.x + i0)[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            xs[2 * k] = w[k] & 0xFFFFu;
            xs[2 * k + 1] = w[k] >> 16;
        }
    } else {
#pragma unroll
        for (uint32_t k = 0; k < kPerThread; ++k) xs[k] = k < m ? p.x[i0 + k] : 0u;
    }
    return m;
}

// Block-wide exclusive sum of one value per thread (256 threads); also the total.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t *scratch, uint32_t &total) {
    const uint32_t t = threadIdx.x;
    scratch[t] = v;
    __syncthreads();
    for (uint32_t d = 1; d < kThreads; d <<= 1) {  // Hillis-Steele inclusive scan
        const uint32_t add = t >= d ? scratch[t - d] : 0u;
        __syncthreads();
        scratch[t] += add;
        __syncthreads();
    }
    total = scratch[kThreads - 1];
    const uint32_t incl = scratch[t];
    __syncthreads();
    return incl - v;
}

// ---------------------------------------------------------------- chunk sums
__global__ void __launch_bounds__(kThreads) sums_kernel(EncParams p) {
    __shared__ uint8_t len[256];
    __shared__ uint32_t scratch[kThreads];
    for (uint32_t e = threadIdx.x; e < 256; e += blockDim.x) len[e] = p.len[e];
    __syncthreads();
    const uint64_t c = blockIdx.x;
    uint32_t xs[kPerThread];
    const uint32_t m = load16(p, c * kChunk + uint64_t{threadIdx.x} * kPerThread, xs);
    uint32_t s = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPerThread; ++k) s += k < m ? len[exponent_of(xs[k])] : 0u;
    uint32_t total;
    (void)block_exclusive_sum(s, scratch, total);
    if (threadIdx.x == 0) p.chunk_sums[c] = total;
}

// ---------------------------------------------------------------- scan
__global__ void __launch_bounds__(kScanThreads) scan_kernel(EncParams p) {
    // Each thread sums a contiguous segment of chunk sums (a multiple of 4
    // long, read 16 bytes at a time, several loads in flight), one block scan
    // of the 1,024 segment sums, then each thread writes its segment's
    // running offsets.
    __shared__ uint64_t part[kScanThreads];
    const uint32_t t = threadIdx.x;
    const uint64_t per = ((p.n_chunks + kScanThreads - 1) / kScanThreads + 3) / 4 * 4;
    const uint64_t b = std::min<uint64_t>(t * per, p.n_chunks), e = std::min<uint64_t>(b + per, p.n_chunks);
    const uint32_t *sums = p.chunk_sums;
    uint64_t s = 0;
    uint64_t c = b;
#pragma unroll 4
    for (; c + 4 <= e; c += 4) {
        const uint4 v = *reinterpret_cast<const uint4 *>(sums + c);  // b is a multiple of 4
        s += uint64_t{v.x} + v.y + v.z + v.w;
    }
    for (; c < e; ++c) s += sums[c];
    part[t] = s;
    __syncthreads();
    for (uint32_t d = 1; d < kScanThreads; d <<= 1) {
        const uint64_t add = t >= d ? part[t - d] : 0u;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    uint64_t run = part[t] - s;  // exclusive prefix of this thread's segment
    c = b;
#pragma unroll 4
    for (; c + 4 <= e; c += 4) {
        const uint4 v = *reinterpret_cast<const uint4 *>(sums + c);
        p.chunk_off[c] = run;
        p.chunk_off[c + 1] = run + v.x;
        p.chunk_off[c + 2] = run + v.x + v.y;
        p.chunk_off[c + 3] = run + v.x + v.y + v.z;
        run += uint64_t{v.x} + v.y + v.z + v.w;
    }
    for (; c < e; ++c) {
        p.chunk_off[c] = run;
        run += sums[c];
    }
    if (t == kScanThreads - 1) p.chunk_off[p.n_chunks] = part[t];
}

// ---------------------------------------------------------------- pack
__global__ void __launch_bounds__(kThreads) pack_kernel(EncParams p) {
    __shared__ uint32_t code[256];
    __shared__ uint8_t len[256];
    __shared__ uint32_t bits[kBitWords];
    __shared__ uint32_t scratch[kThreads];
    for (uint32_t e = threadIdx.x; e < 256; e += blockDim.x) {
        code[e] = p.code[e];
        len[e] = p.len[e];
    }
    for (uint32_t k = threadIdx.x; k < kBitWords; k += blockDim.x) bits[k] = 0;
    __syncthreads();

    const uint64_t c = blockIdx.x;
    const uint64_t i0 = c * kChunk + uint64_t{threadIdx.x} * kPerThread;
    uint32_t xs[kPerThread];
    const uint32_t m = load16(p, i0, xs);

    // sign/mantissa bytes: (sign << 7) | mantissa
    if (m == kPerThread) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t v = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t x = xs[4 * k + j];
                v |= (((x >> 8) & 0x80u) | (x & 0x7Fu)) << (8 * j);
            }
            w[k] = v;
        }
        reinterpret_cast<uint4 *>(p.sm + i0)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        for (uint32_t k = 0; k < m; ++k) p.sm[i0 + k] = static_cast<uint8_t>(((xs[k] >> 8) & 0x80u) | (xs[k] & 0x7Fu));
    }

    // this thread's first bit: chunk offset + block prefix of the thread sums
    uint32_t s = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPerThread; ++k) s += k < m ? len[exponent_of(xs[k])] : 0u;
    uint32_t chunk_bits;
    const uint32_t pre = block_exclusive_sum(s, scratch, chunk_bits);
    const uint64_t cb = p.chunk_off[c];
    uint64_t b = cb + pre;
    const uint32_t lb = static_cast<uint32_t>(cb & 31u) + pre;  // bit index in the LDS buffer
    // the code before this thread's first one (for the first-start rules)
    uint32_t lprev = (m && i0) ? len[exponent_of(p.x[i0 - 1])] : 0u;

    // The thread's codes are one run of bits: gather them MSB-first in a
    // 64-bit register and write whole words.  Words inside the run belong to
    // this thread alone (plain writes); its first and last words may be shared
    // with the neighbouring threads (atomic OR).
    uint64_t acc = 0;
    uint32_t have = lb & 31u;  // bits in acc, counting the word's bits before the run (zeros)
    uint32_t word = lb >> 5;
    bool first_word = true;
    for (uint32_t k = 0; k < m; ++k) {
        const uint32_t e = exponent_of(xs[k]);
        const uint32_t l = len[e];
        const uint64_t i = i0 + k;
        const uint64_t prev = b - lprev;  // start of the previous code
        // (b < total_bits holds when x is the block the plan was made for;
        // the test keeps every index in its buffer when it is not)
        if (b < p.total_bits && (i == 0 || (prev >> 6) != (b >> 6))) {  // first code in window b >> 6
            p.gap8[b >> 6] = static_cast<uint8_t>(b & 63u);
            if (p.counts) p.wfirst[b >> 6] = i;
        }
        if (b < p.total_bits && (i == 0 || (prev >> 12) != (b >> 12))) p.unit_pos[b >> 12] = i;
        acc = (acc << l) | code[e];  // have + l <= 63
        have += l;
        if (have >= 32) {
            const uint32_t w = static_cast<uint32_t>(acc >> (have - 32));
            if (first_word)
                atomicOr(&bits[word], w);
            else
                bits[word] = w;
            first_word = false;
            ++word;
            have -= 32;
        }
        b += l;
        lprev = l;
    }
    if (m && have) atomicOr(&bits[word], static_cast<uint32_t>(acc << (32 - have)));  // the run's last word
    __syncthreads();

    // out to HBM as big-endian words; the first and last words are shared
    // with the neighbouring chunks when the chunk is not word-aligned there
    const uint32_t head = static_cast<uint32_t>(cb & 31u);
    const uint32_t nwords = (head + chunk_bits + 31u) >> 5;
    const bool tail_shared = ((cb + chunk_bits) & 31u) != 0;
    uint32_t *out = reinterpret_cast<uint32_t *>(p.stream) + (cb >> 5);
    const uint64_t room = p.stream_bytes / 4 > (cb >> 5) ? p.stream_bytes / 4 - (cb >> 5) : 0;
    for (uint32_t k = threadIdx.x; k < nwords && k < room; k += blockDim.x) {
        const uint32_t v = __builtin_bswap32(bits[k]);
        if ((k == 0 && head) || (k == nwords - 1 && tail_shared))
            atomicOr(out + k, v);
        else
            out[k] = v;
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
    uint64_t sums, off, gap8, wfirst, bytes;
};

Workspace workspace_layout(uint64_t n, uint64_t n_windows, bool counts) {
    Workspace w{};
    const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
    w.sums = 0;
    w.off = align256(4 * n_chunks);
    w.gap8 = w.off + align256(8 * (n_chunks + 1));
    w.wfirst = w.gap8 + align256(n_windows);
    w.bytes = w.wfirst + (counts ? align256(8 * (n_windows + 1)) : 0);
    return w;
}

bool aligned(const void *ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

// hipLaunchKernel reports the status of this launch only (hipGetLastError
// would also return errors left behind by earlier runtime calls).
template <class... A>
hipError_t launch(void (*kernel)(A...), uint32_t grid, uint32_t block, hipStream_t st, A... args) {
    void *argv[] = {static_cast<void *>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3(grid), dim3(block), argv, 0, st);
}

uint32_t grid_for(uint64_t items, uint32_t cap) {
    const uint64_t g = (items + kThreads - 1) / kThreads;
    return static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>(g, cap)));
}

}  // namespace

extern "C" df11_status df11_gpu_histogram(const uint16_t *x, uint64_t n, uint64_t *hist, void *hip_stream) {
    if (!hist || (n && !x) || !aligned(x, 16) || !aligned(hist, 8)) return DF11_E_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    hipError_t err = launch(hist_zero, 1, 256, st, hist);
    if (err == hipSuccess && n) err = launch(hist_kernel, grid_for(n / 8 + 1, 2048), kThreads, st, x, n, hist);
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

extern "C" df11_status df11_gpu_encode(const df11_gpu_plan *plan, const uint16_t *x, uint8_t *stream,
                                       uint8_t *sign_mant, uint8_t *gaps, uint64_t *unit_pos, uint8_t *counts,
                                       void *workspace, void *hip_stream) {
    if (!plan || !stream || !sign_mant || !gaps || !unit_pos || !workspace) return DF11_E_INVALID_ARG;
    const bool with_counts = (plan->flags & DF11_ENCODE_WINDOW_COUNTS) != 0;
    if (with_counts != (counts != nullptr) || (plan->n_total && !x)) return DF11_E_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(stream, 16) || !aligned(sign_mant, 16) || !aligned(unit_pos, 8) ||
        !aligned(workspace, 16))
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
    p.stream = stream;
    p.sm = sign_mant;
    p.gaps = gaps;
    p.counts = counts;
    p.unit_pos = unit_pos;
    p.chunk_sums = reinterpret_cast<uint32_t *>(wsb + ws.sums);
    p.chunk_off = reinterpret_cast<uint64_t *>(wsb + ws.off);
    p.gap8 = wsb + ws.gap8;
    p.wfirst = with_counts ? reinterpret_cast<uint64_t *>(wsb + ws.wfirst) : nullptr;
    p.n = plan->n_total;
    p.total_bits = plan->total_bits;
    p.n_windows = nw;
    p.n_units = nu;
    p.n_chunks = (plan->n_total + kChunk - 1) / kChunk;
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
    if (err == hipSuccess && chunks) err = launch(sums_kernel, chunks, kThreads, st, p);
    if (err == hipSuccess && chunks) err = launch(scan_kernel, 1, kScanThreads, st, p);
    if (err == hipSuccess && chunks) err = launch(pack_kernel, chunks, kThreads, st, p);
    if (err == hipSuccess && nw) err = launch(finish_kernel, grid_for(nw / 8 + 1, 4096), kThreads, st, p);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int32_t>(err);
        return DF11_E_HIP;
    }
    return DF11_OK;
}
