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
// the prefix sum is a wave-level scan and the stored position is per unit.
// Waves of a workgroup share the decode tables in LDS and each owns a private
// LDS staging area, so no workgroup barrier is needed after the tables are
// loaded.  Workgroups are persistent (grid-stride over groups of units).
// Staging holds the exponent already shifted into place (exponent << 7) as
// 16-bit values; the final merge with the sign/mantissa bytes is one byte
// permute and one bitfield insert per pair of weights, and the output goes out
// as 16-byte stores (16-bit stores only at the two ends of a unit).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "df11_internal.h"

namespace {

constexpr uint32_t kLdsTableMax = 32;     // sub-tables beyond this stay in global memory
constexpr uint32_t kMaxLdsBytes = 65536;  // per workgroup

struct KParams {
    const uint32_t *tables;
    const uint8_t *stream;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint64_t *unit_pos;
    uint16_t *out;
    uint64_t n_total, total_bits, n_windows, n_units;
    uint32_t n_tables;
    uint32_t stage_elems;  // 16-bit staging elements per wave, multiple of 8
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
    h = g ? __builtin_amdgcn_alignbit(w0, w1, 32u - g) : w0;
    l = g ? __builtin_amdgcn_alignbit(w1, w2, 32u - g) : w1;
    r = w2 << g;
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

template <bool kDeepGlobal>
__global__ void __launch_bounds__(1024) df11_decode_kernel(KParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    uint32_t *lut = reinterpret_cast<uint32_t *>(lds);
    const uint32_t lds_tables = kDeepGlobal ? 1u : p.n_tables;
    for (uint32_t i = threadIdx.x; i < lds_tables * 256u; i += blockDim.x) lut[i] = p.tables[i];
    __syncthreads();

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t waves = blockDim.x >> 6;
    uint16_t *stage = reinterpret_cast<uint16_t *>(lds + lds_tables * 1024u) + wave * p.stage_elems;
    const uint64_t n_groups = (p.n_units + waves - 1) / waves;

    for (uint64_t grp = blockIdx.x; grp < n_groups; grp += gridDim.x) {
        const uint64_t u = grp * waves + wave;
        if (u >= p.n_units) continue;  // uniform across the wave

        // ---- window words, gap and end of this lane's window
        const uint64_t w = u * 64 + lane;
        uint32_t w0 = 0, w1 = 0, w2 = 0, gap = 0;
        int end = 0;
        if (w < p.n_windows) {
            const uint2 a = *reinterpret_cast<const uint2 *>(p.stream + 8 * w);
            const uint32_t c = *reinterpret_cast<const uint32_t *>(p.stream + 8 * w + 8);
            w0 = __builtin_bswap32(a.x);
            w1 = __builtin_bswap32(a.y);
            w2 = __builtin_bswap32(c);
            const uint64_t gb = 5 * w;
            const uint8_t *gp = p.gaps + (gb >> 3);
            const uint32_t two = (static_cast<uint32_t>(gp[0]) << 8) | gp[1];
            gap = (two >> (11u - static_cast<uint32_t>(gb & 7))) & 31u;
            const uint64_t left = p.total_bits - 64 * w;
            end = left < 64 ? static_cast<int>(left) : 64;
        }
        uint64_t P1 = p.unit_pos[u + 1];
        uint64_t P0 = p.unit_pos[u];
        P1 = P1 < p.n_total ? P1 : p.n_total;
        P0 = P0 < P1 ? P0 : P1;

        // ---- phase 1: count the codes that start in [gap, end)
        uint32_t h, l, r;
        start_at(w0, w1, w2, gap, h, l, r);
        int pos = static_cast<int>(gap);
        uint32_t cnt = 0;
        while (pos < end) {
            const uint32_t e = lookup<kDeepGlobal>(lut, p.tables, p.n_tables, h);
            consume(e, h, l, r);
            pos += static_cast<int>((e >> 8) & 31u) + 1;
            ++cnt;
        }

        // ---- wave prefix sum of the counts
        uint32_t incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t t = __shfl_up(incl, d, 64);
            if (lane >= static_cast<uint32_t>(d)) incl += t;
        }
        const uint32_t excl = incl - cnt;

        // ---- phase 2: decode again, stage (exponent << 7) at the output slot
        const uint64_t base = P0 & ~uint64_t{7};  // stage[k] holds output base + k
        const uint32_t first = static_cast<uint32_t>(P0 - base) + excl;
        const uint32_t room = first < p.stage_elems ? p.stage_elems - first : 0u;
        const uint32_t n2 = cnt < room ? cnt : room;  // never past this wave's staging
        start_at(w0, w1, w2, gap, h, l, r);
        for (uint32_t j = 0; j < n2; ++j) {
            const uint32_t e = lookup<kDeepGlobal>(lut, p.tables, p.n_tables, h);
            consume(e, h, l, r);
            stage[first + j] = static_cast<uint16_t>(e >> 16);
        }
        wave_sync();

        // ---- merge with sign/mantissa and store [P0, P1)
        uint64_t span = P1 - base;
        span = span < p.stage_elems ? span : p.stage_elems;
        const uint64_t stop = base + span;
        const uint32_t chunks = static_cast<uint32_t>((span + 7) / 8);
        for (uint32_t c = lane; c < chunks; c += 64) {
            const uint64_t g0 = base + 8ull * c;
            const uint4 ev = *reinterpret_cast<const uint4 *>(stage + 8 * c);
            const uint2 s = *reinterpret_cast<const uint2 *>(p.sm + g0);
            uint4 o;
            o.x = merge2(ev.x, s.x, 0x01010000u);
            o.y = merge2(ev.y, s.x, 0x03030202u);
            o.z = merge2(ev.z, s.y, 0x01010000u);
            o.w = merge2(ev.w, s.y, 0x03030202u);
            if (g0 >= P0 && g0 + 8 <= stop) {
                *reinterpret_cast<uint4 *>(p.out + g0) = o;
            } else {
                const uint32_t v[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint64_t g = g0 + k;
                    if (g >= P0 && g < stop) p.out[g] = static_cast<uint16_t>(v[k >> 1] >> (16 * (k & 1)));
                }
            }
        }
        wave_sync();
    }
}

// ------------------------------------------------------------------ host side

thread_local int32_t g_last_hip_error = 0;

struct DeviceInfo {
    int cus = 0;
};

std::mutex g_mu;
DeviceInfo g_dev[64];

int cu_count(int dev) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (dev < 0 || dev >= 64) return 256;
    if (!g_dev[dev].cus) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            v = 256;
        }
        if (v <= 0) v = 256;
        g_dev[dev].cus = v;
    }
    return g_dev[dev].cus;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

df11_status check_block(const df11_device_block *b, const uint16_t *out, uint64_t cap) {
    if (!b) return DF11_E_INVALID_ARG;
    if (b->version != DF11_FORMAT_VERSION) return DF11_E_UNSUPPORTED;
    if (b->n_total == 0) return DF11_OK;
    if (!out || !b->tables || !b->stream || !b->sign_mant || !b->gaps || !b->unit_pos)
        return DF11_E_INVALID_ARG;
    if (cap < b->n_total) return DF11_E_BUFFER_TOO_SMALL;
    if (!aligned(out, 16) || !aligned(b->stream, 16) || !aligned(b->sign_mant, 16) ||
        !aligned(b->unit_pos, 8) || !aligned(b->tables, 16))
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

}  // namespace

extern "C" int32_t df11_last_hip_error(void) { return g_last_hip_error; }

extern "C" const char *df11_hip_error_name(int32_t code) {
    return hipGetErrorName(static_cast<hipError_t>(code));
}

extern "C" df11_status df11_decode_block_ex(const df11_device_block *blk, uint16_t *out_bf16,
                                            uint64_t out_capacity, void *hip_stream,
                                            const df11_launch *launch) {
    df11_status rc = check_block(blk, out_bf16, out_capacity);
    if (rc != DF11_OK || blk->n_total == 0) return rc;
    uint32_t waves = (launch && launch->waves_per_group) ? launch->waves_per_group : 4u;
    if (waves != 1 && waves != 2 && waves != 4 && waves != 8 && waves != 16) return DF11_E_INVALID_ARG;

    const bool deep_global = blk->n_tables > kLdsTableMax;
    const uint32_t lds_tables = deep_global ? 1u : blk->n_tables;
    const uint32_t stage_elems = static_cast<uint32_t>((blk->max_unit_count + 7 + 7) / 8 * 8);
    while (waves > 1 && lds_tables * 1024u + waves * stage_elems * 2u > kMaxLdsBytes) waves >>= 1;
    const uint32_t lds_bytes = lds_tables * 1024u + waves * stage_elems * 2u;
    if (lds_bytes > kMaxLdsBytes) return DF11_E_UNSUPPORTED;

    KParams p;
    p.tables = static_cast<const uint32_t *>(blk->tables);
    p.stream = blk->stream;
    p.sm = blk->sign_mant;
    p.gaps = blk->gaps;
    p.unit_pos = blk->unit_pos;
    p.out = out_bf16;
    p.n_total = blk->n_total;
    p.total_bits = blk->total_bits;
    p.n_windows = blk->n_windows;
    p.n_units = blk->n_units;
    p.n_tables = blk->n_tables;
    p.stage_elems = stage_elems;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const void *fn = deep_global ? reinterpret_cast<const void *>(&df11_decode_kernel<true>)
                                 : reinterpret_cast<const void *>(&df11_decode_kernel<false>);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, static_cast<int>(64 * waves),
                                                     lds_bytes) != hipSuccess) {
        (void)hipGetLastError();  // our own failed query: do not leave it to the caller
        per_cu = 1;
    }
    if (per_cu <= 0) per_cu = 1;
    const uint64_t groups = (blk->n_units + waves - 1) / waves;
    uint64_t grid = std::min<uint64_t>(groups, uint64_t(cu_count(dev)) * uint64_t(per_cu));
    if (launch && launch->max_groups) grid = std::min<uint64_t>(grid, launch->max_groups);
    grid = std::max<uint64_t>(grid, 1);

    // hipLaunchKernel reports the status of this launch only (hipGetLastError
    // would also return errors left behind by earlier runtime calls).
    void *args[] = {&p};
    const hipError_t err = hipLaunchKernel(fn, dim3(static_cast<uint32_t>(grid)), dim3(64 * waves), args,
                                           lds_bytes, static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int32_t>(err);
        return DF11_E_HIP;
    }
    return DF11_OK;
}

extern "C" df11_status df11_decode_block(const df11_device_block *blk, uint16_t *out_bf16,
                                         uint64_t out_capacity, void *hip_stream) {
    return df11_decode_block_ex(blk, out_bf16, out_capacity, hip_stream, nullptr);
}
