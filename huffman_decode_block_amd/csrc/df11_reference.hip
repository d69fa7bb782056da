// Bandwidth references for the block decode (gfx950, HIP): two streaming
// kernels that move the HBM bytes of one df11_decode_block launch without
// decoding anything, so that the decode's rate can be set against what the
// same traffic achieves on the same GPU.
//
// The decode reads the compressed sections once (EncodedExponent, the 5-bit
// gaps, the stored unit positions, PackedSignMantissa) and writes the BF16
// block once, in one coalesced write per group of threads (hada.io summary
// of the DFloat11 paper, section "Noyau GPU en deux etapes et metadonnees
// auxiliaires").  Both references write out[i] = the weight with its
// exponent field zero (sign and mantissa from PackedSignMantissa), a value a
// test can check exactly:
//
//   skeleton: the decode's own access pattern, unit by unit (one 64-lane wave
//     per unit of 64 windows): per lane the 8-byte window word and its 4-byte
//     halo, two gap bytes, the unit's position pair, one unit ahead; the
//     unit's sign/mantissa bytes as 8-byte non-temporal loads; 16-byte
//     non-temporal stores of the whole 64-byte sectors and 2-byte stores of
//     the sectors the unit shares with its neighbours; the same workgroup
//     size, grid rule and unit order (a workgroup's units taken in turn from
//     an LDS counter when its waves have two or more on average).  What it
//     lacks is the decoding itself (tables, counting, scan, staging).
//   stream: the same byte counts in whole tiles of 4,096 weights per wave:
//     the tile's sign/mantissa bytes (8-byte non-temporal loads), its share of
//     the stream and gap bytes (16-byte loads), its 8 KiB of output (16-byte
//     non-temporal stores).  No unit boundaries, no shared sectors: the
//     ceiling of this read/write mix on the GPU.
//   writes, reads: the stream reference's stores alone (zeros) and its loads
//     alone (nothing stored), so that the mix can be set against what each
//     direction reaches by itself.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "df11_internal.h"
#include "df11_wave.h"

namespace {

using df11w::kNonTemporal;
using df11w::kOff;
using df11w::rsrc;
using df11w::Rsrc;
using df11w::v2u;
using df11w::v4u;

constexpr uint64_t kUnitsPerWave = 4;   // as the decode's automatic grid
constexpr uint32_t kTileWeights = 4096;  // stream reference: weights per wave step
constexpr uint64_t kTilesPerWave = 2;    // about as many weights per wave as the decode's 4 units

struct RefParams {
    const uint8_t *stream;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint64_t *unit_pos;
    uint16_t *out;
    uint64_t n_total, n_units, n_tiles;
    uint64_t stream_used, gaps_used;  // section bytes a decode reads
    uint32_t stream_share, gaps_share;  // per tile, multiples of 16 (stream reference)
    uint32_t out_phase;                 // (address of out / 2) mod 32: 64-byte sector phase
    uint32_t unit_queue;                // skeleton: the decode's unit order (units taken in turn)
    uint32_t reads_store_flag;          // stream, reads only: 0 (no store)
};

// Two output values from four sign/mantissa bytes selected by `sel`: the
// exponent field is left zero.
__device__ __forceinline__ uint32_t sm_only2(uint32_t sm4, uint32_t sel) {
    return __builtin_amdgcn_perm(sm4, sm4, sel) & 0x807F807Fu;
}

__device__ __forceinline__ v4u sm_only8(uint32_t lo, uint32_t hi) {
    v4u o;
    o.x = sm_only2(lo, 0x01010000u);
    o.y = sm_only2(lo, 0x03030202u);
    o.z = sm_only2(hi, 0x01010000u);
    o.w = sm_only2(hi, 0x03030202u);
    return o;
}

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

struct UnitLoads {
    uint32_t w0, w1, w2, g0, g1;
    uint64_t pos;  // unit_pos[u] in even lanes, unit_pos[u + 1] in odd lanes
};

__device__ __forceinline__ void load_unit(const RefParams &p, uint64_t u, uint32_t lane, UnitLoads &in) {
    const Rsrc st = rsrc(p.stream + 512 * u, 528);
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
}

constexpr uint32_t kChunksPerPass = 64;
constexpr int kPrefetchChunks = 4;

__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8)))
df11_skeleton_kernel(RefParams p) {
    uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t waves = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    uint64_t u = uniform_u64(uint64_t{blockIdx.x} * waves + wave);
    // as the decode: with the queue, each wave takes the workgroup's next unit
    // position from an LDS counter (positions below `waves` are the first units)
    __shared__ uint32_t s_next_pos;
    if (threadIdx.x == 0) s_next_pos = waves;
    __syncthreads();
    if (u >= p.n_units) return;  // uniform across the wave
    const uint64_t last = p.n_units - 1;
    const uint64_t stride = uniform_u64(uint64_t{gridDim.x} * waves);
    const uint64_t group0 = uniform_u64(uint64_t{blockIdx.x} * waves);
    const uint32_t wshift = __builtin_amdgcn_readfirstlane(31u - __clz(waves));  // waves is a power of two
    UnitLoads cur;
    load_unit(p, u, lane, cur);
    while (true) {
        asm volatile("" : "+v"(lane));
        uint64_t un;
        if (p.unit_queue) {  // uniform
            uint32_t k = 0;
            if (lane == 0) k = atomicAdd(&s_next_pos, 1u);
            k = __builtin_amdgcn_readfirstlane(k);
            un = uniform_u64(group0 + (k & (waves - 1u)) + uint64_t{k >> wshift} * stride);
        } else {
            un = uniform_u64(u + stride);
        }
        UnitLoads nxt;
        load_unit(p, un < last ? un : last, lane, nxt);  // one unit ahead, as the decode
        // the decode's first phase needs the window and gap: wait for them here
        asm volatile("" ::"v"(cur.w0), "v"(cur.w1), "v"(cur.w2), "v"(cur.g0), "v"(cur.g1));

        const uint64_t q1 = lane_u64(cur.pos, 1), q0 = lane_u64(cur.pos, 0);
        const uint64_t P1 = q1 < p.n_total ? q1 : p.n_total;
        const uint64_t P0 = q0 < P1 ? q0 : P1;
        const uint64_t base = P0 & ~uint64_t{7};
        const uint64_t span64 = P1 - base;
        const uint32_t span = span64 < 4104u ? static_cast<uint32_t>(span64) : 4104u;
        const uint32_t lead = static_cast<uint32_t>(P0 - base);
        const uint32_t chunks = (span + 7) / 8;
        const Rsrc smr = rsrc(p.sm + base, 8 * chunks);
        const uint32_t b32 = (p.out_phase + static_cast<uint32_t>(base)) & 31u;
        const uint32_t hs = ((b32 + lead + 31u) & ~31u) - b32;
        const uint32_t ts = b32 + span >= 32u ? ((b32 + span) & ~31u) - b32 : 0u;
        const uint32_t e1 = hs < span ? hs : span;
        const uint32_t e2 = ts > e1 ? ts : e1;
        const uint32_t full_lo = e1 / 8, full_hi = e2 / 8;
        const uint32_t ek = lane < 32 ? lead + lane : e2 + (lane - 32u);
        const bool edge = ek < (lane < 32 ? e1 : span);

        v2u smv[kPrefetchChunks];
        const bool pass3 = chunks > 3 * kChunksPerPass;
#pragma unroll
        for (int k = 0; k < kPrefetchChunks; ++k) {
            if (k == 3 && !pass3) {
                smv[k] = v2u{0u, 0u};
                continue;
            }
            smv[k] = __builtin_amdgcn_raw_buffer_load_b64(smr, 8 * (lane + kChunksPerPass * k), 0, kNonTemporal);
        }
        const uint32_t esm = __builtin_amdgcn_raw_buffer_load_b8(smr, edge ? ek : kOff, 0, 0);
        const Rsrc outr = rsrc(p.out + base, 16 * full_hi);
        v4u outv[kPrefetchChunks];
#pragma unroll
        for (int k = 0; k < kPrefetchChunks; ++k) outv[k] = sm_only8(smv[k].x, smv[k].y);
        const uint32_t eo = __builtin_amdgcn_perm(esm, esm, 0x0c0c0000u) & 0x807Fu;
        asm volatile("" ::"v"(nxt.w0), "v"(nxt.w1), "v"(nxt.w2), "v"(nxt.g0), "v"(nxt.g1), "v"(nxt.pos), "v"(eo));
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const uint32_t c = lane + kChunksPerPass * k;
            __builtin_amdgcn_raw_buffer_store_b128(outv[k], outr, c >= full_lo ? 16 * c : kOff, 0, kNonTemporal);
        }
        if (pass3) {
            const uint32_t c = lane + kChunksPerPass * 3;
            __builtin_amdgcn_raw_buffer_store_b128(outv[3], outr, c >= full_lo ? 16 * c : kOff, 0, kNonTemporal);
        }
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(eo), rsrc(p.out + base, 2 * span),
                                              edge ? 2 * ek : kOff, 0, 0);
        if (chunks > kChunksPerPass * kPrefetchChunks) {
            for (uint32_t c = lane + kChunksPerPass * kPrefetchChunks; c < chunks; c += kChunksPerPass) {
                const v2u t = __builtin_amdgcn_raw_buffer_load_b64(smr, 8 * c, 0, kNonTemporal);
                __builtin_amdgcn_raw_buffer_store_b128(sm_only8(t.x, t.y), outr, c >= full_lo ? 16 * c : kOff, 0,
                                                       kNonTemporal);
            }
        }
        if (un >= p.n_units) break;
        cur = nxt;
        u = un;
    }
}

constexpr uint32_t kTileChunks = kTileWeights / 8;  // 512: 8 per lane

// kMode: kMix moves both the section reads and the output writes; kWrites
// only the output writes (zeros); kReads only the section reads.
enum StreamMode : int { kMix = 0, kWrites = 1, kReads = 2 };

template <int kMode>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8)))
df11_stream_kernel(RefParams p) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t waves = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
    const uint64_t stride = uniform_u64(uint64_t{gridDim.x} * waves);
    for (uint64_t t = uniform_u64(uint64_t{blockIdx.x} * waves + wave); t < p.n_tiles; t += stride) {
        // the tile's share of the stream and gap sections (16-byte loads; the
        // shares of the last tiles may reach past the section, read as zero)
        const uint64_t s0 = t * p.stream_share, g0 = t * p.gaps_share;
        const uint64_t s_left = s0 < p.stream_used ? p.stream_used - s0 : 0;
        const uint64_t g_left = g0 < p.gaps_used ? p.gaps_used - g0 : 0;
        const Rsrc sr = rsrc(p.stream + s0, static_cast<uint32_t>(s_left < p.stream_share ? s_left : p.stream_share));
        const Rsrc gr = rsrc(p.gaps + g0, static_cast<uint32_t>(g_left < p.gaps_share ? g_left : p.gaps_share));
        uint32_t fold = 0;
        if (kMode != kWrites) {
            for (uint32_t off = 16 * lane; off < p.stream_share; off += 1024) {
                const v4u v = __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, 0);
                fold ^= v.x ^ v.y ^ v.z ^ v.w;
            }
            for (uint32_t off = 16 * lane; off < p.gaps_share; off += 1024) {
                const v4u v = __builtin_amdgcn_raw_buffer_load_b128(gr, off, 0, 0);
                fold ^= v.x ^ v.y ^ v.z ^ v.w;
            }
        }
        const uint64_t w0 = t * kTileWeights;
        const uint64_t left = p.n_total - w0;
        const uint32_t n = left < kTileWeights ? static_cast<uint32_t>(left) : kTileWeights;
        const Rsrc smr = rsrc(p.sm + w0, (n + 15u) & ~15u);
        v2u smv[kTileChunks / 64];
#pragma unroll
        for (uint32_t k = 0; k < kTileChunks / 64; ++k)
            smv[k] = kMode == kWrites ? v2u{0u, 0u}
                                      : __builtin_amdgcn_raw_buffer_load_b64(smr, 8 * (lane + 64 * k), 0, kNonTemporal);
        if (kMode == kReads) {
            // the loaded values only decide a store that the host's flag
            // (never set) enables, so that the loads are not dropped
#pragma unroll
            for (uint32_t k = 0; k < kTileChunks / 64; ++k) fold ^= smv[k].x ^ smv[k].y;
            if (p.reads_store_flag && fold == 0) p.out[0] = 0;
            continue;
        }
        asm volatile("" ::"v"(fold));
        const Rsrc full = rsrc(p.out + w0, 16 * (n / 8));
#pragma unroll
        for (uint32_t k = 0; k < kTileChunks / 64; ++k) {
            const uint32_t c = lane + 64 * k;
            const v4u o = sm_only8(smv[k].x, smv[k].y);
            __builtin_amdgcn_raw_buffer_store_b128(o, full, 16 * c, 0, kNonTemporal);
            if (8 * c < n && 8 * c + 8 > n) {  // the block's last, partial chunk
                const Rsrc part = rsrc(p.out + w0, 2 * n);
                const uint32_t e[8] = {o.x, o.x >> 16, o.y, o.y >> 16, o.z, o.z >> 16, o.w, o.w >> 16};
                for (uint32_t j = 0; j < 8; ++j)
                    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(e[j]), part, 2 * (8 * c + j), 0, 0);
            }
        }
    }
}

int occupancy(const void *fn, uint32_t waves) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, static_cast<int>(64 * waves), 0) != hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    return per_cu > 0 ? per_cu : 0;
}

int cu_count() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    return v > 0 ? v : 256;
}

df11_status reference(const df11_device_block *blk, uint16_t *out, uint64_t cap, uint32_t kind, void *hip_stream,
                      const df11_launch *launch) {
    if (kind != DF11_REFERENCE_SKELETON && kind != DF11_REFERENCE_STREAM && kind != DF11_REFERENCE_WRITES &&
        kind != DF11_REFERENCE_READS)
        return DF11_E_INVALID_ARG;
    df11_status rc = df11i::check_device_block(blk, out, cap);
    if (rc != DF11_OK || blk->n_total == 0) return rc;
    if (blk->unit_end || blk->counts) return DF11_E_UNSUPPORTED;  // the pages' format only
    const uint32_t asked = launch ? launch->waves_per_group : 0u;
    if (asked != 0 && asked != 1 && asked != 2 && asked != 4 && asked != 8 && asked != 16) return DF11_E_INVALID_ARG;
    const uint32_t waves = asked ? asked : 16u;

    RefParams p;
    p.stream = blk->stream;
    p.sm = blk->sign_mant;
    p.gaps = blk->gaps;
    p.unit_pos = blk->unit_pos;
    p.out = out;
    p.n_total = blk->n_total;
    p.n_units = blk->n_units;
    p.n_tiles = (blk->n_total + kTileWeights - 1) / kTileWeights;
    p.stream_used = (blk->total_bits + 7) / 8;
    p.gaps_used = (5 * blk->n_windows + 7) / 8;
    auto share = [&](uint64_t bytes) {
        const uint64_t s = (bytes + p.n_tiles - 1) / p.n_tiles;
        return static_cast<uint32_t>((s + 15) / 16 * 16);
    };
    p.stream_share = share(p.stream_used);
    p.gaps_share = share(p.gaps_used);
    p.out_phase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(out) >> 1) & 31u;

    p.reads_store_flag = 0;
    const bool skeleton = kind == DF11_REFERENCE_SKELETON;
    const void *fn = skeleton                          ? reinterpret_cast<const void *>(&df11_skeleton_kernel)
                     : kind == DF11_REFERENCE_STREAM ? reinterpret_cast<const void *>(&df11_stream_kernel<kMix>)
                     : kind == DF11_REFERENCE_WRITES ? reinterpret_cast<const void *>(&df11_stream_kernel<kWrites>)
                                                     : reinterpret_cast<const void *>(&df11_stream_kernel<kReads>);
    const uint64_t items = skeleton ? p.n_units : p.n_tiles;
    const uint64_t per_wave = skeleton ? kUnitsPerWave : kTilesPerWave;
    const uint64_t groups = (items + waves - 1) / waves;
    const uint64_t resident = uint64_t(cu_count()) * uint64_t(std::max(occupancy(fn, waves), 1));
    uint64_t grid;
    if (launch && launch->oversubscribe)
        grid = std::min<uint64_t>(groups, resident * launch->oversubscribe);
    else
        grid = std::min<uint64_t>(groups, std::max<uint64_t>(resident, (groups + per_wave - 1) / per_wave));
    if (launch && launch->max_groups) grid = std::min<uint64_t>(grid, launch->max_groups);
    grid = std::max<uint64_t>(grid, 1);
    p.unit_queue = skeleton && grid * waves * 2 <= p.n_units ? 1u : 0u;  // the decode's rule
    void *args[] = {&p};
    const hipError_t err =
        hipLaunchKernel(fn, dim3(static_cast<uint32_t>(grid)), dim3(64 * waves), args, 0, static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) {
        df11i::last_hip_error = static_cast<int32_t>(err);
        return DF11_E_HIP;
    }
    return DF11_OK;
}

}  // namespace

extern "C" df11_status df11_bandwidth_reference(const df11_device_block *blk, uint16_t *out_bf16,
                                                uint64_t out_capacity, uint32_t kind, void *hip_stream,
                                                const df11_launch *launch) {
    return df11i::guarded([&] { return reference(blk, out_bf16, out_capacity, kind, hip_stream, launch); });
}
