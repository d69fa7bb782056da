// Device building blocks shared by the decode and encode kernels (gfx950,
// 64-lane waves): buffer resources and a wave-wide prefix sum.
#ifndef DF11_WAVE_H
#define DF11_WAVE_H

#include <hip/hip_runtime.h>

#include <cstdint>

namespace df11w {

// Buffer resources: a base address and a size in scalar registers, accessed
// with 32-bit per-lane offsets.  Loads past the size return 0 and stores past
// it are dropped, so masked accesses need an out-of-range offset rather than
// a branch.
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr uint32_t kOff = 0x80000000u;  // an offset past every resource used here
constexpr int kNonTemporal = 2;        // cache policy bit of buffer accesses: non-temporal

__device__ __forceinline__ Rsrc rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (cross-lane moves inside the VALU, no LDS round trip):
// shifts by 1, 2, 3 then 4 and 8 give the scan within each row of 16 lanes;
// broadcasting lane 15 into rows 1 and 3, then lane 31 into rows 2 and 3,
// carries the row totals across.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    uint32_t s = x;
    s += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);  // row_shr:1
    s += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);  // row_shr:2
    s += __builtin_amdgcn_update_dpp(0u, x, 0x113, 0xF, 0xF, true);  // row_shr:3
    s += __builtin_amdgcn_update_dpp(0u, s, 0x114, 0xF, 0xE, false); // row_shr:4, lanes 4..15 of a row
    s += __builtin_amdgcn_update_dpp(0u, s, 0x118, 0xF, 0xC, false); // row_shr:8, lanes 8..15 of a row
    s += __builtin_amdgcn_update_dpp(0u, s, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
    s += __builtin_amdgcn_update_dpp(0u, s, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
    return s;
}

}  // namespace df11w

#endif  // DF11_WAVE_H
