// Internal helpers shared by the libddt HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ddt.h"

#define DDT_CHECK_LAUNCH()                                     \
    do {                                                       \
        if (hipPeekAtLastError() != hipSuccess) {              \
            (void)hipGetLastError();                           \
            return DDT_EHIP;                                   \
        }                                                      \
    } while (0)

namespace ddt {

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin over 8 XCDs

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int elem_bytes(int dtype) { return dtype == DDT_F32 ? 4 : 2; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Remap a linear block id so that each XCD receives one contiguous range of
// logical work items (blocks b, b+8, b+16, ... all land on XCD b % 8).
__host__ __device__ inline int xcd_logical_block(int bid, int nblocks) {
    const int xcd = bid % kXcds;
    const int j = bid / kXcds;
    const int q = nblocks / kXcds, r = nblocks % kXcds;
    return xcd * q + (xcd < r ? xcd : r) + j;
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

}  // namespace ddt
