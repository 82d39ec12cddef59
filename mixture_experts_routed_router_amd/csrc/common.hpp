// common.hpp -- internal helpers shared by the gfx950 kernels of the MoE path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// bf16 <-> fp32. Widening is exact; narrowing rounds to nearest, ties to even
// (finite inputs; a NaN stays a quiet NaN).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The value of lane l ^ 2 / l ^ 1 inside each quad of lanes (DPP quad_perm).
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
}
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // [1,0,3,2]
}

// Lanes of this wave whose 32-bit key equals mine (the whole key is compared
// bit by bit with ballots, so no atomics and no LDS are needed). `nbits` is the
// number of low key bits that can differ.
__device__ __forceinline__ uint64_t match_peers(uint32_t key, int nbits, bool active) {
    uint64_t peers = __ballot(active);
    for (int b = 0; b < nbits; ++b) {
        uint64_t ones = __ballot(active && ((key >> b) & 1u));
        peers &= ((key >> b) & 1u) ? ones : ~ones;
    }
    return peers;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
