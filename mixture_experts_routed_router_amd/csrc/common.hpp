// common.hpp -- internal helpers shared by the gfx950 kernels of the MoE path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// Debug build (-DMOE_DEBUG, relocatable device code): check kernels enqueued ahead
// of a call validate its documented preconditions on device data and, on a
// failure, store a nonzero code in this word; every kernel of the library starts
// by reading it and does nothing once it is set, so a bad input is reported
// instead of faulting [prime-rl PR 3885, Changes: 32-bit row offsets overflowed
// silently]. Release builds read nothing.
#ifdef MOE_DEBUG
extern __device__ int32_t g_moe_debug_word;
#define MOE_DEBUG_GUARD()                                                  \
    do {                                                                   \
        if (*(volatile const int32_t*)&::moe::g_moe_debug_word != 0) return; \
    } while (0)
#else
#define MOE_DEBUG_GUARD() \
    do {                  \
    } while (0)
#endif

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

// SwiGLU backward of 8 elements, 16 bytes of bf16 each of g, u and dh, in fp32:
//   dg = dh u silu'(g),  du = dh silu(g),  silu(g) = g s,  silu'(g) = s (1 + g (1 - s)),
//   s = 1 / (1 + e^-g); results rounded to bf16 (nearest even).
__device__ __forceinline__ void swiglu_bwd_x8(uint4 gv, uint4 uv, uint4 dv, uint4& og, uint4& ou) {
    const uint32_t gp[4] = {gv.x, gv.y, gv.z, gv.w}, up[4] = {uv.x, uv.y, uv.z, uv.w};
    const uint32_t dp[4] = {dv.x, dv.y, dv.z, dv.w};
    uint32_t rg[4], ru[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float dg[2], du[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float g = h ? bf16_hi(gp[q]) : bf16_lo(gp[q]);
            const float u = h ? bf16_hi(up[q]) : bf16_lo(up[q]);
            const float d = h ? bf16_hi(dp[q]) : bf16_lo(dp[q]);
            const float sg = 1.0f / (1.0f + __expf(-g));
            dg[h] = d * u * (sg * (1.0f + g * (1.0f - sg)));
            du[h] = d * (g * sg);
        }
        rg[q] = pack_bf16x2(dg[0], dg[1]);
        ru[q] = pack_bf16x2(du[0], du[1]);
    }
    og = make_uint4(rg[0], rg[1], rg[2], rg[3]);
    ou = make_uint4(ru[0], ru[1], ru[2], ru[3]);
}

}  // namespace moe
