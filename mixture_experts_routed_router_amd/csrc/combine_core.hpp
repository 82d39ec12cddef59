// combine_core.hpp -- one token of the fp32 score-weighted gather-sum (see
// combine.hip), shared by the combine kernel and the fused layer kernel.
//
// out[t, c] = bf16_rne( sum_{j<k} w[t, j] * y[route_row[t*k + j], c] ), fp32 in
// ascending j [prime-rl PR 3885, Changes: one fp32 score-weighted gather-sum
// back]; one wavefront per token, no scatter-add.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kCombinePieces = 2;  // 16-byte column pieces per lane per pass

// Token t by the calling wavefront (wave-uniform t < T), its 16-byte column
// pieces [c_begin, c_end) (c_end < 0: to the end of the row). topk_w NULL:
// weights 1.
template <int KB>  // routes loaded per batch
__device__ __forceinline__ void combine_token(const uint4* __restrict__ y, const int32_t* __restrict__ route_row,
                                              const float* __restrict__ topk_w, int64_t t, int pieces_per_row,
                                              int k, int64_t P_max, uint4* __restrict__ out, int c_begin = 0,
                                              int c_end = -1) {
    constexpr int CP = kCombinePieces;
    const int lane = lane_id();
    const int32_t* rows = route_row + t * k;   // wave-uniform addresses: scalar loads
    const float* ws = topk_w ? topk_w + t * k : nullptr;
    if (c_end < 0) c_end = pieces_per_row;
    for (int c0 = c_begin + lane; c0 < c_end; c0 += kWave * CP) {
        float acc[CP][8];
#pragma unroll
        for (int u = 0; u < CP; ++u)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += KB) {
            uint4 v[CP][KB];
            float w[KB];
#pragma unroll
            for (int jj = 0; jj < KB; ++jj) {
                const int j = j0 + jj;
                const int32_t row = j < k ? rows[j] : -1;
                // a row outside [0, P_max) contributes nothing (never read)
                const bool ok = row >= 0 && row < P_max;
                w[jj] = ok ? (ws ? ws[j] : 1.0f) : 0.0f;
#pragma unroll
                for (int u = 0; u < CP; ++u) {
                    const int c = c0 + u * kWave;
                    // each y row is read by exactly one token: streaming (non-temporal) loads
                    u32x4_t r_ = {0u, 0u, 0u, 0u};
                    if (ok && c < c_end)
                        r_ = __builtin_nontemporal_load((const u32x4_t*)(y + (int64_t)row * pieces_per_row + c));
                    v[u][jj] = make_uint4(r_[0], r_[1], r_[2], r_[3]);
                }
            }
#pragma unroll
            for (int jj = 0; jj < KB; ++jj)
#pragma unroll
                for (int u = 0; u < CP; ++u) {
                    const uint32_t p[4] = {v[u][jj].x, v[u][jj].y, v[u][jj].z, v[u][jj].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[u][2 * q] = fmaf(w[jj], bf16_lo(p[q]), acc[u][2 * q]);
                        acc[u][2 * q + 1] = fmaf(w[jj], bf16_hi(p[q]), acc[u][2 * q + 1]);
                    }
                }
        }
#pragma unroll
        for (int u = 0; u < CP; ++u) {
            const int c = c0 + u * kWave;
            if (c < c_end) {
                uint4 o;
                o.x = pack_bf16x2(acc[u][0], acc[u][1]);
                o.y = pack_bf16x2(acc[u][2], acc[u][3]);
                o.z = pack_bf16x2(acc[u][4], acc[u][5]);
                o.w = pack_bf16x2(acc[u][6], acc[u][7]);
                out[t * pieces_per_row + c] = o;
            }
        }
    }
}

}  // namespace moe
