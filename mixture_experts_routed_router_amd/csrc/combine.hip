// combine.hip -- fp32 score-weighted gather-sum back to token order.
//
// out[t, c] = bf16_rne( sum_{j<k} w[t, j] * y[route_row[t*k + j], c] ), summed in
// fp32 in ascending j [prime-rl PR 3885, Changes: one fp32 score-weighted
// gather-sum back].  Each output element is produced by exactly one lane from
// its k inputs, so there is no scatter-add, no atomic and a fixed order.
//
// One wavefront per token; a lane owns 8 consecutive columns (one 16-byte piece)
// per pass and has all k row pieces of that pass in flight before it sums them.
#include "common.hpp"

namespace moe {

template <int KB>  // routes loaded per batch
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ route_row,
                                                      const float* __restrict__ topk_w,
                                                      int64_t T, int pieces_per_row, int k, int64_t P_max,
                                                      uint4* __restrict__ out) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int lane = lane_id();
    const int32_t* rows = route_row + t * k;   // wave-uniform addresses: scalar loads
    const float* ws = topk_w + t * k;
    for (int c = lane; c < pieces_per_row; c += kWave) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += KB) {
            uint4 v[KB];
            float w[KB];
#pragma unroll
            for (int jj = 0; jj < KB; ++jj) {
                const int j = j0 + jj;
                const int32_t row = j < k ? rows[j] : -1;
                // a row outside [0, P_max) contributes nothing (never read)
                w[jj] = (row >= 0 && row < P_max) ? ws[j] : 0.0f;
                v[jj] = (row >= 0 && row < P_max) ? y[(int64_t)row * pieces_per_row + c]
                                                  : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int jj = 0; jj < KB; ++jj) {
                {
                    const uint32_t p[4] = {v[jj].x, v[jj].y, v[jj].z, v[jj].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[2 * q] = fmaf(w[jj], bf16_lo(p[q]), acc[2 * q]);
                        acc[2 * q + 1] = fmaf(w[jj], bf16_hi(p[q]), acc[2 * q + 1]);
                    }
                }
            }
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        out[t * pieces_per_row + c] = o;
    }
}

hipError_t launch_combine(const uint16_t* y, const int32_t* route_row, const float* topk_w,
                          int64_t T, int H, int k, int64_t P_max, uint16_t* out, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const dim3 grid((unsigned)((T + 3) / 4)), block(256);
    const int pieces = H / 8;
    if (k <= 8)
        hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, stream, (const uint4*)y, route_row,
                           topk_w, T, pieces, k, P_max, (uint4*)out);
    else
        hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, stream, (const uint4*)y, route_row,
                           topk_w, T, pieces, k, P_max, (uint4*)out);
    return hipGetLastError();
}

}  // namespace moe
