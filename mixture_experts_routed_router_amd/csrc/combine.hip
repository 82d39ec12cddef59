// combine.hip -- fp32 score-weighted gather-sum back to token order.
//
// out[t, c] = bf16_rne( sum_{j<k} w[t, j] * y[route_row[t*k + j], c] ), summed in
// fp32 in ascending j [prime-rl PR 3885, Changes: one fp32 score-weighted
// gather-sum back].  Each output element is produced by exactly one lane from
// its k inputs, so there is no scatter-add, no atomic and a fixed order.
//
// One wavefront per token and slice of 128 column pieces (one pass: a lane owns
// two 16-byte pieces, 8 columns each, and has all k row pieces of both in
// flight before it sums them), so a wide row is not summed in passes one after
// another by one wavefront -- at few tokens that was a chain of round trips to
// memory per token. The y
// rows are read with non-temporal loads: nothing reads them again, and on the
// MI355X these loads stream faster than plain ones (a plain read of 1-4 GB runs
// at 5.1-6.0 TB/s, a non-temporal one at 5.6-6.5 TB/s).
//
// With topk_w NULL every weight is 1: the unweighted sum of a token's k layout
// rows is the permute's backward (dx[t] = sum_j dx_perm[route_row[t*k+j]]).
#include <algorithm>

#include "combine_core.hpp"

namespace moe {

constexpr int kCombineSpan = kWave * kCombinePieces;  // column pieces per wavefront

template <int KB>  // routes loaded per batch
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ route_row,
                                                      const float* __restrict__ topk_w,
                                                      int64_t T, int pieces_per_row, int slices, int k,
                                                      int64_t P_max, uint4* __restrict__ out) {
    MOE_DEBUG_GUARD();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t units = T * slices;  // (token, slice), the slices of a token adjacent
    for (int64_t u = (int64_t)blockIdx.x * 4 + wave; u < units; u += (int64_t)gridDim.x * 4) {
        const int64_t t = u / slices;
        const int s = (int)(u - t * slices);
        const int c_begin = s * kCombineSpan;
        combine_token<KB>(y, route_row, topk_w, t, pieces_per_row, k, P_max, out, c_begin,
                          min(pieces_per_row, c_begin + kCombineSpan));
    }
}

hipError_t launch_combine(const uint16_t* y, const int32_t* route_row, const float* topk_w,
                          int64_t T, int H, int k, int64_t P_max, uint16_t* out, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int pieces = H / 8;
    const int slices = (pieces + kCombineSpan - 1) / kCombineSpan;
    // four units per workgroup; past 2^20 workgroups they loop (the grid's work-items stay below 2^32)
    const dim3 grid((unsigned)std::min<int64_t>((T * slices + 3) / 4, (int64_t)1 << 20)), block(256);
    if (k <= 8)
        hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, stream, (const uint4*)y, route_row,
                           topk_w, T, pieces, slices, k, P_max, (uint4*)out);
    else
        hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, stream, (const uint4*)y, route_row,
                           topk_w, T, pieces, slices, k, P_max, (uint4*)out);
    return hipGetLastError();
}

}  // namespace moe
