// route_topk.hip -- top-k routing over router logits, one wavefront per token.
//
// Per token: the k experts with the largest logits, larger first, an exact tie
// going to the lower expert id; weights = softmax over the k selected logits in
// fp32 [PocketLLM "Qwen4-Exp Heterogeneous TP4 Performance", Runtime
// architecture: top-10 of 512 routed experts; prime-rl PR 3885, Changes: the
// top-k scores weight the gather-sum].
//
// Each lane holds E/64 logits of the token in registers; every round a
// butterfly over the wave finds the best (logit, id) not yet taken. The
// comparison is on the fp32 logits themselves (never on exp'd values, which can
// merge distinct logits), with float == so that -0 and +0 tie.
#include "common.hpp"

namespace moe {

__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <int NV>  // logits per lane: ceil(E / 64)
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t T, int E, int k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    const float* row = logits + t * E;

    float v[NV];
    bool live[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + i * kWave;
        live[i] = e < E;
        v[i] = live[i] ? row[e] : 0.0f;
    }

    float my_v = 0.0f;  // lane j keeps the j-th pick
    int my_i = 0;
    float top = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + i * kWave;
            if (live[i] && (bi == 0x7fffffff || ranks_before(v[i], e, bv, bi))) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = kWave / 2; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || ranks_before(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
            }
        }
        // every lane now holds the same winner; its owner retires it
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + i * kWave == bi) live[i] = false;
        if (lane == j) {
            my_v = bv;
            my_i = bi;
        }
        if (j == 0) top = bv;
    }

    const float z = lane < k ? expf(my_v - top) : 0.0f;
    float s = z;
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane < k) {
        topk_idx[t * k + lane] = my_i;
        topk_w[t * k + lane] = z / s;
    }
}

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int waves_per_block = 4;
    const dim3 grid((unsigned)((T + waves_per_block - 1) / waves_per_block));
    const dim3 block(waves_per_block * kWave);
    const int nv = (E + kWave - 1) / kWave;
#define MOE_ROUTE_CASE(N)                                                                  \
    if (nv <= N) {                                                                         \
        hipLaunchKernelGGL(route_topk_kernel<N>, grid, block, 0, stream, logits, T, E, k,  \
                           topk_idx, topk_w);                                              \
        return hipGetLastError();                                                          \
    }
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
    return hipErrorInvalidValue;
}

}  // namespace moe
