// route_topk.hip -- top-k routing over router logits, 8 or 16 lanes per token
// (the per-token algorithm is in topk_core.hpp).
#include "topk_core.hpp"

namespace moe {

constexpr int kRouteThreads = 256;

template <int KL, int VEC, int LPT>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(const float* __restrict__ logits,
                                                                   int64_t T, int E, int k,
                                                                   int32_t* __restrict__ topk_idx,
                                                                   float* __restrict__ topk_w) {
    MOE_DEBUG_GUARD();
    const int sub = lane_id() & (LPT - 1);
    const int64_t t = ((int64_t)blockIdx.x * kRouteThreads + threadIdx.x) / LPT;
    const bool live = t < T;
    topk_token<KL, VEC, LPT>(logits + (live ? t : 0) * E, live, E, k, sub, topk_idx + t * k, topk_w + t * k);
}

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const bool vec4 = (E % 4) == 0 && ((uintptr_t)logits % 16) == 0;
    // 16 lanes per token for wide rows, and when there are too few tokens to give
    // every SIMD two waves at 8 lanes per token (shorter chains, more waves)
    const bool wide = E >= 256 || T <= 16384;
    const int64_t lanes = T * (wide ? 16 : 8);
    const dim3 grid((unsigned)((lanes + kRouteThreads - 1) / kRouteThreads));
    const dim3 block(kRouteThreads);
#define MOE_ROUTE_LAUNCH(KL, VEC, LPT)                                                              \
    hipLaunchKernelGGL((route_topk_kernel<KL, VEC, LPT>), grid, block, 0, stream, logits, T, E, k,  \
                       topk_idx, topk_w)
#define MOE_ROUTE_CASE(KL)                                                                          \
    if (k <= KL) {                                                                                  \
        if (wide) {                                                                                 \
            if (vec4) MOE_ROUTE_LAUNCH(KL, 4, 16); else MOE_ROUTE_LAUNCH(KL, 1, 16);                \
        } else {                                                                                    \
            if (vec4) MOE_ROUTE_LAUNCH(KL, 4, 8); else MOE_ROUTE_LAUNCH(KL, 1, 8);                  \
        }                                                                                           \
        return hipGetLastError();                                                                   \
    }
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(12)  // k = 9..12 (top-10 of 512): shorter lists than 16
    MOE_ROUTE_CASE(16)
    MOE_ROUTE_CASE(32)
#undef MOE_ROUTE_CASE
#undef MOE_ROUTE_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace moe
