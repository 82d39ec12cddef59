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

// 16 lanes per token for wide rows, and when there are too few tokens to give
// every SIMD two waves at 8 lanes per token (shorter chains, more waves)
static bool wide_rows(int64_t T, int E) { return E >= 256 || T <= 16384; }

// Routing with the permute's histogram: the same top-k, and each workgroup's
// routes counted per expert -- hist[b][e] = routes to e among tokens
// [b * tpw, (b + 1) * tpw), tpw = the workgroup's tokens -- so the permute starts
// from these counts instead of re-reading topk_idx to count them [prime-rl PR
// 3885, Changes: a single-pass local layout; PocketLLM "Qwen4-Exp Heterogeneous
// TP4 Performance", Remaining prefill attribution: the router as a phase of its
// own]. Each wave counts a quarter of the workgroup's routes into its own LDS
// histogram with the ballot match of the permute (no atomics); the four are
// summed in a fixed order.
int route_hist_tokens_per_chunk(int64_t T, int E) { return kRouteThreads / (wide_rows(T, E) ? 16 : 8); }

template <int KL, int VEC, int LPT>
__global__ __launch_bounds__(kRouteThreads) void route_topk_hist_kernel(const float* __restrict__ logits,
                                                                        int64_t T, int E, int k,
                                                                        int32_t* __restrict__ topk_idx,
                                                                        float* __restrict__ topk_w,
                                                                        int32_t* __restrict__ hist) {
    MOE_DEBUG_GUARD();
    constexpr int TPW = kRouteThreads / LPT;             // tokens per workgroup
    __shared__ int32_t ids[TPW * 32];                    // k <= 32
    extern __shared__ int32_t wave_hist[];               // [4][E]
    const int sub = lane_id() & (LPT - 1);
    const int64_t t0 = (int64_t)blockIdx.x * TPW;
    const int64_t t = t0 + threadIdx.x / LPT;
    const bool live = t < T;
    const int tl = threadIdx.x / LPT;
    topk_token<KL, VEC, LPT>(logits + (live ? t : 0) * E, live, E, k, sub, topk_idx + t * k, topk_w + t * k,
                             ids + tl * k);
    const int wave = threadIdx.x / kWave, lane = lane_id();
    int32_t* h = wave_hist + wave * E;
    for (int e = lane; e < E; e += kWave) h[e] = 0;
    __syncthreads();
    const int64_t ntok = T - t0 < TPW ? T - t0 : TPW;
    const int routes = (int)ntok * k;
    const int nbits = E <= 1 ? 0 : 32 - __clz(E - 1);
    for (int r0 = wave * kWave; r0 < routes; r0 += kRouteThreads) {  // wave-uniform trip count
        const int r = r0 + lane;
        const bool active = r < routes && (uint32_t)ids[r < routes ? r : 0] < (uint32_t)E;
        const uint32_t key = active ? (uint32_t)ids[r] : 0u;
        const uint64_t peers = match_peers(key, nbits, active);
        if (active && (__ffsll((unsigned long long)peers) - 1) == lane) h[key] += __popcll(peers);
    }
    __syncthreads();
    int32_t* out = hist + (int64_t)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += kRouteThreads)
        out[e] = wave_hist[e] + wave_hist[E + e] + wave_hist[2 * E + e] + wave_hist[3 * E + e];
}

hipError_t launch_route_topk_hist(const float* logits, int64_t T, int E, int k, int32_t* topk_idx, float* topk_w,
                                  int32_t* hist, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const bool vec4 = (E % 4) == 0 && ((uintptr_t)logits % 16) == 0;
    const bool wide = wide_rows(T, E);
    const int64_t blocks = (T + route_hist_tokens_per_chunk(T, E) - 1) / route_hist_tokens_per_chunk(T, E);
    const size_t lds = 4 * (size_t)E * sizeof(int32_t);
#define MOE_ROUTE_LAUNCH(KL, VEC, LPT)                                                                  \
    hipLaunchKernelGGL((route_topk_hist_kernel<KL, VEC, LPT>), dim3((unsigned)blocks), dim3(kRouteThreads), \
                       lds, stream, logits, T, E, k, topk_idx, topk_w, hist)
#define MOE_ROUTE_CASE(KL)                                                                              \
    if (k <= KL) {                                                                                      \
        if (wide) {                                                                                     \
            if (vec4) MOE_ROUTE_LAUNCH(KL, 4, 16); else MOE_ROUTE_LAUNCH(KL, 1, 16);                    \
        } else {                                                                                        \
            if (vec4) MOE_ROUTE_LAUNCH(KL, 4, 8); else MOE_ROUTE_LAUNCH(KL, 1, 8);                      \
        }                                                                                               \
        return hipGetLastError();                                                                       \
    }
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(12)
    MOE_ROUTE_CASE(16)
    MOE_ROUTE_CASE(32)
#undef MOE_ROUTE_CASE
#undef MOE_ROUTE_LAUNCH
    return hipErrorInvalidValue;
}

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const bool vec4 = (E % 4) == 0 && ((uintptr_t)logits % 16) == 0;
    const bool wide = wide_rows(T, E);
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
