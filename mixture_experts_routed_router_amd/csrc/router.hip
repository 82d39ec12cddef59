// router.hip -- the router projection fused with top-k routing: logits = x W_r
// are formed 32 tokens at a time in registers and LDS and never reach HBM
// (unless asked for) [PocketLLM "Qwen4-Exp Heterogeneous TP4 Performance",
// Remaining prefill attribution: the router is a phase of its own; prime-rl
// PR 3885, Changes: top-k weights feed the layer].
//
// The fp32 router weight W_r [H, E] is split once per weight update into two
// bf16 matrices stored expert-major, W_hi = bf16(W_r) and W_lo = bf16(W_r - W_hi)
// ([E, H] each), so x W_r = x W_hi + x W_lo runs on bf16 MFMAs with fp32
// accumulation: x is bf16 and exact, W_hi + W_lo carries 16 significant bits of
// each weight, so the logits are within about 2^-16 relative of the fp32
// projection per product.
//
// One workgroup of four waves per 32 tokens: wave w computes the 32-expert
// blocks w, w+4, ... (v_mfma_f32_32x32x16_bf16, tokens as rows, experts as
// columns, k over H), writes them to an LDS tile [32][E rounded up to 32], and
// after a barrier each token's 8 lanes run the routing step's top-k on its LDS
// row (topk_core.hpp).  Splitting k over more waves per workgroup (2 or 4
// groups, partial tiles added in a fixed order) measured no faster: the time
// goes to streaming W_hi and W_lo through each workgroup, not to load latency.
#include "topk_core.hpp"

namespace moe {

constexpr int kRouterThreads = 256;
constexpr int kRouterTokens = 32;
constexpr int kRouterDepth = 4;  // k steps of loads in flight per wave (divides H / 16)

__global__ __launch_bounds__(256) void router_prepare_kernel(const float* __restrict__ w, int H, int E,
                                                             uint16_t* __restrict__ w_hi,
                                                             uint16_t* __restrict__ w_lo) {
    MOE_DEBUG_GUARD();
    const int64_t n = (int64_t)H * E;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = i / H, h = i - e * H;  // output [E, H]
        const float v = w[h * E + e];
        const uint32_t hi = f32_to_bf16_rne(v);
        const float rest = v - __uint_as_float(hi << 16);
        w_hi[i] = (uint16_t)hi;
        w_lo[i] = (uint16_t)f32_to_bf16_rne(rest);
    }
}

template <int KL>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_hi, const uint16_t* __restrict__ w_lo,
    int64_t T, int H, int E, int k, float* __restrict__ logits_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
    MOE_DEBUG_GUARD();
    extern __shared__ __attribute__((aligned(16))) float lg[];  // [32][ep]
    const int ep = (E + 31) / 32 * 32;
    const int nblk = ep / 32;
    const int64_t t0 = (int64_t)blockIdx.x * kRouterTokens;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int lr = lane & 31, kg = 8 * (lane >> 5);
    // this lane's token row (past the last token: the last one; never stored)
    const int64_t tr = t0 + lr < T ? t0 + lr : T - 1;
    const uint16_t* xa = x + tr * H + kg;
    const int nsteps = H / 16;  // a multiple of kRouterDepth (H % 64 == 0)
    for (int b = wave; b < nblk; b += kRouterThreads / kWave) {
        // k steps of 16 through a ring of kRouterDepth register slots (step s in
        // slot s % kRouterDepth, refilled right after its MFMAs, the scheduling
        // barriers keeping it so), two accumulators so that consecutive MFMAs do
        // not wait on each other
        floatx16_t acc0, acc1;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.0f;
        {
            const int er = b * 32 + lr < E ? b * 32 + lr : E - 1;  // this lane's expert row
            const uint16_t* wh = w_hi + (int64_t)er * H + kg;
            const uint16_t* wl = w_lo + (int64_t)er * H + kg;
            bf16x8_t ra[kRouterDepth], rh[kRouterDepth], rl[kRouterDepth];
#pragma unroll
            for (int d = 0; d < kRouterDepth; ++d) {
                ra[d] = *(const bf16x8_t*)(xa + 16 * d);
                rh[d] = *(const bf16x8_t*)(wh + 16 * d);
                rl[d] = *(const bf16x8_t*)(wl + 16 * d);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int s0 = 0; s0 < nsteps; s0 += kRouterDepth) {
#pragma unroll
                for (int d = 0; d < kRouterDepth; ++d) {
                    floatx16_t& acc = (d & 1) ? acc1 : acc0;
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[d], rh[d], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[d], rl[d], acc, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    // past the last step: re-read the last one (in bounds, never used)
                    const int sn = s0 + d + kRouterDepth < nsteps ? s0 + d + kRouterDepth : nsteps - 1;
                    ra[d] = *(const bf16x8_t*)(xa + 16 * sn);
                    rh[d] = *(const bf16x8_t*)(wh + 16 * sn);
                    rl[d] = *(const bf16x8_t*)(wl + 16 * sn);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        // MFMA 32x32 output: lane l, register r -> token row (r/4)*8 + (l/32)*4 + r%4, expert l%32
        const int col = b * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = (r / 4) * 8 + (lane >> 5) * 4 + r % 4;
            lg[row * ep + col] = col < E ? acc0[r] + acc1[r] : -INFINITY;
        }
    }
    __syncthreads();
    if (logits_out) {
        for (int i = threadIdx.x; i < kRouterTokens * E; i += kRouterThreads) {
            const int row = i / E, col = i - row * E;
            if (t0 + row < T) logits_out[(t0 + row) * E + col] = lg[row * ep + col];
        }
    }
    // 8 lanes per token: token tid / 8 of the tile
    const int tok = threadIdx.x / 8, sub = threadIdx.x & 7;
    const int64_t t = t0 + tok;
    const bool live = t < T;
    topk_token<KL, 4, 8>(lg + tok * ep, live, E, k, sub, topk_idx + t * k, topk_w + t * k);
}

hipError_t launch_router_prepare(const float* w, int H, int E, uint16_t* w_hi, uint16_t* w_lo, hipStream_t stream) {
    const int64_t n = (int64_t)H * E;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(router_prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, H, E, w_hi, w_lo);
    return hipGetLastError();
}

hipError_t launch_router_topk(const uint16_t* x, const uint16_t* w_hi, const uint16_t* w_lo, int64_t T, int H,
                              int E, int k, float* logits, int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int ep = (E + 31) / 32 * 32;
    const size_t lds = (size_t)kRouterTokens * ep * sizeof(float);
    const dim3 grid((unsigned)((T + kRouterTokens - 1) / kRouterTokens)), block(kRouterThreads);
    // more than 64 KB of dynamic LDS (E > 512) has to be allowed per kernel
#define MOE_ROUTER_CASE(KL)                                                                          \
    if (k <= KL) {                                                                                   \
        if (lds > 65536) {                                                                           \
            const hipError_t e_ = hipFuncSetAttribute((const void*)router_topk_kernel<KL>,            \
                                                      hipFuncAttributeMaxDynamicSharedMemorySize,    \
                                                      (int)lds);                                     \
            if (e_ != hipSuccess) return e_;                                                         \
        }                                                                                            \
        hipLaunchKernelGGL((router_topk_kernel<KL>), grid, block, lds, stream, x, w_hi, w_lo, T, H, E, k, \
                           logits, topk_idx, topk_w);                                                \
        return hipGetLastError();                                                                    \
    }
    MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(12)  // k = 9..12 (top-10 of 512): shorter lists than 16
    MOE_ROUTER_CASE(16)
    MOE_ROUTER_CASE(32)
#undef MOE_ROUTER_CASE
    return hipErrorInvalidValue;
}

}  // namespace moe
