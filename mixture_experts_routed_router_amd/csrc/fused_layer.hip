// fused_layer.hip -- the routed-expert layer after routing as one persistent
// kernel: counting sort, scan, scatter, gate/up GEMM (token rows read in place),
// down GEMM and combine, separated by grid-wide barriers [prime-rl PR 3885,
// Changes: the fused "Mega MoE" op that runs dispatch, experts and combine as one
// kernel].
//
// One workgroup per CU (512 threads, the grouped GEMM's shape), launched
// cooperatively so that all of them are resident at once. The phases run the same
// device code as the separate kernels (permute_core.hpp, grouped_gemm_core.hpp,
// combine_core.hpp), so every output equals, bit for bit, that of moe_permute
// (layout only) + moe_grouped_glu_gemm_gather + moe_grouped_down_gemm +
// moe_combine. The page found its fused op slower than the split path on one
// node; this one exists to measure that trade on this chip (no launch gaps, but
// every phase boundary is a grid barrier with a device-wide cache write-back).
//
// The grid barrier: each workgroup makes its writes visible device-wide (an
// agent-scope fence by every thread; the L2s are per XCD), thread 0 adds 1 to a
// counter in the workspace and polls it until every workgroup of this barrier
// has arrived, then every thread fences again before reading. Polls are bounded:
// a workgroup that waits past the limit stores a nonzero error word and leaves,
// and every workgroup leaves as soon as it sees that word, so no wave can spin
// forever whatever happens (moe_fused_layer_status reports it).
#include "combine_core.hpp"
#include "grouped_gemm_core.hpp"
#include "permute_core.hpp"

namespace moe {

constexpr int kFusedThreads = kGemmThreads;  // 512
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr uint32_t kSpinLimit = 1u << 22;    // polls of ~0.3 us: about a second

struct FusedArgs {
    const uint16_t* x;          // [T, H]
    const int32_t* topk_idx;    // [T, k]
    const float* topk_w;        // [T, k]
    const uint16_t* w_gu;       // [E, 2I, H]
    const uint16_t* w_d;        // [E, H, I]
    int64_t T;
    int H, E, k, I, align;
    int64_t P_max;
    int64_t nchunks;
    int32_t* counts;
    int32_t* offsets;
    int32_t* route_row;
    int32_t* row_token;
    uint16_t* h;                // [P_max, I]
    uint16_t* y;                // [P_max, H]
    uint16_t* out;              // [T, H]
    uint32_t* bar;              // workspace: barrier counter
    int32_t* err;               // workspace: error word (0: none)
    int32_t* hist;              // workspace: [nchunks][E]
};

// Arrive, wait for all `nblk` workgroups, return whether the barrier completed.
__device__ __forceinline__ bool grid_sync(const FusedArgs& a, uint32_t& gen, uint32_t nblk) {
    __threadfence();  // this thread's writes reach the device-coherent level
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t target = (gen + 1) * nblk;
        __hip_atomic_fetch_add(a.bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        for (uint32_t spins = 0;; ++spins) {
            if (__hip_atomic_load(a.bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
            if (__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
            if (spins >= kSpinLimit) {
                __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
    }
    ++gen;
    __syncthreads();
    __threadfence();  // and other workgroups' writes are seen from here on
    return __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
}

__global__ void fused_layer_reset_kernel(uint32_t* bar, int32_t* err) {
    if (threadIdx.x == 0) {
        *bar = 0u;
        *err = 0;
    }
}

template <int KB>
__global__ __launch_bounds__(kFusedThreads, 1) void fused_layer_kernel(FusedArgs a) {
    MOE_DEBUG_GUARD();
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsElems];
    __shared__ int32_t tile_start[kMaxE + 1];
    __shared__ int32_t seg_start[kMaxE + 1];
    __shared__ int32_t scan_tmp[kWaves];
    __shared__ __attribute__((aligned(16))) int32_t tok_lds[2 * kWaves * kTokSlots];
    const GemmShared sh{lds, tile_start, seg_start, scan_tmp, tok_lds};
    const uint32_t nblk = gridDim.x;
    const int blk = blockIdx.x, wave = threadIdx.x / kWave;
    const int64_t gwave = (int64_t)blk * kFusedWaves + wave, nwaves = (int64_t)nblk * kFusedWaves;
    const int E = a.E;
    const int64_t R = a.T * a.k;
    // phases 1-3 use the GEMM ring as scratch: per-wave [E] arrays, then the
    // offsets [E+1], the wave totals and the scan's partial sums
    int32_t* scratch = (int32_t*)lds;
    int32_t* wave_arr = scratch + wave * E;
    int32_t* off = scratch + kFusedWaves * E;
    int32_t* wtot = off + E + 1;
    int32_t(*part)[kWave] = (int32_t(*)[kWave])(wtot + kFusedWaves);
    uint32_t gen = 0;

    // 1. per-chunk expert histograms, one wavefront per chunk of 256 routes
    for (int64_t c = gwave; c < a.nchunks; c += nwaves) hist_chunk(a.topk_idx, R, E, c, wave_arr, a.hist + c * E);
    if (!grid_sync(a, gen, nblk)) return;

    // 2. counts and each chunk's earlier routes per expert, a workgroup per 64 experts
    for (int g = blk; g < (E + kWave - 1) / kWave; g += (int)nblk) {
        scan_group<kFusedWaves>(a.hist, a.nchunks, E, a.counts, g, part);
        __syncthreads();
    }
    if (!grid_sync(a, gen, nblk)) return;

    // 3. padded offsets (every workgroup; workgroup 0 publishes them), pad rows'
    // row_token, and route_row / row_token of every route
    padded_offsets(a.counts, E, a.align, off, wtot);
    if (blk == 0)
        for (int e = threadIdx.x; e <= E; e += kFusedThreads) a.offsets[e] = off[e];
    pad_row_tokens(a.counts, off, E, a.P_max, blk, nblk, kFusedThreads, a.row_token);
    for (int64_t c = gwave; c < a.nchunks; c += nwaves)
        scatter_chunk<kSteps>(a.topk_idx, R, E, a.k, c, a.hist, off, wave_arr, a.route_row, a.row_token, kChunk);
    if (!grid_sync(a, gen, nblk)) return;

    // 4. gate/up GEMM with SwiGLU, token rows of x read through row_token
    grouped_gemm_body<true, true, false, false>(sh, a.x, a.row_token, a.w_gu, nullptr, a.offsets, E, a.H, a.I, a.h,
                                                nullptr, INFINITY, (int)a.P_max, blk, (int)nblk);
    if (!grid_sync(a, gen, nblk)) return;

    // 5. down GEMM
    grouped_gemm_body<false, false, false, false>(sh, a.h, nullptr, a.w_d, nullptr, a.offsets, E, a.I, a.H, a.y,
                                                  nullptr, INFINITY, (int)a.P_max, blk, (int)nblk);
    if (!grid_sync(a, gen, nblk)) return;

    // 6. combine, one wavefront per token
    for (int64_t t = gwave; t < a.T; t += nwaves)
        combine_token<KB>((const uint4*)a.y, a.route_row, a.topk_w, t, a.H / 8, a.k, a.P_max, (uint4*)a.out);
}

// workspace: [0, 256) control words, then the histogram
constexpr size_t kFusedControlBytes = 256;

size_t fused_layer_workspace_bytes(int64_t T, int k, int E) {
    const size_t hist = (size_t)((T * k + kChunk - 1) / kChunk) * (size_t)E * sizeof(int32_t);
    return kFusedControlBytes + (hist + 255) / 256 * 256;
}

int fused_layer_grid() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    return (n + 7) / 8 * 8;
}

hipError_t launch_fused_layer(const uint16_t* x, const int32_t* topk_idx, const float* topk_w, const uint16_t* w_gu,
                              const uint16_t* w_d, int64_t T, int H, int E, int k, int I, int align, int64_t P_max,
                              int32_t* counts, int32_t* offsets, int32_t* route_row, int32_t* row_token,
                              uint16_t* h, uint16_t* y, uint16_t* out, void* workspace, hipStream_t stream) {
    int dev = 0, coop = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (err != hipSuccess) return err;
    if (!coop) return hipErrorNotSupported;
    FusedArgs a;
    a.x = x;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.w_gu = w_gu;
    a.w_d = w_d;
    a.T = T;
    a.H = H;
    a.E = E;
    a.k = k;
    a.I = I;
    a.align = align;
    a.P_max = P_max;
    a.nchunks = (T * k + kChunk - 1) / kChunk;
    a.counts = counts;
    a.offsets = offsets;
    a.route_row = route_row;
    a.row_token = row_token;
    a.h = h;
    a.y = y;
    a.out = out;
    a.bar = (uint32_t*)workspace;
    a.err = (int32_t*)workspace + 1;
    a.hist = (int32_t*)((char*)workspace + kFusedControlBytes);
    hipLaunchKernelGGL(fused_layer_reset_kernel, dim3(1), dim3(64), 0, stream, a.bar, a.err);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    void* args[] = {&a};
    const dim3 grid((unsigned)fused_layer_grid()), block(kFusedThreads);
    if (k <= 8)
        return hipLaunchCooperativeKernel((const void*)fused_layer_kernel<8>, grid, block, args, 0, stream);
    return hipLaunchCooperativeKernel((const void*)fused_layer_kernel<16>, grid, block, args, 0, stream);
}

hipError_t fused_layer_read_error(const void* workspace, int32_t* code, hipStream_t stream) {
    hipError_t e = hipMemcpyAsync(code, (const int32_t*)workspace + 1, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(stream);
}

}  // namespace moe
