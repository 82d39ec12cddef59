// grouped_gemm.hip -- the grouped GEMM kernel and its launchers (the device code
// is in grouped_gemm_core.hpp).
#include "grouped_gemm_core.hpp"

namespace moe {

template <bool GLU, bool GATHER, bool W8, bool SWB, bool PK = false>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const void* __restrict__ W, const float* __restrict__ w_scale, const int32_t* __restrict__ offsets,
    int E, int K, int N, uint16_t* __restrict__ C, const uint16_t* __restrict__ gu, float glu_limit,
    int rows_max) {
    MOE_DEBUG_GUARD();
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsElems];
    __shared__ int32_t tile_start[kMaxE + 1];
    __shared__ int32_t seg_start[kMaxE + 1];
    __shared__ int32_t scan_tmp[kWaves];
    __shared__ __attribute__((aligned(16))) int32_t tok_lds[GATHER ? 2 * kWaves * kTokSlots : 1];
    const GemmShared sh{lds, tile_start, seg_start, scan_tmp, tok_lds};
    grouped_gemm_body<GLU, GATHER, W8, SWB, PK>(sh, A, row_token, W, w_scale, offsets, E, K, N, C, gu, glu_limit,
                                                rows_max, blockIdx.x, gridDim.x);
}

static int g_cu_count[64];

static int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (g_cu_count[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_cu_count[dev] = n;
    }
    return g_cu_count[dev];
}

static unsigned persistent_grid() {
    // one workgroup of 8 waves per CU (128 KB of the 160 KB LDS), a multiple of the 8 XCDs
    const int n = cu_count();
    return (unsigned)((n + 7) / 8 * 8);
}

// scale == NULL: bf16 weights; otherwise FP8 (E4M3) weights with one scale per 64 W rows.
hipError_t launch_grouped_glu_gemm(const uint16_t* x_perm, const void* w_gu, const float* scale,
                                   const int32_t* offsets, int E, int H, int I, uint16_t* h, int rows_max,
                                   hipStream_t stream) {
    if (scale)
        hipLaunchKernelGGL((grouped_gemm_kernel<true, false, true, false>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, x_perm, (const int32_t*)nullptr, w_gu, scale,
                           offsets, E, H, I, h, (const uint16_t*)nullptr, INFINITY, rows_max);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<true, false, false, false>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, x_perm, (const int32_t*)nullptr, w_gu, scale,
                           offsets, E, H, I, h, (const uint16_t*)nullptr, INFINITY, rows_max);
    return hipGetLastError();
}

hipError_t launch_grouped_glu_gemm_gather(const uint16_t* x, const int32_t* row_token, const void* w_gu,
                                          const float* scale, const int32_t* offsets, int E, int H,
                                          int I, uint16_t* h, int rows_max, hipStream_t stream) {
    if (scale)
        hipLaunchKernelGGL((grouped_gemm_kernel<true, true, true, false>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, x, row_token, w_gu, scale, offsets, E, H, I, h,
                           (const uint16_t*)nullptr, INFINITY, rows_max);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<true, true, false, false>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, x, row_token, w_gu, scale, offsets, E, H, I, h,
                           (const uint16_t*)nullptr, INFINITY, rows_max);
    return hipGetLastError();
}

hipError_t launch_grouped_down_gemm(const uint16_t* h, const void* w_d, const float* scale,
                                    const int32_t* offsets, int E, int H, int I, uint16_t* y, int rows_max,
                                    hipStream_t stream) {
    if (scale)
        hipLaunchKernelGGL((grouped_gemm_kernel<false, false, true, false>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, h, (const int32_t*)nullptr, w_d, scale,
                           offsets, E, I, H, y, (const uint16_t*)nullptr, INFINITY, rows_max);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<false, false, false, false>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, h, (const int32_t*)nullptr, w_d, scale,
                           offsets, E, I, H, y, (const uint16_t*)nullptr, INFINITY, rows_max);
    return hipGetLastError();
}

// Tiled operands: the weights (bf16 in row pairs, or FP8 codes in row quads, with
// `scale` non-NULL) and, unless gathered, A in 2 x 32 blocks (the layouts
// moe_tile_rows / moe_tile_fp8_rows write); the gate/up GEMM writes h in row-pair
// order, the down GEMM writes y row-major.
hipError_t launch_grouped_glu_gemm_tiled(const uint16_t* x_perm_t, const void* w_gu_t, const float* scale,
                                         const int32_t* offsets, int E, int H, int I, uint16_t* h_t, int rows_max,
                                         hipStream_t stream) {
    if (scale)
        hipLaunchKernelGGL((grouped_gemm_kernel<true, false, true, false, true>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, x_perm_t, (const int32_t*)nullptr, w_gu_t, scale, offsets,
                           E, H, I, h_t, (const uint16_t*)nullptr, INFINITY, rows_max);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<true, false, false, false, true>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, x_perm_t, (const int32_t*)nullptr, w_gu_t, scale, offsets,
                           E, H, I, h_t, (const uint16_t*)nullptr, INFINITY, rows_max);
    return hipGetLastError();
}

// (bf16 weights only: the gathering kernel with tiled FP8 weights runs out of SGPRs)
hipError_t launch_grouped_glu_gemm_gather_tiled(const uint16_t* x, const int32_t* row_token, const void* w_gu_t,
                                                const float* scale, const int32_t* offsets, int E, int H, int I,
                                                uint16_t* h_t, int rows_max, hipStream_t stream) {
    if (scale) return hipErrorInvalidValue;
    hipLaunchKernelGGL((grouped_gemm_kernel<true, true, false, false, true>), dim3(persistent_grid()),
                       dim3(kGemmThreads), 0, stream, x, row_token, w_gu_t, scale, offsets, E, H, I, h_t,
                       (const uint16_t*)nullptr, INFINITY, rows_max);
    return hipGetLastError();
}

hipError_t launch_grouped_down_gemm_tiled(const uint16_t* h_t, const void* w_d_t, const float* scale,
                                          const int32_t* offsets, int E, int H, int I, uint16_t* y, int rows_max,
                                          hipStream_t stream) {
    if (scale)
        hipLaunchKernelGGL((grouped_gemm_kernel<false, false, true, false, true>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, h_t, (const int32_t*)nullptr, w_d_t, scale, offsets, E,
                           I, H, y, (const uint16_t*)nullptr, INFINITY, rows_max);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<false, false, false, false, true>), dim3(persistent_grid()),
                           dim3(kGemmThreads), 0, stream, h_t, (const int32_t*)nullptr, w_d_t, scale, offsets, E,
                           I, H, y, (const uint16_t*)nullptr, INFINITY, rows_max);
    return hipGetLastError();
}

// dgu = SwiGLU backward of dh = dy W_d^T-as-stored, without writing dh: the plain
// GEMM over W_d_t [E, I, H] (K = H, N = I) whose epilogue reads gu [P_max, 2I].
hipError_t launch_grouped_gemm_swiglu_bwd(const uint16_t* dy, const uint16_t* w_d_t, const uint16_t* gu,
                                          const int32_t* offsets, int E, int H, int I, uint16_t* dgu,
                                          int rows_max, hipStream_t stream) {
    hipLaunchKernelGGL((grouped_gemm_kernel<false, false, false, true>), dim3(persistent_grid()),
                       dim3(kGemmThreads), 0, stream, dy, (const int32_t*)nullptr, (const void*)w_d_t,
                       (const float*)nullptr, offsets, E, H, I, dgu, gu, INFINITY, rows_max);
    return hipGetLastError();
}

// The gate/up GEMM with a clamped SwiGLU in its epilogue: h = silu(min(g, limit)) *
// clip(u, -limit, limit), bf16 x_perm and weights.
hipError_t launch_grouped_glu_gemm_clamped(const uint16_t* x_perm, const uint16_t* w_gu, const int32_t* offsets,
                                           int E, int H, int I, float limit, uint16_t* h, int rows_max,
                                           hipStream_t stream) {
    hipLaunchKernelGGL((grouped_gemm_kernel<true, false, false, false>), dim3(persistent_grid()),
                       dim3(kGemmThreads), 0, stream, x_perm, (const int32_t*)nullptr, (const void*)w_gu,
                       (const float*)nullptr, offsets, E, H, I, h, (const uint16_t*)nullptr, limit, rows_max);
    return hipGetLastError();
}

}  // namespace moe
