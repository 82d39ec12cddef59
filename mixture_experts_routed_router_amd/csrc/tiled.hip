// tiled.hip -- the row-pair tiled layout of bf16 matrices, and conversions to and
// from row-major.
//
// A [R, C] matrix (R even, C a multiple of 32) is stored as 2 x 32 blocks of 128
// bytes: element (r, c) sits at
//     ((r / 2) * (C / 32) + c / 32) * 64 + (r % 2) * 32 + c % 32.
// The grouped GEMMs stream their operands through LDS in k stages of 32 columns
// (64 bytes of a row-major row); in this layout one stage's pieces of two
// neighbouring rows fill one whole 128-byte line, so each direct-to-LDS load
// touches half as many lines, which lifts the per-CU operand stream that bounds
// those kernels [Halo "Performance", Levers that help: one grouped matmul over
// all experts -- the layout keeps that, and only changes the order of its
// operands in memory].
#include "common.hpp"

namespace moe {

constexpr int kTileThreads = 256;

// One 16-byte piece (8 elements) per thread and step: piece q = (r, c8) of the
// row-major matrix; its place in the tiled one is block (r/2, c8/4), half r%2,
// 16-byte slot c8%4.
template <bool TO_TILED>
__global__ __launch_bounds__(kTileThreads) void tile_rows_kernel(const uint4* __restrict__ src, int64_t rows,
                                                                 int cols, uint4* __restrict__ dst) {
    MOE_DEBUG_GUARD();
    const int ppr = cols / 8;
    const int64_t total = rows * (int64_t)ppr;
    const int64_t stride = (int64_t)gridDim.x * kTileThreads;
    for (int64_t q = (int64_t)blockIdx.x * kTileThreads + threadIdx.x; q < total; q += stride) {
        const int64_t r = q / ppr;
        const int c = (int)(q - r * ppr);
        const int64_t t = ((r >> 1) * (ppr >> 2) + (c >> 2)) * 8 + (r & 1) * 4 + (c & 3);
        if (TO_TILED) dst[t] = src[q];
        else dst[q] = src[t];
    }
}

hipError_t launch_tile_rows(const uint16_t* src, int64_t rows, int cols, uint16_t* dst, bool to_tiled,
                            hipStream_t stream) {
    const int64_t total = rows * (int64_t)(cols / 8);
    if (total == 0) return hipGetLastError();
    const int64_t want = (total + kTileThreads - 1) / kTileThreads;
    const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
    if (to_tiled)
        hipLaunchKernelGGL(tile_rows_kernel<true>, dim3(grid), dim3(kTileThreads), 0, stream, (const uint4*)src,
                           rows, cols, (uint4*)dst);
    else
        hipLaunchKernelGGL(tile_rows_kernel<false>, dim3(grid), dim3(kTileThreads), 0, stream, (const uint4*)src,
                           rows, cols, (uint4*)dst);
    return hipGetLastError();
}

// FP8 codes [R, K] (R % 4 == 0, K % 32 == 0) in 4-row tiled order: 4 x 32-byte
// blocks, code (r, c) at ((r / 4) * (K / 32) + c / 32) * 128 + (r % 4) * 32 + c % 32.
// Thread step: 16-byte piece q = (r, c16) -> slot ((r/4)(K/32) + c16/2) * 8 + (r%4) * 2 + c16 % 2.
template <bool TO_TILED>
__global__ __launch_bounds__(kTileThreads) void tile_quads_kernel(const uint4* __restrict__ src, int64_t rows,
                                                                  int cols, uint4* __restrict__ dst) {
    MOE_DEBUG_GUARD();
    const int ppr = cols / 16;
    const int64_t total = rows * (int64_t)ppr;
    const int64_t stride = (int64_t)gridDim.x * kTileThreads;
    for (int64_t q = (int64_t)blockIdx.x * kTileThreads + threadIdx.x; q < total; q += stride) {
        const int64_t r = q / ppr;
        const int c = (int)(q - r * ppr);
        const int64_t t = ((r >> 2) * (ppr >> 1) + (c >> 1)) * 8 + (r & 3) * 2 + (c & 1);
        if (TO_TILED) dst[t] = src[q];
        else dst[q] = src[t];
    }
}

hipError_t launch_tile_fp8_rows(const uint8_t* src, int64_t rows, int cols, uint8_t* dst, bool to_tiled,
                                hipStream_t stream) {
    const int64_t total = rows * (int64_t)(cols / 16);
    if (total == 0) return hipGetLastError();
    const int64_t want = (total + kTileThreads - 1) / kTileThreads;
    const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
    if (to_tiled)
        hipLaunchKernelGGL(tile_quads_kernel<true>, dim3(grid), dim3(kTileThreads), 0, stream, (const uint4*)src,
                           rows, cols, (uint4*)dst);
    else
        hipLaunchKernelGGL(tile_quads_kernel<false>, dim3(grid), dim3(kTileThreads), 0, stream, (const uint4*)src,
                           rows, cols, (uint4*)dst);
    return hipGetLastError();
}

}  // namespace moe
