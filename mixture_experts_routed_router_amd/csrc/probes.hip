// probes.hip -- measurement kernels that give the chip's own roofs beside its
// published ones: a device copy (HBM read + write stream), a read-only stream and
// a register-only bf16 MFMA loop. Neither is part of the layer; the bench reports each kernel's
// roofline fraction against both the spec and these measured roofs [PocketLLM
// "Qwen4-Exp Heterogeneous TP4 Performance", Theoretical ceilings / Hardware roofs:
// measured copy and GEMM roofs quoted beside the spec figures].
#include "common.hpp"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kCopyPieces = 4;  // 16-byte pieces per lane in flight

// dst[i] = src[i] over n 16-byte pieces: grid-stride, kCopyPieces loads issued
// before the stores, non-temporal both ways (every byte is touched once).
__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4_t* __restrict__ src,
                                                                   u32x4_t* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads * kCopyPieces;
    for (int64_t base = (int64_t)blockIdx.x * kProbeThreads * kCopyPieces + threadIdx.x; base < n;
         base += stride) {
        u32x4_t v[kCopyPieces];
#pragma unroll
        for (int u = 0; u < kCopyPieces; ++u) {
            const int64_t i = base + (int64_t)u * kProbeThreads;
            if (i < n) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kCopyPieces; ++u) {
            const int64_t i = base + (int64_t)u * kProbeThreads;
            if (i < n) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

// Read-only stream: the same grid-stride walk as the copy, kCopyPieces non-temporal
// 16-byte loads in flight per lane; each thread XORs what it read and writes the
// result to its own 16 bytes of sink, so every load is live.
constexpr int kReadBlocksPerCu = 8;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_t* __restrict__ src, int64_t n,
                                                                   u32x4_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads * kCopyPieces;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (int64_t base = (int64_t)blockIdx.x * kProbeThreads * kCopyPieces + threadIdx.x; base < n;
         base += stride) {
        u32x4_t v[kCopyPieces];
#pragma unroll
        for (int u = 0; u < kCopyPieces; ++u) {
            const int64_t i = base + (int64_t)u * kProbeThreads;
            v[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kCopyPieces; ++u) acc ^= v[u];
    }
    sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

int probe_read_blocks(int cus) { return cus * kReadBlocksPerCu; }

hipError_t launch_probe_read(const void* src, size_t bytes, void* sink, int cus, hipStream_t stream) {
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)probe_read_blocks(cus)), dim3(kProbeThreads), 0, stream,
                       (const u32x4_t*)src, (int64_t)(bytes / 16), (u32x4_t*)sink);
    return hipGetLastError();
}

// Register-only bf16 MFMA loop: each wave runs kChains independent accumulator
// chains of v_mfma_f32_32x32x16_bf16 (so no MFMA waits on the previous one's
// result), `iters` rounds; the operands depend on the lane so nothing folds, and
// each lane writes the sum of its accumulators so nothing is dead.
constexpr int kChains = 4;
constexpr int kProbeMfmaBlocksPerCu = 2;  // 8 waves per CU, two per SIMD

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(float* __restrict__ sink, int iters) {
    const int lane = lane_id();
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1.0f + 0.001f * (float)((lane + i) & 7));
        b[i] = (__bf16)(0.5f - 0.001f * (float)((lane * 3 + i) & 7));
    }
    floatx16_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = floatx16_t{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, int cus, hipStream_t stream) {
    const int64_t n = (int64_t)(bytes / 16);
    const unsigned grid = (unsigned)(cus * 8);  // 8 workgroups of 256 threads per CU
    hipLaunchKernelGGL(probe_copy_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, (const u32x4_t*)src,
                       (u32x4_t*)dst, n);
    return hipGetLastError();
}

int probe_mfma_blocks(int cus) { return cus * kProbeMfmaBlocksPerCu; }

double probe_mfma_flops(int cus, int iters) {
    // 2 * 32 * 32 * 16 flops per MFMA, kChains per round, per wave
    return 2.0 * 32 * 32 * 16 * (double)kChains * (double)iters * (double)(probe_mfma_blocks(cus) * (kProbeThreads / kWave));
}

hipError_t launch_probe_mfma(float* sink, int iters, int cus, hipStream_t stream) {
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)probe_mfma_blocks(cus)), dim3(kProbeThreads), 0, stream,
                       sink, iters);
    return hipGetLastError();
}

}  // namespace moe
