// debug.hip -- the debug build's checks of the preconditions the release kernels
// trust [prime-rl PR 3885, Changes: 32-bit row offsets overflowed silently -- a bad
// index must be reported, not turned into a stray write]. Compiled into the debug
// library only (-DMOE_DEBUG); the release library holds none of this.
//
// Each check kernel reads its input and, if a precondition fails, stores that
// check's code into g_moe_debug_word with ordinary vector stores (every failing
// lane stores the same code; no atomics). Check kernels are enqueued on the
// call's stream before its own kernels; those, and every kernel of later calls,
// begin by reading the word and do nothing once it is nonzero. A check kernel
// also returns at once when the word is already set, so the first failure's code
// is kept until moe_debug_reset.
#include "common.hpp"

#ifdef MOE_DEBUG

namespace moe {

__device__ int32_t g_moe_debug_word = 0;

constexpr int kCheckThreads = 256;

__device__ __forceinline__ void flag(int32_t code) { *(volatile int32_t*)&g_moe_debug_word = code; }

// every value of logits[0 .. n) is finite (code 1)
__global__ __launch_bounds__(kCheckThreads) void debug_check_finite(const float* __restrict__ v, int64_t n) {
    MOE_DEBUG_GUARD();
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kCheckThreads)
        bad |= !__builtin_isfinite(v[i]);
    if (bad) flag(1);
}

// topk_idx [T, k]: every id in [0, E) (code 2) and the k ids of a token distinct (code 3)
__global__ __launch_bounds__(kCheckThreads) void debug_check_topk(const int32_t* __restrict__ idx, int64_t T,
                                                                   int k, int E) {
    MOE_DEBUG_GUARD();
    const int64_t t = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
    if (t >= T) return;
    const int32_t* row = idx + t * k;
    int32_t code = 0;
    for (int j = 0; j < k; ++j) {
        const int32_t e = row[j];
        if (e < 0 || e >= E) code = 2;
        for (int i = 0; i < j && code == 0; ++i)
            if (row[i] == e) code = 3;
    }
    if (code) flag(code);
}

// offsets [E+1] and counts [E] (code 4): offsets[0] == 0, non-decreasing,
// offsets[E] <= P_max, and 0 <= counts[e] <= offsets[e+1] - offsets[e]
__global__ __launch_bounds__(kCheckThreads) void debug_check_offsets(const int32_t* __restrict__ counts,
                                                                      const int32_t* __restrict__ offsets, int E,
                                                                      int64_t P_max) {
    MOE_DEBUG_GUARD();
    bool bad = false;
    for (int e = threadIdx.x; e < E; e += kCheckThreads) {
        const int64_t o0 = offsets[e], o1 = offsets[e + 1];
        if (e == 0 && o0 != 0) bad = true;
        if (o1 < o0 || o1 > P_max) bad = true;
        if (counts) {
            const int64_t c = counts[e];
            if (c < 0 || c > o1 - o0) bad = true;
        }
    }
    if (bad) flag(4);
}

// rows [0 .. n): every value in [lo, hi) (route_row: code 5, row_token: code 6)
__global__ __launch_bounds__(kCheckThreads) void debug_check_range(const int32_t* __restrict__ v, int64_t n,
                                                                    int64_t lo, int64_t hi, int32_t code) {
    MOE_DEBUG_GUARD();
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kCheckThreads) {
        const int64_t x = v[i];
        bad |= x < lo || x >= hi;
    }
    if (bad) flag(code);
}

__global__ void debug_reset_kernel() {
    if (threadIdx.x == 0) flag(0);
}

static unsigned grid_for(int64_t n) {
    const int64_t b = (n + kCheckThreads - 1) / kCheckThreads;
    return (unsigned)(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

hipError_t debug_check_logits(const float* logits, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(debug_check_finite, dim3(grid_for(n)), dim3(kCheckThreads), 0, s, logits, n);
    return hipGetLastError();
}

hipError_t debug_check_ids(const int32_t* idx, int64_t T, int k, int E, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(debug_check_topk, dim3((unsigned)((T + kCheckThreads - 1) / kCheckThreads)),
                       dim3(kCheckThreads), 0, s, idx, T, k, E);
    return hipGetLastError();
}

hipError_t debug_check_layout(const int32_t* counts, const int32_t* offsets, int E, int64_t P_max, hipStream_t s) {
    hipLaunchKernelGGL(debug_check_offsets, dim3(1), dim3(kCheckThreads), 0, s, counts, offsets, E, P_max);
    return hipGetLastError();
}

hipError_t debug_check_rows(const int32_t* v, int64_t n, int64_t lo, int64_t hi, int32_t code, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(debug_check_range, dim3(grid_for(n)), dim3(kCheckThreads), 0, s, v, n, lo, hi, code);
    return hipGetLastError();
}

hipError_t debug_read(int32_t* code, hipStream_t s) {
    hipError_t e = hipMemcpyFromSymbolAsync(code, HIP_SYMBOL(g_moe_debug_word), sizeof(int32_t), 0,
                                            hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(s);
}

hipError_t debug_reset(hipStream_t s) {
    hipLaunchKernelGGL(debug_reset_kernel, dim3(1), dim3(64), 0, s);
    return hipGetLastError();
}

}  // namespace moe

#endif  // MOE_DEBUG
