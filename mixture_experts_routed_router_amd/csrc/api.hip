// api.hip -- the C ABI of the MoE path: argument validation on the host, then
// launches on the caller's stream.  Nothing is enqueued unless every check passes.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/moe_mi355x.h"
#include "common.hpp"

namespace moe {
hipError_t launch_route_topk(const float*, int64_t, int, int, int32_t*, float*, hipStream_t);
hipError_t launch_route_topk_hist(const float*, int64_t, int, int, int32_t*, float*, int32_t*, hipStream_t);
size_t route_hist_workspace_bytes(int64_t T, int E);
hipError_t launch_permute_from_hist(const uint16_t*, const int32_t*, int64_t, int, int, int, int, int64_t, int32_t*,
                                   int32_t*, int32_t*, int32_t*, uint16_t*, void*, hipStream_t);
hipError_t launch_permute(const uint16_t*, const int32_t*, int64_t, int, int, int, int, int64_t,
                          int32_t*, int32_t*, int32_t*, int32_t*, uint16_t*, void*, bool, hipStream_t);
hipError_t launch_tile_rows(const uint16_t*, int64_t, int, uint16_t*, bool, hipStream_t);
hipError_t launch_tile_fp8_rows(const uint8_t*, int64_t, int, uint8_t*, bool, hipStream_t);
hipError_t launch_grouped_glu_gemm_tiled(const uint16_t*, const void*, const float*, const int32_t*, int, int, int,
                                         uint16_t*, int, hipStream_t);
hipError_t launch_grouped_glu_gemm_gather_tiled(const uint16_t*, const int32_t*, const void*, const float*,
                                                const int32_t*, int, int, int, uint16_t*, int, hipStream_t);
hipError_t launch_grouped_down_gemm_tiled(const uint16_t*, const void*, const float*, const int32_t*, int, int, int,
                                          uint16_t*, int, hipStream_t);
size_t permute_workspace_bytes(int64_t R, int E);
size_t permute_scratch_bytes();
hipError_t launch_permute_noalloc(const uint16_t*, const int32_t*, int64_t, int, int, int, int, int64_t, int32_t*,
                                  int32_t*, int32_t*, int32_t*, uint16_t*, hipStream_t);
hipError_t launch_grouped_glu_gemm(const uint16_t*, const void*, const float*, const int32_t*, int,
                                   int, int, uint16_t*, int, hipStream_t);
hipError_t launch_grouped_glu_gemm_gather(const uint16_t*, const int32_t*, const void*, const float*,
                                          const int32_t*, int, int, int, uint16_t*, int, hipStream_t);
hipError_t launch_grouped_down_gemm(const uint16_t*, const void*, const float*, const int32_t*, int,
                                    int, int, uint16_t*, int, hipStream_t);
hipError_t launch_quantize_fp8(const uint16_t*, int64_t, int, int, uint8_t*, float*, hipStream_t);
hipError_t launch_grouped_gemm_small(bool, const uint16_t*, const int32_t*, const void*, const float*,
                                     const int32_t*, int, int, int, uint16_t*, int, hipStream_t);
hipError_t launch_combine_bwd(const uint16_t*, const uint16_t*, const int32_t*, const float*, const int32_t*,
                              const int32_t*, int64_t, int, int, int, int64_t, uint16_t*, float*, hipStream_t);
hipError_t launch_route_bwd(const int32_t*, const float*, const float*, int64_t, int, int, float*, hipStream_t);
hipError_t launch_grouped_glu_gemm_clamped(const uint16_t*, const uint16_t*, const int32_t*, int, int, int, float,
                                           uint16_t*, int, hipStream_t);
hipError_t launch_grouped_gemm_swiglu_bwd(const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, int,
                                          int, int, uint16_t*, int, hipStream_t);
hipError_t launch_swiglu(const uint16_t*, const uint16_t*, const int32_t*, int, int, int64_t, uint16_t*,
                         hipStream_t, bool tiled_out);
hipError_t launch_transpose(const uint16_t*, int64_t, int, int, uint16_t*, hipStream_t);
hipError_t launch_router_prepare(const float*, int, int, uint16_t*, uint16_t*, hipStream_t);
hipError_t launch_router_topk(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int, int, int, float*,
                              int32_t*, float*, hipStream_t);
hipError_t launch_wgrad(const uint16_t*, const uint16_t*, const int32_t*, const int32_t*, int, int, int,
                        int rows_max, float*, hipStream_t, bool a_tiled, bool b_tiled);
hipError_t launch_combine(const uint16_t*, const int32_t*, const float*, int64_t, int, int,
                          int64_t, uint16_t*, hipStream_t);
hipError_t launch_probe_copy(const void*, void*, size_t, int, hipStream_t);
size_t fused_layer_workspace_bytes(int64_t, int, int);
hipError_t launch_fused_layer(const uint16_t*, const int32_t*, const float*, const uint16_t*, const uint16_t*, int64_t,
                              int, int, int, int, int, int64_t, int32_t*, int32_t*, int32_t*, int32_t*, uint16_t*,
                              uint16_t*, uint16_t*, void*, hipStream_t);
hipError_t fused_layer_read_error(const void*, int32_t*, hipStream_t);
hipError_t launch_probe_mfma(float*, int, int, hipStream_t);
hipError_t launch_probe_read(const void*, size_t, void*, int, hipStream_t);
int probe_read_blocks(int);
int probe_mfma_blocks(int);
double probe_mfma_flops(int, int);
#ifdef MOE_DEBUG
hipError_t debug_check_logits(const float*, int64_t, hipStream_t);
hipError_t debug_check_ids(const int32_t*, int64_t, int, int, hipStream_t);
hipError_t debug_check_layout(const int32_t*, const int32_t*, int, int64_t, hipStream_t);
hipError_t debug_check_rows(const int32_t*, int64_t, int64_t, int64_t, int32_t, hipStream_t);
hipError_t debug_read(int32_t*, hipStream_t);
hipError_t debug_reset(hipStream_t);
#endif
}  // namespace moe

namespace {

thread_local char g_err[512];

moe_status fail(moe_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

moe_status ok() {
    g_err[0] = '\0';
    return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Debug build: enqueue a precondition check ahead of the call's kernels (see
// debug.hip); release builds compile these to nothing.
#ifdef MOE_DEBUG
#define DEBUG_CHECK(expr)                                                  \
    do {                                                                   \
        const hipError_t e_ = (expr);                                      \
        if (e_ != hipSuccess) return hip_status(e_, "debug check launch"); \
    } while (0)
#else
#define DEBUG_CHECK(expr) \
    do {                  \
    } while (0)
#endif

#define REQUIRE_PTR(p)                                                             \
    do {                                                                           \
        if (!(p)) return fail(MOE_ERR_NULL_POINTER, "%s is NULL", #p);             \
        if (!aligned16(p))                                                         \
            return fail(MOE_ERR_MISALIGNED_POINTER, "%s is not 16-byte aligned", #p); \
    } while (0)

// Buffers whose size is proportional to T may be NULL when T == 0 (an empty
// allocation has no address); alignment is still required when present.
#define REQUIRE_PTR_UNLESS_EMPTY(p, empty)                                         \
    do {                                                                           \
        if (!(empty)) REQUIRE_PTR(p);                                              \
        else if ((p) && !aligned16(p))                                             \
            return fail(MOE_ERR_MISALIGNED_POINTER, "%s is not 16-byte aligned", #p); \
    } while (0)

moe_status check_ek(int32_t E, int32_t k) {
    if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_INVALID_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_E);
    if (k < 1 || k > MOE_MAX_K || k > E)
        return fail(MOE_ERR_INVALID_SHAPE, "k=%d outside [1, min(E=%d, %d)]", k, E, MOE_MAX_K);
    return MOE_OK;
}

moe_status check_dim64(const char* name, int32_t v) {
    if (v < 64 || v % 64 != 0)
        return fail(MOE_ERR_INVALID_SHAPE, "%s=%d must be a positive multiple of 64", name, v);
    return MOE_OK;
}

// FP8 weights and few rows per expert (P_max <= 64 E): the weight-streaming
// kernel; otherwise 256-row tiles. P_max bounds the layout's rows, so the host
// can choose without knowing the counts.
constexpr int64_t kSmallRowsPerExpert = 64;
bool use_small_m(int64_t P_max, int32_t E, const float* scale) {
    return scale != nullptr && P_max <= kSmallRowsPerExpert * E;
}

// gate/up: C = h from W [E, 2I, H]; down: C = y from W [E, H, I]. scale NULL: bf16 weights.
hipError_t launch_glu(const uint16_t* a, const int32_t* row_token, const void* w, const float* scale,
                      const int32_t* offsets, int32_t E, int32_t H, int32_t I, int64_t P_max, uint16_t* h,
                      hipStream_t stream) {
    if (use_small_m(P_max, E, scale))
        return moe::launch_grouped_gemm_small(true, a, row_token, w, scale, offsets, E, H, I, h, (int)P_max, stream);
    if (row_token)
        return moe::launch_grouped_glu_gemm_gather(a, row_token, w, scale, offsets, E, H, I, h, (int)P_max, stream);
    return moe::launch_grouped_glu_gemm(a, w, scale, offsets, E, H, I, h, (int)P_max, stream);
}

hipError_t launch_down(const uint16_t* h, const void* w, const float* scale, const int32_t* offsets,
                       int32_t E, int32_t H, int32_t I, int64_t P_max, uint16_t* y, hipStream_t stream) {
    if (use_small_m(P_max, E, scale))
        return moe::launch_grouped_gemm_small(false, h, nullptr, w, scale, offsets, E, I, H, y, (int)P_max, stream);
    return moe::launch_grouped_down_gemm(h, w, scale, offsets, E, H, I, y, (int)P_max, stream);
}

// compute units of the current device (256 on an MI355X)
int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

moe_status check_pmax(int64_t P_max) {
    if (P_max < 1 || P_max >= ((int64_t)1 << 31))
        return fail(MOE_ERR_SIZE_OVERFLOW, "P_max=%lld outside [1, 2^31)", (long long)P_max);
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL_POINTER: return "MOE_ERR_NULL_POINTER";
        case MOE_ERR_INVALID_SHAPE: return "MOE_ERR_INVALID_SHAPE";
        case MOE_ERR_INVALID_ALIGN: return "MOE_ERR_INVALID_ALIGN";
        case MOE_ERR_SIZE_OVERFLOW: return "MOE_ERR_SIZE_OVERFLOW";
        case MOE_ERR_MISALIGNED_POINTER: return "MOE_ERR_MISALIGNED_POINTER";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        case MOE_ERR_INVALID_VALUE: return "MOE_ERR_INVALID_VALUE";
        case MOE_ERR_PRECONDITION: return "MOE_ERR_PRECONDITION";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char* moe_last_error_message(void) { return g_err; }

int64_t moe_padded_rows_max(int64_t T, int32_t k, int32_t E, int32_t align) {
    if (T < 0 || k < 1 || E < 1 || align < 1 || T > ((int64_t)1 << 40)) return -1;
    return T * k + (int64_t)E * (align - 1);
}

moe_status moe_permute_workspace_size(int64_t T, int32_t k, int32_t E, size_t* bytes) {
    if (!bytes) return fail(MOE_ERR_NULL_POINTER, "bytes is NULL");
    if (T < 0) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld < 0", (long long)T);
    moe_status s = check_ek(E, k);
    if (s != MOE_OK) return s;
    *bytes = moe::permute_workspace_bytes(T * k, E);
    return ok();
}

moe_status moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
                          float* topk_w, moe_stream_t stream) {
    REQUIRE_PTR_UNLESS_EMPTY(logits, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(topk_idx, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(topk_w, T == 0);
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    moe_status s = check_ek(E, k);
    if (s != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_logits(logits, T * (int64_t)E, (hipStream_t)stream));
    return hip_status(moe::launch_route_topk(logits, T, E, k, topk_idx, topk_w, (hipStream_t)stream),
                      "moe_route_topk launch");
}

static moe_status check_gather(const int32_t* row_token, int64_t T, int32_t H) {
    REQUIRE_PTR(row_token);
    if (T < 1) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld < 1", (long long)T);
    if ((uint64_t)T * (uint64_t)H * 2u >= ((uint64_t)1 << 32))
        return fail(MOE_ERR_SIZE_OVERFLOW, "T*H*2 = %llu bytes of x reach 2^32 (32-bit offsets)",
                    (unsigned long long)((uint64_t)T * (uint64_t)H * 2u));
    return MOE_OK;
}

static moe_status check_permute(const moe_bf16* x, const int32_t* topk_idx, int64_t T, int32_t H, int32_t E,
                                int32_t k, int32_t align, int64_t P_max, const int32_t* expert_counts,
                                const int32_t* expert_offsets, const int32_t* route_row, const int32_t* row_token,
                                const moe_bf16* x_perm) {
    // x_perm == NULL: the layout only (no gather), and x is not read
    REQUIRE_PTR_UNLESS_EMPTY(x, T == 0 || !x_perm);
    REQUIRE_PTR_UNLESS_EMPTY(topk_idx, T == 0);
    REQUIRE_PTR(expert_counts);
    REQUIRE_PTR(expert_offsets);
    REQUIRE_PTR_UNLESS_EMPTY(route_row, T == 0);
    REQUIRE_PTR(row_token);
    REQUIRE_PTR_UNLESS_EMPTY(x_perm, true);
    if (T < 0) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld < 0", (long long)T);
    moe_status s = check_ek(E, k);
    if (s != MOE_OK) return s;
    if ((s = check_dim64("H", H)) != MOE_OK) return s;
    if (align < 1 || align > MOE_MAX_ALIGN || (align & (align - 1)) != 0)
        return fail(MOE_ERR_INVALID_ALIGN, "align=%d is not a power of two in [1, %d]", align, MOE_MAX_ALIGN);
    if ((s = check_pmax(P_max)) != MOE_OK) return s;
    const int64_t need = moe_padded_rows_max(T, k, E, align);
    if (need < 0 || need > P_max)
        return fail(MOE_ERR_SIZE_OVERFLOW, "P_max=%lld < T*k + E*(align-1) = %lld", (long long)P_max,
                    (long long)need);
    return MOE_OK;
}

moe_status moe_permute(const moe_bf16* x, const int32_t* topk_idx, int64_t T, int32_t H, int32_t E,
                       int32_t k, int32_t align, int64_t P_max, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* route_row, int32_t* row_token,
                       moe_bf16* x_perm, void* workspace, size_t workspace_bytes,
                       moe_stream_t stream) {
    moe_status s = check_permute(x, topk_idx, T, H, E, k, align, P_max, expert_counts, expert_offsets, route_row,
                                 row_token, x_perm);
    if (s != MOE_OK) return s;
    REQUIRE_PTR_UNLESS_EMPTY(workspace, T == 0);
    const size_t ws = moe::permute_workspace_bytes(T * k, E);
    if (workspace_bytes < ws)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, ws);
    DEBUG_CHECK(moe::debug_check_ids(topk_idx, T, k, E, (hipStream_t)stream));
    return hip_status(moe::launch_permute(x, topk_idx, T, H, E, k, align, P_max, expert_counts,
                                          expert_offsets, route_row, row_token, x_perm, workspace, false,
                                          (hipStream_t)stream),
                      "moe_permute launch");
}

// ---- row-pair tiled layouts (tiled.hip) ------------------------------------------------

static moe_status check_even_pmax(int64_t P_max) {
    if (P_max & 1) return fail(MOE_ERR_INVALID_SHAPE, "P_max=%lld must be even for row-pair tiled rows", (long long)P_max);
    return MOE_OK;
}

static moe_status tile_or_untile(const moe_bf16* src, int64_t rows, int32_t cols, moe_bf16* dst, bool to_tiled,
                                 moe_stream_t stream) {
    REQUIRE_PTR_UNLESS_EMPTY(src, rows == 0);
    REQUIRE_PTR_UNLESS_EMPTY(dst, rows == 0);
    if (rows < 0 || (rows & 1)) return fail(MOE_ERR_INVALID_SHAPE, "rows=%lld must be even and >= 0", (long long)rows);
    if (cols < 32 || cols % 32 != 0) return fail(MOE_ERR_INVALID_SHAPE, "cols=%d must be a positive multiple of 32", cols);
    if (rows == 0) return ok();  // nothing to do, nothing enqueued
    if (src == dst) return fail(MOE_ERR_INVALID_VALUE, "src and dst must not be the same buffer");
    return hip_status(moe::launch_tile_rows(src, rows, cols, dst, to_tiled, (hipStream_t)stream),
                      to_tiled ? "moe_tile_rows launch" : "moe_untile_rows launch");
}

moe_status moe_tile_rows(const moe_bf16* src, int64_t rows, int32_t cols, moe_bf16* dst, moe_stream_t stream) {
    return tile_or_untile(src, rows, cols, dst, true, stream);
}

moe_status moe_untile_rows(const moe_bf16* src, int64_t rows, int32_t cols, moe_bf16* dst, moe_stream_t stream) {
    return tile_or_untile(src, rows, cols, dst, false, stream);
}

moe_status moe_permute_tiled(const moe_bf16* x, const int32_t* topk_idx, int64_t T, int32_t H, int32_t E,
                             int32_t k, int32_t align, int64_t P_max, int32_t* expert_counts,
                             int32_t* expert_offsets, int32_t* route_row, int32_t* row_token,
                             moe_bf16* x_perm, void* workspace, size_t workspace_bytes,
                             moe_stream_t stream) {
    moe_status s = check_permute(x, topk_idx, T, H, E, k, align, P_max, expert_counts, expert_offsets, route_row,
                                 row_token, x_perm);
    if (s != MOE_OK) return s;
    if ((s = check_even_pmax(P_max)) != MOE_OK) return s;
    REQUIRE_PTR_UNLESS_EMPTY(workspace, T == 0);
    const size_t ws = moe::permute_workspace_bytes(T * k, E);
    if (workspace_bytes < ws)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, ws);
    DEBUG_CHECK(moe::debug_check_ids(topk_idx, T, k, E, (hipStream_t)stream));
    return hip_status(moe::launch_permute(x, topk_idx, T, H, E, k, align, P_max, expert_counts,
                                          expert_offsets, route_row, row_token, x_perm, workspace, true,
                                          (hipStream_t)stream),
                      "moe_permute_tiled launch");
}

moe_status moe_route_hist_workspace_size(int64_t T, int32_t k, int32_t E, size_t* bytes) {
    if (!bytes) return fail(MOE_ERR_NULL_POINTER, "bytes is NULL");
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    moe_status s = check_ek(E, k);
    if (s != MOE_OK) return s;
    *bytes = moe::route_hist_workspace_bytes(T, E);
    return ok();
}

moe_status moe_route_topk_hist(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
                               float* topk_w, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
    REQUIRE_PTR_UNLESS_EMPTY(logits, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(topk_idx, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(topk_w, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(workspace, T == 0);
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    moe_status s = check_ek(E, k);
    if (s != MOE_OK) return s;
    const size_t ws = moe::route_hist_workspace_bytes(T, E);
    if (T > 0 && workspace_bytes < ws)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, ws);
    DEBUG_CHECK(moe::debug_check_logits(logits, T * (int64_t)E, (hipStream_t)stream));
    return hip_status(moe::launch_route_topk_hist(logits, T, E, k, topk_idx, topk_w, (int32_t*)workspace,
                                                  (hipStream_t)stream),
                      "moe_route_topk_hist launch");
}

moe_status moe_permute_from_hist(const moe_bf16* x, const int32_t* topk_idx, int64_t T, int32_t H, int32_t E,
                                 int32_t k, int32_t align, int64_t P_max, int32_t* expert_counts,
                                 int32_t* expert_offsets, int32_t* route_row, int32_t* row_token,
                                 moe_bf16* x_perm, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
    moe_status s = check_permute(x, topk_idx, T, H, E, k, align, P_max, expert_counts, expert_offsets, route_row,
                                 row_token, x_perm);
    if (s != MOE_OK) return s;
    if (T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    REQUIRE_PTR_UNLESS_EMPTY(workspace, T == 0);
    const size_t ws = moe::route_hist_workspace_bytes(T, E);
    if (T > 0 && workspace_bytes < ws)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, ws);
    DEBUG_CHECK(moe::debug_check_ids(topk_idx, T, k, E, (hipStream_t)stream));
    return hip_status(moe::launch_permute_from_hist(x, topk_idx, T, H, E, k, align, P_max, expert_counts,
                                                    expert_offsets, route_row, row_token, x_perm, workspace,
                                                    (hipStream_t)stream),
                      "moe_permute_from_hist launch");
}

moe_status moe_fused_layer_workspace_size(int64_t T, int32_t k, int32_t E, size_t* bytes) {
    if (!bytes) return fail(MOE_ERR_NULL_POINTER, "bytes is NULL");
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    moe_status s = check_ek(E, k);
    if (s != MOE_OK) return s;
    *bytes = moe::fused_layer_workspace_bytes(T, k, E);
    return ok();
}

moe_status moe_fused_layer(const moe_bf16* x, const int32_t* topk_idx, const float* topk_w,
                           const moe_bf16* w_gate_up, const moe_bf16* w_down, int64_t T, int32_t H, int32_t E,
                           int32_t k, int32_t I, int32_t align, int64_t P_max, int32_t* expert_counts,
                           int32_t* expert_offsets, int32_t* route_row, int32_t* row_token, moe_bf16* h,
                           moe_bf16* y, moe_bf16* out, void* workspace, size_t workspace_bytes,
                           moe_stream_t stream) {
    REQUIRE_PTR(x);  // read by the gathering GEMM (check_permute needs x only with x_perm)
    if (T < 1) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld < 1", (long long)T);
    moe_status s = check_permute(x, topk_idx, T, H, E, k, align, P_max, expert_counts, expert_offsets, route_row,
                                 row_token, nullptr);
    if (s != MOE_OK) return s;
    REQUIRE_PTR(topk_w);
    REQUIRE_PTR(w_gate_up);
    REQUIRE_PTR(w_down);
    REQUIRE_PTR(h);
    REQUIRE_PTR(y);
    REQUIRE_PTR(out);
    REQUIRE_PTR(workspace);
    if ((s = check_dim64("I", I)) != MOE_OK) return s;
    if ((uint64_t)H * (uint64_t)I * 4u >= ((uint64_t)1 << 32))
        return fail(MOE_ERR_SIZE_OVERFLOW, "one expert's weights (2*I*H bf16, H=%d, I=%d) reach 2^32 bytes", H, I);
    if ((s = check_gather(row_token, T, H)) != MOE_OK) return s;
    const size_t ws = moe::fused_layer_workspace_bytes(T, k, E);
    if (workspace_bytes < ws)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, ws);
    DEBUG_CHECK(moe::debug_check_ids(topk_idx, T, k, E, (hipStream_t)stream));
    return hip_status(moe::launch_fused_layer(x, topk_idx, topk_w, w_gate_up, w_down, T, H, E, k, I, align, P_max,
                                              expert_counts, expert_offsets, route_row, row_token, h, y, out,
                                              workspace, (hipStream_t)stream),
                      "moe_fused_layer launch");
}

moe_status moe_fused_layer_status(const void* workspace, moe_stream_t stream) {
    REQUIRE_PTR(workspace);
    int32_t code = 0;
    moe_status s = hip_status(moe::fused_layer_read_error(workspace, &code, (hipStream_t)stream),
                              "moe_fused_layer_status");
    if (s != MOE_OK) return s;
    if (code != 0)
        return fail(MOE_ERR_HIP, "moe_fused_layer: a grid barrier timed out (a workgroup never arrived); "
                                 "the outputs of that call are incomplete");
    return ok();
}

size_t moe_permute_noalloc_max_workspace(void) { return moe::permute_scratch_bytes(); }

moe_status moe_permute_noalloc(const moe_bf16* x, const int32_t* topk_idx, int64_t T, int32_t H, int32_t E,
                               int32_t k, int32_t align, int64_t P_max, int32_t* expert_counts,
                               int32_t* expert_offsets, int32_t* route_row, int32_t* row_token,
                               moe_bf16* x_perm, moe_stream_t stream) {
    moe_status s = check_permute(x, topk_idx, T, H, E, k, align, P_max, expert_counts, expert_offsets, route_row,
                                 row_token, x_perm);
    if (s != MOE_OK) return s;
    const size_t ws = moe::permute_workspace_bytes(T * k, E);
    if (ws > moe::permute_scratch_bytes())
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                    "moe_permute_noalloc: T*k=%lld routes over E=%d experts need %zu bytes of scratch, more than "
                    "the library's fixed %zu (use moe_permute with a workspace)",
                    (long long)(T * k), E, ws, moe::permute_scratch_bytes());
    DEBUG_CHECK(moe::debug_check_ids(topk_idx, T, k, E, (hipStream_t)stream));
    return hip_status(moe::launch_permute_noalloc(x, topk_idx, T, H, E, k, align, P_max, expert_counts,
                                                  expert_offsets, route_row, row_token, x_perm,
                                                  (hipStream_t)stream),
                      "moe_permute_noalloc launch");
}

static moe_status check_gemm(const void* a, const void* w, const int32_t* counts,
                             const int32_t* offsets, int32_t E, int32_t H, int32_t I,
                             int64_t P_max, const void* out) {
    REQUIRE_PTR(a);
    REQUIRE_PTR(w);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(offsets);
    REQUIRE_PTR(out);
    if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_INVALID_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_E);
    moe_status s;
    if ((s = check_dim64("H", H)) != MOE_OK) return s;
    if ((s = check_dim64("I", I)) != MOE_OK) return s;
    // the kernels address one expert's weights with 32-bit byte offsets
    if ((uint64_t)H * (uint64_t)I * 4u >= ((uint64_t)1 << 32))
        return fail(MOE_ERR_SIZE_OVERFLOW, "one expert's weights (2*I*H bf16, H=%d, I=%d) reach 2^32 bytes", H, I);
    return check_pmax(P_max);
}

moe_status moe_grouped_glu_gemm(const moe_bf16* x_perm, const moe_bf16* w_gate_up,
                                const int32_t* expert_counts, const int32_t* expert_offsets,
                                int32_t E, int32_t H, int32_t I, int64_t P_max, moe_bf16* h,
                                moe_stream_t stream) {
    moe_status s = check_gemm(x_perm, w_gate_up, expert_counts, expert_offsets, E, H, I, P_max, h);
    if (s != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(launch_glu(x_perm, nullptr, w_gate_up, nullptr, expert_offsets, E, H, I, P_max, h,
                                 (hipStream_t)stream),
                      "moe_grouped_glu_gemm launch");
}


moe_status moe_grouped_glu_gemm_clamped(const moe_bf16* x_perm, const moe_bf16* w_gate_up,
                                        const int32_t* expert_counts, const int32_t* expert_offsets, int32_t E,
                                        int32_t H, int32_t I, int64_t P_max, float limit, moe_bf16* h,
                                        moe_stream_t stream) {
    moe_status s = check_gemm(x_perm, w_gate_up, expert_counts, expert_offsets, E, H, I, P_max, h);
    if (s != MOE_OK) return s;
    if (!(limit >= 0.0f)) return fail(MOE_ERR_INVALID_VALUE, "limit=%g must be >= 0", (double)limit);
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_grouped_glu_gemm_clamped(x_perm, w_gate_up, expert_offsets, E, H, I, limit, h,
                                                           (int)P_max, (hipStream_t)stream),
                      "moe_grouped_glu_gemm_clamped launch");
}

moe_status moe_grouped_glu_gemm_gather(const moe_bf16* x, const int32_t* row_token,
                                       const moe_bf16* w_gate_up, const int32_t* expert_counts,
                                       const int32_t* expert_offsets, int64_t T, int32_t E, int32_t H,
                                       int32_t I, int64_t P_max, moe_bf16* h, moe_stream_t stream) {
    moe_status s = check_gemm(x, w_gate_up, expert_counts, expert_offsets, E, H, I, P_max, h);
    if (s != MOE_OK) return s;
    if ((s = check_gather(row_token, T, H)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    DEBUG_CHECK(moe::debug_check_rows(row_token, P_max, -1, T, 6, (hipStream_t)stream));
    return hip_status(launch_glu(x, row_token, w_gate_up, nullptr, expert_offsets, E, H, I, P_max, h,
                                 (hipStream_t)stream),
                      "moe_grouped_glu_gemm_gather launch");
}

moe_status moe_grouped_down_gemm(const moe_bf16* h, const moe_bf16* w_down,
                                 const int32_t* expert_counts, const int32_t* expert_offsets,
                                 int32_t E, int32_t H, int32_t I, int64_t P_max, moe_bf16* y,
                                 moe_stream_t stream) {
    moe_status s = check_gemm(h, w_down, expert_counts, expert_offsets, E, H, I, P_max, y);
    if (s != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(launch_down(h, w_down, nullptr, expert_offsets, E, H, I, P_max, y, (hipStream_t)stream),
                      "moe_grouped_down_gemm launch");
}

moe_status moe_grouped_glu_gemm_tiled(const moe_bf16* x_perm, const moe_bf16* w_gate_up,
                                      const int32_t* expert_counts, const int32_t* expert_offsets, int32_t E,
                                      int32_t H, int32_t I, int64_t P_max, moe_bf16* h, moe_stream_t stream) {
    moe_status s = check_gemm(x_perm, w_gate_up, expert_counts, expert_offsets, E, H, I, P_max, h);
    if (s != MOE_OK) return s;
    if ((s = check_even_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_grouped_glu_gemm_tiled(x_perm, w_gate_up, nullptr, expert_offsets, E, H, I, h,
                                                         (int)P_max, (hipStream_t)stream),
                      "moe_grouped_glu_gemm_tiled launch");
}

moe_status moe_grouped_glu_gemm_gather_tiled(const moe_bf16* x, const int32_t* row_token,
                                             const moe_bf16* w_gate_up, const int32_t* expert_counts,
                                             const int32_t* expert_offsets, int64_t T, int32_t E, int32_t H,
                                             int32_t I, int64_t P_max, moe_bf16* h, moe_stream_t stream) {
    moe_status s = check_gemm(x, w_gate_up, expert_counts, expert_offsets, E, H, I, P_max, h);
    if (s != MOE_OK) return s;
    if ((s = check_even_pmax(P_max)) != MOE_OK) return s;
    if ((s = check_gather(row_token, T, H)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    DEBUG_CHECK(moe::debug_check_rows(row_token, P_max, -1, T, 6, (hipStream_t)stream));
    return hip_status(moe::launch_grouped_glu_gemm_gather_tiled(x, row_token, w_gate_up, nullptr, expert_offsets, E,
                                                                H, I, h, (int)P_max, (hipStream_t)stream),
                      "moe_grouped_glu_gemm_gather_tiled launch");
}

moe_status moe_grouped_down_gemm_tiled(const moe_bf16* h, const moe_bf16* w_down, const int32_t* expert_counts,
                                       const int32_t* expert_offsets, int32_t E, int32_t H, int32_t I,
                                       int64_t P_max, moe_bf16* y, moe_stream_t stream) {
    moe_status s = check_gemm(h, w_down, expert_counts, expert_offsets, E, H, I, P_max, y);
    if (s != MOE_OK) return s;
    if ((s = check_even_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_grouped_down_gemm_tiled(h, w_down, nullptr, expert_offsets, E, H, I, y, (int)P_max,
                                                          (hipStream_t)stream),
                      "moe_grouped_down_gemm_tiled launch");
}

moe_status moe_quantize_fp8(const moe_bf16* w, int64_t E, int32_t R, int32_t K, uint8_t* w8,
                            float* scale, moe_stream_t stream) {
    REQUIRE_PTR(w);
    REQUIRE_PTR(w8);
    REQUIRE_PTR(scale);
    if (E < 1 || E > ((int64_t)1 << 20)) return fail(MOE_ERR_INVALID_SHAPE, "E=%lld outside [1, 2^20]", (long long)E);
    moe_status s;
    if ((s = check_dim64("R", R)) != MOE_OK) return s;
    if ((s = check_dim64("K", K)) != MOE_OK) return s;
    if (E * (R / 64) >= ((int64_t)1 << 31))
        return fail(MOE_ERR_SIZE_OVERFLOW, "E*R/64 = %lld blocks reach 2^31", (long long)(E * (R / 64)));
    return hip_status(moe::launch_quantize_fp8(w, E, R, K, w8, scale, (hipStream_t)stream),
                      "moe_quantize_fp8 launch");
}

moe_status moe_grouped_glu_gemm_fp8w(const moe_bf16* x_perm, const uint8_t* w8_gate_up,
                                     const float* scale_gate_up, const int32_t* expert_counts,
                                     const int32_t* expert_offsets, int32_t E, int32_t H, int32_t I,
                                     int64_t P_max, moe_bf16* h, moe_stream_t stream) {
    moe_status s = check_gemm(x_perm, w8_gate_up, expert_counts, expert_offsets, E, H, I, P_max, h);
    if (s != MOE_OK) return s;
    REQUIRE_PTR(scale_gate_up);
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(launch_glu(x_perm, nullptr, w8_gate_up, scale_gate_up, expert_offsets, E, H, I, P_max,
                                 h, (hipStream_t)stream),
                      "moe_grouped_glu_gemm_fp8w launch");
}

moe_status moe_grouped_glu_gemm_gather_fp8w(const moe_bf16* x, const int32_t* row_token,
                                            const uint8_t* w8_gate_up, const float* scale_gate_up,
                                            const int32_t* expert_counts,
                                            const int32_t* expert_offsets, int64_t T, int32_t E,
                                            int32_t H, int32_t I, int64_t P_max, moe_bf16* h,
                                            moe_stream_t stream) {
    moe_status s = check_gemm(x, w8_gate_up, expert_counts, expert_offsets, E, H, I, P_max, h);
    if (s != MOE_OK) return s;
    REQUIRE_PTR(scale_gate_up);
    if ((s = check_gather(row_token, T, H)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    DEBUG_CHECK(moe::debug_check_rows(row_token, P_max, -1, T, 6, (hipStream_t)stream));
    return hip_status(launch_glu(x, row_token, w8_gate_up, scale_gate_up, expert_offsets, E, H, I, P_max, h,
                                 (hipStream_t)stream),
                      "moe_grouped_glu_gemm_gather_fp8w launch");
}

moe_status moe_grouped_down_gemm_fp8w(const moe_bf16* h, const uint8_t* w8_down, const float* scale_down,
                                      const int32_t* expert_counts, const int32_t* expert_offsets,
                                      int32_t E, int32_t H, int32_t I, int64_t P_max, moe_bf16* y,
                                      moe_stream_t stream) {
    moe_status s = check_gemm(h, w8_down, expert_counts, expert_offsets, E, H, I, P_max, y);
    if (s != MOE_OK) return s;
    REQUIRE_PTR(scale_down);
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(launch_down(h, w8_down, scale_down, expert_offsets, E, H, I, P_max, y,
                                  (hipStream_t)stream),
                      "moe_grouped_down_gemm_fp8w launch");
}

static moe_status tile_fp8(const uint8_t* src, int64_t rows, int32_t cols, uint8_t* dst, bool to_tiled,
                          moe_stream_t stream) {
    REQUIRE_PTR_UNLESS_EMPTY(src, rows == 0);
    REQUIRE_PTR_UNLESS_EMPTY(dst, rows == 0);
    if (rows < 0 || (rows & 3)) return fail(MOE_ERR_INVALID_SHAPE, "rows=%lld must be a multiple of 4, >= 0", (long long)rows);
    if (cols < 32 || cols % 32 != 0) return fail(MOE_ERR_INVALID_SHAPE, "cols=%d must be a positive multiple of 32", cols);
    if (rows == 0) return ok();
    if (src == dst) return fail(MOE_ERR_INVALID_VALUE, "src and dst must not be the same buffer");
    return hip_status(moe::launch_tile_fp8_rows(src, rows, cols, dst, to_tiled, (hipStream_t)stream),
                      to_tiled ? "moe_tile_fp8_rows launch" : "moe_untile_fp8_rows launch");
}

moe_status moe_tile_fp8_rows(const uint8_t* src, int64_t rows, int32_t cols, uint8_t* dst, moe_stream_t stream) {
    return tile_fp8(src, rows, cols, dst, true, stream);
}

moe_status moe_untile_fp8_rows(const uint8_t* src, int64_t rows, int32_t cols, uint8_t* dst, moe_stream_t stream) {
    return tile_fp8(src, rows, cols, dst, false, stream);
}

moe_status moe_grouped_glu_gemm_fp8w_tiled(const moe_bf16* x_perm, const uint8_t* w8_gate_up,
                                           const float* scale_gate_up, const int32_t* expert_counts,
                                           const int32_t* expert_offsets, int32_t E, int32_t H, int32_t I,
                                           int64_t P_max, moe_bf16* h, moe_stream_t stream) {
    moe_status s = check_gemm(x_perm, w8_gate_up, expert_counts, expert_offsets, E, H, I, P_max, h);
    if (s != MOE_OK) return s;
    REQUIRE_PTR(scale_gate_up);
    if ((s = check_even_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_grouped_glu_gemm_tiled(x_perm, w8_gate_up, scale_gate_up, expert_offsets, E, H, I, h,
                                                         (int)P_max, (hipStream_t)stream),
                      "moe_grouped_glu_gemm_fp8w_tiled launch");
}

moe_status moe_grouped_down_gemm_fp8w_tiled(const moe_bf16* h, const uint8_t* w8_down, const float* scale_down,
                                            const int32_t* expert_counts, const int32_t* expert_offsets, int32_t E,
                                            int32_t H, int32_t I, int64_t P_max, moe_bf16* y, moe_stream_t stream) {
    moe_status s = check_gemm(h, w8_down, expert_counts, expert_offsets, E, H, I, P_max, y);
    if (s != MOE_OK) return s;
    REQUIRE_PTR(scale_down);
    if ((s = check_even_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_grouped_down_gemm_tiled(h, w8_down, scale_down, expert_offsets, E, H, I, y,
                                                          (int)P_max, (hipStream_t)stream),
                      "moe_grouped_down_gemm_fp8w_tiled launch");
}

moe_status moe_grouped_gemm(const moe_bf16* a, const moe_bf16* w, const int32_t* expert_counts,
                            const int32_t* expert_offsets, int32_t E, int32_t K, int32_t N, int64_t P_max,
                            moe_bf16* c, moe_stream_t stream) {
    // the down GEMM's kernel is the plain grouped GEMM: (H, I) = (N, K)
    moe_status s = check_gemm(a, w, expert_counts, expert_offsets, E, N, K, P_max, c);
    if (s != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(launch_down(a, w, nullptr, expert_offsets, E, N, K, P_max, c, (hipStream_t)stream),
                      "moe_grouped_gemm launch");
}

moe_status moe_grouped_gemm_tiled(const moe_bf16* a, const moe_bf16* w, const int32_t* expert_counts,
                                  const int32_t* expert_offsets, int32_t E, int32_t K, int32_t N, int64_t P_max,
                                  moe_bf16* c, moe_stream_t stream) {
    moe_status s = check_gemm(a, w, expert_counts, expert_offsets, E, N, K, P_max, c);
    if (s != MOE_OK) return s;
    if ((s = check_even_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_grouped_down_gemm_tiled(a, w, nullptr, expert_offsets, E, N, K, c, (int)P_max,
                                                          (hipStream_t)stream),
                      "moe_grouped_gemm_tiled launch");
}

static moe_status check_swiglu(const int32_t* offsets, int32_t E, int32_t I, int64_t P_max) {
    REQUIRE_PTR(offsets);
    if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_INVALID_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_E);
    moe_status s;
    if ((s = check_dim64("I", I)) != MOE_OK) return s;
    return check_pmax(P_max);
}

moe_status moe_swiglu(const moe_bf16* gu, const int32_t* expert_offsets, int32_t E, int32_t I,
                      int64_t P_max, moe_bf16* h, moe_stream_t stream) {
    REQUIRE_PTR(gu);
    REQUIRE_PTR(h);
    moe_status s = check_swiglu(expert_offsets, E, I, P_max);
    if (s != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(nullptr, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_swiglu(gu, nullptr, expert_offsets, E, I, P_max, h, (hipStream_t)stream, false),
                      "moe_swiglu launch");
}

moe_status moe_swiglu_backward(const moe_bf16* dh, const moe_bf16* gu, const int32_t* expert_offsets,
                               int32_t E, int32_t I, int64_t P_max, moe_bf16* dgu, moe_stream_t stream) {
    REQUIRE_PTR(dh);
    REQUIRE_PTR(gu);
    REQUIRE_PTR(dgu);
    moe_status s = check_swiglu(expert_offsets, E, I, P_max);
    if (s != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(nullptr, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_swiglu(gu, dh, expert_offsets, E, I, P_max, dgu, (hipStream_t)stream, false),
                      "moe_swiglu_backward launch");
}

moe_status moe_swiglu_tiled(const moe_bf16* gu, const int32_t* expert_offsets, int32_t E, int32_t I,
                            int64_t P_max, moe_bf16* h, moe_stream_t stream) {
    REQUIRE_PTR(gu);
    REQUIRE_PTR(h);
    moe_status s = check_swiglu(expert_offsets, E, I, P_max);
    if (s != MOE_OK) return s;
    if ((s = check_even_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(nullptr, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_swiglu(gu, nullptr, expert_offsets, E, I, P_max, h, (hipStream_t)stream, true),
                      "moe_swiglu_tiled launch");
}

moe_status moe_swiglu_backward_tiled(const moe_bf16* dh, const moe_bf16* gu, const int32_t* expert_offsets,
                                     int32_t E, int32_t I, int64_t P_max, moe_bf16* dgu, moe_stream_t stream) {
    REQUIRE_PTR(dh);
    REQUIRE_PTR(gu);
    REQUIRE_PTR(dgu);
    moe_status s = check_swiglu(expert_offsets, E, I, P_max);
    if (s != MOE_OK) return s;
    if ((s = check_even_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(nullptr, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_swiglu(gu, dh, expert_offsets, E, I, P_max, dgu, (hipStream_t)stream, true),
                      "moe_swiglu_backward_tiled launch");
}

moe_status moe_grouped_gemm_swiglu_backward(const moe_bf16* dy, const moe_bf16* w_down_t, const moe_bf16* gu,
                                            const int32_t* expert_counts, const int32_t* expert_offsets, int32_t E,
                                            int32_t H, int32_t I, int64_t P_max, moe_bf16* dgu, moe_stream_t stream) {
    moe_status s = check_gemm(dy, w_down_t, expert_counts, expert_offsets, E, H, I, P_max, dgu);
    if (s != MOE_OK) return s;
    REQUIRE_PTR(gu);
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_grouped_gemm_swiglu_bwd(dy, w_down_t, gu, expert_offsets, E, H, I, dgu,
                                                          (int)P_max, (hipStream_t)stream),
                      "moe_grouped_gemm_swiglu_backward launch");
}

moe_status moe_transpose_experts(const moe_bf16* w, int64_t E, int32_t R, int32_t C, moe_bf16* wt,
                                 moe_stream_t stream) {
    REQUIRE_PTR(w);
    REQUIRE_PTR(wt);
    if (E < 1 || E > ((int64_t)1 << 20)) return fail(MOE_ERR_INVALID_SHAPE, "E=%lld outside [1, 2^20]", (long long)E);
    moe_status s;
    if ((s = check_dim64("R", R)) != MOE_OK) return s;
    if ((s = check_dim64("C", C)) != MOE_OK) return s;
    if (E * (R / 64) * (C / 64) >= ((int64_t)1 << 31))
        return fail(MOE_ERR_SIZE_OVERFLOW, "E*R*C/4096 tiles reach 2^31");
    return hip_status(moe::launch_transpose(w, E, R, C, wt, (hipStream_t)stream), "moe_transpose_experts launch");
}

moe_status moe_combine_backward(const moe_bf16* dout, const moe_bf16* y, const int32_t* route_row,
                                const float* topk_w, const int32_t* row_token, const int32_t* expert_offsets,
                                int64_t T, int32_t H, int32_t E, int32_t k, int64_t P_max, moe_bf16* dy,
                                float* dw, moe_stream_t stream) {
    REQUIRE_PTR_UNLESS_EMPTY(dout, T == 0);
    REQUIRE_PTR(y);
    REQUIRE_PTR_UNLESS_EMPTY(route_row, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(topk_w, T == 0);
    REQUIRE_PTR(row_token);
    REQUIRE_PTR(expert_offsets);
    REQUIRE_PTR(dy);
    REQUIRE_PTR_UNLESS_EMPTY(dw, T == 0);
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    moe_status s = check_ek(E, k);
    if (s != MOE_OK) return s;
    if ((s = check_dim64("H", H)) != MOE_OK) return s;
    if ((s = check_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(nullptr, expert_offsets, E, P_max, (hipStream_t)stream));
    DEBUG_CHECK(moe::debug_check_rows(route_row, T * (int64_t)k, -1, P_max, 5, (hipStream_t)stream));
    return hip_status(moe::launch_combine_bwd(dout, y, route_row, topk_w, row_token, expert_offsets, T, H, k, E,
                                              P_max, dy, dw, (hipStream_t)stream),
                      "moe_combine_backward launch");
}

moe_status moe_route_backward(const int32_t* topk_idx, const float* topk_w, const float* dw, int64_t T,
                              int32_t E, int32_t k, float* dlogits, moe_stream_t stream) {
    REQUIRE_PTR_UNLESS_EMPTY(topk_idx, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(topk_w, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(dw, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(dlogits, T == 0);
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    moe_status s = check_ek(E, k);
    if (s != MOE_OK) return s;
    return hip_status(moe::launch_route_bwd(topk_idx, topk_w, dw, T, E, k, dlogits, (hipStream_t)stream),
                      "moe_route_backward launch");
}

moe_status moe_permute_backward(const moe_bf16* dx_perm, const int32_t* route_row, int64_t T, int32_t H,
                                int32_t k, int64_t P_max, moe_bf16* dx, moe_stream_t stream) {
    // the combine kernel with every weight 1
    REQUIRE_PTR(dx_perm);
    REQUIRE_PTR_UNLESS_EMPTY(route_row, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(dx, T == 0);
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    if (k < 1 || k > MOE_MAX_K) return fail(MOE_ERR_INVALID_SHAPE, "k=%d outside [1, %d]", k, MOE_MAX_K);
    moe_status s;
    if ((s = check_dim64("H", H)) != MOE_OK) return s;
    if ((s = check_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_rows(route_row, T * (int64_t)k, -1, P_max, 5, (hipStream_t)stream));
    return hip_status(moe::launch_combine(dx_perm, route_row, nullptr, T, H, k, P_max, dx, (hipStream_t)stream),
                      "moe_permute_backward launch");
}

static moe_status check_wgrad(const moe_bf16* a, const moe_bf16* b, const int32_t* row_token,
                              const int32_t* expert_counts, const int32_t* expert_offsets, int32_t E, int32_t M,
                              int32_t N, int64_t P_max, float* dw) {
    REQUIRE_PTR(a);
    REQUIRE_PTR(b);
    REQUIRE_PTR(expert_counts);
    REQUIRE_PTR(expert_offsets);
    REQUIRE_PTR(dw);
    if (!aligned16(dw)) return fail(MOE_ERR_MISALIGNED_POINTER, "dw is not 16-byte aligned");
    if (row_token && !aligned16(row_token))
        return fail(MOE_ERR_MISALIGNED_POINTER, "row_token is not 16-byte aligned");
    if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_INVALID_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_E);
    moe_status s;
    if ((s = check_dim64("M", M)) != MOE_OK) return s;
    if ((s = check_dim64("N", N)) != MOE_OK) return s;
    if ((s = check_pmax(P_max)) != MOE_OK) return s;
    const int64_t tiles = (int64_t)E * ((M + 255) / 256) * ((N + 255) / 256);
    if (tiles >= ((int64_t)1 << 31)) return fail(MOE_ERR_SIZE_OVERFLOW, "E*M*N/65536 tiles reach 2^31");
    return ok();
}

moe_status moe_grouped_wgrad(const moe_bf16* a, const moe_bf16* b, const int32_t* row_token,
                             const int32_t* expert_counts, const int32_t* expert_offsets, int32_t E, int32_t M,
                             int32_t N, int64_t P_max, float* dw, moe_stream_t stream) {
    moe_status s = check_wgrad(a, b, row_token, expert_counts, expert_offsets, E, M, N, P_max, dw);
    if (s != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_wgrad(a, b, row_token, expert_offsets, E, M, N, (int)P_max, dw,
                                        (hipStream_t)stream, false, false),
                      "moe_grouped_wgrad launch");
}

moe_status moe_grouped_wgrad_tiled(const moe_bf16* a, int32_t a_tiled, const moe_bf16* b, int32_t b_tiled,
                                   const int32_t* expert_counts, const int32_t* expert_offsets, int32_t E, int32_t M,
                                   int32_t N, int64_t P_max, float* dw, moe_stream_t stream) {
    moe_status s = check_wgrad(a, b, nullptr, expert_counts, expert_offsets, E, M, N, P_max, dw);
    if (s != MOE_OK) return s;
    if ((a_tiled != 0 && a_tiled != 1) || (b_tiled != 0 && b_tiled != 1))
        return fail(MOE_ERR_INVALID_SHAPE, "a_tiled=%d, b_tiled=%d: each must be 0 or 1", a_tiled, b_tiled);
    if ((a_tiled || b_tiled) && (s = check_even_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_layout(expert_counts, expert_offsets, E, P_max, (hipStream_t)stream));
    return hip_status(moe::launch_wgrad(a, b, nullptr, expert_offsets, E, M, N, (int)P_max, dw, (hipStream_t)stream,
                                        a_tiled != 0, b_tiled != 0),
                      "moe_grouped_wgrad_tiled launch");
}

moe_status moe_router_prepare(const float* w_router, int32_t H, int32_t E, moe_bf16* w_hi, moe_bf16* w_lo,
                              moe_stream_t stream) {
    REQUIRE_PTR(w_router);
    REQUIRE_PTR(w_hi);
    REQUIRE_PTR(w_lo);
    if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_INVALID_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_E);
    moe_status s;
    if ((s = check_dim64("H", H)) != MOE_OK) return s;
    return hip_status(moe::launch_router_prepare(w_router, H, E, w_hi, w_lo, (hipStream_t)stream),
                      "moe_router_prepare launch");
}

moe_status moe_router_topk(const moe_bf16* x, const moe_bf16* w_hi, const moe_bf16* w_lo, int64_t T, int32_t H,
                           int32_t E, int32_t k, float* logits, int32_t* topk_idx, float* topk_w,
                           moe_stream_t stream) {
    REQUIRE_PTR_UNLESS_EMPTY(x, T == 0);
    REQUIRE_PTR(w_hi);
    REQUIRE_PTR(w_lo);
    REQUIRE_PTR_UNLESS_EMPTY(topk_idx, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(topk_w, T == 0);
    if (logits && !aligned16(logits)) return fail(MOE_ERR_MISALIGNED_POINTER, "logits is not 16-byte aligned");
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    moe_status s = check_ek(E, k);
    if (s != MOE_OK) return s;
    if ((s = check_dim64("H", H)) != MOE_OK) return s;
    return hip_status(moe::launch_router_topk(x, w_hi, w_lo, T, H, E, k, logits, topk_idx, topk_w,
                                              (hipStream_t)stream),
                      "moe_router_topk launch");
}

moe_status moe_combine(const moe_bf16* y, const int32_t* route_row, const float* topk_w, int64_t T,
                       int32_t H, int32_t k, int64_t P_max, moe_bf16* out, moe_stream_t stream) {
    REQUIRE_PTR(y);
    REQUIRE_PTR_UNLESS_EMPTY(route_row, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(topk_w, T == 0);
    REQUIRE_PTR_UNLESS_EMPTY(out, T == 0);
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_SHAPE, "T=%lld outside [0, 2^31)", (long long)T);
    if (k < 1 || k > MOE_MAX_K) return fail(MOE_ERR_INVALID_SHAPE, "k=%d outside [1, %d]", k, MOE_MAX_K);
    moe_status s;
    if ((s = check_dim64("H", H)) != MOE_OK) return s;
    if ((s = check_pmax(P_max)) != MOE_OK) return s;
    DEBUG_CHECK(moe::debug_check_rows(route_row, T * (int64_t)k, -1, P_max, 5, (hipStream_t)stream));
    return hip_status(moe::launch_combine(y, route_row, topk_w, T, H, k, P_max, out, (hipStream_t)stream),
                      "moe_combine launch");
}

moe_status moe_probe_copy(const void* src, void* dst, size_t bytes, moe_stream_t stream) {
    REQUIRE_PTR(src);
    REQUIRE_PTR(dst);
    if (bytes == 0 || bytes % 16 != 0)
        return fail(MOE_ERR_INVALID_SHAPE, "bytes=%zu must be a positive multiple of 16", bytes);
    return hip_status(moe::launch_probe_copy(src, dst, bytes, device_cus(), (hipStream_t)stream),
                      "moe_probe_copy launch");
}

moe_status moe_probe_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, moe_stream_t stream) {
    REQUIRE_PTR(src);
    REQUIRE_PTR(sink);
    if (bytes == 0 || bytes % 16 != 0)
        return fail(MOE_ERR_INVALID_SHAPE, "bytes=%zu must be a positive multiple of 16", bytes);
    if (!aligned16(src) || !aligned16(sink)) return fail(MOE_ERR_MISALIGNED_POINTER, "src or sink not 16-byte aligned");
    const int cus = device_cus();
    const size_t need = (size_t)moe::probe_read_blocks(cus) * 256 * 16;
    if (sink_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "sink holds %zu bytes < %zu needed", sink_bytes, need);
    return hip_status(moe::launch_probe_read(src, bytes, sink, cus, (hipStream_t)stream), "moe_probe_read launch");
}

size_t moe_probe_read_sink_bytes(void) { return (size_t)moe::probe_read_blocks(device_cus()) * 256 * 16; }

moe_status moe_probe_mfma_bf16(float* sink, int64_t sink_floats, int32_t iters, double* flops,
                               moe_stream_t stream) {
    REQUIRE_PTR(sink);
    if (!flops) return fail(MOE_ERR_NULL_POINTER, "flops is NULL");
    if (iters < 1) return fail(MOE_ERR_INVALID_VALUE, "iters=%d < 1", iters);
    const int cus = device_cus();
    const int64_t need = (int64_t)moe::probe_mfma_blocks(cus) * 256;
    if (sink_floats < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "sink holds %lld floats < %lld needed", (long long)sink_floats,
                    (long long)need);
    *flops = moe::probe_mfma_flops(cus, iters);
    return hip_status(moe::launch_probe_mfma(sink, iters, cus, (hipStream_t)stream), "moe_probe_mfma_bf16 launch");
}

int64_t moe_probe_mfma_sink_floats(void) { return (int64_t)moe::probe_mfma_blocks(device_cus()) * 256; }

int moe_debug_build(void) {
#ifdef MOE_DEBUG
    return 1;
#else
    return 0;
#endif
}

moe_status moe_debug_status(moe_stream_t stream) {
#ifdef MOE_DEBUG
    int32_t code = 0;
    moe_status s = hip_status(moe::debug_read(&code, (hipStream_t)stream), "moe_debug_status");
    if (s != MOE_OK) return s;
    switch (code) {
        case 0: return ok();
        case 1: return fail(MOE_ERR_PRECONDITION, "moe_route_topk: a logit is not finite");
        case 2: return fail(MOE_ERR_PRECONDITION, "moe_permute: a top-k id is outside [0, E)");
        case 3: return fail(MOE_ERR_PRECONDITION, "moe_permute: a token's top-k ids are not distinct");
        case 4: return fail(MOE_ERR_PRECONDITION,
                            "expert_offsets/expert_counts: offsets[0] != 0, decreasing offsets, offsets[E] > P_max, "
                            "or a count outside [0, its segment's rows]");
        case 5: return fail(MOE_ERR_PRECONDITION, "route_row: a value outside [-1, P_max)");
        case 6: return fail(MOE_ERR_PRECONDITION, "row_token: a value outside [-1, T)");
        default: return fail(MOE_ERR_PRECONDITION, "unknown check code %d", code);
    }
#else
    (void)stream;
    g_err[0] = '\0';
    snprintf(g_err, sizeof g_err, "release build: device-side preconditions are not checked");
    return MOE_OK;
#endif
}

moe_status moe_debug_reset(moe_stream_t stream) {
#ifdef MOE_DEBUG
    return hip_status(moe::debug_reset((hipStream_t)stream), "moe_debug_reset");
#else
    (void)stream;
    return ok();
#endif
}

}  // extern "C"
