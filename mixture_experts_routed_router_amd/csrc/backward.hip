// backward.hip -- the memory-bound steps of the backward pass, and the saved
// SwiGLU of the training forward.
//
// Backward of the path [prime-rl PR 3885, Changes: the single-pass layout gathers
// in backward too; the forward keeps the gate/up output so that the backward
// does not recompute it]. With dout = dL/dout [T, H]:
//   combine    dw[t,j] = <dout[t], y[route_row[t*k+j]]>;  dy[route_row[t*k+j]] =
//              w[t,j] dout[t]; every pad row of a segment is zeroed, so the K-grouped
//              weight-gradient GEMMs may sum over whole padded segments
//   routing    dlogits[t, idx[t,j]] = w[t,j] (dw[t,j] - sum_i w[t,i] dw[t,i]), 0 for
//              the experts not selected (softmax over the selected logits)
//   SwiGLU     forward h = silu(g) u from gu = [g | u]; backward dgu = [dh u silu'(g) |
//              dh silu(g)], silu'(g) = s (1 + g (1 - s)), s = sigmoid(g)
//   transpose  expert weights [E, R, C] -> [E, C, R] once per weight update, so
//              the input-gradient GEMMs are the forward's grouped GEMM
// fp32 arithmetic, bf16 storage (rounded to nearest even), fp32 dw and dlogits.
// Every reduction runs in a fixed order (no atomics): results are deterministic.
#include "common.hpp"

namespace moe {

// 16 bytes with a non-temporal load: for rows that nothing reads again.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4_t r = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ---- combine backward: one wavefront per token, its k routes in ascending j ----
// Passes of 4 pieces per lane (256 pieces, 4 KB of the row): the token's dout
// pieces are loaded once per pass, and route j+1's y pieces are loaded before
// route j's are used. Each lane accumulates its dot products over its pieces in
// ascending order, and the k wave reductions run after the last pass. A row
// outside [0, P_max) (no layout row) is neither read nor written.
constexpr int kCbU = 4;  // pieces per lane and pass

template <int KL>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint4* __restrict__ dout,
                                                          const uint4* __restrict__ y,
                                                          const int32_t* __restrict__ route_row,
                                                          const float* __restrict__ topk_w, int64_t T,
                                                          int pieces, int k, int64_t P_max,
                                                          uint4* __restrict__ dy, float* __restrict__ dw) {
    MOE_DEBUG_GUARD();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int lane = lane_id();
    const uint4* g = dout + t * pieces;
    float dot[KL];
#pragma unroll
    for (int j = 0; j < KL; ++j) dot[j] = 0.0f;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int c0 = 0; c0 < pieces; c0 += kWave * kCbU) {
        uint4 gv[kCbU], yv[kCbU], yn[kCbU];
        int64_t row = route_row[t * k];  // wave-uniform
        bool ok = row >= 0 && row < P_max;
#pragma unroll
        for (int u = 0; u < kCbU; ++u) {
            const int c = c0 + u * kWave + lane;
            gv[u] = c < pieces ? g[c] : zero;
            yn[u] = ok && c < pieces ? ld_nt(y + row * pieces + c) : zero;
        }
#pragma unroll
        for (int j = 0; j < KL; ++j) {
            if (j < k) {
                const float w = topk_w[t * k + j];
                const int64_t cur = row;
                const bool cur_ok = ok;
#pragma unroll
                for (int u = 0; u < kCbU; ++u) yv[u] = yn[u];
                if (j + 1 < k) {  // the next route's pieces, before this route's are used
                    row = route_row[t * k + j + 1];
                    ok = row >= 0 && row < P_max;
#pragma unroll
                    for (int u = 0; u < kCbU; ++u) {
                        const int c = c0 + u * kWave + lane;
                        yn[u] = ok && c < pieces ? ld_nt(y + row * pieces + c) : zero;
                    }
                }
#pragma unroll
                for (int u = 0; u < kCbU; ++u) {
                    const int c = c0 + u * kWave + lane;
                    if (!cur_ok || c >= pieces) continue;
                    const uint32_t gp[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
                    const uint32_t yp[4] = {yv[u].x, yv[u].y, yv[u].z, yv[u].w};
                    uint32_t o[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float g0 = bf16_lo(gp[q]), g1 = bf16_hi(gp[q]);
                        dot[j] = fmaf(g0, bf16_lo(yp[q]), dot[j]);
                        dot[j] = fmaf(g1, bf16_hi(yp[q]), dot[j]);
                        o[q] = pack_bf16x2(w * g0, w * g1);
                    }
                    dy[cur * pieces + c] = make_uint4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        if (j < k) {
            const float s = wave_sum(dot[j]);
            if (lane == 0) dw[t * k + j] = s;
        }
    }
}

// Pad rows of the used layout -> 0: one workgroup per expert. A segment's pad rows
// (row_token == -1) are its last rows, fewer than align of them: the first wave
// finds where they start, 64 rows per ballot from the end, then the workgroup
// zeroes their 16-byte pieces.
__global__ __launch_bounds__(256) void zero_pad_rows_kernel(const int32_t* __restrict__ row_token,
                                                            const int32_t* __restrict__ offsets, int pieces,
                                                            int64_t rows_max, uint4* __restrict__ dst) {
    MOE_DEBUG_GUARD();
    __shared__ int64_t pad0;
    const int e = blockIdx.x;
    // the segment clamped to [0, rows_max): offsets that break their contract cannot
    // make it read or write outside row_token or dst
    const int64_t s0 = min(max((int64_t)offsets[e], (int64_t)0), rows_max);
    const int64_t s1 = max(min((int64_t)offsets[e + 1], rows_max), s0);
    if (threadIdx.x < kWave) {
        const int lane = lane_id();
        int64_t start = s1;  // first pad row
        for (int64_t hi = s1; hi > s0; hi -= kWave) {
            const int64_t p = hi - 1 - lane;
            const bool pad = p >= s0 && row_token[p] < 0;
            const uint64_t m = __ballot(pad);  // lane i: row hi-1-i
            const uint64_t run = ~m;           // lanes from 0 that are pad rows form the suffix
            const int n = run == 0 ? kWave : __ffsll((unsigned long long)run) - 1;
            start = hi - n;
            if (n < kWave) break;
        }
        if (lane == 0) pad0 = start;
    }
    __syncthreads();
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t i = pad0 * pieces + threadIdx.x; i < s1 * pieces; i += blockDim.x) dst[i] = z;
}

// ---- routing backward: one wavefront per token ----
__global__ __launch_bounds__(256) void route_bwd_kernel(const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ topk_w,
                                                        const float* __restrict__ dw, int64_t T, int E,
                                                        int k, float* __restrict__ dlogits) {
    MOE_DEBUG_GUARD();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int lane = lane_id();
    const float wl = lane < k ? topk_w[t * k + lane] : 0.0f;
    const float dl = lane < k ? dw[t * k + lane] : 0.0f;
    const float s = wave_sum(wl * dl);
    for (int e = lane; e < E; e += kWave) {
        float v = 0.0f;
        for (int j = 0; j < k; ++j)  // wave-uniform loads
            if (topk_idx[t * k + j] == e) v = topk_w[t * k + j] * (dw[t * k + j] - s);
        dlogits[t * E + e] = v;
    }
}

// ---- SwiGLU forward (BWD false) and backward (BWD true) over used rows ----
// gu [P_max, 2I] and dh [P_max, I] row-major. TO: the output (h, or dgu = [dg | du])
// in row pairs (element (p, c) of a C-column matrix at (p/2)*2C + (c/32)*64 +
// (p%2)*32 + c%32, the order moe_tile_rows writes), produced in storage order: the
// forward's i-th 16-byte piece is h's i-th; the backward's i-th is dg's piece of the
// pair's first I columns, du's sits 2I/8 pieces after it. A row of the last pair at
// or past the used rows is written as zeros.
__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <bool BWD, bool TO>
__global__ __launch_bounds__(256) void swiglu_kernel(const uint4* __restrict__ gu, const uint4* __restrict__ dh,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     int64_t P_max, int pieces_i, uint4* __restrict__ out) {
    MOE_DEBUG_GUARD();
    const int64_t used = min((int64_t)offsets[E], P_max);
    // TO: pieces over whole pairs (2 * pieces_i per pair: I/32 blocks of 8 pieces)
    const int64_t n = TO ? (used + 1) / 2 * 2 * pieces_i : used * pieces_i;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t p;
        int c;
        if (TO) {
            const int64_t pr = i / (2 * pieces_i);
            const int rem = (int)(i - pr * 2 * pieces_i);  // block rem / 8, piece rem % 8 of the block
            p = 2 * pr + ((rem >> 2) & 1);
            c = (rem >> 3) * 4 + (rem & 3);  // the row's 16-byte piece (8 columns)
        } else {
            p = i / pieces_i;
            c = (int)(i - p * pieces_i);
        }
        // where the output piece(s) go
        const int64_t o_g = TO ? (BWD ? i + (i / (2 * pieces_i)) * 2 * pieces_i : i) : (BWD ? p * 2 * pieces_i + c : i);
        const int64_t o_u = TO ? o_g + 2 * pieces_i : o_g + pieces_i;
        if (TO && p >= used) {
            out[o_g] = zero;
            if (BWD) out[o_u] = zero;
            continue;
        }
        const uint4 gv = gu[p * 2 * pieces_i + c], uv = gu[p * 2 * pieces_i + pieces_i + c];
        const uint32_t gp[4] = {gv.x, gv.y, gv.z, gv.w}, up[4] = {uv.x, uv.y, uv.z, uv.w};
        if (!BWD) {
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack_bf16x2(silu_f(bf16_lo(gp[q])) * bf16_lo(up[q]),
                                   silu_f(bf16_hi(gp[q])) * bf16_hi(up[q]));
            out[o_g] = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
            uint4 og, ou;
            swiglu_bwd_x8(gv, uv, dh[p * pieces_i + c], og, ou);
            out[o_g] = og;
            out[o_u] = ou;
        }
    }
}

// ---- expert weight transpose [E, R, C] -> [E, C, R], 64x64 tiles through LDS ----
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ w, int R, int C,
                                                        uint16_t* __restrict__ wt) {
    MOE_DEBUG_GUARD();
    __shared__ uint16_t tile[64][64 + 2];
    const int tiles_c = C / 64, tiles_r = R / 64;
    const int64_t b = blockIdx.x;
    const int64_t e = b / ((int64_t)tiles_r * tiles_c);
    const int rem = (int)(b - e * tiles_r * tiles_c);
    const int r0 = (rem / tiles_c) * 64, c0 = (rem % tiles_c) * 64;
    const uint16_t* src = w + e * R * C;
    uint16_t* dst = wt + e * R * C;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = tid / 8 + 32 * i, cp = (tid % 8) * 8;
        const uint4 v = *(const uint4*)(src + (int64_t)(r0 + r) * C + c0 + cp);
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tile[r][cp + 2 * j] = (uint16_t)(q[j] & 0xffffu);
            tile[r][cp + 2 * j + 1] = (uint16_t)(q[j] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid / 8 + 32 * i, rp = (tid % 8) * 8;
        uint32_t q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            q[j] = (uint32_t)tile[rp + 2 * j][c] | ((uint32_t)tile[rp + 2 * j + 1][c] << 16);
        *(uint4*)(dst + (int64_t)(c0 + c) * R + r0 + rp) = make_uint4(q[0], q[1], q[2], q[3]);
    }
}

static unsigned grid_for(int64_t n, int64_t cap) {
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

hipError_t launch_combine_bwd(const uint16_t* dout, const uint16_t* y, const int32_t* route_row,
                              const float* topk_w, const int32_t* row_token, const int32_t* offsets,
                              int64_t T, int H, int k, int E, int64_t P_max, uint16_t* dy, float* dw,
                              hipStream_t stream) {
    const int pieces = H / 8;
    hipLaunchKernelGGL(zero_pad_rows_kernel, dim3((unsigned)E), dim3(256), 0, stream, row_token, offsets, pieces,
                       P_max, (uint4*)dy);
    if (T > 0) {
        const dim3 grid((unsigned)((T + 3) / 4)), block(256);
#define MOE_CB_LAUNCH(KL)                                                                              \
        hipLaunchKernelGGL(combine_bwd_kernel<KL>, grid, block, 0, stream, (const uint4*)dout, (const uint4*)y, \
                           route_row, topk_w, T, pieces, k, P_max, (uint4*)dy, dw)
        if (k <= 8) MOE_CB_LAUNCH(8);
        else if (k <= 16) MOE_CB_LAUNCH(16);
        else MOE_CB_LAUNCH(32);
#undef MOE_CB_LAUNCH
    }
    return hipGetLastError();
}

hipError_t launch_route_bwd(const int32_t* topk_idx, const float* topk_w, const float* dw, int64_t T, int E,
                            int k, float* dlogits, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(route_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, topk_idx,
                       topk_w, dw, T, E, k, dlogits);
    return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t* gu, const uint16_t* dh, const int32_t* offsets, int E, int I,
                         int64_t P_max, uint16_t* out, hipStream_t stream, bool tiled_out) {
    const int pi = I / 8;
    const dim3 grid(grid_for(P_max * pi, 8192)), block(256);
#define MOE_SWIGLU_LAUNCH(BWD, TO)                                                                     \
    hipLaunchKernelGGL((swiglu_kernel<BWD, TO>), grid, block, 0, stream, (const uint4*)gu, (const uint4*)dh, \
                       offsets, E, P_max, pi, (uint4*)out)
    if (dh && tiled_out) MOE_SWIGLU_LAUNCH(true, true);
    else if (dh) MOE_SWIGLU_LAUNCH(true, false);
    else if (tiled_out) MOE_SWIGLU_LAUNCH(false, true);
    else MOE_SWIGLU_LAUNCH(false, false);
#undef MOE_SWIGLU_LAUNCH
    return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t* w, int64_t E, int R, int C, uint16_t* wt, hipStream_t stream) {
    const int64_t blocks = E * (R / 64) * (C / 64);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, R, C, wt);
    return hipGetLastError();
}

}  // namespace moe
