// wgrad.hip -- expert weight gradients, K-grouped over each expert's rows.
//
//   dW[e, m, n] = sum over the rows p of expert e's padded segment of A[p, m] B[p, n]
//
// with A, B row-major over the layout rows (dW_down: A = dy, B = h; dW_gate_up:
// A = dgu, B = x_perm, or the token rows x[row_token[p]] read in place), fp32
// accumulation and fp32 output [prime-rl PR 3885, Changes: weight-gradient GEMMs
// write straight into fp32 accumulators; one K-grouped GEMM launch per weight].
// Pad rows of a segment contribute nothing: the backward zeroes them in A.
//
// The reduction runs over rows, which are the strided dimension of both operands,
// so each 32-row chunk is transposed on its way into LDS: a thread loads 16 bytes
// (8 columns) of two consecutive rows and writes the 8 (row, row+1) pairs as
// 32-bit words at [column][row], so the MFMA fragments (8 consecutive rows of
// one column) are single 128-bit LDS reads. Tile 128 x 128 per workgroup of four
// waves (2 x 2 waves of 64 x 64, v_mfma_f32_32x32x16_bf16), LDS double-buffered
// with the next chunk's global loads in flight during the MFMAs. One workgroup
// per (expert, tile); an expert with no rows writes zeros.
#include "common.hpp"

namespace moe {

constexpr int kWgBM = 128, kWgBN = 128, kWgBK = 32;
constexpr int kWgStride = kWgBK + 8;  // bf16 per LDS row (80 bytes: 16-byte aligned, spreads banks)

template <bool GATHER_B>
__global__ __launch_bounds__(256) void wgrad_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                    const int32_t* __restrict__ row_token,
                                                    const int32_t* __restrict__ offsets, int M, int N,
                                                    int tiles_m, int tiles_n, float* __restrict__ dW) {
    __shared__ __attribute__((aligned(16))) uint16_t at[2][kWgBM][kWgStride];
    __shared__ __attribute__((aligned(16))) uint16_t bt[2][kWgBN][kWgStride];

    const int64_t b = blockIdx.x;
    const int e = (int)(b / ((int64_t)tiles_m * tiles_n));
    const int rem = (int)(b - (int64_t)e * tiles_m * tiles_n);
    const int m0 = (rem / tiles_n) * kWgBM, n0 = (rem % tiles_n) * kWgBN;
    const int seg0 = offsets[e], seg1 = offsets[e + 1];
    const int nchunks = (seg1 - seg0 + kWgBK - 1) / kWgBK;

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = tid / kWave, wm = wave >> 1, wn = wave & 1;
    // staging: thread -> row pair (2pp, 2pp+1) of the chunk, 16-byte column piece cp
    const int pp = tid & 15, cp = tid >> 4;
    const int ca = m0 + 8 * cp, cb = n0 + 8 * cp;
    const bool a_col = ca < M, b_col = cb < N;

    u32x4_t ra[2], rb[2];
    auto load = [&](int ch) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int p = seg0 + ch * kWgBK + 2 * pp + h;
            const bool in = p < seg1;
            ra[h] = (in && a_col) ? *(const u32x4_t*)(A + (int64_t)p * M + ca) : u32x4_t{0u, 0u, 0u, 0u};
            int64_t rowb = p;
            bool okb = in && b_col;
            if (GATHER_B) {
                const int32_t tk = in ? row_token[p] : -1;
                okb = okb && tk >= 0;
                rowb = tk;
            }
            rb[h] = okb ? *(const u32x4_t*)(B + rowb * N + cb) : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    // (row 2pp, row 2pp+1) pairs of column 8cp+q as one 32-bit word at [8cp+q][2pp]
    auto store = [&](int buf) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t alo = __builtin_amdgcn_perm(ra[1][d], ra[0][d], 0x05040100u);  // col 2d
            const uint32_t ahi = __builtin_amdgcn_perm(ra[1][d], ra[0][d], 0x07060302u);  // col 2d+1
            const uint32_t blo = __builtin_amdgcn_perm(rb[1][d], rb[0][d], 0x05040100u);
            const uint32_t bhi = __builtin_amdgcn_perm(rb[1][d], rb[0][d], 0x07060302u);
            *(uint32_t*)&at[buf][8 * cp + 2 * d][2 * pp] = alo;
            *(uint32_t*)&at[buf][8 * cp + 2 * d + 1][2 * pp] = ahi;
            *(uint32_t*)&bt[buf][8 * cp + 2 * d][2 * pp] = blo;
            *(uint32_t*)&bt[buf][8 * cp + 2 * d + 1][2 * pp] = bhi;
        }
    };

    floatx16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nchunks > 0) {
        load(0);
        store(0);
        __syncthreads();
    }
    const int lrow = lane & 31, kh = 8 * (lane >> 5);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        if (ch + 1 < nchunks) load(ch + 1);
#pragma unroll
        for (int ks = 0; ks < kWgBK / 16; ++ks) {
            bf16x8_t fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[i] = *(const bf16x8_t*)&at[buf][wm * 64 + i * 32 + lrow][ks * 16 + kh];
                fb[i] = *(const bf16x8_t*)&bt[buf][wn * 64 + i * 32 + lrow][ks * 16 + kh];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (ch + 1 < nchunks) store(buf ^ 1);
        __syncthreads();
    }

    // MFMA 32x32 output: lane l, register r -> row (r/4)*8 + (l/32)*4 + r%4, column l%32
    float* out = dW + (int64_t)e * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + j * 32 + lrow;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + (r / 4) * 8 + (lane >> 5) * 4 + r % 4;
                if (m < M) out[(int64_t)m * N + n] = acc[i][j][r];
            }
        }
}

hipError_t launch_wgrad(const uint16_t* A, const uint16_t* B, const int32_t* row_token, const int32_t* offsets,
                        int E, int M, int N, float* dW, hipStream_t stream) {
    const int tm = (M + kWgBM - 1) / kWgBM, tn = (N + kWgBN - 1) / kWgBN;
    const int64_t blocks = (int64_t)E * tm * tn;
    if (row_token)
        hipLaunchKernelGGL(wgrad_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, A, B, row_token,
                           offsets, M, N, tm, tn, dW);
    else
        hipLaunchKernelGGL(wgrad_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, A, B,
                           (const int32_t*)nullptr, offsets, M, N, tm, tn, dW);
    return hipGetLastError();
}

}  // namespace moe
