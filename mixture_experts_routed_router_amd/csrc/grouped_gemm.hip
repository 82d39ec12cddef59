// grouped_gemm.hip -- grouped expert GEMMs on bf16 MFMA (gfx950), fp32 accumulate.
//
// One launch computes every expert's GEMM over its segment of the padded,
// expert-grouped layout [Halo "Performance", Levers that help: one batched expert
// matmul instead of a per-expert loop]:
//
//   C[p, n] = sum_k A[p, k] * W[e, n, k]       for p in expert e's segment
//
// GLU variant (gate/up projections): W[e] holds 2N rows, gate rows [0, N) and up
// rows [N, 2N); each tile loads matching gate and up rows, so each wave holds
// g and u for the same (row, column) in the same register and the SwiGLU
// h = silu(g) * u runs in the epilogue without leaving registers [Halo,
// Levers that help: fused GLU; prime-rl PR 3885, Changes: gate and up as one
// GEMM ahead of a clamped SwiGLU -- here unclamped].
//
// Scheduling: a persistent grid walks the tile list in expert-major order
// (expert, then column tile, then row tile), so an expert's weights are read
// about once and stay in L2 while its row tiles run [prime-rl PR 3885,
// Required kernel commits: expert-major task order].  Tiles are dealt in
// contiguous runs per XCD (workgroup b runs on XCD b % 8), so each expert's
// tiles share one XCD's L2.  Counts and offsets are read on the device; an
// expert with no rows owns no tiles and reads no weights [PocketLLM "Qwen4-Exp
// Heterogeneous TP4 Performance", Confirmed architecture decisions].  No
// workgroup ever waits on another.
//
// Tile: 128 rows x 128 W-rows x 64 k, 4 waves in a 2x2 grid, each wave 64 rows x
// two 32-column MFMA blocks (v_mfma_f32_32x32x16_bf16), LDS double-buffered with
// an XOR swizzle of 16-byte pieces so the MFMA operand reads are free of bank
// conflicts.  The output tile goes through LDS so that global stores are whole
// 16-byte pieces.
#include "common.hpp"

namespace moe {

constexpr int BM = 128;  // rows per tile
constexpr int BN = 128;  // W rows per tile (GLU: 64 gate + 64 up)
constexpr int BK = 64;   // k per stage
constexpr int kGemmThreads = 256;
constexpr int kMaxE = 1024;
constexpr int kTileElems = BM * BK;  // bf16 elements of one operand tile

// Piece (16 bytes = 8 bf16) c of row `row` of a [rows][64] tile lives at piece
// c ^ swz(row). Consecutive 8 rows get 8 distinct pieces; rows r and r+8 of a
// 16-row group land in opposite halves of a 256-byte bank window.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int tile_off(int row, int piece) {
    return row * BK + ((piece ^ swz(row)) << 3);
}

// Exclusive scan of one int per thread over a 256-thread block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp /* >= 4 ints */) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) tmp[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += tmp[w];
    __syncthreads();
    return before + incl - v;
}

template <bool GLU>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ offsets, int E, int K, int N, uint16_t* __restrict__ C) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kTileElems];  // [stage][A,B]
    __shared__ int32_t tile_start[kMaxE + 1];
    __shared__ int32_t seg_start[kMaxE + 1];
    __shared__ int32_t scan_tmp[4];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int NT = GLU ? N / 64 : (N + BN - 1) / BN;    // column tiles per expert
    const int NW = GLU ? 2 * N : N;                     // W rows per expert
    const int64_t w_stride = (int64_t)NW * K;

    // ---- per-expert tile counts -> prefix (each workgroup computes its own copy)
    {
        const int per = (E + kGemmThreads - 1) / kGemmThreads;  // <= 4
        int local = 0;
        for (int i = 0; i < per; ++i) {
            const int e = tid * per + i;
            if (e < E) {
                const int32_t o0 = offsets[e], o1 = offsets[e + 1];
                seg_start[e] = o0;
                local += (o1 - o0 + BM - 1) / BM * NT;
            }
        }
        int run = block_exclusive_scan(local, scan_tmp);
        for (int i = 0; i < per; ++i) {
            const int e = tid * per + i;
            if (e < E) {
                tile_start[e] = run;
                run += (offsets[e + 1] - offsets[e] + BM - 1) / BM * NT;
            }
        }
        if (tid == 0) seg_start[E] = offsets[E];
        if (tid == kGemmThreads - 1) tile_start[E] = run;
        __syncthreads();
    }
    const int total = tile_start[E];

    // ---- XCD-aware split: XCD x takes the contiguous run [x*chunk, (x+1)*chunk)
    const int nxcd = 8;
    const int xcd = blockIdx.x % nxcd, slot = blockIdx.x / nxcd;
    const int per_xcd = (int)(gridDim.x / nxcd);
    const int chunk = (total + nxcd - 1) / nxcd;
    const int t_end = min(total, (xcd + 1) * chunk);

    for (int t = xcd * chunk + slot; t < t_end; t += per_xcd) {
        // expert e: the last e with tile_start[e] <= t (experts with no tiles repeat a value)
        int lo = 0, hi = E;  // invariant: tile_start[lo] <= t < tile_start[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tile_start[mid] <= t) lo = mid; else hi = mid;
        }
        const int e = lo;
        const int seg0 = seg_start[e], seg1 = seg_start[e + 1];
        const int mt_e = (seg1 - seg0 + BM - 1) / BM;
        const int q = t - tile_start[e];
        const int nt = q / mt_e, mt = q - nt * mt_e;
        const int row0 = seg0 + mt * BM;
        const int rows_valid = min(BM, seg1 - row0);
        const uint16_t* We = W + (int64_t)e * w_stride;

        // global -> register staging: thread owns pieces tid + 256*i of each tile.
        // Row/column validity and W row indices do not depend on k: compute once.
        const uint16_t* pa[4];
        const uint16_t* pb[4];
        bool oka[4], okb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = tid + i * kGemmThreads;
            const int row = id >> 3, pc = id & 7;
            oka[i] = row < rows_valid;
            pa[i] = A + (int64_t)(row0 + (oka[i] ? row : 0)) * K + pc * 8;
            int wrow;
            if (GLU) {
                wrow = row < 64 ? nt * 64 + row : N + nt * 64 + (row - 64);
                okb[i] = true;
            } else {
                wrow = nt * BN + row;
                okb[i] = wrow < N;
            }
            pb[i] = We + (int64_t)(okb[i] ? wrow : 0) * K + pc * 8;
        }
        uint4 ra[4], rb[4];
#define MOE_LOAD_STAGE(kt)                                                              \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                 \
            ra[i] = oka[i] ? *(const uint4*)(pa[i] + (kt) * BK) : make_uint4(0u, 0u, 0u, 0u); \
            rb[i] = okb[i] ? *(const uint4*)(pb[i] + (kt) * BK) : make_uint4(0u, 0u, 0u, 0u); \
        }
#define MOE_STORE_STAGE(buf)                                                            \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                 \
            const int id = tid + i * kGemmThreads;                                      \
            const int off = tile_off(id >> 3, id & 7);                                  \
            *(uint4*)(&lds[(buf)][0][off]) = ra[i];                                     \
            *(uint4*)(&lds[(buf)][1][off]) = rb[i];                                     \
        }

        floatx16_t acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        // which 32-row blocks / 32-column blocks this wave computes
        const bool mb_on[2] = {wm * 64 < rows_valid, wm * 64 + 32 < rows_valid};
        int brow[2];
        bool nb_on[2];
        if (GLU) {
            brow[0] = wn * 32;          // gate block
            brow[1] = 64 + wn * 32;     // up block
            nb_on[0] = nb_on[1] = true;
        } else {
            brow[0] = wn * 64;
            brow[1] = wn * 64 + 32;
            nb_on[0] = nt * BN + brow[0] < N;
            nb_on[1] = nt * BN + brow[1] < N;
        }

        const int nk = K / BK;
        __syncthreads();  // previous tile's epilogue is done with the LDS
        MOE_LOAD_STAGE(0)
        MOE_STORE_STAGE(0)
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < nk) { MOE_LOAD_STAGE(kt + 1) }
            const uint16_t* sa = lds[buf][0];
            const uint16_t* sb = lds[buf][1];
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const int pc = ks * 2 + (lane >> 5);
                bf16x8_t a[2], b[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = wm * 64 + i * 32 + (lane & 31);
                    a[i] = *(const bf16x8_t*)(sa + tile_off(row, pc));
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int row = brow[j] + (lane & 31);
                    b[j] = *(const bf16x8_t*)(sb + tile_off(row, pc));
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        if (mb_on[i] && nb_on[j])
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j],
                                                                                 acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < nk) { MOE_STORE_STAGE(buf ^ 1) }
            __syncthreads();
        }

        // ---- epilogue: accumulators -> bf16 -> LDS (per-wave region) -> 16-byte stores.
        // MFMA 32x32 output layout: lane l, register r holds
        //   row = (r / 4) * 8 + (l / 32) * 4 + r % 4,  column = l % 32.
        constexpr int OC = GLU ? 32 : 64;  // output columns per wave
        uint16_t* so = &lds[0][0][0] + wave * (64 * OC);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (GLU) {
                    const float g = acc[i][0][r], u = acc[i][1][r];
                    const float hval = g / (1.0f + __expf(-g)) * u;
                    so[row * OC + (lane & 31)] = (uint16_t)f32_to_bf16_rne(hval);
                } else {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        so[row * OC + j * 32 + (lane & 31)] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes have landed
        __builtin_amdgcn_wave_barrier();
        constexpr int PPR = OC / 8;           // 16-byte pieces per output row of the wave
        const int col0 = GLU ? nt * 64 + wn * 32 : nt * BN + wn * 64;
#pragma unroll
        for (int i = 0; i < (64 * PPR) / kWave; ++i) {
            const int id = lane + i * kWave;
            const int row = id / PPR, pc = id % PPR;
            const int grow = wm * 64 + row;
            const int gcol = col0 + pc * 8;
            if (grow < rows_valid && gcol < N)
                *(uint4*)(C + (int64_t)(row0 + grow) * N + gcol) = *(const uint4*)(so + row * OC + pc * 8);
        }
    }
#undef MOE_LOAD_STAGE
#undef MOE_STORE_STAGE
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
    // two workgroups per CU (LDS: 2 x ~72 KB of 160 KB), a multiple of the 8 XCDs
    const int n = cu_count() * 2;
    return (unsigned)((n + 7) / 8 * 8);
}

hipError_t launch_grouped_glu_gemm(const uint16_t* x_perm, const uint16_t* w_gu,
                                   const int32_t* offsets, int E, int H, int I, uint16_t* h,
                                   hipStream_t stream) {
    hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(persistent_grid()), dim3(kGemmThreads), 0,
                       stream, x_perm, w_gu, offsets, E, H, I, h);
    return hipGetLastError();
}

hipError_t launch_grouped_down_gemm(const uint16_t* h, const uint16_t* w_d, const int32_t* offsets,
                                    int E, int H, int I, uint16_t* y, hipStream_t stream) {
    hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(persistent_grid()), dim3(kGemmThreads), 0,
                       stream, h, w_d, offsets, E, I, H, y);
    return hipGetLastError();
}

}  // namespace moe
