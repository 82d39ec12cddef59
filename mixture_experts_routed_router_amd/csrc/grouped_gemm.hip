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
// g and u for the same (row, column) in the same register position and the
// SwiGLU h = silu(g) * u runs in the epilogue without leaving registers [Halo,
// Levers that help: fused GLU; prime-rl PR 3885, Changes: gate and up as one
// GEMM ahead of a SwiGLU].
//
// Scheduling: a persistent grid (one workgroup per CU) walks the tile list in
// expert-major order (expert, then column tile, then row tile), so an expert's
// weights are read about once and stay in L2 while its row tiles run [prime-rl
// PR 3885, Required kernel commits: expert-major task order].  The tile list is
// dealt in contiguous runs per XCD (workgroup b runs on XCD b % 8), so each
// expert's tiles share one XCD's L2.  Counts and offsets are read on the device;
// an expert with no rows owns no tiles and reads no weights [PocketLLM "Qwen4-Exp
// Heterogeneous TP4 Performance", Confirmed architecture decisions].  No
// workgroup ever waits on another.
//
// Tile: 256 rows x 256 W-rows, k in steps of 32 through a 4-stage LDS ring that
// is filled by direct global->LDS loads (no register staging). 8 waves (two per
// SIMD, so one wave's MFMAs cover the other's waits) in a 2x4 grid; each wave
// owns 128 rows x 64 W-rows = 4x2 blocks of v_mfma_f32_32x32x16_bf16 (128
// accumulator registers).  16-byte pieces are XOR-swizzled in LDS so that the
// MFMA operand reads are conflict-free.  The output tile is staged through LDS
// so global stores are whole 16-byte pieces.
#include "common.hpp"

namespace moe {

constexpr int BM = 256;       // rows per tile
constexpr int BN = 256;       // W rows per tile (GLU: 128 gate + 128 up)
#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 32
#endif
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 4
#endif
constexpr int BK = MOE_GEMM_BK;          // k per stage
constexpr int STAGES = MOE_GEMM_STAGES;  // LDS ring depth
constexpr int PR = BK / 8;               // 16-byte pieces per row of a stage
constexpr int RPB = 64 / PR;             // rows filled by one wave-wide 1 KB load
constexpr int KSTEPS = BK / 16;          // MFMA k-steps per stage
#ifndef MOE_GEMM_WAVES
#define MOE_GEMM_WAVES 8
#endif
constexpr int kWaves = MOE_GEMM_WAVES;             // 4 (one per SIMD) or 8 (two per SIMD)
constexpr int kGemmThreads = kWaves * 64;
constexpr int WGN = kWaves / 2;                    // wave grid: 2 (rows) x WGN (W rows)
constexpr int WTN = BN / WGN;                      // W rows (output columns) per wave
constexpr int NBN = WTN / 32;                      // 32-column MFMA blocks per wave
static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves");
constexpr int kMaxE = 1024;
constexpr int kAElems = BM * BK;                   // bf16 elements of one A stage (16 KB)
constexpr int kBElems = BN * BK;                   // one B stage (16 KB)
constexpr int kStageElems = kAElems + kBElems;
constexpr int kLdsElems = STAGES * kStageElems;    // 128 KB
constexpr int kPiecesPerThread = (BM * PR) / kGemmThreads;  // of A (and of B) per stage
constexpr int kLoadsPerStage = 2 * kPiecesPerThread;        // per thread: A + B 16-byte loads
static_assert(BM == BN, "A and B stages share one load layout");
static_assert(kLoadsPerStage * (STAGES - 2) < 64, "vmcnt is 6 bits");
// The epilogue stages each wave's 128 x WTN bf16 output tile through the LDS ring;
// it must fit, or it would overwrite the tile tables that follow the ring in LDS.
static_assert(kWaves * 128 * WTN <= kLdsElems, "epilogue staging must fit in the LDS ring");

// Rows of a stage are BK bf16 = PR pieces of 16 bytes. Piece p of row r is stored
// at piece p ^ swz(r). For the same logical piece of any 8 consecutive rows (a
// 128-byte, 32-bank window) and of any 16 consecutive rows (a 256-byte, 64-bank
// window), the physical 16-byte slots are all distinct.
__device__ __forceinline__ int swz(int row) {
    if (PR == 4) return ((row >> 1) ^ (row >> 2)) & 3;
    return (row ^ (row >> 3)) & 7;  // PR == 8
}
static_assert(PR == 4 || PR == 8, "BK must be 32 or 64");

// Exclusive scan of one int per thread over the workgroup.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp /* >= kWaves ints */) {
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

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) const uint16_t*)p;
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4,
// SGPR base + VGPR byte offset): lane l's piece lands at LDS byte lds_base + 16*l.
// Issued through inline asm so that the compiler neither waits for these loads
// before unrelated LDS reads nor counts them; every wait is explicit below.
// M0 is written only here in this kernel (checked in its ISA).
__device__ __forceinline__ void dma16(uint32_t lds_base, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_base), "v"(voff), "s"(sbase) : "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroup barrier after this wave's LDS reads have returned. Unlike
// __syncthreads() it does not drain the in-flight global->LDS loads.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Everything one tile needs that does not depend on the live row-block count.
struct TileArgs {
    const uint16_t* a_tile;   // A + row0 * K
    const uint16_t* w_exp;    // W + e * (W rows per expert) * K
    uint16_t* c_tile;         // C + row0 * N
    int K, N, nt, rows_valid;
};

// One tile: the k loop through the LDS ring, then the epilogue. NV = number of
// this wave's 32-row blocks that hold segment rows (compile-time, so every MFMA
// in the loop is unconditional and the accumulators never leave AGPRs).
template <bool GLU, int NV>
__device__ __forceinline__ void run_tile(const TileArgs& ta, uint16_t* lds, int wave, int lane,
                                         const int (&rd_off)[KSTEPS]) {
    const int wm = wave / WGN, wn = wave % WGN;
    const int K = ta.K, N = ta.N, nt = ta.nt, rows_valid = ta.rows_valid;

    // ---- this thread's A and B pieces of every stage. Wave w, load i fills LDS
    // rows [RPB*(n*w+i), +RPB) (n = kPiecesPerThread); lane l fills row
    // RPB*(n*w+i) + l/PR, physical piece l%PR, i.e. logical piece (l%PR) ^ swz(row). Rows past the
    // segment (or past N) read a valid row instead; those results are never stored.
    // Byte offsets are relative to the tile's row 0 (A) and the expert (W), so they
    // stay fixed while the k stage moves the SGPR base.
    uint32_t offa[kPiecesPerThread], offb[kPiecesPerThread];
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i) {
        const int r = RPB * (kPiecesPerThread * wave + i) + lane / PR;
        const int piece = (lane % PR) ^ swz(r);
        const int ar = r < rows_valid ? r : 0;
        offa[i] = (uint32_t)((ar * K + piece * 8) * 2);
        int wr;
        if (GLU) {
            const int c = nt * 128 + (r & 127);  // output column of this W row
            const int cc = c < N ? c : N - 1;
            wr = r < 128 ? cc : N + cc;
        } else {
            const int c = nt * BN + r;
            wr = c < N ? c : N - 1;
        }
        offb[i] = (uint32_t)(((int64_t)wr * K + piece * 8) * 2);
    }
    const uint32_t lds0 = lds_addr(lds);
    auto issue_stage = [&](int kt) {
        const uint32_t sa = lds0 + (uint32_t)((kt % STAGES) * kStageElems * 2);
        const uint32_t sb = sa + kAElems * 2;
        const uint16_t* ga = ta.a_tile + kt * BK;
        const uint16_t* gb = ta.w_exp + kt * BK;
#pragma unroll
        for (int i = 0; i < kPiecesPerThread; ++i) {
            dma16(sa + (kPiecesPerThread * wave + i) * 1024, ga, offa[i]);
            dma16(sb + (kPiecesPerThread * wave + i) * 1024, gb, offb[i]);
        }
    };

    // LDS B row of each of this wave's 32-column blocks. GLU: the first half of
    // the blocks are gate columns, the second half the matching up columns.
    int brow[NBN];
#pragma unroll
    for (int j = 0; j < NBN; ++j)
        brow[j] = GLU ? (j < NBN / 2 ? 0 : 128) + wn * (WTN / 2) + (j % (NBN / 2)) * 32
                      : wn * WTN + j * 32;

    floatx16_t acc[NV > 0 ? NV : 1][NBN];
#pragma unroll
    for (int i = 0; i < (NV > 0 ? NV : 1); ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---- main loop: two wave groups in ping-pong. Group 0 (waves 0-3) and group 1
    // (waves 4-7) put one wave on each SIMD. Stage s is computed by group 0 in
    // phase 2s and by group 1 in phase 2s+1; in each phase the other group is the
    // memory group: it reads its fragments of the stage it computes next from LDS
    // and issues its half of the direct-to-LDS loads of a stage three or four
    // ahead. So in every phase one wave per SIMD issues nothing but its MFMAs, from
    // registers, while the other wave's memory traffic overlaps them.
    //   buffer of stage s: read by group 0 in phase 2s-1 and group 1 in phase 2s;
    //   group 1's half of stage s+3 is issued in phase 2s (buffer of s-1 is free),
    //   group 0's half of stage s+4 in phase 2s+1 (buffer of s is free);
    //   each group waits for its own half of stage s+1 by the end of phase 2s.
    static_assert(KSTEPS == 2, "the ping-pong schedule is written for BK = 32");
    static_assert(kWaves == 8, "the ping-pong schedule needs two waves per SIMD");
    constexpr int NA = NV > 0 ? NV : 1;
    const int grp = wave >> 2;  // == wm
    bf16x8_t fa[2][NA], fb[2][NBN];
#define MOE_LOAD_STAGE_FRAGS(stage)                                                           \
    do {                                                                                      \
        const uint16_t* sa_ = lds + ((stage) % STAGES) * kStageElems;                         \
        const uint16_t* sb_ = sa_ + kAElems;                                                  \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                    \
            _Pragma("unroll") for (int i = 0; i < NV; ++i)                                    \
                fa[ks][i] = *(const bf16x8_t*)(sa_ + ((2 * i + wm) * 32) * BK + rd_off[ks]);   \
            _Pragma("unroll") for (int j = 0; j < NBN; ++j)                                   \
                fb[ks][j] = *(const bf16x8_t*)(sb_ + brow[j] * BK + rd_off[ks]);               \
        }                                                                                     \
    } while (0)
#define MOE_MMA_STAGE()                                                                       \
    do {                                                                                      \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks)                                      \
            _Pragma("unroll") for (int i = 0; i < NV; ++i)                                    \
                _Pragma("unroll") for (int j = 0; j < NBN; ++j)                               \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0); \
    } while (0)
    // outstanding halves of later stages this group may leave in flight when it
    // needs stage s+1: group 0 has issued up to s+3, group 1 up to s+3 as well
#define MOE_WAIT_NEXT(s)                                                                      \
    do {                                                                                      \
        const int later_ = min(2, nk - 2 - (s));                                              \
        if (later_ >= 2) wait_vmcnt<2 * kLoadsPerStage>();                                    \
        else if (later_ == 1) wait_vmcnt<kLoadsPerStage>();                                   \
        else wait_vmcnt<0>();                                                                 \
    } while (0)

    const int nk = K / BK;
    // The previous tile's epilogue stores must be done before this tile's loads are
    // issued: a compiler-visible wait here means the compiler sees no vector-memory
    // operation pending inside the k loop (the loop's own loads are invisible to
    // it), so it adds no drain of the prefetch there.
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();  // the previous tile's epilogue is done with the LDS
    // prologue: both groups issue their halves of stages 0..2, group 0 also of 3
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue_stage(s);
    if (grp == 0 && STAGES - 1 < nk) issue_stage(STAGES - 1);
    {
        // stage 0 in: later stages of this group still allowed in flight
        const int issued = min(nk, grp == 0 ? STAGES : STAGES - 1);
        if (issued >= 4) wait_vmcnt<3 * kLoadsPerStage>();
        else if (issued == 3) wait_vmcnt<2 * kLoadsPerStage>();
        else if (issued == 2) wait_vmcnt<kLoadsPerStage>();
        else wait_vmcnt<0>();
    }
    lds_barrier();
    if (grp == 0 && NV > 0) MOE_LOAD_STAGE_FRAGS(0);
    lds_barrier();

    // Each group runs its own straight-line loop; both pass two barriers per stage.
    if (grp == 0) {
        for (int kt = 0; kt < nk; ++kt) {
            // phase 2kt: compute stage kt (fragments read in the previous phase)
            __builtin_amdgcn_s_setprio(1);
            if (NV > 0) MOE_MMA_STAGE();
            __builtin_amdgcn_s_setprio(0);
            MOE_WAIT_NEXT(kt);  // own half of stage kt+1 in; kt+2, kt+3 may stay in flight
            lds_barrier();
            // phase 2kt+1: refill the buffer of stage kt (both groups have read it)
            // with stage kt+4, and read stage kt+1
            if (kt + STAGES < nk) issue_stage(kt + STAGES);
            if (NV > 0 && kt + 1 < nk) MOE_LOAD_STAGE_FRAGS(kt + 1);
            lds_barrier();
        }
    } else {
        for (int kt = 0; kt < nk; ++kt) {
            // phase 2kt: read stage kt; issue stage kt+3 into the buffer of stage kt-1
            if (NV > 0) MOE_LOAD_STAGE_FRAGS(kt);
            if (kt + STAGES - 1 < nk) issue_stage(kt + STAGES - 1);
            MOE_WAIT_NEXT(kt);  // own half of stage kt+1 in; kt+2, kt+3 may stay in flight
            lds_barrier();
            // phase 2kt+1: compute stage kt
            __builtin_amdgcn_s_setprio(1);
            if (NV > 0) MOE_MMA_STAGE();
            __builtin_amdgcn_s_setprio(0);
            lds_barrier();
        }
    }
#undef MOE_LOAD_STAGE_FRAGS
#undef MOE_MMA_STAGE
#undef MOE_WAIT_NEXT

    // ---- epilogue: accumulators -> bf16 -> LDS (per-wave region) -> 16-byte stores.
    // MFMA 32x32 output layout: lane l, register r holds
    //   row = (r / 4) * 8 + (l / 32) * 4 + r % 4,  column = l % 32.
    lds_barrier();  // all waves are done reading the last stage
    if (NV == 0) return;
    constexpr int OC = GLU ? WTN / 2 : WTN;  // output columns per wave
    const int lrow = lane & 31;
    uint16_t* so = lds + wave * (128 * OC);
#pragma unroll
    for (int i = 0; i < (NV > 0 ? NV : 1); ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            if (GLU) {
#pragma unroll
                for (int j = 0; j < NBN / 2; ++j) {
                    const float g = acc[i][j][r], u = acc[i][j + NBN / 2][r];
                    const float hval = g / (1.0f + __expf(-g)) * u;
                    so[row * OC + j * 32 + lrow] = (uint16_t)f32_to_bf16_rne(hval);
                }
            } else {
#pragma unroll
                for (int j = 0; j < NBN; ++j)
                    so[row * OC + j * 32 + lrow] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes have landed
    __builtin_amdgcn_wave_barrier();
    constexpr int PPR = OC / 8;  // 16-byte pieces per output row of the wave
    const int col0 = GLU ? nt * 128 + wn * (WTN / 2) : nt * BN + wn * WTN;
#pragma unroll 4
    for (int i = 0; i < (NV * 32 * PPR) / kWave; ++i) {
        const int id = lane + i * kWave;
        const int row = id / PPR, pc = id % PPR;
        const int grow = ((row >> 5) * 2 + wm) * 32 + (row & 31);  // block row>>5 is block 2i+wm
        const int gcol = col0 + pc * 8;
        if (grow < rows_valid && gcol < N)
            *(uint4*)(ta.c_tile + (int64_t)grow * N + gcol) = *(const uint4*)(so + row * OC + pc * 8);
    }
}

template <bool GLU>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ offsets, int E, int K, int N, uint16_t* __restrict__ C) {
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsElems];
    __shared__ int32_t tile_start[kMaxE + 1];
    __shared__ int32_t seg_start[kMaxE + 1];
    __shared__ int32_t scan_tmp[kWaves];

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / WGN;
    // column tiles per expert: GLU tiles cover 128 output columns (128 gate + 128 up rows)
    const int NT = GLU ? (N + 127) / 128 : (N + BN - 1) / BN;
    const int NW = GLU ? 2 * N : N;  // W rows per expert
    const int64_t w_stride = (int64_t)NW * K;

    // ---- per-expert tile counts -> prefix (every workgroup builds its own copy)
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

    // lane-constant parts of the MFMA operand addresses: logical piece
    // (2*ks + lane/32) of row (lane % 32) of each 32-row block
    const int lrow = lane & 31;
    int rd_off[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) rd_off[ks] = lrow * BK + (((2 * ks + (lane >> 5)) ^ swz(lrow)) << 3);

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
        TileArgs ta;
        ta.a_tile = A + (int64_t)row0 * K;
        ta.w_exp = W + (int64_t)e * w_stride;
        ta.c_tile = C + (int64_t)row0 * N;
        ta.K = K;
        ta.N = N;
        ta.nt = nt;
        ta.rows_valid = min(BM, seg1 - row0);
        // live 32-row blocks of this wave: wave row wm owns blocks 2i + wm
        const int nvb = max(0, min(4, ((ta.rows_valid + 31) / 32 - wm + 1) / 2));
        switch (nvb) {
            case 4: run_tile<GLU, 4>(ta, lds, wave, lane, rd_off); break;
            case 3: run_tile<GLU, 3>(ta, lds, wave, lane, rd_off); break;
            case 2: run_tile<GLU, 2>(ta, lds, wave, lane, rd_off); break;
            case 1: run_tile<GLU, 1>(ta, lds, wave, lane, rd_off); break;
            default: run_tile<GLU, 0>(ta, lds, wave, lane, rd_off); break;
        }
    }
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
