// grouped_gemm_core.hpp -- grouped expert GEMMs on bf16 MFMA (gfx950), fp32 accumulate:
// the device code, shared by grouped_gemm.hip's kernel and the fused layer kernel.
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
// expert-major order (expert, then row tile, then column tile), so an expert's
// weights are read about once and stay in cache while its row tiles run [prime-rl
// PR 3885, Required kernel commits: expert-major task order]; consecutive tiles
// share a row tile of A.  An expert's rows are cut into ceil(rows / 256) row
// tiles of nearly equal size (whole 32-row blocks), not 256-row tiles and a
// remainder.  The tile list is
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
// MFMA operand reads are conflict-free.  The ring runs on from one tile to the
// next (the next tile's first stages load during the last k steps), and the
// output is written straight from registers while the next tile runs (plain
// GEMM: 16 bytes per lane, whole 128-byte rows per instruction; GLU: 8 bytes per
// lane, as a wave owns 32 output columns). Variants of the epilogue: SwiGLU
// (GLU, optionally clamped at a runtime limit) and the SwiGLU backward of the
// plain GEMM's output (SWB: dh = dy W_d never leaves registers).
//
// FP8-weight variant (W8): W holds OCP E4M3 codes with one fp32 scale per 64
// consecutive W rows of an expert [Halo "Performance", Levers that do not help
// here: the bytes of fine-grained experts' weights are what bounds them, and
// fp8 halves them; prime-rl, Changes: blockwise FP8 expert weights]. A B stage
// is then 32 bytes per W row (half the bytes), each lane reads its 16 codes
// from LDS with one 16-byte read and widens them to bf16 exactly
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1), and the MFMAs run on bf16 as
// before. The block scale is constant along k, so it multiplies the fp32
// accumulator once in the epilogue.
#pragma once
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
// A wave's epilogue issues at most 4 blocks x NBN column blocks x 4 store
// instructions; a wait may leave those and 3 stages of loads in flight.
constexpr int kMaxStoresPerTile = 4 * NBN * 4;
static_assert(3 * kLoadsPerStage + kMaxStoresPerTile < 64, "vmcnt is 6 bits");
// FP8 weights: a B stage is BN rows x BK bytes (8 KB), one 16-byte piece per thread.
constexpr int kLoadsPerStageW8 = kPiecesPerThread + 1;
static_assert(BN * BK == 16 * kGemmThreads, "one fp8 B piece per thread and stage");

// Rows of a stage are BK bf16 = PR pieces of 16 bytes. Piece p of row r is stored
// at piece p ^ swz(r). For the same logical piece of any 8 consecutive rows (a
// 128-byte, 32-bank window) and of any 16 consecutive rows (a 256-byte, 64-bank
// window), the physical 16-byte slots are all distinct.
__device__ __forceinline__ int swz(int row) {
    if (PR == 4) return ((row >> 1) ^ (row >> 2)) & 3;
    return (row ^ (row >> 3)) & 7;  // PR == 8
}
static_assert(PR == 4 || PR == 8, "BK must be 32 or 64");

// FP8 B stage: a row is BK = 32 bytes, two 16-byte pieces; piece p of row r is
// stored at p ^ swz8(r). A wave's operand read covers 16 consecutive rows with
// one piece each; flipping the piece every 8 rows puts the two halves of those
// 512 bytes on disjoint banks.
__device__ __forceinline__ int swz8(int row) { return (row >> 3) & 1; }

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

// Wait until at most n of this wave's vector-memory operations are in flight;
// n is rounded down to a multiple of 4 (waiting for more is always safe).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    switch (n >> 2) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<4>(); break;
        case 2: wait_vmcnt<8>(); break;
        case 3: wait_vmcnt<12>(); break;
        case 4: wait_vmcnt<16>(); break;
        case 5: wait_vmcnt<20>(); break;
        case 6: wait_vmcnt<24>(); break;
        case 7: wait_vmcnt<28>(); break;
        case 8: wait_vmcnt<32>(); break;
        case 9: wait_vmcnt<36>(); break;
        case 10: wait_vmcnt<40>(); break;
        case 11: wait_vmcnt<44>(); break;
        case 12: wait_vmcnt<48>(); break;
        case 13: wait_vmcnt<52>(); break;
        case 14: wait_vmcnt<56>(); break;
        default: wait_vmcnt<60>(); break;
    }
}

// Lane exchange inside each quad of lanes (DPP quad_perm): partner lane ^ 2 or ^ 1.

// The value of lane l ^ 4 (same 16-lane DPP row): row_shl:4 gives lane l the
// value of lane l + 4, row_shr:4 that of lane l - 4; `odd` = lane bit 2.
__device__ __forceinline__ uint32_t lane_xor4(uint32_t v, bool odd) {
    const uint32_t from_up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x104, 0xF, 0xF, true);
    const uint32_t from_dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x114, 0xF, 0xF, true);
    return odd ? from_dn : from_up;
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;  // round to nearest even (v_cvt_pk_bf16_f32)
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// 4x4 transpose of bf16 values inside a quad of lanes. On entry lane p (= lane % 4)
// holds column p of the block, v[m] = element (m, p); on exit it holds row p as
// w0 = (p,0) | (p,1) << 16 and w1 = (p,2) | (p,3) << 16. Rows are swapped in
// pairs with lane p^2, then single values with lane p^1; the byte selectors of
// v_perm_b32 (bytes 0-3 of the second operand, 4-7 of the first) depend only on
// the lane and are built once (QuadSel).
struct QuadSel {
    bool h;              // p & 2
    uint32_t give;       // p odd: (kp.lo, y.lo), even: (kp.hi, y.hi)
    uint32_t pa;         // columns {p, p^1} in order, from kp and t
    uint32_t pb;         // columns {p^2, p^3} in order, from y and t
};

__device__ __forceinline__ QuadSel quad_sel(int lane) {
    const int p = lane & 3;
    const bool g = (p & 1) != 0;
    QuadSel q;
    q.h = (p & 2) != 0;
    q.give = g ? 0x01000504u : 0x03020706u;
    q.pa = g ? 0x07060100u : 0x01000504u;
    q.pb = g ? 0x07060302u : 0x03020504u;
    return q;
}

__device__ __forceinline__ void quad_transpose_bf16(float v0, float v1, float v2, float v3,
                                                    const QuadSel& qs, uint32_t& w0, uint32_t& w1) {
    const uint32_t b01 = pack2_bf16(v0, v1), b23 = pack2_bf16(v2, v3);  // lo = even row
    const uint32_t kp = qs.h ? b23 : b01;           // rows 2h, 2h+1 of column p
    const uint32_t y = quad_xor2(qs.h ? b01 : b23); // rows 2h, 2h+1 of column p^2
    // this lane ends with row 2h+g; the partner p^1 needs row 2h+1-g of both
    const uint32_t t = quad_xor1(__builtin_amdgcn_perm(kp, y, qs.give));  // row 2h+g of p^1 (lo), p^3 (hi)
    const uint32_t pa = __builtin_amdgcn_perm(kp, t, qs.pa);
    const uint32_t pb = __builtin_amdgcn_perm(y, t, qs.pb);
    w0 = qs.h ? pb : pa;
    w1 = qs.h ? pa : pb;
}

// Everything one tile needs.
struct TileArgs {
    const uint16_t* a_tile;   // A + row0 * K (gathering A: the token matrix x itself)
    const char* w_exp;        // W + e * (W rows per expert) * K elements (as bytes)
    const float* w_scale;     // FP8 weights: the expert's scales, one per 64 W rows
    uint16_t* c_tile;         // C + row0 * N (SwiGLU backward: dgu + row0 * 2N)
    const uint16_t* gu_tile;  // SwiGLU backward: gu + row0 * 2N
    int row0, nt, rows_valid;
    int nvb;                  // this wave's 32-row blocks that hold segment rows (0..4)
};

// This thread's byte offsets of its A and B pieces of a stage, relative to the
// tile's row 0 (A) and the expert (W), so they stay fixed while the k stage moves
// the SGPR base. Wave w, load i fills LDS rows [RPB*(n*w+i), +RPB)
// (n = kPiecesPerThread); lane l fills row RPB*(n*w+i) + l/PR, physical piece
// l%PR, i.e. logical piece (l%PR) ^ swz(row). Rows past the segment (or past N)
// read a valid row instead; those results are never stored.
struct StageOffsets {
    uint32_t a[kPiecesPerThread], b[kPiecesPerThread];
};

// GATHER: A is the token matrix x [T, K], and layout row p reads token row
// row_token[p] -- the permute's gather folded into the loads. `tok` holds this
// thread's token of each of its rows (issue_token_loads); a pad row (-1) reads
// token 0 instead, its results are never read.
//
// PK (tiled operands): A (unless gathering) and bf16 W are stored as 2 x 32
// blocks, row pair q and k block b at 128 * (q * K/32 + b) bytes, the even row's 64
// bytes first; FP8 W as 4 x 32-byte blocks, row quad q and k block b at
// 128 * (q * K/32 + b). A stage's pieces of two (four) neighbouring rows then fill
// one 128-byte line instead of halves (quarters) of two (four). The offsets here
// are those of stage 0; stage s adds 128 s bytes (through the SGPR base, or part
// of it through the lane offset).
template <bool GLU, bool GATHER, bool W8, bool PK = false>
__device__ __forceinline__ StageOffsets stage_offsets(const TileArgs& ta, int K, int N, int wave, int lane,
                                                      const uint32_t (&tok)[kPiecesPerThread]) {
    StageOffsets o;
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i) {
        const int r = RPB * (kPiecesPerThread * wave + i) + lane / PR;
        const int piece = (lane % PR) ^ swz(r);
        uint32_t ar;
        if (GATHER) ar = (int32_t)tok[i] < 0 ? 0u : tok[i];
        else ar = (uint32_t)(r < ta.rows_valid ? r : 0);
        // 32-bit byte offset: the host guarantees rows * K * 2 < 2^32 (T * H * 2 when gathering)
        if (PK && !GATHER) {
            // row ar of the tile is layout row row0 + ar; a_tile points at row0's pair
            const uint32_t rr = ar + (uint32_t)(ta.row0 & 1);
            o.a[i] = (rr >> 1) * (uint32_t)K * 4u + (rr & 1u) * 64u + (uint32_t)piece * 16u;
        } else {
            o.a[i] = (ar * (uint32_t)K + (uint32_t)(piece * 8)) * 2u;
        }
        int wr;
        if (GLU) {
            const int c = ta.nt * 128 + (r & 127);  // output column of this W row
            const int cc = c < N ? c : N - 1;
            wr = r < 128 ? cc : N + cc;
        } else {
            const int c = ta.nt * BN + r;
            wr = c < N ? c : N - 1;
        }
        if (!W8) {
            if (PK) o.b[i] = (uint32_t)(wr >> 1) * (uint32_t)K * 4u + (uint32_t)(wr & 1) * 64u + (uint32_t)piece * 16u;
            else o.b[i] = (uint32_t)(((int64_t)wr * K + piece * 8) * 2);
        }
    }
    if (W8) {
        // FP8 B: wave w fills W rows 32w .. 32w+31 of the stage, lane l row
        // 32w + l/2, physical piece l%2 (logical (l%2) ^ swz8(row)). Byte offsets
        // inside one expert's weights fit 32 bits (checked on the host).
        const int r = 32 * wave + lane / 2;
        const int piece = (lane & 1) ^ swz8(r);
        int wr;
        if (GLU) {
            const int c = ta.nt * 128 + (r & 127);
            const int cc = c < N ? c : N - 1;
            wr = r < 128 ? cc : N + cc;
        } else {
            const int c = ta.nt * BN + r;
            wr = c < N ? c : N - 1;
        }
        // PK: the codes in 4-row tiled order, 4 rows x 32 bytes per 128-byte block
        if (PK) o.b[0] = (uint32_t)(wr >> 2) * (uint32_t)K * 4u + (uint32_t)(wr & 3) * 32u + (uint32_t)piece * 16u;
        else o.b[0] = (uint32_t)wr * (uint32_t)K + (uint32_t)(piece * 16);
    }
    return o;
}

// Gathering A: the tokens of a tile's rows go from row_token straight into LDS
// (global_load_lds_dword, one instruction per wave, counted by vmcnt like the
// stage loads; no register is written asynchronously). Wave w loads the tokens
// of rows 32w .. 32w+31 -- the rows its stage loads cover -- into its own 64-slot
// region (lanes 32..63 repeat them); rows past the segment read the tile's first
// row. After the wave's own wait, read_tokens picks each thread's two rows; no
// other wave touches the region, so no barrier is needed.
constexpr int kTokSlots = 64;  // per wave and buffer

__device__ __forceinline__ void issue_token_loads(const TileArgs& ta, const int32_t* row_token, int wave,
                                                  int lane, uint32_t lds_region) {
    const int r = 32 * wave + (lane & 31);
    const uint32_t off = (uint32_t)(r < ta.rows_valid ? r : 0) * 4u;
    const int32_t* base = row_token + ta.row0;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(lds_region), "v"(off), "s"(base) : "memory");
}

__device__ __forceinline__ void read_tokens(const int32_t* region, int lane,
                                            uint32_t (&tok)[kPiecesPerThread]) {
    static_assert(kPiecesPerThread * RPB == 32, "a wave's stage loads cover 32 rows");
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i) tok[i] = (uint32_t)region[RPB * i + lane / PR];
}

// This thread's share of one stage: A and B pieces of k-stage kt of a tile into ring
// slot `slot`. bx: bytes added to every W piece's offset (tiled W in the gathering
// variant: the part of its 128-byte stride the SGPR base does not take).
template <bool W8>
__device__ __forceinline__ void issue_stage(uint32_t lds0, int slot, int wave, const uint16_t* ga,
                                            const char* gb, const StageOffsets& o, uint32_t bx) {
    const uint32_t sa = lds0 + (uint32_t)(slot * kStageElems * 2);
    const uint32_t sb = sa + kAElems * 2;
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i) {
        dma16(sa + (kPiecesPerThread * wave + i) * 1024, ga, o.a[i]);
        if (!W8) dma16(sb + (kPiecesPerThread * wave + i) * 1024, gb, o.b[i] + bx);
    }
    if (W8) dma16(sb + wave * 1024, gb, o.b[0] + bx);
}

// 8 E4M3 codes (two dwords, k order) -> 8 bf16, exactly (every E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A compile-time bool passed as a value (selects a copy of a generic lambda).
template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// Wave-constant values of the whole launch.
struct WaveCtx {
    uint16_t* lds;
    uint32_t lds0;
    int K, N, nk;
    int wave, lane, wm, wn, grp;
    int rd_off[KSTEPS];
    int rd8_off;         // FP8 B: byte offset of this lane's 16 codes within a 32-row block
    int32_t* tok_lds;    // gathering A: [2][kWaves][kTokSlots] token buffers
    float glu_limit;     // GLU: clamp limit (+inf: the plain SwiGLU)
};

// One tile: the k loop through the LDS ring, then the epilogue. NV = number of
// this wave's 32-row blocks that hold segment rows (compile-time, so every MFMA
// in the loop is unconditional and the accumulators stay in registers).
//
// The ring runs on across tiles: stage kt of a tile lives in slot (base + kt) % 4,
// and when pf_next is set, the loads of the next tile's first stages are issued
// during this tile's last k steps (group 1 issues stages 0-2, group 0 stages 0-3,
// exactly what a prologue would). The next tile then starts with `prefetched` set
// and no prologue.
//
// The epilogue writes straight from registers (no LDS): after a 4x4 transpose
// inside each quad of lanes, a lane holds 4 consecutive bf16 of one output row
// (the gate/up GEMM stores those 8 bytes; the plain GEMM first trades halves with
// lane ^ 4 and stores 16). This wave's stores of the previous tile (s_prev of
// them) were issued after the prefetched stages; vector-memory operations
// complete in issue order, so a wait for a prefetched stage may leave those
// stores in flight.
template <bool GLU, bool GATHER, bool W8, bool SWB, bool PK, int NV>
__device__ __forceinline__ int run_tile(const WaveCtx& w, const TileArgs& ta, const TileArgs& tn,
                                        int base, bool prefetched, bool pf_next, int s_prev,
                                        const int32_t* __restrict__ row_token, int tb) {
    const int K = w.K, N = w.N, nk = w.nk, wave = w.wave, lane = w.lane, wm = w.wm, wn = w.wn;
    const int grp = w.grp;
    // Gathering A: this tile's tokens are in token buffer tb (loaded during the
    // previous tile when it prefetched this one, else loaded here); the next
    // tile's go to buffer tb^1 now and are waited for just before its first stage
    // is issued.
    const int32_t* tok_cur = w.tok_lds + (tb * kWaves + wave) * kTokSlots;
    const int32_t* tok_nxt = w.tok_lds + ((tb ^ 1) * kWaves + wave) * kTokSlots;
    uint32_t tok[kPiecesPerThread] = {0u, 0u}, tkn[kPiecesPerThread] = {0u, 0u};
    int n_tok = 0;  // token loads of the next tile in flight (issued after any prefetched stage)
    if (GATHER) {
        if (!prefetched) issue_token_loads(ta, row_token, wave, lane, lds_addr((const uint16_t*)tok_cur));
        if (pf_next) {
            issue_token_loads(tn, row_token, wave, lane, lds_addr((const uint16_t*)tok_nxt));
            n_tok = 1;
        }
        if (!prefetched) {
            if (n_tok) wait_vmcnt<1>();
            else wait_vmcnt<0>();
        }
        read_tokens(tok_cur, lane, tok);
    }
    const StageOffsets oc = stage_offsets<GLU, GATHER, W8, PK>(ta, K, N, wave, lane, tok);
    constexpr int LPS = W8 ? kLoadsPerStageW8 : kLoadsPerStage;  // this thread's loads per stage
    constexpr int WB = W8 ? 1 : 2;                                // bytes per weight
    // per k stage: A elements and W bytes the SGPR bases move, and bytes added to W's
    // lane offsets (row-pair tiled operands move 128 bytes per stage)
    constexpr int AST = (PK && !GATHER) ? 2 * BK : BK;
    // (the gathering variant keeps W's base stride and adds the rest per lane: with the
    // full stride in the base, the compiler runs out of SGPRs for it)
    constexpr int WST = (PK && !GATHER) ? 4 * BK : BK * WB;
    constexpr uint32_t WX = (PK && GATHER) ? (uint32_t)(4 * BK - BK * WB) : 0u;

    // LDS B row of each of this wave's 32-column blocks. GLU: the first half of
    // the blocks are gate columns, the second half the matching up columns.
    int brow[NBN];
#pragma unroll
    for (int j = 0; j < NBN; ++j)
        brow[j] = GLU ? (j < NBN / 2 ? 0 : 128) + wn * (WTN / 2) + (j % (NBN / 2)) * 32
                      : wn * WTN + j * 32;

    // Accumulators: the first k-step of stage 0 starts each from a zero operand
    // (no separate clearing pass); a wave with no rows never uses them.
    floatx16_t acc[NV > 0 ? NV : 1][NBN];

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
    // Stages kt >= nk are the next tile's stages kt - nk.
    static_assert(KSTEPS == 2, "the ping-pong schedule is written for BK = 32");
    static_assert(kWaves == 8, "the ping-pong schedule needs two waves per SIMD");
    constexpr int NA = NV > 0 ? NV : 1;
    bf16x8_t fa[2][NA], fb[2][NBN];
#define MOE_ISSUE(s)                                                                              \
    do {                                                                                          \
        const int s_ = (s);                                                                       \
        const int slot_ = (base + s_) & (STAGES - 1);                                             \
        if (s_ < nk)                                                                              \
            issue_stage<W8>(w.lds0, slot_, wave, ta.a_tile + s_ * AST, ta.w_exp + s_ * WST, oc, \
                            (uint32_t)s_ * WX);                                           \
        else if (pf_next) {                                                                       \
            const StageOffsets on_ = stage_offsets<GLU, GATHER, W8, PK>(tn, K, N, wave, lane, tkn); \
            issue_stage<W8>(w.lds0, slot_, wave, tn.a_tile + (s_ - nk) * AST,                     \
                            tn.w_exp + (s_ - nk) * WST, on_, (uint32_t)(s_ - nk) * WX);       \
        }                                                                                         \
    } while (0)
#define MOE_LOAD_STAGE_FRAGS(stage)                                                           \
    do {                                                                                      \
        const uint16_t* sa_ = w.lds + ((base + (stage)) & (STAGES - 1)) * kStageElems;        \
        const uint16_t* sb_ = sa_ + kAElems;                                                  \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                    \
            _Pragma("unroll") for (int i = 0; i < NV; ++i)                                    \
                fa[ks][i] = *(const bf16x8_t*)(sa_ + ((2 * i + wm) * 32) * BK + w.rd_off[ks]); \
            if (!W8) {                                                                        \
                _Pragma("unroll") for (int j = 0; j < NBN; ++j)                               \
                    fb[ks][j] = *(const bf16x8_t*)(sb_ + brow[j] * BK + w.rd_off[ks]);         \
            }                                                                                 \
        }                                                                                     \
        if (W8) {                                                                             \
            const char* s8_ = (const char*)sb_;                                               \
            u32x4_t raw_[NBN];                                                                \
            _Pragma("unroll") for (int j = 0; j < NBN; ++j)                                   \
                raw_[j] = *(const u32x4_t*)(s8_ + brow[j] * BK + w.rd8_off);                  \
            _Pragma("unroll") for (int j = 0; j < NBN; ++j) {                                 \
                fb[0][j] = fp8x8_to_bf16(raw_[j][0], raw_[j][1]);                             \
                fb[1][j] = fp8x8_to_bf16(raw_[j][2], raw_[j][3]);                             \
            }                                                                                 \
        }                                                                                     \
    } while (0)
#define MOE_MMA_STAGE(FIRST)                                                                  \
    do {                                                                                      \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks)                                      \
            _Pragma("unroll") for (int i = 0; i < NV; ++i)                                    \
                _Pragma("unroll") for (int j = 0; j < NBN; ++j)                               \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                      \
                        fa[ks][i], fb[ks][j], ((FIRST) && ks == 0) ? floatx16_t{} : acc[i][j], 0, 0, 0); \
    } while (0)
    // Before this group's first load of the next tile (issued at iteration FIRST_),
    // wait for the next tile's token loads: since they were issued, this group has
    // issued PRO_ prologue stages (none when this tile was prefetched) and one
    // stage in each earlier iteration, all of which may stay in flight.
#define MOE_WAIT_TOKENS(kt, FIRST_, PRO_)                                                     \
    do {                                                                                      \
        if (GATHER && pf_next && (kt) == (FIRST_)) {                                          \
            const int younger_ = ((prefetched ? 0 : (PRO_)) + (kt)) * LPS;                     \
            wait_vmcnt_dyn(younger_ < 60 ? younger_ : 60);                                    \
            read_tokens(tok_nxt, lane, tkn);                                                  \
        }                                                                                     \
    } while (0)
    // Wait for this group's half of stage kt+1. Its later stages kt+2, kt+3 (where
    // they exist) may stay in flight, and so may the previous tile's stores when
    // stage kt+1 was issued before them (prefetched stages 0..P).
#define MOE_WAIT_NEXT(kt, P)                                                                  \
    do {                                                                                      \
        const int s2_ = (kt) + 2;                                                             \
        const int later_ = (s2_ < nk || pf_next ? 1 : 0) + (s2_ + 1 < nk || pf_next ? 1 : 0);  \
        if (prefetched && (kt) + 1 <= (P))                                                    \
            wait_vmcnt_dyn(later_ * LPS + s_prev + n_tok);                                    \
        else if (later_ >= 2) wait_vmcnt<2 * LPS>();                                          \
        else if (later_ == 1) wait_vmcnt<LPS>();                                              \
        else wait_vmcnt<0>();                                                                 \
    } while (0)

    if (!prefetched) {
        // prologue: all waves are done with the ring; both groups issue their halves
        // of stages 0..2, group 0 also of 3; wait for stage 0 (older stores of the
        // previous tile complete first)
        lds_barrier();
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nk) MOE_ISSUE(s);
        if (grp == 0 && STAGES - 1 < nk) MOE_ISSUE(STAGES - 1);
        const int issued = min(nk, grp == 0 ? STAGES : STAGES - 1);
        if (issued >= 4) wait_vmcnt<3 * LPS>();
        else if (issued == 3) wait_vmcnt<2 * LPS>();
        else if (issued == 2) wait_vmcnt<LPS>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (grp == 0) MOE_LOAD_STAGE_FRAGS(0);
        lds_barrier();
    } else if (grp == 0) {
        // the stage is in (the previous tile's last wait and barrier); group 0 reads
        // its fragments ahead of its first MFMAs, group 1 in its first phase as usual
        MOE_LOAD_STAGE_FRAGS(0);
    }

    // Each group runs its own straight-line loop; both pass two barriers per stage.
    // The middle stages -- every stage the group issues is inside this tile, both
    // later stages are in flight, and no wait can leave older stores or token
    // loads outstanding -- run a copy of the loop body with those waits and
    // issues fixed, without the branches that pick them at the edges.
#define MOE_G0_BODY(kt, STEADY, FIRST)                                                            \
    do {                                                                                          \
        /* phase 2kt: compute stage kt (fragments read in the previous phase) */                  \
        __builtin_amdgcn_s_setprio(1);                                                            \
        if (NV > 0) MOE_MMA_STAGE(FIRST);                                                         \
        __builtin_amdgcn_s_setprio(0);                                                            \
        if (STEADY) wait_vmcnt<2 * LPS>();                                                        \
        else MOE_WAIT_NEXT(kt, 3);                                                                \
        lds_barrier();                                                                            \
        /* phase 2kt+1: refill the buffer of stage kt (both groups have read it) with */          \
        /* stage kt+4, and read stage kt+1 */                                                     \
        if (STEADY) {                                                                             \
            issue_stage<W8>(w.lds0, (base + (kt) + STAGES) & (STAGES - 1), wave,                  \
                            ta.a_tile + ((kt) + STAGES) * AST, ta.w_exp + ((kt) + STAGES) * WST, oc, \
                            (uint32_t)((kt) + STAGES) * WX);                                      \
            MOE_LOAD_STAGE_FRAGS((kt) + 1);                                                       \
        } else {                                                                                  \
            MOE_WAIT_TOKENS(kt, nk - STAGES, STAGES);                                             \
            MOE_ISSUE((kt) + STAGES);                                                             \
            if ((kt) + 1 < nk) MOE_LOAD_STAGE_FRAGS((kt) + 1);                                    \
        }                                                                                         \
        lds_barrier();                                                                            \
    } while (0)
#define MOE_G1_BODY(kt, STEADY, FIRST)                                                            \
    do {                                                                                          \
        /* phase 2kt: read stage kt; issue stage kt+3 into the buffer of stage kt-1 */            \
        MOE_LOAD_STAGE_FRAGS(kt);                                                                 \
        if (STEADY) {                                                                             \
            issue_stage<W8>(w.lds0, (base + (kt) + STAGES - 1) & (STAGES - 1), wave,              \
                            ta.a_tile + ((kt) + STAGES - 1) * AST,                                \
                            ta.w_exp + ((kt) + STAGES - 1) * WST, oc,                         \
                            (uint32_t)((kt) + STAGES - 1) * WX);                                  \
            wait_vmcnt<2 * LPS>();                                                                \
        } else {                                                                                  \
            MOE_WAIT_TOKENS(kt, nk - STAGES + 1, STAGES - 1);                                     \
            MOE_ISSUE((kt) + STAGES - 1);                                                         \
            MOE_WAIT_NEXT(kt, 2);                                                                 \
        }                                                                                         \
        lds_barrier();                                                                            \
        /* phase 2kt+1: compute stage kt */                                                       \
        __builtin_amdgcn_s_setprio(1);                                                            \
        if (NV > 0) MOE_MMA_STAGE(FIRST);                                                         \
        __builtin_amdgcn_s_setprio(0);                                                            \
        lds_barrier();                                                                            \
    } while (0)
    static_assert(STAGES == 4, "the steady ranges below assume a four-stage ring");
    if (grp == 0) {
        // steady: kt >= 3 (stage kt+1 >= 4 was issued in this tile, after any
        // stores of the previous one) and kt + 4 < nk (stage kt+4 is this tile's)
        const int lo = min(3, nk), hi = max(lo, nk - 4);
        MOE_G0_BODY(0, false, true);  // nk >= 2 (K >= 64)
        int kt = 1;
        for (; kt < lo; ++kt) MOE_G0_BODY(kt, false, false);
        for (; kt < hi; ++kt) MOE_G0_BODY(kt, true, false);
        for (; kt < nk; ++kt) MOE_G0_BODY(kt, false, false);
    } else {
        // steady: kt >= 2 (stage kt+1 >= 3 issued in this tile) and kt + 3 < nk
        const int lo = min(2, nk), hi = max(lo, nk - 3);
        MOE_G1_BODY(0, false, true);
        int kt = 1;
        for (; kt < lo; ++kt) MOE_G1_BODY(kt, false, false);
        for (; kt < hi; ++kt) MOE_G1_BODY(kt, true, false);
        for (; kt < nk; ++kt) MOE_G1_BODY(kt, false, false);
    }
#undef MOE_G0_BODY
#undef MOE_G1_BODY
#undef MOE_ISSUE
#undef MOE_LOAD_STAGE_FRAGS
#undef MOE_MMA_STAGE
#undef MOE_WAIT_NEXT
#undef MOE_WAIT_TOKENS

    // ---- epilogue: accumulators -> bf16 -> global, straight from registers.
    // MFMA 32x32 output layout: lane l, register r holds
    //   row = (r / 4) * 8 + (l / 32) * 4 + r % 4,  column = l % 32,
    // so registers 4q..4q+3 of the quad of lanes 4c..4c+3 form the 4x4 block of rows
    // 8q + 4(l/32) + 0..3 and columns 4c + 0..3. Every store instruction covers 8 rows
    // of the wave's columns (GLU: one 32-column block; plain: both blocks, 64
    // columns); those with no row inside the segment are not issued, and the rest
    // are counted.
    int stores = 0;
    if (NV > 0) {
        // The tile's scalars pass through an empty asm here, so the compiler cannot
        // compute the epilogue's addresses ahead of the k loop and hold them in
        // registers across it.
        int rows_valid = ta.rows_valid, n_cols = N, nt = ta.nt, zero = 0;
        int ln = lane;
        asm volatile("" : "+s"(rows_valid), "+s"(n_cols), "+s"(nt), "+s"(zero), "+v"(ln));
        const float* w_scale = ta.w_scale + zero;
        uint16_t* c_tile = ta.c_tile + zero;
        const uint16_t* gu_tile = ta.gu_tile + zero;
        const QuadSel qs = quad_sel(ln);
        const int out_row = (ln >> 5) * 4 + (ln & 3);  // this lane's row in an 8-row group
        // byte offset of this lane's 8 bytes from the group's (row 0, column 0).
        // PK (GLU output): h is row-pair tiled and c_tile points at row0's pair; the
        // group of tile rows r0.. (r0 even) and columns cb.. starts r0 * N + 2 cb
        // elements in, and this lane's row lies lp = (row0 & 1) + out_row rows past
        // it: pair lp / 2 (2N elements each), half lp % 2 of each 2 x 32 block
        const int lp = (ta.row0 & 1) + out_row;
        const uint32_t out_off =
            PK && GLU ? (uint32_t)(((lp >> 1) * 2 * n_cols + (lp & 1) * 32 + ((ln & 31) >> 2) * 4) * 2)
                      : (uint32_t)((out_row * n_cols + ((ln & 31) >> 2) * 4) * 2);
        constexpr int OB = GLU ? NBN / 2 : NBN;    // 32-column output blocks per wave
        const int col0 = GLU ? nt * 128 + wn * (WTN / 2) : nt * BN + wn * WTN;
        if (GLU) {
            // The clamp is a separate copy of the loop, picked by a branch on the
            // launch-uniform limit: as one loop with a runtime test, the compiler
            // computed the clamp for every element and then selected.
            const float lim = w.glu_limit;
            auto glu_epilogue = [&](auto clamp_tag) {
                constexpr bool CLAMP = decltype(clamp_tag)::value;
#pragma unroll
                for (int i = 0; i < NV; ++i) {
#pragma unroll
                    for (int jb = 0; jb < OB; ++jb) {
                        const int cb = col0 + jb * 32;
                        if (cb >= n_cols) continue;
                        // FP8 weights: a 32-column block lies inside one 64-row scale block
                        // (gate rows cb.., up rows n_cols + cb..), so its scales are wave-uniform
                        float sg = 1.0f, su = 1.0f;
                        if (W8) {
                            sg = w_scale[cb >> 6];
                            su = w_scale[(n_cols + cb) >> 6];
                        }
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r0 = (2 * i + wm) * 32 + q * 8;
                            if (r0 >= rows_valid) continue;
                            float v[4];
#pragma unroll
                            for (int m = 0; m < 4; ++m) {
                                float g = acc[i][jb][4 * q + m], u = acc[i][jb + NBN / 2][4 * q + m];
                                if (W8) {
                                    g *= sg;
                                    u *= su;
                                }
                                if (CLAMP) {  // gate capped at +limit, up clipped to [-limit, limit]
                                    g = __builtin_amdgcn_fmed3f(g, -INFINITY, lim);
                                    u = __builtin_amdgcn_fmed3f(u, -lim, lim);
                                }
                                // silu(g) = g * 1/(1 + e^-g) with the hardware reciprocal
                                // (v_rcp_f32, within 1 ulp): 2-6% faster than IEEE division
                                // here, an error far below h's bf16 rounding
                                v[m] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
                            }
                            uint32_t w0, w1;
                            quad_transpose_bf16(v[0], v[1], v[2], v[3], qs, w0, w1);
                            char* grp0 = (char*)(c_tile + ((int64_t)r0 * n_cols + (PK ? 2 * cb : cb)));
                            if (out_row < rows_valid - r0)
                                *(uint2*)(grp0 + out_off) = make_uint2(w0, w1);
                            ++stores;
                        }
                    }
                }
            };
            if (lim < INFINITY) glu_epilogue(BoolTag<true>{});
            else glu_epilogue(BoolTag<false>{});
        } else if (col0 < n_cols) {
            // Plain GEMM: the wave's two 32-column blocks are adjacent (64 columns, one
            // 128-byte line per row; N is a multiple of 64, so both exist). After the
            // quad transposes a lane holds columns 4c..4c+3 of both blocks for one row;
            // lanes c = 2j and 2j+1 (lane ^ 4) trade halves, so the even lane holds
            // columns 8j..8j+7 and the odd one 32+8j..32+8j+7, and each store
            // instruction writes 8 whole 128-byte rows, 16 bytes per lane. (Stores of
            // 8 bytes per lane, 64 bytes per row and instruction, made the down GEMM
            // about 25% slower.)
            static_assert(GLU || OB == 2, "two 32-column blocks per wave");
            const bool odd = (ln & 4) != 0;
            // byte offset of this lane's 16 bytes from the group's (row 0, column 0)
            const int st_off_col = (odd ? 32 : 0) + ((ln & 31) >> 3) * 8;  // this lane's first column
            const uint32_t st_off = (uint32_t)((out_row * n_cols + st_off_col) * 2);
            float s0 = 1.0f, s1 = 1.0f;
            if (W8) {
                s0 = w_scale[col0 >> 6];
                s1 = w_scale[(col0 + 32) >> 6];
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r0 = (2 * i + wm) * 32 + q * 8;
                    if (r0 >= rows_valid) continue;
                    float v0[4], v1[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        v0[m] = W8 ? acc[i][0][4 * q + m] * s0 : acc[i][0][4 * q + m];
                        v1[m] = W8 ? acc[i][1][4 * q + m] * s1 : acc[i][1][4 * q + m];
                    }
                    uint32_t a0, a1, b0, b1;
                    quad_transpose_bf16(v0[0], v0[1], v0[2], v0[3], qs, a0, a1);
                    quad_transpose_bf16(v1[0], v1[1], v1[2], v1[3], qs, b0, b1);
                    const uint32_t g0 = lane_xor4(odd ? a0 : b0, odd);
                    const uint32_t g1 = lane_xor4(odd ? a1 : b1, odd);
                    const uint4 o = odd ? make_uint4(g0, g1, b0, b1) : make_uint4(a0, a1, g0, g1);
                    if (SWB) {
                        // o = this lane's 8 columns of dh (bf16, as the unfused path stores
                        // them); g and u at the same row and columns of gu [rows, 2N] give
                        // dg and du, written to the same places of dgu
                        const int64_t roff = (int64_t)(r0 + out_row) * (2 * n_cols) + col0 + (st_off_col);
                        if (out_row < rows_valid - r0) {
                            const uint4 gv = *(const uint4*)(gu_tile + roff);
                            const uint4 uv = *(const uint4*)(gu_tile + roff + n_cols);
                            uint4 og, ou;
                            swiglu_bwd_x8(gv, uv, o, og, ou);
                            *(uint4*)(c_tile + roff) = og;
                            *(uint4*)(c_tile + roff + n_cols) = ou;
                        }
                        stores += 2;
                    } else {
                        // Non-temporal: each tile round writes about an L2's worth of
                        // output per XCD, which would otherwise evict the operands
                        // (down GEMM 2-8% faster; the gate/up output, 4x smaller per
                        // tile, gained nothing and keeps plain stores)
                        char* grp0 = (char*)(c_tile + ((int64_t)r0 * n_cols + col0));
                        if (out_row < rows_valid - r0) {
                            const u32x4_t o4 = {o.x, o.y, o.z, o.w};
                            __builtin_nontemporal_store(o4, (u32x4_t*)(grp0 + st_off));
                        }
                        ++stores;
                    }
                }
            }
        }
    }
    return stores;
}

// The LDS one workgroup of the grouped GEMM uses (declared by the kernel that
// runs it: the grouped GEMM kernel, or the fused layer kernel between its phases).
struct GemmShared {
    uint16_t* lds;         // the operand ring, kLdsElems, 1024-byte aligned
    int32_t* tile_start;   // [kMaxE + 1]
    int32_t* seg_start;    // [kMaxE + 1]
    int32_t* scan_tmp;     // [kWaves]
    int32_t* tok_lds;      // gathering A: [2][kWaves][kTokSlots], 16-byte aligned
};

// One workgroup's share of a grouped GEMM launch: workgroup `blk` of `nblk`
// (a multiple of the 8 XCDs; workgroup b runs on XCD b % 8).
template <bool GLU, bool GATHER, bool W8, bool SWB, bool PK = false>
__device__ __forceinline__ void grouped_gemm_body(
    const GemmShared& sh, const uint16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const void* __restrict__ W, const float* __restrict__ w_scale, const int32_t* __restrict__ offsets,
    int E, int K, int N, uint16_t* __restrict__ C, const uint16_t* __restrict__ gu, float glu_limit,
    int rows_max, int blk, int nblk) {
    static_assert(!SWB || (!GLU && !GATHER && !W8), "the SwiGLU backward epilogue follows the plain bf16 GEMM");
    static_assert(!PK || !SWB, "row-pair tiled operands are for the forward GEMMs");
    uint16_t* lds = sh.lds;
    int32_t* tile_start = sh.tile_start;
    int32_t* seg_start = sh.seg_start;
    int32_t* scan_tmp = sh.scan_tmp;
    int32_t* tok_lds = sh.tok_lds;

    const int tid = threadIdx.x;
    // column tiles per expert: GLU tiles cover 128 output columns (128 gate + 128 up rows)
    const int NT = GLU ? (N + 127) / 128 : (N + BN - 1) / BN;
    const int NW = GLU ? 2 * N : N;  // W rows per expert
    const int64_t w_stride = (int64_t)NW * K * (W8 ? 1 : 2);  // bytes per expert

    // ---- per-expert tile counts -> prefix (every workgroup builds its own copy)
    // Segments are clamped to [0, rows_max) (rows_max = P_max, the rows of A and
    // C), and an expert whose end lies before its start gets none: offsets that
    // break their contract cannot make a tile read or write outside the buffers.
    auto seg_bound = [&](int e) { return min(max(offsets[e], 0), rows_max); };
    {
        const int per = (E + kGemmThreads - 1) / kGemmThreads;  // <= 2
        int local = 0;
        for (int i = 0; i < per; ++i) {
            const int e = tid * per + i;
            if (e < E) {
                const int32_t o0 = seg_bound(e), o1 = max(seg_bound(e + 1), o0);
                seg_start[e] = o0;
                local += (o1 - o0 + BM - 1) / BM * NT;
            }
        }
        int run = block_exclusive_scan(local, scan_tmp);
        for (int i = 0; i < per; ++i) {
            const int e = tid * per + i;
            if (e < E) {
                tile_start[e] = run;
                const int32_t o0 = seg_bound(e), o1 = max(seg_bound(e + 1), o0);
                run += (o1 - o0 + BM - 1) / BM * NT;
            }
        }
        if (tid == 0) seg_start[E] = seg_bound(E);
        if (tid == kGemmThreads - 1) tile_start[E] = run;
        __syncthreads();
    }
    const int total = tile_start[E];

    WaveCtx w;
    w.lds = lds;
    w.lds0 = lds_addr(lds);
    w.K = K;
    w.N = N;
    w.nk = K / BK;
    w.lane = lane_id();
    w.wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    w.wm = w.wave / WGN;
    w.wn = w.wave % WGN;
    w.grp = w.wave >> 2;  // == wm
    w.tok_lds = tok_lds;
    w.glu_limit = glu_limit;
    // lane-constant parts of the MFMA operand addresses: logical piece
    // (2*ks + lane/32) of row (lane % 32) of each 32-row block
    {
        const int lrow = w.lane & 31;
        // The k order inside a stage only has to match between A and B. bf16 B:
        // k-step ks, lane half h reads k = 16ks + 8h + 0..7 (logical piece 2ks + h).
        // FP8 B: lane half h reads the 16 codes k = 16h .. 16h+15 at once, so
        // k-step ks takes k = 16h + 8ks + 0..7 of both operands (piece 2h + ks).
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const int piece = W8 ? 2 * (w.lane >> 5) + ks : 2 * ks + (w.lane >> 5);
            w.rd_off[ks] = lrow * BK + ((piece ^ swz(lrow)) << 3);
        }
        w.rd8_off = lrow * BK + (((w.lane >> 5) ^ swz8(lrow)) << 4);
    }

    // ---- XCD-aware split: XCD x takes the contiguous run [x*chunk, (x+1)*chunk)
    const int nxcd = 8;
    const int xcd = blk % nxcd, slot = blk / nxcd;
    const int per_xcd = nblk / nxcd;
    const int chunk = (total + nxcd - 1) / nxcd;
    const int t_end = min(total, (xcd + 1) * chunk);

    auto tile_args = [&](int t) {
        // expert e: the last e with tile_start[e] <= t (experts with no tiles repeat a value)
        int lo = 0, hi = E;  // invariant: tile_start[lo] <= t < tile_start[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tile_start[mid] <= t) lo = mid; else hi = mid;
        }
        // every value below is uniform over the wave: keep it in scalar registers
        const int e = __builtin_amdgcn_readfirstlane(lo);
        const int seg0 = __builtin_amdgcn_readfirstlane(seg_start[e]);
        const int seg1 = max(__builtin_amdgcn_readfirstlane(seg_start[e + 1]), seg0);
        const int q = t - __builtin_amdgcn_readfirstlane(tile_start[e]);
        // The segment's 32-row blocks are spread evenly over its ceil(rows / 256)
        // row tiles (17 blocks -> 6, 6, 5 rather than 8, 8, 1): the same MFMA
        // work, but no nearly empty tile that still streams all of its weights.
        const int nb = (seg1 - seg0 + 31) / 32;
        const int m = (nb + BM / 32 - 1) / (BM / 32);
        const int mt = q / NT, nt = q - mt * NT;  // row tile, then column tile
        const int bq = nb / m, br = nb - bq * m;  // row tile mt has bq + (mt < br) blocks
        const int row0 = seg0 + 32 * (mt * bq + min(mt, br));
        TileArgs ta;
        // PK: A (and a GLU's h) tiled in row pairs; the tile's base is row0's pair
        const int64_t rowb = PK ? (int64_t)(row0 >> 1) * 2 : (int64_t)row0;
        ta.a_tile = GATHER ? A : A + rowb * K;
        ta.row0 = row0;
        ta.w_exp = (const char*)W + (int64_t)e * w_stride;
        ta.w_scale = W8 ? w_scale + (int64_t)e * (NW / 64) : w_scale;
        ta.c_tile = C + (PK && GLU ? rowb : (int64_t)row0) * (SWB ? 2 * N : N);
        ta.gu_tile = SWB ? gu + (int64_t)row0 * 2 * N : gu;
        ta.nt = nt;
        ta.rows_valid = min(32 * (bq + (mt < br ? 1 : 0)), seg1 - row0);
        // live 32-row blocks of this wave: wave row wm owns blocks 2i + wm
        ta.nvb = max(0, min(4, ((ta.rows_valid + 31) / 32 - w.wm + 1) / 2));
        return ta;
    };

    // The next tile's first stages are prefetched when the ring can hold them
    // (at least 4 k stages per tile).
    const bool cross = w.nk >= STAGES;
    int tb = 0;  // gathering A: the current tile's token buffer
    int t = xcd * chunk + slot;
    if (t >= t_end) return;
    TileArgs cur = tile_args(t);
    int base = 0, s_prev = 0;
    bool prefetched = false;
    for (;;) {
        const int tn = t + per_xcd;
        const bool has_next = tn < t_end;
        const TileArgs nxt = has_next ? tile_args(tn) : cur;
        const bool pf_next = has_next && cross;
        int s;
        switch (cur.nvb) {
            case 4: s = run_tile<GLU, GATHER, W8, SWB, PK, 4>(w, cur, nxt, base, prefetched, pf_next, s_prev, row_token, tb); break;
            case 3: s = run_tile<GLU, GATHER, W8, SWB, PK, 3>(w, cur, nxt, base, prefetched, pf_next, s_prev, row_token, tb); break;
            case 2: s = run_tile<GLU, GATHER, W8, SWB, PK, 2>(w, cur, nxt, base, prefetched, pf_next, s_prev, row_token, tb); break;
            case 1: s = run_tile<GLU, GATHER, W8, SWB, PK, 1>(w, cur, nxt, base, prefetched, pf_next, s_prev, row_token, tb); break;
            default: s = run_tile<GLU, GATHER, W8, SWB, PK, 0>(w, cur, nxt, base, prefetched, pf_next, s_prev, row_token, tb); break;
        }
        if (!has_next) break;
        s_prev = s;
        prefetched = pf_next;
        base = (base + w.nk) & (STAGES - 1);
        tb ^= 1;
        cur = nxt;
        t = tn;
    }
}


}  // namespace moe
