// wgrad.hip -- expert weight gradients, K-grouped over each expert's rows.
//
// Two kernels: wgrad_pp_kernel (below the first; B read from the layout) and
// wgrad_kernel (B gathered through row_token). Both compute every output with the
// same MFMAs in the same order, so their results are identical bit for bit.
//
//   dW[e, m, n] = sum over the rows p of expert e's padded segment of A[p, m] B[p, n]
//
// with A, B row-major over the layout rows (dW_down: A = dy, B = h; dW_gate_up:
// A = dgu, B = x_perm, or the token rows x[row_token[p]] read in place), fp32
// accumulation and fp32 output [prime-rl PR 3885, Changes: weight-gradient GEMMs
// write straight into fp32 accumulators; one K-grouped GEMM launch per weight].
// Pad rows of a segment contribute nothing: the backward zeroes them in A.
//
// The reduction runs over rows, which are the strided dimension of both operands.
// Each 32-row chunk goes into LDS as it is in memory ([row][column], 16-byte
// stores of the 16-byte loads), and the MFMA fragments -- 8 consecutive rows of
// one column -- are read transposed with gfx950's ds_read_b64_tr_b16: within each
// group of 16 lanes, lane i receives element i % 4 of the 8-byte pieces addressed
// by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12, so when lane q addresses row
// kb + q/4, columns c + 4 (q % 4) .. +3, lane i gets rows kb .. kb+3 of column
// c + i; two such reads make a fragment. (The version before this wrote the rows
// transposed, as 32-bit (row, row+1) pairs at [column][row]: 4-byte LDS stores
// with 2-way bank conflicts, 29% of its LDS cycles.) A row is padded to 576 bytes
// so that the four rows a half-wave reads sit in four different 64-byte bank
// groups. Tile 256 x 256 per workgroup of eight
// waves (2 x 4 waves of 128 x 64, v_mfma_f32_32x32x16_bf16: 12 fragment reads per
// 16 MFMAs; a 128 x 128 tile of four 64 x 64 waves read 8 per 8 and was bound by
// LDS traffic). LDS is double-buffered, and the chunks' global loads go through
// a ring of kWgDepth register slots, so the loads of the next kWgDepth chunks are
// in flight during the MFMAs (one chunk ahead left every chunk waiting on its
// loads). One workgroup per (expert, tile), tiles dealt to the XCDs in
// contiguous runs so that an expert's tiles, which read the same rows, share an
// L2; an expert with no rows writes zeros.
#include "common.hpp"

namespace moe {

constexpr int kWgBM = 256, kWgBN = 256, kWgBK = 32;
constexpr int kWgThreads = 512;
constexpr int kWgDepth = 3;  // chunks of global loads in flight

// Workgroup barrier after this wave's LDS accesses have completed. Unlike
// __syncthreads() it does not wait for the global loads in flight (those land
// in registers, and the compiler waits for each before its first use), so the
// load ring stays full across barriers.
__device__ __forceinline__ void wg_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
constexpr int kWgStride = kWgBM + 32;  // bf16 per LDS row: 576 bytes, 64 bytes past a 256-byte multiple

// 4 bf16 of one column, 4 consecutive rows (see above); p: this lane's 8-byte piece
__device__ __forceinline__ v4i16_t ds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
}

// rows 0..3 and 4..7 of a fragment's column, as one 8 x bf16 operand
__device__ __forceinline__ bf16x8_t frag_of(v4i16_t lo, v4i16_t hi) {
    const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

template <bool GATHER_B>
__global__ __launch_bounds__(kWgThreads, 1) void wgrad_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                    const int32_t* __restrict__ row_token,
                                                    const int32_t* __restrict__ offsets, int M, int N,
                                                    int tiles_m, int tiles_n, int rows_max, float* __restrict__ dW) {
    MOE_DEBUG_GUARD();
    __shared__ __attribute__((aligned(16))) uint16_t at[2][kWgBK][kWgStride];
    __shared__ __attribute__((aligned(16))) uint16_t bt[2][kWgBK][kWgStride];
    static_assert(kWgBM == kWgBN, "A and B chunks share the staging layout");

    // XCD-aware order: block b runs on XCD b % 8; XCD x takes tiles
    // [start_x, start_x + count_x) in order, count_x = blocks on XCD x
    const int64_t nb = gridDim.x, bx = blockIdx.x % 8;
    int64_t b = blockIdx.x / 8;
    for (int x = 0; x < bx; ++x) b += (nb - x + 7) / 8;
    const int e = (int)(b / ((int64_t)tiles_m * tiles_n));
    const int rem = (int)(b - (int64_t)e * tiles_m * tiles_n);
    const int m0 = (rem / tiles_n) * kWgBM, n0 = (rem % tiles_n) * kWgBN;
    // the segment clamped to [0, rows_max): offsets that break their contract cannot
    // make a load leave A or B
    const int seg0 = min(max(offsets[e], 0), rows_max), seg1 = max(min(offsets[e + 1], rows_max), seg0);
    const int nchunks = (seg1 - seg0 + kWgBK - 1) / kWgBK;

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = tid / kWave, wm = wave >> 2, wn = wave & 3;
    // staging: thread -> row pair (2pp, 2pp+1) of the chunk, 16-byte column piece cp
    // (0..31); a wavefront's 32 lanes of one row read and write 512 contiguous bytes
    const int cp = tid & 31, pp = tid >> 5;
    const int ca = m0 + 8 * cp, cb = n0 + 8 * cp;
    const bool a_col = ca < M, b_col = cb < N;

    // Chunk ch's loads go to register slot ch % kWgDepth. The loads themselves are
    // unconditional (a row past the segment, or a chunk past the last, reads the
    // segment's first row; a column past the matrix reads column 0) and the values
    // are zeroed when they are used, so no load sits under a branch and the
    // compiler's waits keep the ring in flight. (Gathering B needs the token
    // before its row can be read; that variant waits for it.)
    u32x4_t ra[kWgDepth][2], rb[kWgDepth][2];
    bool oka[kWgDepth][2], okb[kWgDepth][2];
    const int ca_ld = a_col ? ca : 0, cb_ld = b_col ? cb : 0;
#define MOE_WG_LOAD(slot, ch)                                                                     \
    do {                                                                                          \
        _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                           \
            const int p = seg0 + (ch) * kWgBK + 2 * pp + h;                                       \
            const bool in = p < seg1;                                                             \
            const int pl = in ? p : seg0;                                                         \
            ra[slot][h] = *(const u32x4_t*)(A + (int64_t)pl * M + ca_ld);                         \
            oka[slot][h] = in && a_col;                                                           \
            if (GATHER_B) {                                                                       \
                const int32_t tk = in ? row_token[p] : -1;                                        \
                okb[slot][h] = in && b_col && tk >= 0;                                            \
                rb[slot][h] = okb[slot][h] ? *(const u32x4_t*)(B + (int64_t)tk * N + cb)          \
                                           : u32x4_t{0u, 0u, 0u, 0u};                             \
            } else {                                                                              \
                rb[slot][h] = *(const u32x4_t*)(B + (int64_t)pl * N + cb_ld);                     \
                okb[slot][h] = in && b_col;                                                       \
            }                                                                                     \
        }                                                                                         \
    } while (0)
    // rows 2pp, 2pp+1, columns 8cp .. 8cp+7 as loaded (zero where out of range)
    auto store = [&](const u32x4_t (&ra2)[2], const u32x4_t (&rb2)[2], const bool (&oa)[2],
                     const bool (&ob)[2], int buf) {
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            *(u32x4_t*)&at[buf][2 * pp + h][8 * cp] = oa[h] ? ra2[h] : z;
            *(u32x4_t*)&bt[buf][2 * pp + h][8 * cp] = ob[h] ? rb2[h] : z;
        }
    };

    floatx16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // transposed fragment reads: lane l (group g = l / 16, q = l % 16) addresses row
    // 8 (g / 2) + q / 4 (+ 4 for the second half of the fragment, + 16 ks) and
    // columns 16 (g % 2) + 4 (q % 4) .. +3 of the 32-column block; it receives
    // column l % 32 of the block, rows 8 (l / 32) .. +7 of the k step
    const int tr_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    if (nchunks > 0) {
        // chunk 0 straight to LDS buffer 0; chunks 1 .. kWgDepth into their slots
        MOE_WG_LOAD(0, 0);
        store(ra[0], rb[0], oka[0], okb[0], 0);
#pragma unroll
        for (int d = 1; d < kWgDepth; ++d) MOE_WG_LOAD(d, d);
        MOE_WG_LOAD(0, kWgDepth);
        wg_lds_barrier();
    }
    // iteration ch: MFMAs on LDS buffer ch & 1; chunk ch+1 from its slot into the
    // other buffer (free since the last barrier); that slot refilled with chunk
    // ch+1+kWgDepth; one barrier. Full rounds of kWgDepth chunks run without
    // branches (a branch inside the ring makes the compiler's waits drain it);
    // the last partial round is guarded. Scheduling barriers keep each chunk's
    // store where it is: hoisted to the top of a round, the stores of later
    // chunks would wait there for loads issued only one chunk earlier.
#define MOE_WG_CHUNK(d, ch)                                                                       \
    do {                                                                                          \
        const int buf_ = (ch) & 1;                                                                \
        _Pragma("unroll") for (int ks = 0; ks < kWgBK / 16; ++ks) {                               \
            bf16x8_t fa[4], fb[2];                                                                \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                       \
                const uint16_t* pa_ = &at[buf_][ks * 16 + tr_row][wm * 128 + i * 32 + tr_col];    \
                fa[i] = frag_of(ds_read_tr16(pa_), ds_read_tr16(pa_ + 4 * kWgStride));            \
            }                                                                                     \
            _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                       \
                const uint16_t* pb_ = &bt[buf_][ks * 16 + tr_row][wn * 64 + j * 32 + tr_col];     \
                fb[j] = frag_of(ds_read_tr16(pb_), ds_read_tr16(pb_ + 4 * kWgStride));            \
            }                                                                                     \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                         \
                _Pragma("unroll") for (int j = 0; j < 2; ++j)                                     \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0); \
        }                                                                                         \
        constexpr int nxt_ = ((d) + 1) % kWgDepth;                                                \
        __builtin_amdgcn_sched_barrier(0);                                                        \
        store(ra[nxt_], rb[nxt_], oka[nxt_], okb[nxt_], buf_ ^ 1);                                \
        MOE_WG_LOAD(nxt_, (ch) + 1 + kWgDepth);                                                   \
        wg_lds_barrier();                                                                         \
        __builtin_amdgcn_sched_barrier(0);                                                        \
    } while (0)
    static_assert(kWgDepth == 3, "the chunk loop below is unrolled for a ring of 3");
    int ch0 = 0;
    for (; ch0 + kWgDepth <= nchunks; ch0 += kWgDepth) {
        MOE_WG_CHUNK(0, ch0);
        MOE_WG_CHUNK(1, ch0 + 1);
        MOE_WG_CHUNK(2, ch0 + 2);
    }
    if (ch0 < nchunks) MOE_WG_CHUNK(0, ch0);
    if (ch0 + 1 < nchunks) MOE_WG_CHUNK(1, ch0 + 1);
#undef MOE_WG_CHUNK
#undef MOE_WG_LOAD

    // MFMA 32x32 output: lane l, register r -> row (r/4)*8 + (l/32)*4 + r%4, column l%32.
    // Registers 4q..4q+3 of the quad of lanes 4c..4c+3 are the 4x4 block of rows
    // 8q + 4(l/32) + 0..3 and columns 4c..4c+3; a transpose inside the quad (an
    // exchange with lane ^ 1, then with lane ^ 2) leaves lane 4c+p with row
    // 8q + 4(l/32) + p, columns 4c..4c+3: one 16-byte store per lane, 8 whole
    // 128-byte rows per instruction (4-byte stores, 2 rows per instruction, took
    // four times the store instructions).
    float* out = dW + (int64_t)e * M * N;
    const bool p0 = (lane & 1) != 0, p1 = (lane & 2) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int nb = n0 + wn * 64 + j * 32;  // N % 64 == 0: a block is all in or all out
            if (nb >= N) continue;
            const int n = nb + ((lane & 31) >> 2) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = m0 + wm * 128 + i * 32 + q * 8 + (lane >> 5) * 4 + (lane & 3);
                const uint32_t v0 = __float_as_uint(acc[i][j][4 * q + 0]), v1 = __float_as_uint(acc[i][j][4 * q + 1]);
                const uint32_t v2 = __float_as_uint(acc[i][j][4 * q + 2]), v3 = __float_as_uint(acc[i][j][4 * q + 3]);
                // lane ^ 1: the odd lane takes its partner's even rows, the even lane its partner's odd rows
                const uint32_t x0 = quad_xor1(p0 ? v0 : v1), x1 = quad_xor1(p0 ? v2 : v3);
                const uint32_t t0 = p0 ? x0 : v0, t1 = p0 ? v1 : x0, t2 = p0 ? x1 : v2, t3 = p0 ? v3 : x1;
                // lane ^ 2: the same for pairs of rows
                const uint32_t y0 = quad_xor2(p1 ? t0 : t2), y1 = quad_xor2(p1 ? t1 : t3);
                const uint4 o = p1 ? make_uint4(y0, y1, t2, t3) : make_uint4(t0, t1, y0, y1);
                if (m < M) *(uint4*)(out + (int64_t)m * N + n) = o;
            }
        }
}

// ---- the ping-pong weight-gradient kernel (B not gathered) ----------------------------
//
// The same tile and MFMA shapes as wgrad_kernel, on the grouped GEMM's pipeline:
// each 32-row chunk ("stage") of A and B goes straight from global memory into a
// four-stage LDS ring with direct-to-LDS loads (global_load_lds_dwordx4, no
// register staging), rows as they are in memory, and the fragments are read with
// the transposing LDS read. Two groups of four waves (one wave of each per SIMD)
// alternate: while one group runs its MFMAs on a stage held in registers, the
// other reads its fragments of that stage and issues its half of a later stage's
// loads, so each SIMD's MFMA pipe is fed by one wave while the other waits on
// memory. Per stage s: group 0 computes in phase 2s, group 1 in phase 2s+1; group
// 1 issues its half of stage s+3 in phase 2s (into stage s-1's slot), group 0 its
// half of stage s+4 in phase 2s+1 (into stage s's slot); each group waits for its
// own half of stage s+1 by the end of phase 2s. One tile (expert, 256 x 256 block
// of dW) per workgroup.
//
// In LDS a stage row is 256 bf16 (512 bytes) of one layout row; its 16-byte piece p
// sits in slot p ^ 4 (row % 4), so the four rows a half-wave's transposing read
// touches fall in four different 64-byte bank groups. A chunk that ends past the
// expert's segment (segments not a multiple of 32 rows) is loaded whole and its
// rows past the segment are overwritten with zeros by the waves that loaded them,
// after their loads land and before the barrier that precedes any read.
//
// Order: experts ranked by rows (descending, ties to the lower id; E <= 256,
// else by id). A work unit is one row of an expert's tiles (tiles_n tiles that
// read the same A columns and all of B's, and share one L2): tile row i of rank r
// is unit u = tiles_m r + i. The units are dealt to the 8 XCDs in rounds of eight,
// forward in even rounds and backward in odd ones (XCD x takes unit 8k + x, then
// 8(k+1) + 7 - x, ...), and each XCD runs its units in order, a unit's tiles one
// after another: the longest tiles start first, and under skewed routing no XCD
// collects the largest unit of every round. (Dealing whole experts, rank r to XCD
// r % 8, left the busiest XCD 1.47x the mean work under Zipf(1.2) routing; the
// weight gradients of that layer took 21% and 15% longer.)
constexpr int kPpStages = 4;
constexpr int kPpRowElems = kWgBM;                  // 256 bf16 per stage row
constexpr int kPpOpElems = kWgBK * kPpRowElems;     // one operand's stage, 16 KB
constexpr int kPpStageElems = 2 * kPpOpElems;       // A then B, 32 KB
constexpr int kPpLoads = 4;                         // this thread's loads per stage (2 A + 2 B)
constexpr int kPpRankMaxE = 256;

__device__ __forceinline__ uint32_t pp_lds_addr(const uint16_t* p) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) const uint16_t*)p;
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane
// (M0 holds the wave's LDS base). Every wait on these loads is an explicit vmcnt.
__device__ __forceinline__ void pp_dma16(uint32_t lds_base, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" :: "s"(lds_base), "v"(voff), "s"(sbase)
                 : "memory");
}
template <int N>
__device__ __forceinline__ void pp_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// at most `later` stages of this thread's loads left in flight
__device__ __forceinline__ void pp_wait_stages(int later) {
    if (later >= 3) pp_wait_vmcnt<3 * kPpLoads>();
    else if (later == 2) pp_wait_vmcnt<2 * kPpLoads>();
    else if (later == 1) pp_wait_vmcnt<kPpLoads>();
    else pp_wait_vmcnt<0>();
}

// AT / BT: A / B stored in row pairs (element (p, c) of a C-column operand at
// (p/2)*2C + (c/32)*64 + (p%2)*32 + c%32, the order moe_tile_rows writes). Only the
// global addresses change: a 32-row stage still starts 32*C elements after the
// previous one, and each lane's 16 bytes land in the same LDS slot as for a
// row-major operand, so the MFMAs and every result bit are the same.
template <bool AT, bool BT>
__global__ __launch_bounds__(kWgThreads, 1) void wgrad_pp_kernel(const uint16_t* __restrict__ A,
                                                                 const uint16_t* __restrict__ B,
                                                                 const int32_t* __restrict__ offsets, int E, int M,
                                                                 int N, int tiles_m, int tiles_n, int rows_max,
                                                                 float* __restrict__ dW) {
    MOE_DEBUG_GUARD();
    __shared__ __attribute__((aligned(1024))) uint16_t ring[kPpStages * kPpStageElems];
    __shared__ int32_t rows_lds[kPpRankMaxE];
    __shared__ int32_t pick;

    // ---- this block's tile: unit u (round k of its XCD), tile tile_n of the unit
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int k = slot / tiles_n, tile_n = slot - k * tiles_n;
    const int u = 8 * k + ((k & 1) ? 7 - xcd : xcd);
    const int r = u / tiles_m;  // the expert rank this block serves
    if (r >= E) return;         // uniform over the block
    const int tile_m = u - r * tiles_m;
    const int tid = threadIdx.x;
    int e = r;
    if (E <= kPpRankMaxE) {
        for (int i = tid; i < E; i += kWgThreads) rows_lds[i] = max(offsets[i + 1] - offsets[i], 0);
        __syncthreads();
        if (tid < E) {
            const int mine = rows_lds[tid];
            int rank = 0;
            for (int i = 0; i < E; ++i) {
                const int o = rows_lds[i];
                rank += (o > mine) || (o == mine && i < tid);
            }
            if (rank == r) pick = tid;
        }
        __syncthreads();
        e = pick;
    }
    const int m0 = tile_m * kWgBM, n0 = tile_n * kWgBN;
    // the segment clamped to [0, rows_max), as in wgrad_kernel
    const int seg0 = min(max(offsets[e], 0), rows_max);
    const int rows = max(min(offsets[e + 1], rows_max) - seg0, 0);
    const int nk = (rows + kWgBK - 1) / kWgBK;
    const int valid_last = rows - (nk - 1) * kWgBK;  // rows of the last stage inside the segment

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave >> 2, wn = wave & 3, grp = wm;
    const uint32_t ring0 = pp_lds_addr(ring);

    // ---- this thread's load pieces: wave w, load i fills stage rows 4w + 2i + (0, 1);
    // lane l: row 4w + 2i + l/32, physical slot l%32 = logical piece (l%32) ^ 4 (row%4)
    // (the last stage's rows past the segment read its last row inside it instead --
    // never a row past P_max -- and are zeroed in LDS once loaded; columns past M or N
    // read column 0, and their results are never stored)
    // (row pairs: the bases are the pair of the segment's first row, and a stage row r
    // lies r + seg0 % 2 rows past it)
    const int par = seg0 & 1;
    // element offset of (row r, column c) from the base of a C-column operand
    auto off_of = [](bool tiled, int r, int c, int C) {
        return tiled ? (r >> 1) * 2 * C + (c >> 5) * 64 + (r & 1) * 32 + (c & 31) : r * C + c;
    };
    uint32_t a_off[2], b_off[2], a_off_last[2], b_off_last[2];
    int ld_row[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 4 * wave + 2 * i + (lane >> 5);
        const int row_last = row < valid_last ? row : valid_last - 1;
        const int piece = (lane & 31) ^ (4 * (row & 3));
        const int ca = m0 + 8 * piece, cb = n0 + 8 * piece;
        const int cca = ca < M ? ca : 0, ccb = cb < N ? cb : 0;
        ld_row[i] = row;
        a_off[i] = (uint32_t)off_of(AT, AT ? row + par : row, cca, M) * 2u;
        b_off[i] = (uint32_t)off_of(BT, BT ? row + par : row, ccb, N) * 2u;
        a_off_last[i] = (uint32_t)off_of(AT, AT ? row_last + par : row_last, cca, M) * 2u;
        b_off_last[i] = (uint32_t)off_of(BT, BT ? row_last + par : row_last, ccb, N) * 2u;
    }
    const char* a_base = (const char*)(A + (int64_t)(AT ? seg0 - par : seg0) * M);
    const char* b_base = (const char*)(B + (int64_t)(BT ? seg0 - par : seg0) * N);
    const int64_t a_step = (int64_t)kWgBK * M * 2, b_step = (int64_t)kWgBK * N * 2;  // bytes per stage

    auto issue = [&](int st) {  // this thread's pieces of stage st
        const uint32_t sa = ring0 + (uint32_t)((st & (kPpStages - 1)) * kPpStageElems * 2);
        const bool last = st == nk - 1;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            pp_dma16(sa + (uint32_t)((2 * wave + i) * 1024), a_base + st * a_step, last ? a_off_last[i] : a_off[i]);
            pp_dma16(sa + (uint32_t)(kPpOpElems * 2 + (2 * wave + i) * 1024), b_base + st * b_step,
                     last ? b_off_last[i] : b_off[i]);
        }
    };
    // after this thread's loads of the last stage landed: zero its rows past the segment
    auto zero_tail = [&](int st) {
        if (valid_last >= kWgBK || st != nk - 1) return;
        uint16_t* sa = ring + (st & (kPpStages - 1)) * kPpStageElems;
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 2; ++i)
            if (ld_row[i] >= valid_last) {
                const int off = ld_row[i] * kPpRowElems + 8 * (lane & 31);
                *(u32x4_t*)(sa + off) = z;
                *(u32x4_t*)(sa + kPpOpElems + off) = z;
            }
    };

    // ---- fragment reads (transposing): lane l addresses row 8 (l/32) + (l%16)/4 (+4 for
    // the upper half) of the k step and columns 16 ((l/16)%2) + 4 (l%4) .. +3 of a
    // 32-column block; the row's swizzle 4 (row%4) depends on (l%16)/4 alone
    const int tr_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int tr_swz = 4 * (((lane & 15) >> 2) & 3);
    const int tr_colp = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // piece within the 32-column block
    const int tr_half = 4 * (lane & 1);                              // element offset within the piece
    // element offset of this lane's 8-byte piece for the 32-column block starting at piece pb
    auto tr_off = [&](int pb, int ks) {
        return (ks * 16 + tr_row) * kPpRowElems + (((pb + tr_colp) ^ tr_swz) << 3) + tr_half;
    };
    bf16x8_t fa[2][4], fb[2][2];
    // (macros rather than lambdas: a lambda capturing the fragments or accumulators by
    // reference kept them in scratch memory)
#define MOE_PP_READ_FRAGS(st)                                                                   \
    do {                                                                                        \
        const uint16_t* sa_ = ring + ((st) & (kPpStages - 1)) * kPpStageElems;                  \
        const uint16_t* sb_ = sa_ + kPpOpElems;                                                 \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                      \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                     \
                const uint16_t* pa_ = sa_ + tr_off(wm * 16 + i * 4, ks);                        \
                fa[ks][i] = frag_of(ds_read_tr16(pa_), ds_read_tr16(pa_ + 4 * kPpRowElems));    \
            }                                                                                   \
            _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                     \
                const uint16_t* pb_ = sb_ + tr_off(wn * 8 + j * 4, ks);                         \
                fb[ks][j] = frag_of(ds_read_tr16(pb_), ds_read_tr16(pb_ + 4 * kPpRowElems));    \
            }                                                                                   \
        }                                                                                       \
    } while (0)
    floatx16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = floatx16_t{};
#define MOE_PP_MMA()                                                                            \
    do {                                                                                        \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks)                                        \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                       \
                _Pragma("unroll") for (int j = 0; j < 2; ++j)                                   \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0); \
    } while (0)
    // stages st+1.. of this group still in flight after its loads up to stage `upto`
    auto later = [&](int st, int upto) { return max(0, min(upto, nk - 1) - st); };

    if (nk > 0) {
        // prologue: both groups issue their halves of stages 0..2, group 0 also of 3
        for (int st = 0; st < kPpStages - 1; ++st)
            if (st < nk) issue(st);
        if (grp == 0 && kPpStages - 1 < nk) issue(kPpStages - 1);
        pp_wait_stages(later(0, grp == 0 ? kPpStages - 1 : kPpStages - 2));
        zero_tail(0);
        wg_lds_barrier();
        if (grp == 0) MOE_PP_READ_FRAGS(0);
        wg_lds_barrier();
        // each group runs its own loop (a branch on the group inside one loop made the
        // compiler keep two copies of the accumulators)
        if (grp == 0) {
            for (int kt = 0; kt < nk; ++kt) {
                // phase 2kt: compute stage kt; wait for own half of stage kt+1
                __builtin_amdgcn_s_setprio(1);
                MOE_PP_MMA();
                __builtin_amdgcn_s_setprio(0);
                if (kt + 1 < nk) {
                    pp_wait_stages(later(kt + 1, kt + 3));
                    zero_tail(kt + 1);
                }
                wg_lds_barrier();
                // phase 2kt+1: refill stage kt's slot with stage kt+4; read stage kt+1
                if (kt + 4 < nk) issue(kt + 4);
                if (kt + 1 < nk) MOE_PP_READ_FRAGS(kt + 1);
                wg_lds_barrier();
            }
        } else {
            for (int kt = 0; kt < nk; ++kt) {
                // phase 2kt: read stage kt; issue stage kt+3 into stage kt-1's slot; wait for kt+1
                MOE_PP_READ_FRAGS(kt);
                if (kt + 3 < nk) issue(kt + 3);
                if (kt + 1 < nk) {
                    pp_wait_stages(later(kt + 1, kt + 3));
                    zero_tail(kt + 1);
                }
                wg_lds_barrier();
                // phase 2kt+1: compute stage kt
                __builtin_amdgcn_s_setprio(1);
                MOE_PP_MMA();
                __builtin_amdgcn_s_setprio(0);
                wg_lds_barrier();
            }
        }
    }

#undef MOE_PP_READ_FRAGS
#undef MOE_PP_MMA

    // ---- epilogue (as wgrad_kernel's): 16-byte fp32 stores, 8 whole 128-byte rows each
    float* out = dW + (int64_t)e * M * N;
    const bool p0 = (lane & 1) != 0, p1 = (lane & 2) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int nb = n0 + wn * 64 + j * 32;
            if (nb >= N) continue;
            const int n = nb + ((lane & 31) >> 2) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = m0 + wm * 128 + i * 32 + q * 8 + (lane >> 5) * 4 + (lane & 3);
                const uint32_t v0 = __float_as_uint(acc[i][j][4 * q + 0]), v1 = __float_as_uint(acc[i][j][4 * q + 1]);
                const uint32_t v2 = __float_as_uint(acc[i][j][4 * q + 2]), v3 = __float_as_uint(acc[i][j][4 * q + 3]);
                const uint32_t x0 = quad_xor1(p0 ? v0 : v1), x1 = quad_xor1(p0 ? v2 : v3);
                const uint32_t t0 = p0 ? x0 : v0, t1 = p0 ? v1 : x0, t2 = p0 ? x1 : v2, t3 = p0 ? v3 : x1;
                const uint32_t y0 = quad_xor2(p1 ? t0 : t2), y1 = quad_xor2(p1 ? t1 : t3);
                const uint4 o = p1 ? make_uint4(y0, y1, t2, t3) : make_uint4(t0, t1, y0, y1);
                if (m < M) *(uint4*)(out + (int64_t)m * N + n) = o;
            }
        }
}

hipError_t launch_wgrad(const uint16_t* A, const uint16_t* B, const int32_t* row_token, const int32_t* offsets,
                        int E, int M, int N, int rows_max, float* dW, hipStream_t stream, bool a_tiled,
                        bool b_tiled) {
    const int tm = (M + kWgBM - 1) / kWgBM, tn = (N + kWgBN - 1) / kWgBN;
    const int64_t blocks = (int64_t)E * tm * tn;
    if (row_token) {
        if (a_tiled || b_tiled) return hipErrorInvalidValue;  // the gathering kernel reads row-major A
        hipLaunchKernelGGL(wgrad_kernel<true>, dim3((unsigned)blocks), dim3(kWgThreads), 0, stream, A, B, row_token,
                           offsets, M, N, tm, tn, rows_max, dW);
    } else {
        // E * tm units (tile rows) dealt to the 8 XCDs, 8 * ceil(E * tm / 8) of them;
        // blocks past the last unit return at once
        const int64_t units = ((int64_t)E * tm + 7) / 8 * 8;
        const int64_t pp_blocks = units * tn;
        const dim3 grid((unsigned)pp_blocks), block(kWgThreads);
        if (a_tiled && b_tiled)
            hipLaunchKernelGGL((wgrad_pp_kernel<true, true>), grid, block, 0, stream, A, B, offsets, E, M, N, tm, tn,
                               rows_max, dW);
        else if (a_tiled)
            hipLaunchKernelGGL((wgrad_pp_kernel<true, false>), grid, block, 0, stream, A, B, offsets, E, M, N, tm, tn,
                               rows_max, dW);
        else if (b_tiled)
            hipLaunchKernelGGL((wgrad_pp_kernel<false, true>), grid, block, 0, stream, A, B, offsets, E, M, N, tm, tn,
                               rows_max, dW);
        else
            hipLaunchKernelGGL((wgrad_pp_kernel<false, false>), grid, block, 0, stream, A, B, offsets, E, M, N, tm, tn,
                               rows_max, dW);
    }
    return hipGetLastError();
}

}  // namespace moe
