// grouped_gemm_small.hip -- grouped expert GEMMs when experts hold few rows.
//
// With a handful of rows per expert a grouped GEMM is bound by reading the
// expert weights, not by its flops [Halo "Performance", Levers that do not help
// here: small-M experts are weight-bandwidth-bound]. With FP8 weights the
// 256-row tiles of grouped_gemm.hip spend two of every three loads on the
// (mostly repeated) rows and stream weights at about 3 TB/s there; here the
// weights stream from HBM straight into registers, many loads deep, and meet the
// expert's few rows, which every wave re-reads from L2. (With bf16 weights the
// tiled kernel already streams at the rate of a plain read and is kept.)
//
//   - one wave is one unit: 16*NB W rows of one expert (gate/up: NB/2 blocks of
//     gate rows and the matching up rows; down: that many columns of y); every
//     A load feeds NB MFMAs per chunk, so more of the loads in flight carry
//     weights (the rows' own loads come from L2, but each still takes a slot);
//   - the expert's padded segment is taken 32 rows per pass, in chunks of 16
//     rows (v_mfma_f32_16x16x32_bf16); a pass reads the unit's weights once, so
//     an expert with at most 32 rows reads its weights exactly once (more rows:
//     more passes, which re-read the weights mostly from cache -- correct for
//     any count, weight-optimal only for few rows);
//   - each lane loads 16 bytes of a W row per k-step, kSmallDepth k-steps ahead;
//   - no LDS and no barriers: the waves of a workgroup are independent.
//
// Results are the same functions as grouped_gemm.hip's (same rows written, pad
// rows of the segment included); only the summation order differs. FP8 weights
// (E4M3 codes, one fp32 scale per 64 W rows) take 64 k per step: a lane's 16
// codes widen exactly to two bf16 operands, and the scale multiplies the fp32
// sum in the epilogue.
#include "common.hpp"

namespace moe {

constexpr int kSmallThreads = 256;  // 4 waves, one unit each
constexpr int kSmallDepth = 4;      // k-steps of loads in flight per wave
constexpr int kSmallChunks = 2;     // 16-row chunks per pass (32 rows; a 32-aligned small
                                    // expert's whole segment, with registers for 2 waves per SIMD)
// 16-row W blocks per wave: 4 for gate/up (two gate blocks, two up blocks), 2 for
// down. More blocks per A load leave more of the loads in flight to weights; the
// down GEMM has half the W rows, and at 4 blocks too few waves to keep HBM busy.
constexpr int kSmallBlocksGlu = 4;
constexpr int kSmallBlocksDown = 2;

// 8 E4M3 codes -> 8 bf16 (exact), k order kept.
__device__ __forceinline__ bf16x8_t small_fp8x8(uint32_t lo, uint32_t hi) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One pass over a unit's weights for rows [pr0, pr0 + 16*NC) of the segment.
// MFMA 16x16x32 operands: lane l gives row (A) or column (B) l % 16 and the 8
// k-values of group l / 16; the k order inside a step only has to agree between
// A and B. bf16 step (32 k): lane group g takes k = 8g .. 8g+7. FP8 step (64 k):
// group g's 16 codes are k = 16g .. 16g+15, sub-step s takes k = 16g + 8s + 0..7.
// Output: lane l, register r holds row 4*(l/16) + r, column l % 16.
template <bool GLU, bool GATHER, bool W8, int NC, int NB>
__device__ __forceinline__ void small_pass(const uint16_t* __restrict__ A,
                                           const int32_t* __restrict__ row_token,
                                           const char* const (&wr)[NB], int K, int seg0,
                                           int seg1, int pr0, int lane,
                                           const float (&sc)[NB], uint16_t* __restrict__ C,
                                           int ldc, int c0) {
    static_assert(NB % 2 == 0, "gate and up blocks come in pairs");
    constexpr int D = kSmallDepth;
    constexpr int SUB = W8 ? 2 : 1;       // MFMAs per step
    constexpr int KS = 32 * SUB;          // k per step
    const int n = lane & 15, g = lane >> 4;
    const int nsteps = K / KS;

    // this lane's A row of each chunk (rows past the segment read its first row;
    // a gathered pad row reads token 0; neither result is stored or used)
    const uint16_t* arow[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        int p = pr0 + 16 * c + n;
        if (p >= seg1) p = seg0;
        int64_t r = p;
        if (GATHER) {
            const int32_t tk = row_token[p];
            r = tk < 0 ? 0 : tk;
        }
        arow[c] = A + r * K + (W8 ? 16 * g : 8 * g);
    }
    // W: 64 bytes per step per row for both formats; this lane's 16 at byte 16g
    // `zero` is opaque per pass: otherwise the first steps' weight loads, which do
    // not depend on the pass, are hoisted out of the pass loop and the waits in the
    // k loop then count a queue in another order (an integer, not the pointers,
    // goes through the asm, so the loads stay global loads)
    int zero = 0;
    asm volatile("" : "+s"(zero));
    const char* wb[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) wb[j] = wr[j] + 16 * g + zero;

    u32x4_t bq[D][NB];
    bf16x8_t aq[D][NC][SUB];
    floatx4_t acc[NC][NB];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[c][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

#define MOE_SMALL_LOAD(d, s)                                                                   \
    do {                                                                                       \
        const int64_t s_ = (s);                                                                \
        _Pragma("unroll") for (int j = 0; j < NB; ++j)                                         \
            bq[d][j] = *(const u32x4_t*)(wb[j] + s_ * 64);                                     \
        _Pragma("unroll") for (int c = 0; c < NC; ++c)                                         \
            _Pragma("unroll") for (int u = 0; u < SUB; ++u)                                    \
                aq[d][c][u] = *(const bf16x8_t*)(arow[c] + s_ * KS + 8 * u);                   \
    } while (0)
#define MOE_SMALL_MMA(d)                                                                       \
    do {                                                                                       \
        _Pragma("unroll") for (int u = 0; u < SUB; ++u) {                                      \
            _Pragma("unroll") for (int j = 0; j < NB; ++j) {                                   \
                const bf16x8_t b_ = W8 ? small_fp8x8(bq[d][j][2 * u], bq[d][j][2 * u + 1])     \
                                       : __builtin_bit_cast(bf16x8_t, bq[d][j]);              \
                _Pragma("unroll") for (int c = 0; c < NC; ++c)                                 \
                    acc[c][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[d][c][u], b_, acc[c][j], 0, 0, 0); \
            }                                                                                  \
        }                                                                                      \
    } while (0)

    // Ring of D register slots: step s lives in slot s % D. Loads past the last
    // step re-read the last step (in bounds, from cache) so the loop needs no
    // branches; those slots are never used. The scheduling barriers keep each
    // slot's refill right after its MFMAs, so D - 1 steps stay in flight and the
    // refill can reuse the slot's registers (left alone, the scheduler gathers
    // the loads into bursts or hoists them above the MFMAs that still read the
    // slot, and the register copies and waits that follow drain the pipeline).
#pragma unroll
    for (int d = 0; d < D; ++d) {
        MOE_SMALL_LOAD(d, min(d, nsteps - 1));  // in slot order, as in the loop, so that
        __builtin_amdgcn_sched_barrier(0);      // the waits at its head count the same queue
    }
    int s0_ = 0;
    for (; s0_ + D <= nsteps; s0_ += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            MOE_SMALL_MMA(d);
            __builtin_amdgcn_sched_barrier(0);
            MOE_SMALL_LOAD(d, min(s0_ + d + D, nsteps - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    const int rem = nsteps - s0_;
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < rem) MOE_SMALL_MMA(d);
#undef MOE_SMALL_LOAD
#undef MOE_SMALL_MMA

    // epilogue: 2-byte stores, 16 lanes write 32 consecutive bytes of a row
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int p = pr0 + 16 * c + 4 * g + r;
            if (p >= seg1) continue;
            uint16_t* out = C + (int64_t)p * ldc + c0 + n;
            if (GLU) {
#pragma unroll
                for (int j = 0; j < NB / 2; ++j) {
                    const float gv = acc[c][j][r] * sc[j], uv = acc[c][j + NB / 2][r] * sc[j + NB / 2];
                    out[16 * j] = (uint16_t)f32_to_bf16_rne(gv / (1.0f + __expf(-gv)) * uv);
                }
            } else {
#pragma unroll
                for (int j = 0; j < NB; ++j) out[16 * j] = (uint16_t)f32_to_bf16_rne(acc[c][j][r] * sc[j]);
            }
        }
    }
}

// A [rows, K] bf16 (GATHER: the token matrix, row p read as row_token[p]);
// W [E, NW, K] (bf16, or E4M3 codes with scale [E, NW/64]); NW = 2N for GLU.
// C [rows, N]. Units per expert: GLU N / (8 NB) (8 NB columns of h each), down
// N / (16 NB).
template <bool GLU, bool GATHER, bool W8>
__global__ __launch_bounds__(kSmallThreads) void grouped_gemm_small_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ row_token, const void* __restrict__ W,
    const float* __restrict__ w_scale, const int32_t* __restrict__ offsets, int E, int K, int N,
    uint16_t* __restrict__ C, int rows_max) {
    MOE_DEBUG_GUARD();
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    constexpr int NB = GLU ? kSmallBlocksGlu : kSmallBlocksDown;
    constexpr int COLS = GLU ? 8 * NB : 16 * NB;  // output columns per unit
    const int units = N / COLS;                   // per expert (host checks N % COLS == 0)
    const int unit = blockIdx.x * (kSmallThreads / kWave) + wave;
    const int e = unit / units;
    if (e >= E) return;
    const int u = unit - e * units;
    // clamped to [0, rows_max) (rows_max = P_max): offsets that break their
    // contract cannot make the kernel read or write outside A or C
    const int seg0 = min(max(offsets[e], 0), rows_max), seg1 = min(max(offsets[e + 1], 0), rows_max);
    if (seg1 <= seg0) return;  // no rows: none of this expert's weights are read

    const int NW = GLU ? 2 * N : N;
    const int n = lane & 15;
    const int c0 = COLS * u;  // first output column of the unit
    const int64_t wrow = (int64_t)K * (W8 ? 1 : 2);  // bytes per W row
    const char* wexp = (const char*)W + (int64_t)e * NW * wrow;
    // this lane's W row of block j: GLU gate blocks first, then the matching up blocks
    const char* wr[NB];
    float sc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int row0 = GLU ? (j < NB / 2 ? c0 + 16 * j : N + c0 + 16 * (j - NB / 2)) : c0 + 16 * j;
        wr[j] = wexp + (row0 + n) * wrow;
        sc[j] = W8 ? w_scale[(int64_t)e * (NW / 64) + (row0 >> 6)] : 1.0f;  // 16-row block in one 64-row scale block
    }
    // Every pass takes two chunks, also when the rest of the segment fits one:
    // the one-chunk loop compiles to register copies that drain the load
    // pipeline, and a spare chunk costs only cached A reads and MFMAs.
    static_assert(kSmallChunks == 2, "passes of two 16-row chunks");
    for (int pr0 = seg0; pr0 < seg1; pr0 += 16 * kSmallChunks)
        small_pass<GLU, GATHER, W8, kSmallChunks, NB>(A, row_token, wr, K, seg0, seg1, pr0, lane, sc, C, N,
                                                      c0);
}

// glu: C = h [rows, N = I] from W [E, 2I, K = H]; down: C = y [rows, N = H] from W [E, H, K = I].
hipError_t launch_grouped_gemm_small(bool glu, const uint16_t* A, const int32_t* row_token, const void* W,
                                     const float* scale, const int32_t* offsets, int E, int K, int N,
                                     uint16_t* C, int rows_max, hipStream_t stream) {
    const int64_t units = (int64_t)E * (N / (glu ? 8 * kSmallBlocksGlu : 16 * kSmallBlocksDown));
    const int waves = kSmallThreads / kWave;
    const dim3 grid((unsigned)((units + waves - 1) / waves)), block(kSmallThreads);
#define MOE_SMALL_LAUNCH(G, GA, W8)                                                                 \
    hipLaunchKernelGGL((grouped_gemm_small_kernel<G, GA, W8>), grid, block, 0, stream, A, row_token, W, \
                       scale, offsets, E, K, N, C, rows_max)
    // FP8 weights only: with bf16 weights the 256-row tiles of the tiled kernel
    // stream the weights faster at few rows per expert (32-expert small-M layer:
    // gate/up 222 against 260 us, down 131 against 155 us on one box), so no bf16
    // instantiation is built
    if (scale == nullptr) return hipErrorInvalidValue;
    const bool gather = row_token != nullptr;
    if (glu) {
        if (gather) MOE_SMALL_LAUNCH(true, true, true); else MOE_SMALL_LAUNCH(true, false, true);
    } else {
        MOE_SMALL_LAUNCH(false, false, true);
    }
#undef MOE_SMALL_LAUNCH
    return hipGetLastError();
}

}  // namespace moe
