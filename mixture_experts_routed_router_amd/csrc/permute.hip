// permute.hip -- atomic-free counting sort of the routes into a padded,
// expert-grouped row layout, and the gather of token rows into it.
//
// [Halo "Performance", Levers that help: the atomic-free expert permute;
//  prime-rl PR 3885, Changes: one gather into the padded expert-grouped layout]
//
// The flat routes r = t*k + j are cut into chunks of kChunk routes, one chunk
// per wavefront. Inside a wave, lanes holding the same expert id find each other
// with ballots over the id's bits (match_peers): the lowest such lane is the
// group's leader and popcount gives the group size and each lane's rank. Every
// wave keeps its own histogram / cursor array in LDS, so no two lanes ever
// update the same counter in one step and nothing needs an atomic.
//
//   1. hist:    per chunk c and expert e, the count hist[c][e]        (workspace)
//   2. scan:    per expert e, counts[e] = sum_c hist[c][e], and hist[c][e] becomes
//               the number of e's routes in chunks before c (one workgroup per 64
//               experts)
//   3. scatter: every workgroup derives offsets = exclusive scan of the counts
//               rounded up to align; route_row[r] = offsets[e] + hist[c][e] + rank
//               among earlier equal ids (stable in r), row_token[route_row[r]] =
//               r / k; offsets are published and pad rows get row_token = -1
//   4. gather:  x_perm[p] = x[row_token[p]] (zero row if -1), written token-major:
//               each token's row is read once and stored to its k rows (the
//               row-pair tiled layout: each route row's whole pair, see
//               permute_copy_token_pairs_kernel)
//
// A small batch runs all four steps in one launch (permute_small_kernel), each
// workgroup building the layout in its own LDS with the same device functions.
#include <algorithm>
#include <mutex>

#include "permute_core.hpp"

namespace moe {

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / kWave;

__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ topk_idx,
                                                           int64_t R, int E, int64_t nchunks,
                                                           int32_t* __restrict__ hist) {
    MOE_DEBUG_GUARD();
    extern __shared__ int32_t lds_hist[];  // [4][E]
    const int wave = threadIdx.x / kWave;
    const int64_t c = (int64_t)blockIdx.x * 4 + wave;
    if (c >= nchunks) return;
    hist_chunk(topk_idx, R, E, c, lds_hist + wave * E, hist + c * E);
}

// One workgroup of 1024 threads per 64 experts (scan_group), so each load reads
// 256 consecutive bytes of a hist row and the passes over the histogram are
// spread over E / 64 CUs.
__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(int32_t* __restrict__ hist,
                                                                    int64_t nchunks, int E,
                                                                    int32_t* __restrict__ counts) {
    MOE_DEBUG_GUARD();
    __shared__ int32_t part[kScanWaves][kWave];
    scan_group<kScanWaves>(hist, nchunks, E, counts, blockIdx.x, part);
}

// Every workgroup first derives the padded expert offsets from the counts;
// workgroup 0 publishes them, and each workgroup writes row_token = -1 on its
// share of the pad rows. Then one wavefront per chunk (scatter_chunk).
constexpr int kScatterThreads = 256;

template <int STEPS>
__global__ __launch_bounds__(kScatterThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ topk_idx, int64_t R, int E, int k, int align, int64_t nchunks,
    int64_t P_max, const int32_t* __restrict__ base, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ route_row, int32_t* __restrict__ row_token,
    int chunk_routes) {
    MOE_DEBUG_GUARD();
    extern __shared__ int32_t lds_cursor[];  // [4][E] cursors, [E+1] offsets, [4] wave totals
    int32_t* off = lds_cursor + 4 * E;
    int32_t* wtot = off + E + 1;
    const int tid = threadIdx.x, wave = tid / kWave;
    padded_offsets(counts, E, align, off, wtot);
    if (blockIdx.x == 0)
        for (int e = tid; e <= E; e += kScatterThreads) offsets[e] = off[e];
    pad_row_tokens(counts, off, E, P_max, blockIdx.x, gridDim.x, kScatterThreads, row_token);
    const int64_t c = (int64_t)blockIdx.x * 4 + wave;
    if (c >= nchunks) return;
    scatter_chunk<STEPS>(topk_idx, R, E, k, c, base, off, lds_cursor + wave * E, route_row, row_token,
                         chunk_routes);
}

// The gather, token-major: one wavefront per token reads the token's row of x
// once (kCopyUnroll 16-byte pieces per lane in flight, 1 KB per wave-wide load)
// and writes it to the token's k layout rows (route_row), so x is read once
// rather than k times; each store instruction writes 1 KB of one row. The last
// E workgroups zero the pad rows of the experts' segments. A layout far larger
// than the 256 MB Infinity Cache is written with non-temporal stores (NT).
constexpr int kCopyUnroll = 4;
constexpr int kCopyThreads = 256;
constexpr int kCopyWaves = kCopyThreads / kWave;
constexpr int64_t kStreamingLayoutBytes = 512ll << 20;

template <bool NT>
__device__ __forceinline__ void store_piece(uint4* dst, const uint4& v) {
    if (NT) {
        const u32x4_t t4 = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(t4, (u32x4_t*)dst);
    } else {
        *dst = v;
    }
}

template <bool NT>
__global__ __launch_bounds__(kCopyThreads) void permute_copy_rows_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ route_row, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int64_t T, int k, int ppr, int64_t token_blocks,
    uint4* __restrict__ x_perm) {
    MOE_DEBUG_GUARD();
    const int lane = lane_id();
    if ((int64_t)blockIdx.x >= token_blocks) {
        // pad rows [offsets[e] + counts[e], offsets[e+1]) of expert e
        const int e = (int)((int64_t)blockIdx.x - token_blocks);
        const int64_t p0 = (int64_t)offsets[e] + counts[e], p1 = offsets[e + 1];
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        for (int64_t q = p0 * ppr + threadIdx.x; q < p1 * ppr; q += kCopyThreads) store_piece<NT>(x_perm + q, z);
        return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = (int64_t)blockIdx.x * kCopyWaves + wave;
    if (t >= T) return;
    const uint4* src = x + t * ppr;
    for (int c0 = 0; c0 < ppr; c0 += kWave * kCopyUnroll) {
        uint4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int c = c0 + u * kWave + lane;
            // x is read once here: streaming (non-temporal) loads
            u32x4_t r_ = {0u, 0u, 0u, 0u};
            if (c < ppr) r_ = __builtin_nontemporal_load((const u32x4_t*)(src + c));
            v[u] = make_uint4(r_[0], r_[1], r_[2], r_[3]);
        }
        for (int j = 0; j < k; ++j) {
            const int32_t row = __builtin_amdgcn_readfirstlane(route_row[t * k + j]);  // wave-uniform
            if (row < 0) continue;  // an out-of-range expert id has no row
            uint4* dst = x_perm + (int64_t)row * ppr;
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) {
                const int c = c0 + u * kWave + lane;
                if (c < ppr) store_piece<NT>(dst + c, v[u]);
            }
        }
    }
}

// The gather into the row-pair tiled layout (tiled.hip), token-major: one
// wavefront per token, and per route row p the wavefront writes p's whole pair
// -- its own row and the partner row p ^ 1, read through row_token (a pad or
// past-the-end partner: zeros) -- unless p is odd and its partner is a routed
// row, whose token writes the pair instead. So every pair is written by exactly
// one wavefront, 1 KB of whole 128-byte lines per store. In a pair's 2H
// contiguous elements 16-byte slot i holds piece (i/8)*4 + i%4 of row
// 2q + (i/4)%2. Pairs of two pad rows -- inside one segment's padding, or its
// last pad row and row offsets[E] -- are zeroed by the last E workgroups, each
// pair by its even row.
//
// Token blocks are dealt to the XCDs in contiguous runs (workgroup b runs on
// XCD b % 8), so the tokens in flight on one XCD are neighbours: a pair's
// partner is usually a nearby token of the same expert, whose row this XCD's
// L2 has just read. Timed alone, back to back (x resident in the Infinity
// Cache), the whole permute went from 297 to 248 us on the skewed layer's 1 GB
// layout, 99 -> 86 us at the bench-sized layer and 153 -> 136 us at 512
// experts against plain token order (a pair-major copy, one wavefront per pair
// reading both token rows, took 326, 94 and 147 us). Inside the layer, where x
// comes from HBM, the skewed permute is bound by its HBM writes (290 -> 287 us);
// the other two gain 4 and 7 us over the pair-major copy.
template <bool NT>
__global__ __launch_bounds__(kCopyThreads) void permute_copy_token_pairs_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ route_row, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int64_t T, int k, int ppr,
    int64_t token_blocks, uint4* __restrict__ x_perm) {
    MOE_DEBUG_GUARD();
    const int lane = lane_id();
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    const int n = 2 * ppr;  // 16-byte slots of a pair
    if ((int64_t)blockIdx.x >= token_blocks) {
        // expert e's pad rows [p0, p1): zero each pair whose even row is a pad row
        // and whose odd row is a pad row or past the used rows (row_token -1)
        const int e = (int)((int64_t)blockIdx.x - token_blocks);
        const int64_t p0 = (int64_t)offsets[e] + counts[e], p1 = offsets[e + 1];
        for (int64_t q = (p0 + 1) & ~(int64_t)1; q < p1; q += 2) {
            if (row_token[q + 1] >= 0) continue;
            uint4* dst = x_perm + (q >> 1) * n;
            for (int i = threadIdx.x; i < n; i += kCopyThreads) store_piece<NT>(dst + i, z);
        }
        return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    int64_t tb = blockIdx.x;  // token block: XCD-contiguous runs over the first whole multiple of 8 blocks
    const int64_t nb8 = token_blocks / 8 * 8;
    if (tb < nb8) tb = (tb % 8) * (nb8 / 8) + tb / 8;
    const int64_t t = tb * kCopyWaves + wave;
    if (t >= T) return;
    const uint4* src = x + t * ppr;
    for (int j = 0; j < k; ++j) {
        const int32_t row = __builtin_amdgcn_readfirstlane(route_row[t * k + j]);
        if (row < 0) continue;  // an out-of-range expert id has no row
        const int odd = row & 1;
        const int32_t tp = __builtin_amdgcn_readfirstlane(row_token[row ^ 1]);
        if (odd && tp >= 0) continue;  // the partner's token writes this pair
        const uint4* srcp = x + (int64_t)(tp < 0 ? 0 : tp) * ppr;
        uint4* dst = x_perm + (int64_t)(row >> 1) * n;
        for (int i0 = 0; i0 < n; i0 += kWave * kCopyUnroll) {
            uint4 v[kCopyUnroll];
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) {
                const int i = i0 + u * kWave + lane;
                const int half = (i >> 2) & 1;
                const int c = ((i >> 3) << 2) | (i & 3);
                v[u] = z;
                if (i < n) {
                    if (half == odd) v[u] = src[c];
                    else if (tp >= 0) v[u] = srcp[c];
                }
            }
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) {
                const int i = i0 + u * kWave + lane;
                if (i < n) store_piece<NT>(dst + i, v[u]);
            }
        }
    }
}

int64_t permute_chunks(int64_t R) { return (R + kChunk - 1) / kChunk; }

// The permute of a small batch in one launch (at most kSmallRoutes routes, a
// layout bound of at most kSmallRows rows), where the four launches of the split
// path would cost more than their work. Every workgroup builds the whole layout
// in its own LDS with the split path's own steps -- per-chunk histograms
// (hist_chunk), the scan over chunks, padded_offsets and the stable scatter
// (scatter_chunk) -- so the results are the same bits. Workgroup 0 then
// publishes counts, offsets, route_row and the used rows of row_token, every
// workgroup writes row_token = -1 on its share of the rows from offsets[E] to
// P_max, and gathers its share of the used layout rows (TILED: row pairs, as
// the split path's copy lays them out) from row_token in LDS. Nothing is read from
// another workgroup, so no workgroup waits on another.
constexpr int64_t kSmallRoutes = 2048;
constexpr int64_t kSmallRows = 8192;
constexpr int kSmallThreads = 256;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr size_t kSmallLdsBytes = 64 << 10;

static size_t small_permute_lds_bytes(int64_t R, int E, int64_t rows_cap) {
    const int64_t nchunks = (R + kChunk - 1) / kChunk;
    // hist [nchunks][E], cur [4][E], off [E + 1], wtot [4], cnt [E], route_row [R], row_token [rows_cap]
    return (size_t)(nchunks * E + kSmallWaves * E + (E + 1) + 4 + E + R + rows_cap) * sizeof(int32_t);
}

static bool use_small_permute(int64_t R, int E, int64_t rows_cap) {
    return R > 0 && R <= kSmallRoutes && rows_cap <= kSmallRows &&
           small_permute_lds_bytes(R, E, rows_cap) <= kSmallLdsBytes;
}

template <bool TILED>
__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ topk_idx, int64_t R, int E, int k, int align,
    int64_t P_max, int rows_cap, int ppr, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ route_row, int32_t* __restrict__ row_token, uint4* __restrict__ x_perm) {
    MOE_DEBUG_GUARD();
    extern __shared__ int32_t lds_small[];
    const int nchunks = (int)((R + kChunk - 1) / kChunk);
    int32_t* hist = lds_small;               // [nchunks][E]
    int32_t* cur = hist + nchunks * E;       // [kSmallWaves][E], per wave
    int32_t* off = cur + kSmallWaves * E;    // [E + 1]
    int32_t* wtot = off + E + 1;             // [4]
    int32_t* cnt = wtot + 4;                 // [E]
    int32_t* rrow = cnt + E;                 // [R]
    int32_t* rtok = rrow + R;                // [rows_cap]
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();

    // 1. per-chunk histograms; every row starts as a pad row
    for (int c = wave; c < nchunks; c += kSmallWaves) hist_chunk(topk_idx, R, E, c, cur + wave * E, hist + c * E);
    for (int p = tid; p < rows_cap; p += kSmallThreads) rtok[p] = -1;
    __syncthreads();
    // 2. per expert: its count, and each chunk's routes to it in earlier chunks
    for (int e = tid; e < E; e += kSmallThreads) {
        int32_t run = 0;
        for (int c = 0; c < nchunks; ++c) {
            const int32_t v = hist[c * E + e];
            hist[c * E + e] = run;
            run += v;
        }
        cnt[e] = run;
    }
    __syncthreads();
    // 3. the padded offsets (two barriers inside)
    padded_offsets(cnt, E, align, off, wtot);
    // 4. the stable scatter, into LDS
    for (int c = wave; c < nchunks; c += kSmallWaves)
        scatter_chunk<kSteps>(topk_idx, R, E, k, c, hist, off, cur + wave * E, rrow, rtok, (int)kChunk);
    __syncthreads();
    const int64_t used = off[E];

    // 5. publish the layout
    if (blockIdx.x == 0) {
        for (int e = tid; e <= E; e += kSmallThreads) {
            offsets[e] = off[e];
            if (e < E) counts[e] = cnt[e];
        }
        for (int64_t r = tid; r < R; r += kSmallThreads) route_row[r] = rrow[r];
        for (int64_t p = tid; p < used; p += kSmallThreads) row_token[p] = rtok[p];
    }
    for (int64_t p = used + (int64_t)blockIdx.x * kSmallThreads + tid; p < P_max;
         p += (int64_t)gridDim.x * kSmallThreads)
        row_token[p] = -1;
    if (!x_perm) return;  // the layout only

    // 6. the gather: one wavefront per slice of kWave * kCopyUnroll 16-byte slots
    // of a layout row (TILED: of a row pair), all of its loads in flight at once
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    const int n = TILED ? 2 * ppr : ppr;  // 16-byte slots per row (pair)
    const int slices = (n + kWave * kCopyUnroll - 1) / (kWave * kCopyUnroll);
    const int64_t units = (TILED ? (used + 1) / 2 : used) * slices;
    for (int64_t w = (int64_t)blockIdx.x * kSmallWaves + wave; w < units; w += (int64_t)gridDim.x * kSmallWaves) {
        const int64_t q = w / slices;
        const int i0 = (int)(w - q * slices) * kWave * kCopyUnroll;
        const int64_t p0 = TILED ? 2 * q : q;
        const int32_t t0 = rtok[p0];
        const int32_t t1 = TILED && p0 + 1 < used ? rtok[p0 + 1] : -1;
        const uint4* src0 = x + (int64_t)(t0 < 0 ? 0 : t0) * ppr;
        const uint4* src1 = x + (int64_t)(t1 < 0 ? 0 : t1) * ppr;
        uint4* dst = x_perm + q * n;
        {
            uint4 v[kCopyUnroll];
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) {
                const int i = i0 + u * kWave + lane;
                // tiled: slot i holds piece (i/8)*4 + i%4 of the pair's row (i/4)%2
                const bool second = TILED && ((i >> 2) & 1);
                const int c = TILED ? (((i >> 3) << 2) | (i & 3)) : i;
                const int32_t t = second ? t1 : t0;
                v[u] = z;
                if (i < n && t >= 0) v[u] = *((second ? src1 : src0) + c);
            }
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) {
                const int i = i0 + u * kWave + lane;
                if (i < n) dst[i] = v[u];
            }
        }
    }
}

static hipError_t launch_permute_small(const uint16_t* x, const int32_t* topk_idx, int64_t R, int H, int E, int k,
                                       int align, int64_t P_max, int64_t rows_cap, int32_t* counts,
                                       int32_t* offsets, int32_t* route_row, int32_t* row_token, uint16_t* x_perm,
                                       bool tiled, hipStream_t stream) {
    const int ppr = H / 8;
    const int n = tiled ? 2 * ppr : ppr;
    const int64_t slices = (n + kWave * kCopyUnroll - 1) / (kWave * kCopyUnroll);
    const int64_t units = x_perm ? (tiled ? (rows_cap + 1) / 2 : rows_cap) * slices : 0;
    // one wavefront per gather unit, up to 1024 workgroups; at least one (it publishes the layout)
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(1024, (units + kSmallWaves - 1) / kSmallWaves));
    const size_t lds = small_permute_lds_bytes(R, E, rows_cap);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kSmallThreads), lds, stream, (const uint4*)x, topk_idx,
                           R, E, k, align, P_max, (int)rows_cap, ppr, counts, offsets, route_row, row_token,
                           (uint4*)x_perm);
    };
    if (tiled) go(permute_small_kernel<true>);
    else go(permute_small_kernel<false>);
    return hipGetLastError();
}


hipError_t launch_permute_copy(const uint16_t* x, int64_t T, int H, int E, int k, int64_t P_max,
                               const int32_t* counts, const int32_t* offsets, const int32_t* route_row,
                               const int32_t* row_token, uint16_t* x_perm, bool tiled, hipStream_t stream);

size_t permute_workspace_bytes(int64_t R, int E) {
    const size_t b = (size_t)permute_chunks(R) * (size_t)E * sizeof(int32_t);
    return (b + 255) / 256 * 256;
}

hipError_t launch_permute(const uint16_t* x, const int32_t* topk_idx, int64_t T, int H, int E,
                          int k, int align, int64_t P_max, int32_t* counts, int32_t* offsets,
                          int32_t* route_row, int32_t* row_token, uint16_t* x_perm,
                          void* workspace, bool tiled, hipStream_t stream) {
    const int64_t R = T * k;
    const int64_t rows_cap = R + (int64_t)E * (align - 1);  // no layout is longer
    if (use_small_permute(R, E, rows_cap))
        return launch_permute_small(x, topk_idx, R, H, E, k, align, P_max, rows_cap, counts, offsets, route_row,
                                    row_token, x_perm, tiled, stream);
    const int64_t nchunks = permute_chunks(R);
    int32_t* hist = (int32_t*)workspace;
    const size_t lds = 4 * (size_t)E * sizeof(int32_t);
    if (nchunks > 0) {
        hipLaunchKernelGGL(permute_hist_kernel, dim3((unsigned)((nchunks + 3) / 4)), dim3(256), lds,
                           stream, topk_idx, R, E, nchunks, hist);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(permute_scan_kernel, dim3((unsigned)((E + kWave - 1) / kWave)), dim3(kScanThreads), 0,
                       stream, hist, nchunks, E, counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // at least one workgroup: it also publishes the offsets and the pad rows
    const int64_t scatter_blocks = nchunks > 0 ? (nchunks + 3) / 4 : 1;
    const size_t scatter_lds = (4 * (size_t)E + E + 1 + 4) * sizeof(int32_t);
    hipLaunchKernelGGL(permute_scatter_kernel<kSteps>, dim3((unsigned)scatter_blocks), dim3(kScatterThreads),
                       scatter_lds, stream, topk_idx, R, E, k, align, nchunks, P_max, (const int32_t*)hist,
                       (const int32_t*)counts, offsets, route_row, row_token, kChunk);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_permute_copy(x, T, H, E, k, P_max, counts, offsets, route_row, row_token, x_perm, tiled, stream);
}

// The permute from a histogram the routing kernel already wrote (hist [nchunks][E],
// chunk c = tokens [c * tpw, (c + 1) * tpw)): scan, scatter, gather -- no counting pass.
int route_hist_tokens_per_chunk(int64_t T, int E);

size_t route_hist_workspace_bytes(int64_t T, int E) {
    const int64_t tpw = route_hist_tokens_per_chunk(T, E);
    const size_t b = (size_t)((T + tpw - 1) / tpw) * (size_t)E * sizeof(int32_t);
    return (b + 255) / 256 * 256;
}

hipError_t launch_permute_from_hist(const uint16_t* x, const int32_t* topk_idx, int64_t T, int H, int E, int k,
                                   int align, int64_t P_max, int32_t* counts, int32_t* offsets,
                                   int32_t* route_row, int32_t* row_token, uint16_t* x_perm, void* workspace,
                                   hipStream_t stream) {
    const int64_t R = T * k;
    const int tpw = route_hist_tokens_per_chunk(T, E);
    const int64_t nchunks = T > 0 ? (T + tpw - 1) / tpw : 0;
    int32_t* hist = (int32_t*)workspace;
    hipLaunchKernelGGL(permute_scan_kernel, dim3((unsigned)((E + kWave - 1) / kWave)), dim3(kScanThreads), 0,
                       stream, hist, nchunks, E, counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t scatter_blocks = nchunks > 0 ? (nchunks + 3) / 4 : 1;
    const size_t scatter_lds = (4 * (size_t)E + E + 1 + 4) * sizeof(int32_t);
    // tpw * k <= 32 * 32 routes per chunk: 16 steps of 64
    hipLaunchKernelGGL(permute_scatter_kernel<16>, dim3((unsigned)scatter_blocks), dim3(kScatterThreads),
                       scatter_lds, stream, topk_idx, R, E, k, align, nchunks, P_max, (const int32_t*)hist,
                       (const int32_t*)counts, offsets, route_row, row_token, tpw * k);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_permute_copy(x, T, H, E, k, P_max, counts, offsets, route_row, row_token, x_perm, false,
                               stream);
}

hipError_t launch_permute_copy(const uint16_t* x, int64_t T, int H, int E, int k, int64_t P_max,
                               const int32_t* counts, const int32_t* offsets, const int32_t* route_row,
                               const int32_t* row_token, uint16_t* x_perm, bool tiled, hipStream_t stream) {
    if (!x_perm) return hipGetLastError();  // the layout only
    const int ppr = H / 8;  // 16-byte pieces per row
    // one wavefront per token, then one workgroup per expert for its pad rows
    const int64_t token_blocks = (T + kCopyWaves - 1) / kCopyWaves;
    const dim3 grid((unsigned)(token_blocks + E));
    const bool nt = P_max * (int64_t)H * 2 > kStreamingLayoutBytes;
    if (tiled) {
        // token-major, whole pairs (P_max is even); then the pad-pair workgroups
        auto go_pairs = [&](auto kern) {
            hipLaunchKernelGGL(kern, grid, dim3(kCopyThreads), 0, stream, (const uint4*)x, route_row, row_token,
                               counts, offsets, T, k, ppr, token_blocks, (uint4*)x_perm);
        };
        if (nt) go_pairs(permute_copy_token_pairs_kernel<true>);
        else go_pairs(permute_copy_token_pairs_kernel<false>);
        return hipGetLastError();
    }
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(kCopyThreads), 0, stream, (const uint4*)x, (const int32_t*)route_row,
                           (const int32_t*)counts, (const int32_t*)offsets, T, k, ppr, token_blocks,
                           (uint4*)x_perm);
    };
    if (nt) go(permute_copy_rows_kernel<true>);
    else go(permute_copy_rows_kernel<false>);
    return hipGetLastError();
}

// ---- the allocation-free permute ------------------------------------------------------
//
// For callers that cannot allocate (code under graph capture, serving loops): the
// per-chunk histogram lives in a file-scope device array instead of a caller
// workspace. Each device that runs this holds its own copy, for the life of the
// process. Host code never uses the array's name as an address: its device
// address is looked up once per device (with that device current) and kept.
// The histogram is fully rewritten by every call before it is read, so nothing
// needs clearing; calls that overlap on one device share the array and race.
constexpr size_t kScratchBytes = 4u << 20;  // 4 MiB: nchunks * E int32 counters
static __device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

size_t permute_scratch_bytes() { return kScratchBytes; }

hipError_t launch_permute_noalloc(const uint16_t* x, const int32_t* topk_idx, int64_t T, int H, int E, int k,
                                  int align, int64_t P_max, int32_t* counts, int32_t* offsets,
                                  int32_t* route_row, int32_t* row_token, uint16_t* x_perm, hipStream_t stream) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            err = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
            if (err != hipSuccess) {
                g_scratch_ptr[dev] = nullptr;
                return err;
            }
        }
        ptr = g_scratch_ptr[dev];
    }
    return launch_permute(x, topk_idx, T, H, E, k, align, P_max, counts, offsets, route_row, row_token, x_perm,
                          ptr, false, stream);
}

}  // namespace moe
