// permute_core.hpp -- the pieces of the atomic-free counting sort (see
// permute.hip), shared by the permute kernels and the fused layer kernel. Each
// piece is the work of one wavefront (a chunk of routes) or of one workgroup (a
// group of 64 experts, the padded offsets).
//
// [Halo "Performance", Levers that help: the atomic-free expert permute;
//  prime-rl PR 3885, Changes: one gather into the padded expert-grouped layout]
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kChunk = 256;             // routes per wavefront chunk
constexpr int kSteps = kChunk / kWave;  // all of a chunk's ids are loaded before any is used

__device__ __forceinline__ int key_bits(int E) { return E <= 1 ? 0 : 32 - __clz(E - 1); }

// Chunk c of kChunk routes by one wavefront: hist_row[e] = routes to expert e in
// the chunk. h is this wave's private LDS histogram [E]. Lanes with equal ids
// find each other with ballots (match_peers); the lowest one adds the group's size.
__device__ __forceinline__ void hist_chunk(const int32_t* __restrict__ topk_idx, int64_t R, int E, int64_t c,
                                           int32_t* h, int32_t* __restrict__ hist_row) {
    const int lane = lane_id();
    for (int e = lane; e < E; e += kWave) h[e] = 0;
    const int nbits = key_bits(E);
    const int64_t r0 = c * kChunk;
    uint32_t ids[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int64_t r = r0 + s * kWave + lane;
        ids[s] = r < R ? (uint32_t)topk_idx[r] : 0xffffffffu;
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const bool active = ids[s] < (uint32_t)E;  // out-of-range ids take no part
        const uint32_t key = active ? ids[s] : 0u;
        const uint64_t peers = match_peers(key, nbits, active);
        if (active && (__ffsll((unsigned long long)peers) - 1) == lane) h[key] += __popcll(peers);
    }
    for (int e = lane; e < E; e += kWave) hist_row[e] = h[e];
}

// Experts [64 g, 64 g + 64) by one workgroup of NW waves: lane l of every wave
// owns expert 64 g + l, wave w a contiguous range of chunks. counts[e] = sum_c
// hist[c][e], and hist[c][e] becomes the number of e's routes in chunks before c.
// part: LDS [NW][64]. Every thread of the workgroup calls this (two barriers).
template <int NW>
__device__ __forceinline__ void scan_group(int32_t* __restrict__ hist, int64_t nchunks, int E,
                                           int32_t* __restrict__ counts, int g, int32_t (*part)[kWave]) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int e = g * kWave + lane;
    const bool live = e < E && wave < NW;
    const int64_t per = (nchunks + NW - 1) / NW;
    const int64_t c0 = min(nchunks, (int64_t)wave * per), c1 = min(nchunks, c0 + per);
    int32_t sum = 0;
    if (live) {
#pragma unroll 8
        for (int64_t c = c0; c < c1; ++c) sum += hist[c * E + e];
    }
    if (wave < NW) part[wave][lane] = sum;
    __syncthreads();
    if (wave == 0) {  // per expert: exclusive scan over the waves' ranges, and the total
        int32_t run = 0;
        for (int w = 0; w < NW; ++w) {
            const int32_t v = part[w][lane];
            part[w][lane] = run;
            run += v;
        }
        if (e < E) counts[e] = run;
    }
    __syncthreads();
    if (live) {
        int32_t run = part[wave][lane];
#pragma unroll 8
        for (int64_t c = c0; c < c1; ++c) {
            const int32_t v = hist[c * E + e];
            hist[c * E + e] = run;
            run += v;
        }
    }
}

// The padded offsets from the counts, into LDS off[0 .. E] (E <= 1024): the
// first 256 threads take experts 4i .. 4i+3 each, then a workgroup scan. wtot:
// LDS [4]. Every thread of the workgroup calls this (two barriers).
__device__ __forceinline__ void padded_offsets(const int32_t* __restrict__ counts, int E, int align, int32_t* off,
                                               int32_t* wtot) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const bool mine = tid < 256;
    int32_t pc[4], local = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        pc[q] = mine && e < E ? (counts[e] + align - 1) / align * align : 0;
        local += pc[q];
    }
    int32_t incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (mine && lane == kWave - 1) wtot[wave] = incl;
    __syncthreads();
    if (mine) {
        for (int w = 0; w < wave; ++w) incl += wtot[w];
        int32_t run = incl - local;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * tid + q;
            if (e < E) off[e] = run;
            run += pc[q];
        }
        if (tid == 255) off[E] = incl;
    }
    __syncthreads();
}

// row_token = -1 on the pad rows of experts b, b + nb, ... and on this
// workgroup's share of the rows from off[E] to P_max (b = this workgroup among nb).
__device__ __forceinline__ void pad_row_tokens(const int32_t* __restrict__ counts, const int32_t* off, int E,
                                               int64_t P_max, int64_t b, int64_t nb, int nthreads,
                                               int32_t* __restrict__ row_token) {
    const int tid = threadIdx.x;
    for (int64_t e = b; e < E; e += nb)
        for (int64_t p = (int64_t)off[e] + counts[e] + tid; p < off[e + 1]; p += nthreads) row_token[p] = -1;
    for (int64_t p = (int64_t)off[E] + b * nthreads + tid; p < P_max; p += nb * nthreads) row_token[p] = -1;
}

// Chunk c of chunk_routes routes (at most STEPS * 64) by one wavefront: route_row
// and row_token of its routes, stable in r. base: the chunk's earlier routes per
// expert (from scan_group); off: the padded offsets; cur: this wave's LDS [E].
template <int STEPS>
__device__ __forceinline__ void scatter_chunk(const int32_t* __restrict__ topk_idx, int64_t R, int E, int k,
                                              int64_t c, const int32_t* __restrict__ base, const int32_t* off,
                                              int32_t* cur, int32_t* __restrict__ route_row,
                                              int32_t* __restrict__ row_token, int chunk_routes) {
    const int lane = lane_id();
    for (int e = lane; e < E; e += kWave) cur[e] = base[c * E + e] + off[e];
    const int nbits = key_bits(E);
    const uint64_t lt = lanemask_lt();
    const int64_t r0 = c * chunk_routes;
    const int64_t r_end = r0 + chunk_routes < R ? r0 + chunk_routes : R;
    const int steps = (chunk_routes + kWave - 1) / kWave;
    uint32_t ids[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int64_t r = r0 + s * kWave + lane;
        ids[s] = s < steps && r < r_end ? (uint32_t)topk_idx[r] : 0xffffffffu;
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        if (s < steps) {  // wave-uniform
            const int64_t r = r0 + s * kWave + lane;
            const bool active = ids[s] < (uint32_t)E;
            const uint32_t key = active ? ids[s] : 0u;
            const uint64_t peers = match_peers(key, nbits, active);
            if (active) {
                const int32_t dest = cur[key] + __popcll(peers & lt);
                route_row[r] = dest;
                row_token[dest] = (int32_t)(r / k);
            } else if (r < r_end) {
                route_row[r] = -1;  // an out-of-range id gets no row
            }
            if (active && (__ffsll((unsigned long long)peers) - 1) == lane) cur[key] += __popcll(peers);
        }
    }
}

}  // namespace moe
