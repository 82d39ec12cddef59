// topk_core.hpp -- the per-token top-k of the routing step, shared by the routing
// kernel (logits from global memory) and the fused router (logits from LDS).
//
// Per token: the k experts with the largest logits, larger first, an exact tie
// going to the lower expert id; weights = softmax over the k selected logits in
// fp32 [PocketLLM "Qwen4-Exp Heterogeneous TP4 Performance", Runtime
// architecture: top-10 of 512 routed experts; prime-rl PR 3885, Changes: the
// top-k scores weight the gather-sum].
//
// A token's logits are split over a group of L = 8 lanes (16 for wide rows):
// lane s reads experts 4s..4s+3, then 4L further on, ..., so each load
// instruction reads 16L consecutive bytes of the row. Every lane keeps the best
// KL (>= k) of its own logits as a list sorted best first. Then k rounds pick the
// best head of the L lists with DPP exchanges (partners lane^1, lane^2, the
// mirrored half-row, the mirrored row), and the owner of the winner drops its
// head. The comparison is on the fp32 logits themselves (never on exp'd values,
// which can merge distinct logits), with float == so that -0 and +0 tie. Logits
// must be finite.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kNoExpert = 0x7fffffff;  // empty list slot (value -inf)

// Bitwise, not short-circuit: the lanes' comparisons combine as masks instead of
// as branches around each list slot.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    return (va > vb) | ((va == vb) & (ia < ib));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// Keep (v, e) in the sorted list if it ranks among the best KL: every slot takes
// its own entry, its predecessor's, or the new one (no branches, no dynamic
// register indexing).
template <int KL>
__device__ __forceinline__ void insert_sorted(float (&lv)[KL], int (&li)[KL], float v, int e) {
    bool before_prev = ranks_before(v, e, lv[0], li[0]);
    float pv = lv[0];
    int pi = li[0];
    lv[0] = before_prev ? v : pv;
    li[0] = before_prev ? e : pi;
#pragma unroll
    for (int j = 1; j < KL; ++j) {
        const bool before = ranks_before(v, e, lv[j], li[j]);
        const float cv = lv[j];
        const int ci = li[j];
        lv[j] = before ? (before_prev ? pv : v) : cv;
        li[j] = before ? (before_prev ? pi : e) : ci;
        before_prev = before;
        pv = cv;
        pi = ci;
    }
}

// (hv, hi) <- the better of itself and its DPP partner's
template <int CTRL>
__device__ __forceinline__ void best_with(float& hv, int& hi) {
    const float ov = dpp_f<CTRL>(hv);
    const int oi = dpp_i<CTRL>(hi);
    const bool take = ranks_before(ov, oi, hv, hi);
    hv = take ? ov : hv;
    hi = take ? oi : hi;
}

// The top-k of one token's row of E logits, computed by the LPT consecutive lanes
// of its group (sub = this lane's index in the group; live = the token exists --
// groups past the last token run the exchanges on empty lists). KL >= k list slots
// per lane; VEC logits per load (4 needs E % 4 == 0 and a 16-byte aligned row).
// Writes idx_out[j], w_out[j] for j < k (only when live), and idx_lds[j] too when
// idx_lds is not NULL (an LDS copy of the ids).
template <int KL, int VEC, int LPT>
__device__ __forceinline__ void topk_token(const float* row, bool live, int E, int k, int sub,
                                           int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                           int32_t* idx_lds = nullptr) {
    constexpr int kLanesPerToken = LPT;
    static_assert(LPT == 8 || LPT == 16, "8 or 16 lanes per token");
    float lv[KL];
    int li[KL];
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        lv[j] = -INFINITY;
        li[j] = kNoExpert;
    }
    if (live) {
        for (int e0 = sub * VEC; e0 < E; e0 += kLanesPerToken * VEC) {
            if (VEC == 4) {
                const float4 q = *(const float4*)(row + e0);
                insert_sorted<KL>(lv, li, q.x, e0);
                insert_sorted<KL>(lv, li, q.y, e0 + 1);
                insert_sorted<KL>(lv, li, q.z, e0 + 2);
                insert_sorted<KL>(lv, li, q.w, e0 + 3);
            } else {
                insert_sorted<KL>(lv, li, row[e0], e0);
            }
        }
    }

    // k rounds: the best head of the group's L lists; its owner drops it. Lane s
    // records picks s, s+L, ... and every lane adds up the softmax terms.
    constexpr int kOwn = (KL + kLanesPerToken - 1) / kLanesPerToken;
    float own_z[kOwn];
    int own_i[kOwn];
    float top = 0.0f, sum = 0.0f;
#pragma unroll
    for (int jj = 0; jj < kOwn; ++jj) {
#pragma unroll
        for (int u = 0; u < kLanesPerToken; ++u) {
            const int j = jj * kLanesPerToken + u;
            if (j >= k) continue;  // k <= KL: the loop unrolls fully
            float hv = lv[0];
            int hi = li[0];
            best_with<0xB1>(hv, hi);   // quad_perm [1,0,3,2]: lane ^ 1
            best_with<0x4E>(hv, hi);   // quad_perm [2,3,0,1]: lane ^ 2
            best_with<0x141>(hv, hi);  // row_half_mirror: the other quad of the 8
            if (LPT == 16) best_with<0x140>(hv, hi);  // row_mirror: the other 8 of the 16
            if (li[0] == hi) {
#pragma unroll
                for (int m = 0; m + 1 < KL; ++m) {
                    lv[m] = lv[m + 1];
                    li[m] = li[m + 1];
                }
                lv[KL - 1] = -INFINITY;
                li[KL - 1] = kNoExpert;
            }
            if (j == 0) top = hv;
            const float z = expf(hv - top);
            sum += z;
            if (sub == u) {
                own_z[jj] = z;
                own_i[jj] = hi;
            }
        }
    }
    if (live) {
#pragma unroll
        for (int jj = 0; jj < kOwn; ++jj) {
            const int j = jj * kLanesPerToken + sub;
            if (j < k) {
                idx_out[j] = own_i[jj];
                w_out[j] = own_z[jj] / sum;
                if (idx_lds) idx_lds[j] = own_i[jj];  // the same ids, for the caller's histogram
            }
        }
    }
}

}  // namespace moe
