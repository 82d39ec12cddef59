/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of the routed-expert
 * forward path of a Mixture-of-Experts layer. Only the test suite, the smoke
 * check and the bench's CPU-baseline leg may load it; the product path never
 * does, and this file shares no code, header or constant with the GPU library.
 *
 * Sources (page title, section):
 *   [Halo]      Halo, "Performance": Levers that help; Levers that do not help here
 *   [PocketLLM] "Qwen4-Exp Heterogeneous TP4 Performance": Runtime architecture;
 *               Decode ceiling
 *   [prime-rl]  prime-rl pull request 3885 (DeepSeek-V4.1 Flash performance work):
 *               Changes; Known numerics
 *
 * What is computed, for T tokens of hidden size H, E experts, top-k routing and
 * expert intermediate size I (all tensors row-major) -- the forward below, and
 * its backward further down:
 *   routing   per token, the k experts with the largest router logits, and their
 *             weights = softmax over those k logits;
 *   layout    a padded, expert-grouped row layout of the routed tokens, built by a
 *             stable counting sort of the flat routes r = t*k + j;
 *   experts   per routed row, h = silu(x W_gate^T) * (x W_up^T) and y = h W_down^T;
 *   combine   per token, the score-weighted sum of its k expert outputs, gathered.
 *
 * Precision: bf16 inputs are widened exactly; all arithmetic is in double and
 * no intermediate is rounded, so these functions give the exact value that the
 * GPU path reaches with bf16 storage and fp32 accumulation. Sums run in plain
 * ascending index order.
 *
 * Every function returns 0 on success and a negative code on invalid
 * arguments (nothing is written then).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EINVAL (-1)
#define ORACLE_ENONFINITE (-2)
#define ORACLE_ERANGE (-3)

/* bf16 -> double: a bf16 value is the top 16 bits of an IEEE binary32. */
static double bf(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* silu(g) = g * sigmoid(g) = g / (1 + exp(-g)).  SwiGLU is silu(gate) * up
 * [prime-rl, Changes: fused FP8 shared expert -- gate and up projections feed
 * a SwiGLU whose output is the down projection's input]. */
static double silu(double g) { return g / (1.0 + exp(-g)); }

/* "a is ranked before b" in the routing order: larger logit first, and on an
 * exact tie (float ==, so -0 == +0) the lower expert id first. */
static int ranks_before(float la, int32_t a, float lb, int32_t b) {
    if (la > lb) return 1;
    if (la < lb) return 0;
    return a < b;
}

/*
 * Top-k routing [PocketLLM, Runtime architecture: 512 routed experts with
 * top-10 routing; prime-rl, Changes: top-k weights feed a score-weighted sum].
 * Per token t: k passes, each picking the best expert not yet picked; then
 * w[t,j] = exp(L_j - L_0) / sum_i exp(L_i - L_0) over the k picks (softmax over
 * the selected logits; L_0 is the largest, so every exponent is <= 0).
 * Logits must be finite.
 */
int moe_oracle_route_topk(const float *logits, int64_t T, int32_t E, int32_t k,
                          int32_t *topk_idx, double *topk_w) {
    if (!logits || !topk_idx || !topk_w || T < 0 || E < 1 || k < 1 || k > E)
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < T * (int64_t)E; ++i)
        if (!isfinite(logits[i])) return ORACLE_ENONFINITE;
    char *taken = (char *)malloc((size_t)E);
    if (!taken) return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        const float *L = logits + t * (int64_t)E;
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(L[e], e, L[best], best)) best = e;
            }
            taken[best] = 1;
            topk_idx[t * k + j] = best;
        }
        double m = (double)L[topk_idx[t * k]];
        double s = 0.0;
        for (int32_t j = 0; j < k; ++j) s += exp((double)L[topk_idx[t * k + j]] - m);
        for (int32_t j = 0; j < k; ++j)
            topk_w[t * k + j] = exp((double)L[topk_idx[t * k + j]] - m) / s;
    }
    free(taken);
    return 0;
}

/*
 * Router projection [PocketLLM, Remaining prefill attribution: the router is a
 * phase of its own]: logits[t,e] = sum_h x[t,h] W_r[h,e], x bf16 [T, H] widened
 * exactly, W_r fp32 [H, E], summed in double in ascending h.
 */
int moe_oracle_router_logits(const uint16_t *x, const float *w_r, int64_t T, int32_t H, int32_t E,
                             double *logits) {
    if (!x || !w_r || !logits || T < 0 || H < 1 || E < 1) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int32_t h = 0; h < H; ++h) s += bf(x[t * H + h]) * (double)w_r[(int64_t)h * E + e];
            logits[t * E + e] = s;
        }
    return 0;
}

/*
 * Padded expert-grouped layout [prime-rl, Changes: single-pass local layout --
 * one gather into the padded expert-grouped layout; Halo, Levers that help:
 * the atomic-free expert permute].
 *   counts[e]      number of routes r with topk_idx[r] == e
 *   offsets[0]     0
 *   offsets[e+1]   offsets[e] + counts[e] rounded up to a multiple of align
 *   route_row[r]   the row of route r: routes of expert e fill rows
 *                  offsets[e], offsets[e]+1, ... in ascending r (a stable sort)
 *   row_token[p]   r / k for the row p = route_row[r]; -1 on every other row
 *                  in [0, P_max)
 * Requires every topk_idx in [0, E) and offsets[E] <= P_max < 2^31.
 */
int moe_oracle_layout(const int32_t *topk_idx, int64_t T, int32_t k, int32_t E,
                      int32_t align, int64_t P_max, int32_t *counts, int32_t *offsets,
                      int32_t *route_row, int32_t *row_token) {
    if (!topk_idx || !counts || !offsets || !route_row || !row_token || T < 0 ||
        k < 1 || E < 1 || align < 1 || P_max < 0 || P_max >= ((int64_t)1 << 31))
        return ORACLE_EINVAL;
    const int64_t R = T * (int64_t)k;
    for (int64_t r = 0; r < R; ++r)
        if (topk_idx[r] < 0 || topk_idx[r] >= E) return ORACLE_ERANGE;
    int64_t *cnt = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int64_t *off = (int64_t *)calloc((size_t)E + 1, sizeof(int64_t));
    if (!cnt || !off) { free(cnt); free(off); return ORACLE_EINVAL; }
    for (int64_t r = 0; r < R; ++r) cnt[topk_idx[r]] += 1;
    off[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        off[e + 1] = off[e] + (cnt[e] + align - 1) / align * align;
    if (off[E] > P_max) { free(cnt); free(off); return ORACLE_ERANGE; }
    for (int32_t e = 0; e < E; ++e) counts[e] = (int32_t)cnt[e];
    for (int32_t e = 0; e <= E; ++e) offsets[e] = (int32_t)off[e];
    for (int64_t p = 0; p < P_max; ++p) row_token[p] = -1;
    /* cursor[e] walks expert e's rows; visiting r in ascending order makes the
     * placement stable. */
    int64_t *cursor = off; /* reuse: off is no longer needed as such */
    for (int64_t r = 0; r < R; ++r) {
        int32_t e = topk_idx[r];
        int64_t p = cursor[e]++;
        route_row[r] = (int32_t)p;
        row_token[p] = (int32_t)(r / k);
    }
    free(cnt);
    free(off);
    return 0;
}

/* Gather of token rows into the layout: x_perm[p] = x[row_token[p]] bit for
 * bit, and a zero row where row_token[p] == -1.  rows = how many rows to fill. */
int moe_oracle_gather(const uint16_t *x, const int32_t *row_token, int64_t T, int64_t rows,
                      int32_t H, uint16_t *x_perm) {
    if (!x || !row_token || !x_perm || rows < 0 || H < 1) return ORACLE_EINVAL;
    for (int64_t p = 0; p < rows; ++p) {
        int32_t t = row_token[p];
        if (t >= T) return ORACLE_ERANGE;
        for (int32_t c = 0; c < H; ++c)
            x_perm[p * H + c] = (t >= 0) ? x[(int64_t)t * H + c] : (uint16_t)0;
    }
    return 0;
}

/*
 * Gate/up projections and SwiGLU for every routed row of every expert
 * [Halo, Levers that help: one grouped matmul over all experts computes what a
 * per-expert loop computes -- this is that loop].  W_gu[e] is [2I, H]: rows
 * [0, I) are the gate projection and rows [I, 2I) the up projection.
 *   g = sum_c x_perm[p,c] W_gu[e,i,c];  u = sum_c x_perm[p,c] W_gu[e,I+i,c]
 *   h[p,i] = silu(g) * u
 * Only rows offsets[e] .. offsets[e]+counts[e]-1 are written.
 */
int moe_oracle_glu(const uint16_t *x_perm, const uint16_t *w_gu, const int32_t *counts,
                   const int32_t *offsets, int32_t E, int32_t H, int32_t I, double *h) {
    if (!x_perm || !w_gu || !counts || !offsets || !h || E < 1 || H < 1 || I < 1)
        return ORACLE_EINVAL;
    for (int32_t e = 0; e < E; ++e) {
        const uint16_t *W = w_gu + (int64_t)e * 2 * I * H;
        int64_t p0 = offsets[e], n = counts[e];
#pragma omp parallel for schedule(static)
        for (int64_t p = p0; p < p0 + n; ++p) {
            const uint16_t *xr = x_perm + p * H;
            for (int32_t i = 0; i < I; ++i) {
                const uint16_t *wg = W + (int64_t)i * H;
                const uint16_t *wu = W + (int64_t)(I + i) * H;
                double g = 0.0, u = 0.0;
                for (int32_t c = 0; c < H; ++c) {
                    g += bf(xr[c]) * bf(wg[c]);
                    u += bf(xr[c]) * bf(wu[c]);
                }
                h[p * I + i] = silu(g) * u;
            }
        }
    }
    return 0;
}

/*
 * Down projection for every routed row: y[p,c] = sum_i h[p,i] W_d[e,c,i], with
 * W_d[e] = [H, I].  h is taken as double so that the oracle's own chain never
 * rounds; a bf16 input is widened by the caller.
 */
int moe_oracle_down(const double *h, const uint16_t *w_d, const int32_t *counts,
                    const int32_t *offsets, int32_t E, int32_t H, int32_t I, double *y) {
    if (!h || !w_d || !counts || !offsets || !y || E < 1 || H < 1 || I < 1)
        return ORACLE_EINVAL;
    for (int32_t e = 0; e < E; ++e) {
        const uint16_t *W = w_d + (int64_t)e * H * I;
        int64_t p0 = offsets[e], n = counts[e];
#pragma omp parallel for schedule(static)
        for (int64_t p = p0; p < p0 + n; ++p) {
            const double *hr = h + p * I;
            for (int32_t c = 0; c < H; ++c) {
                const uint16_t *wr = W + (int64_t)c * I;
                double s = 0.0;
                for (int32_t i = 0; i < I; ++i) s += hr[i] * bf(wr[i]);
                y[p * H + c] = s;
            }
        }
    }
    return 0;
}

/*
 * Score-weighted gather-sum back to token order [prime-rl, Changes: one
 * score-weighted gather-sum back]: out[t,c] = sum_{j<k} w[t,j] y[route_row[t*k+j], c],
 * summed over j ascending.  A gather per token, not a scatter-add.
 */
int moe_oracle_combine(const double *y, const int32_t *route_row, const double *topk_w,
                       int64_t T, int32_t H, int32_t k, int64_t P_max, double *out) {
    if (!y || !route_row || !topk_w || !out || T < 0 || H < 1 || k < 1) return ORACLE_EINVAL;
    for (int64_t r = 0; r < T * (int64_t)k; ++r)
        if (route_row[r] < 0 || route_row[r] >= P_max) return ORACLE_ERANGE;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t c = 0; c < H; ++c) {
            double s = 0.0;
            for (int32_t j = 0; j < k; ++j)
                s += topk_w[t * k + j] * y[(int64_t)route_row[t * k + j] * H + c];
            out[t * H + c] = s;
        }
    }
    return 0;
}

/*
 * The whole layer as a plain per-token loop (the definition the grouped path
 * reorganises): for each token, route it, run each of its k experts on it and
 * add the expert output scaled by its routing weight.  No layout is built.
 * tokens: the token ids to evaluate (NULL = all T, in order); out is
 * [n_tokens, H] in the order of `tokens`.
 */
int moe_oracle_forward(const uint16_t *x, const float *logits, const uint16_t *w_gu,
                       const uint16_t *w_d, int64_t T, int32_t H, int32_t E, int32_t k,
                       int32_t I, const int64_t *tokens, int64_t n_tokens, double *out) {
    if (!x || !logits || !w_gu || !w_d || !out || T < 0 || H < 1 || E < 1 || k < 1 ||
        k > E || I < 1)
        return ORACLE_EINVAL;
    if (!tokens) n_tokens = T;
    for (int64_t n = 0; n < n_tokens; ++n) {
        int64_t t = tokens ? tokens[n] : n;
        if (t < 0 || t >= T) return ORACLE_ERANGE;
        for (int32_t e = 0; e < E; ++e)
            if (!isfinite(logits[t * E + e])) return ORACLE_ENONFINITE;
    }
    int err = 0;
#pragma omp parallel
    {
        int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        double *w = (double *)malloc(sizeof(double) * (size_t)k);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        if (!idx || !w || !a) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t n = 0; n < n_tokens; ++n) {
                int64_t t = tokens ? tokens[n] : n;
                const uint16_t *xr = x + t * H;
                moe_oracle_route_topk(logits + t * E, 1, E, k, idx, w);
                double *acc = out + n * H;
                for (int32_t c = 0; c < H; ++c) acc[c] = 0.0;
                for (int32_t j = 0; j < k; ++j) {
                    const uint16_t *Wgu = w_gu + (int64_t)idx[j] * 2 * I * H;
                    const uint16_t *Wd = w_d + (int64_t)idx[j] * H * I;
                    for (int32_t i = 0; i < I; ++i) {
                        double g = 0.0, u = 0.0;
                        for (int32_t c = 0; c < H; ++c) {
                            g += bf(xr[c]) * bf(Wgu[(int64_t)i * H + c]);
                            u += bf(xr[c]) * bf(Wgu[(int64_t)(I + i) * H + c]);
                        }
                        a[i] = silu(g) * u;
                    }
                    for (int32_t c = 0; c < H; ++c) {
                        double y = 0.0;
                        for (int32_t i = 0; i < I; ++i) y += a[i] * bf(Wd[(int64_t)c * I + i]);
                        acc[c] += w[j] * y;
                    }
                }
            }
        }
        free(idx);
        free(w);
        free(a);
    }
    return err ? ORACLE_EINVAL : 0;
}

/*
 * FP8 expert weights [Halo, "Performance", Levers that do not help here: lower
 * precision shrinks expert-weight bytes (fp8: by half) rather than matmul time;
 * prime-rl, Changes: FP8 expert weights quantized once per optimizer step,
 * blockwise FP8 grouped GEMMs].
 *
 * Format: OCP 8-bit float E4M3 ("E4M3FN"): sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; the
 * all-ones code S.1111.111 is NaN and there is no infinity, so the largest
 * finite magnitude is 1.75 * 2^8 = 448.
 */
static double e4m3_value(uint8_t c) {
    const int e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);
    return (c & 0x80) ? -v : v;
}

/* round to nearest, ties to even, of a non-negative double holding an integer + fraction */
static double rne(double q) {
    double f = floor(q);
    double d = q - f;
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

/* Nearest E4M3 code to v, ties to the even code; |v| must not exceed 448. */
static int e4m3_encode(float v, uint8_t *out) {
    if (!isfinite(v) || fabsf(v) > 448.0f) return ORACLE_ERANGE;
    const uint8_t sign = signbit(v) ? 0x80 : 0;
    const double a = fabs((double)v);
    if (a < ldexp(1.0, -6)) {               /* subnormal range: step 2^-9 */
        const double n = rne(a * 512.0);    /* 0..8; 8 is the smallest normal, code 8 */
        *out = sign | (uint8_t)n;
        return 0;
    }
    int e;
    (void)frexp(a, &e);
    e -= 1;                                 /* a = 1.f * 2^e */
    double n = rne(ldexp(a, 3 - e));        /* 8 <= n <= 16 */
    if (n >= 16.0) { n = 8.0; e += 1; }
    *out = sign | (uint8_t)(((e + 7) << 3) | ((int)n - 8));
    return 0;
}

int moe_oracle_fp8_encode(const float *v, int64_t n, uint8_t *out) {
    if (!v || !out || n < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        if (e4m3_encode(v[i], &out[i]) != 0) return ORACLE_ERANGE;
    return 0;
}

int moe_oracle_fp8_decode(const uint8_t *c, int64_t n, double *out) {
    if (!c || !out || n < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(c[i]);
    return 0;
}

/*
 * Block-scaled quantization of expert weights w [E, R, K] (bf16), one scale per
 * block of 64 consecutive rows (output channels) over all K:
 *   scale[e, b] = max |w[e, 64b .. 64b+63, :]| / 448      (fp32 division; 1 if
 *                 the block is all zero)
 *   w8[e, r, c] = E4M3 nearest-even of clamp(w[e, r, c] / scale[e, r / 64], +-448)
 *                 (fp32 division; the clamp only catches a quotient one rounding
 *                 past 448, which rounds to 448 anyway)
 * and dequantizes to scale * e4m3_value(w8).
 */
int moe_oracle_quantize_fp8(const uint16_t *w, int64_t E, int32_t R, int32_t K, uint8_t *w8,
                            float *scale) {
    if (!w || !w8 || !scale || E < 1 || R < 64 || R % 64 != 0 || K < 1) return ORACLE_EINVAL;
    const int32_t nb = R / 64;
    for (int64_t e = 0; e < E; ++e) {
        for (int32_t b = 0; b < nb; ++b) {
            const int64_t base = (e * R + (int64_t)b * 64) * K;
            float amax = 0.0f;
            for (int64_t i = 0; i < (int64_t)64 * K; ++i) {
                const float a = fabsf((float)bf(w[base + i]));
                if (a > amax) amax = a;
            }
            const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            scale[e * nb + b] = s;
            for (int64_t i = 0; i < (int64_t)64 * K; ++i) {
                float q = (float)bf(w[base + i]) / s;
                if (q > 448.0f) q = 448.0f;   /* amax / fl(amax / 448) can land an ulp past 448 */
                if (q < -448.0f) q = -448.0f;
                if (e4m3_encode(q, &w8[base + i]) != 0) return ORACLE_ERANGE;
            }
        }
    }
    return 0;
}

/* The dequantized weights in double: scale[e, r / 64] * e4m3_value(w8[e, r, c]). */
int moe_oracle_dequantize_fp8(const uint8_t *w8, const float *scale, int64_t E, int32_t R,
                              int32_t K, double *w) {
    if (!w8 || !scale || !w || E < 1 || R < 64 || R % 64 != 0 || K < 1) return ORACLE_EINVAL;
    const int32_t nb = R / 64;
    for (int64_t e = 0; e < E; ++e)
        for (int32_t r = 0; r < R; ++r) {
            const double s = (double)scale[e * nb + r / 64];
            const int64_t base = (e * R + r) * (int64_t)K;
            for (int32_t c = 0; c < K; ++c) w[base + c] = s * e4m3_value(w8[base + c]);
        }
    return 0;
}

/* moe_oracle_glu with weights given in double (dequantized FP8 weights). */
int moe_oracle_glu_w64(const uint16_t *x_perm, const double *w_gu, const int32_t *counts,
                       const int32_t *offsets, int32_t E, int32_t H, int32_t I, double *h) {
    if (!x_perm || !w_gu || !counts || !offsets || !h || E < 1 || H < 1 || I < 1)
        return ORACLE_EINVAL;
    for (int32_t e = 0; e < E; ++e) {
        const double *W = w_gu + (int64_t)e * 2 * I * H;
        int64_t p0 = offsets[e], n = counts[e];
#pragma omp parallel for schedule(static)
        for (int64_t p = p0; p < p0 + n; ++p) {
            const uint16_t *xr = x_perm + p * H;
            for (int32_t i = 0; i < I; ++i) {
                const double *wg = W + (int64_t)i * H;
                const double *wu = W + (int64_t)(I + i) * H;
                double g = 0.0, u = 0.0;
                for (int32_t c = 0; c < H; ++c) {
                    g += bf(xr[c]) * wg[c];
                    u += bf(xr[c]) * wu[c];
                }
                h[p * I + i] = silu(g) * u;
            }
        }
    }
    return 0;
}

/* moe_oracle_down with weights given in double (dequantized FP8 weights). */
int moe_oracle_down_w64(const double *h, const double *w_d, const int32_t *counts,
                        const int32_t *offsets, int32_t E, int32_t H, int32_t I, double *y) {
    if (!h || !w_d || !counts || !offsets || !y || E < 1 || H < 1 || I < 1)
        return ORACLE_EINVAL;
    for (int32_t e = 0; e < E; ++e) {
        const double *W = w_d + (int64_t)e * H * I;
        int64_t p0 = offsets[e], n = counts[e];
#pragma omp parallel for schedule(static)
        for (int64_t p = p0; p < p0 + n; ++p) {
            const double *hr = h + p * I;
            for (int32_t c = 0; c < H; ++c) {
                const double *wr = W + (int64_t)c * I;
                double s = 0.0;
                for (int32_t i = 0; i < I; ++i) s += hr[i] * wr[i];
                y[p * H + c] = s;
            }
        }
    }
    return 0;
}

/*
 * ---------------------------------------------------------------------------
 * Backward of the path [prime-rl PR 3885, Changes: the single-pass layout gathers
 * in backward too; grouped GEMMs for the forward, dgrad and wgrad; weight
 * gradients accumulated in fp32; the forward keeps its gate/up output so that
 * the backward does not recompute it].  For a loss with gradient dout [T, H]
 * with respect to the layer output (chain rule through each forward step):
 *   combine   dw[t,j] = <dout[t], y[route_row[t*k+j]]>
 *             dy[route_row[t*k+j]] = w[t,j] dout[t]      (every other row 0)
 *   routing   softmax over the k selected logits:
 *             dlogits[t, idx[t,j]] = w[t,j] (dw[t,j] - sum_i w[t,i] dw[t,i]);
 *             0 for the experts not selected (the selection is piecewise constant)
 *   down      dh[p] = dy[p] W_d[e]            dW_d[e] = sum_p dy[p]^T h[p]
 *   SwiGLU    h = silu(g) u:  dg = dh u silu'(g),  du = dh silu(g),
 *             silu'(g) = s (1 + g (1 - s)) with s = sigmoid(g)
 *   gate/up   dx_perm[p] = dg[p] W_gate[e] + du[p] W_up[e]
 *             dW_gu[e] = sum_p [dg[p], du[p]]^T x_perm[p]
 *   permute   dx[t] = sum_j dx_perm[route_row[t*k+j]]   (a gather per token)
 * Sums over rows p run over an expert's routed rows in ascending order, which
 * is ascending token order (the layout is stable), so the step functions and
 * the per-token loop add the same terms in the same order.
 * ---------------------------------------------------------------------------
 */

int moe_oracle_combine_bwd(const double *dout, const double *y, const int32_t *route_row,
                           const double *topk_w, int64_t T, int32_t H, int32_t k, int64_t P_max,
                           double *dy, double *dw) {
    if (!dout || !y || !route_row || !topk_w || !dy || !dw || T < 0 || H < 1 || k < 1 || P_max < 0)
        return ORACLE_EINVAL;
    for (int64_t r = 0; r < T * (int64_t)k; ++r)
        if (route_row[r] < 0 || route_row[r] >= P_max) return ORACLE_ERANGE;
    for (int64_t i = 0; i < P_max * (int64_t)H; ++i) dy[i] = 0.0;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double *g = dout + t * H;
        for (int32_t j = 0; j < k; ++j) {
            const int64_t p = route_row[t * k + j];
            const double w = topk_w[t * k + j];
            double s = 0.0;
            for (int32_t c = 0; c < H; ++c) {
                s += g[c] * y[p * H + c];
                dy[p * H + c] = w * g[c];
            }
            dw[t * k + j] = s;
        }
    }
    return 0;
}

int moe_oracle_route_bwd(const int32_t *topk_idx, const double *topk_w, const double *dw, int64_t T,
                         int32_t E, int32_t k, double *dlogits) {
    if (!topk_idx || !topk_w || !dw || !dlogits || T < 0 || E < 1 || k < 1 || k > E)
        return ORACLE_EINVAL;
    for (int64_t r = 0; r < T * (int64_t)k; ++r)
        if (topk_idx[r] < 0 || topk_idx[r] >= E) return ORACLE_ERANGE;
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int32_t j = 0; j < k; ++j) s += topk_w[t * k + j] * dw[t * k + j];
        for (int32_t e = 0; e < E; ++e) dlogits[t * E + e] = 0.0;
        for (int32_t j = 0; j < k; ++j)
            dlogits[t * E + topk_idx[t * k + j]] = topk_w[t * k + j] * (dw[t * k + j] - s);
    }
    return 0;
}

/* derivative of silu: d/dg [g sigmoid(g)] = s + g s (1 - s) */
static double silu_grad(double g) {
    const double s = 1.0 / (1.0 + exp(-g));
    return s * (1.0 + g * (1.0 - s));
}

/* SwiGLU forward and backward on rows of gu = [g | u] ([rows, 2I]):
 *   h[p,i] = silu(g) u;   dgu[p,i] = dh u silu'(g),  dgu[p,I+i] = dh silu(g). */
int moe_oracle_swiglu(const double *gu, int64_t rows, int32_t I, double *h) {
    if (!gu || !h || rows < 0 || I < 1) return ORACLE_EINVAL;
    for (int64_t p = 0; p < rows; ++p)
        for (int32_t i = 0; i < I; ++i)
            h[p * I + i] = silu(gu[p * 2 * I + i]) * gu[p * 2 * I + I + i];
    return 0;
}

/* Clamped SwiGLU on rows of gu = [g | u] [prime-rl PR 3885, Changes: the
 * DeepSeek-V4.1 recipes run a clamped SwiGLU]. The page names the clamp but not
 * its form or constant; read here as a cap of the gate pre-activation at +limit
 * and a clip of the up projection to [-limit, +limit] ahead of the plain SwiGLU:
 *   h[p,i] = silu(min(g, limit)) * min(max(u, -limit), limit),   limit >= 0.
 * limit = +inf is the plain SwiGLU. */
int moe_oracle_swiglu_clamped(const double *gu, int64_t rows, int32_t I, double limit, double *h) {
    if (!gu || !h || rows < 0 || I < 1 || !(limit >= 0.0)) return ORACLE_EINVAL;
    for (int64_t p = 0; p < rows; ++p)
        for (int32_t i = 0; i < I; ++i) {
            double g = gu[p * 2 * I + i], u = gu[p * 2 * I + I + i];
            if (g > limit) g = limit;
            if (u > limit) u = limit;
            if (u < -limit) u = -limit;
            h[p * I + i] = silu(g) * u;
        }
    return 0;
}

int moe_oracle_swiglu_bwd(const double *dh, const double *gu, int64_t rows, int32_t I, double *dgu) {
    if (!dh || !gu || !dgu || rows < 0 || I < 1) return ORACLE_EINVAL;
    for (int64_t p = 0; p < rows; ++p)
        for (int32_t i = 0; i < I; ++i) {
            const double g = gu[p * 2 * I + i], u = gu[p * 2 * I + I + i], d = dh[p * I + i];
            dgu[p * 2 * I + i] = d * u * silu_grad(g);
            dgu[p * 2 * I + I + i] = d * silu(g);
        }
    return 0;
}

/* Grouped GEMM with the weight as stored (dgrad): C[p,n] = sum_k A[p,k] W[e,k,n],
 * W [E, K, N], on each expert's routed rows.  dh = dy W_d uses W_d [E, H, I];
 * dx_perm = dgu W_gu uses W_gu [E, 2I, H]. */
int moe_oracle_gemm_nn(const double *A, const uint16_t *W, const int32_t *counts,
                       const int32_t *offsets, int32_t E, int32_t K, int32_t N, double *C) {
    if (!A || !W || !counts || !offsets || !C || E < 1 || K < 1 || N < 1) return ORACLE_EINVAL;
    for (int32_t e = 0; e < E; ++e) {
        const uint16_t *We = W + (int64_t)e * K * N;
        const int64_t p0 = offsets[e], n = counts[e];
#pragma omp parallel for schedule(static)
        for (int64_t p = p0; p < p0 + n; ++p)
            for (int32_t c = 0; c < N; ++c) {
                double s = 0.0;
                for (int32_t kk = 0; kk < K; ++kk) s += A[p * K + kk] * bf(We[(int64_t)kk * N + c]);
                C[p * N + c] = s;
            }
    }
    return 0;
}

/* Weight gradient, K-grouped over each expert's rows:
 *   dW[e,m,n] = sum over routed rows p of e (ascending) of A[p,m] B[p,n]
 * A [rows, M], B [rows, N], dW [E, M, N]; an expert with no rows gets zeros. */
int moe_oracle_wgrad(const double *A, const double *B, const int32_t *counts,
                     const int32_t *offsets, int32_t E, int32_t M, int32_t N, double *dW) {
    if (!A || !B || !counts || !offsets || !dW || E < 1 || M < 1 || N < 1) return ORACLE_EINVAL;
    for (int32_t e = 0; e < E; ++e) {
        double *D = dW + (int64_t)e * M * N;
        const int64_t p0 = offsets[e], n = counts[e];
#pragma omp parallel for schedule(static)
        for (int32_t m = 0; m < M; ++m)
            for (int32_t c = 0; c < N; ++c) {
                double s = 0.0;
                for (int64_t p = p0; p < p0 + n; ++p) s += A[p * M + m] * B[p * N + c];
                D[(int64_t)m * N + c] = s;
            }
    }
    return 0;
}

/* The permute's backward: dx[t,c] = sum_j dx_perm[route_row[t*k+j], c], j ascending. */
int moe_oracle_permute_bwd(const double *dx_perm, const int32_t *route_row, int64_t T, int32_t H,
                           int32_t k, int64_t P_max, double *dx) {
    if (!dx_perm || !route_row || !dx || T < 0 || H < 1 || k < 1) return ORACLE_EINVAL;
    for (int64_t r = 0; r < T * (int64_t)k; ++r)
        if (route_row[r] < 0 || route_row[r] >= P_max) return ORACLE_ERANGE;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int32_t c = 0; c < H; ++c) {
            double s = 0.0;
            for (int32_t j = 0; j < k; ++j) s += dx_perm[(int64_t)route_row[t * k + j] * H + c];
            dx[t * H + c] = s;
        }
    return 0;
}

/*
 * The whole backward as a per-token loop (no layout): route the token, recompute
 * each of its k experts (g, u, h, y), then apply the chain rule above; weight
 * gradients accumulate over tokens in ascending order.  dout [T, H] in double;
 * outputs dx [T, H], dlogits [T, E], dw_gu [E, 2I, H], dw_d [E, H, I].
 *
 * A token's input gradients (dx, dlogits) depend on no other token.  When both
 * weight-gradient outputs are NULL only those are computed, and the tokens run in
 * parallel; each token's arithmetic is the same either way.
 */
typedef struct {
    int32_t *idx;
    double *w, *dwt, *g, *u, *a, *dh;
} BwdScratch;

static int bwd_scratch_alloc(BwdScratch *sc, int32_t k, int32_t I) {
    sc->idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    sc->w = (double *)malloc(sizeof(double) * (size_t)k);
    sc->dwt = (double *)malloc(sizeof(double) * (size_t)k);
    sc->g = (double *)malloc(sizeof(double) * (size_t)I * k);
    sc->u = (double *)malloc(sizeof(double) * (size_t)I * k);
    sc->a = (double *)malloc(sizeof(double) * (size_t)I * k);
    sc->dh = (double *)malloc(sizeof(double) * (size_t)I);
    return sc->idx && sc->w && sc->dwt && sc->g && sc->u && sc->a && sc->dh;
}

static void bwd_scratch_free(BwdScratch *sc) {
    free(sc->idx); free(sc->w); free(sc->dwt); free(sc->g); free(sc->u); free(sc->a); free(sc->dh);
}

/* Token t's dx and dlogits rows; adds its share to dw_gu, dw_d unless they are NULL. */
static void backward_token(int64_t t, const uint16_t *x, const float *logits, const uint16_t *w_gu,
                           const uint16_t *w_d, const double *dout, int32_t H, int32_t E, int32_t k,
                           int32_t I, double *dx, double *dlogits, double *dw_gu, double *dw_d,
                           const BwdScratch *sc) {
    int32_t *idx = sc->idx;
    double *w = sc->w, *dwt = sc->dwt, *g = sc->g, *u = sc->u, *a = sc->a, *dh = sc->dh;
    const uint16_t *xr = x + t * H;
    const double *gr = dout + t * H;
    moe_oracle_route_topk(logits + t * E, 1, E, k, idx, w);
    /* forward of each route, and dw */
    for (int32_t j = 0; j < k; ++j) {
        const uint16_t *Wgu = w_gu + (int64_t)idx[j] * 2 * I * H;
        const uint16_t *Wd = w_d + (int64_t)idx[j] * H * I;
        for (int32_t i = 0; i < I; ++i) {
            double gg = 0.0, uu = 0.0;
            for (int32_t c = 0; c < H; ++c) {
                gg += bf(xr[c]) * bf(Wgu[(int64_t)i * H + c]);
                uu += bf(xr[c]) * bf(Wgu[(int64_t)(I + i) * H + c]);
            }
            g[j * I + i] = gg;
            u[j * I + i] = uu;
            a[j * I + i] = silu(gg) * uu;
        }
        double s = 0.0;
        for (int32_t c = 0; c < H; ++c) {
            double yc = 0.0;
            for (int32_t i = 0; i < I; ++i) yc += a[j * I + i] * bf(Wd[(int64_t)c * I + i]);
            s += gr[c] * yc;
        }
        dwt[j] = s;
    }
    double sw = 0.0;
    for (int32_t j = 0; j < k; ++j) sw += w[j] * dwt[j];
    for (int32_t e = 0; e < E; ++e) dlogits[t * E + e] = 0.0;
    for (int32_t j = 0; j < k; ++j) dlogits[t * E + idx[j]] = w[j] * (dwt[j] - sw);
    for (int32_t c = 0; c < H; ++c) dx[t * H + c] = 0.0;
    /* backward of each route */
    for (int32_t j = 0; j < k; ++j) {
        const uint16_t *Wd = w_d + (int64_t)idx[j] * H * I;
        double *dWgu = dw_gu ? dw_gu + (int64_t)idx[j] * 2 * I * H : NULL;
        double *dWd = dw_d ? dw_d + (int64_t)idx[j] * H * I : NULL;
        for (int32_t i = 0; i < I; ++i) {
            double sdh = 0.0;
            for (int32_t c = 0; c < H; ++c) sdh += (w[j] * gr[c]) * bf(Wd[(int64_t)c * I + i]);
            dh[i] = sdh;
        }
        if (dWd)
            for (int32_t c = 0; c < H; ++c)
                for (int32_t i = 0; i < I; ++i) dWd[(int64_t)c * I + i] += (w[j] * gr[c]) * a[j * I + i];
        for (int32_t i = 0; i < I; ++i) {
            const double dg = dh[i] * u[j * I + i] * silu_grad(g[j * I + i]);
            const double du = dh[i] * silu(g[j * I + i]);
            if (dWgu)
                for (int32_t c = 0; c < H; ++c) {
                    dWgu[(int64_t)i * H + c] += dg * bf(xr[c]);
                    dWgu[(int64_t)(I + i) * H + c] += du * bf(xr[c]);
                }
            g[j * I + i] = dg; /* keep dg, du for dx below */
            u[j * I + i] = du;
        }
    }
    /* dx[t] = sum_j of that route's dx_perm row, j ascending */
    for (int32_t j = 0; j < k; ++j) {
        const uint16_t *Wgu = w_gu + (int64_t)idx[j] * 2 * I * H;
        for (int32_t c = 0; c < H; ++c) {
            double s = 0.0;
            for (int32_t i = 0; i < 2 * I; ++i) {
                const double d = i < I ? g[j * I + i] : u[j * I + i - I];
                s += d * bf(Wgu[(int64_t)i * H + c]);
            }
            dx[t * H + c] += s;
        }
    }
}

int moe_oracle_backward(const uint16_t *x, const float *logits, const uint16_t *w_gu,
                        const uint16_t *w_d, const double *dout, int64_t T, int32_t H, int32_t E,
                        int32_t k, int32_t I, double *dx, double *dlogits, double *dw_gu,
                        double *dw_d) {
    if (!x || !logits || !w_gu || !w_d || !dout || !dx || !dlogits || (!dw_gu) != (!dw_d) || T < 0 ||
        H < 1 || E < 1 || k < 1 || k > E || I < 1)
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < T * (int64_t)E; ++i)
        if (!isfinite(logits[i])) return ORACLE_ENONFINITE;
    if (dw_gu) {
        for (int64_t i = 0; i < (int64_t)E * 2 * I * H; ++i) dw_gu[i] = 0.0;
        for (int64_t i = 0; i < (int64_t)E * H * I; ++i) dw_d[i] = 0.0;
        BwdScratch sc;
        int ok = bwd_scratch_alloc(&sc, k, I);
        if (ok)
            for (int64_t t = 0; t < T; ++t)
                backward_token(t, x, logits, w_gu, w_d, dout, H, E, k, I, dx, dlogits, dw_gu, dw_d, &sc);
        bwd_scratch_free(&sc);
        return ok ? 0 : ORACLE_EINVAL;
    }
    int failed = 0;
#pragma omp parallel
    {
        BwdScratch sc;
        const int ok = bwd_scratch_alloc(&sc, k, I);
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t)
            if (ok) backward_token(t, x, logits, w_gu, w_d, dout, H, E, k, I, dx, dlogits, NULL, NULL, &sc);
        bwd_scratch_free(&sc);
    }
    return failed ? ORACLE_EINVAL : 0;
}

/* Threads the OpenMP loops above use (for reporting the oracle's CPU time). */
int moe_oracle_num_threads(void) { return omp_get_max_threads(); }

/* Threads later calls from this thread run on (timing the oracle on one core). */
void moe_oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
