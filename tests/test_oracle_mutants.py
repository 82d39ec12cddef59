"""Plants plausible mistakes in copies of the CPU oracle (never in the oracle
itself) and checks that the pins in test_oracle_pins.py catch each one.  CPU only."""
from __future__ import annotations

import pytest

import oracle
from oracle.build import build_variant
from mixture_experts_routed_router_amd import inputs as gen

import test_oracle_pins as pins

MUTANTS = {
    # clamped SwiGLU: the up projection clipped from above only
    "clamp_up_one_sided": ([("            if (u < -limit) u = -limit;\n", "")], [pins.check_swiglu_clamped]),
    # clamped SwiGLU: the gate clipped from below too
    "clamp_gate_both_sides": ([("            if (g > limit) g = limit;\n",
                                "            if (g > limit) g = limit;\n            if (g < -limit) g = -limit;\n")],
                              [pins.check_swiglu_clamped]),
    # clamped SwiGLU: the cap applied to silu(g) instead of g
    "clamp_after_silu": ([("            if (g > limit) g = limit;\n", ""),
                          ("if (u < -limit) u = -limit;\n            h[p * I + i] = silu(g) * u;",
                           "if (u < -limit) u = -limit;\n            h[p * I + i] = fmin(silu(g), limit) * u;")],
                         [pins.check_swiglu_clamped]),
    # routing: ties to the higher id instead of the lower
    "tie_to_higher_id": ([("return a < b;", "return a > b;")], [pins.check_topk_brute_force]),
    # routing: a dropped term in the softmax denominator
    "softmax_drops_last_pick": ([("for (int32_t j = 0; j < k; ++j) s += exp(",
                                  "for (int32_t j = 0; j < k - 1; ++j) s += exp(")],
                                [pins.check_softmax_weights]),
    # layout: unpadded offsets
    "offsets_unpadded": ([("off[e + 1] = off[e] + (cnt[e] + align - 1) / align * align;",
                           "off[e + 1] = off[e] + cnt[e];")], [pins.check_layout_cases]),
    # layout: pad rows not marked -1
    "pad_rows_not_marked": ([("row_token[p] = -1;", "row_token[p] = 0;")], [pins.check_layout_cases]),
    # layout: placement not stable (routes visited in descending order)
    "unstable_placement": ([("for (int64_t r = 0; r < R; ++r) {\n        int32_t e = topk_idx[r];",
                             "for (int64_t r = R - 1; r >= 0; --r) {\n        int32_t e = topk_idx[r];")],
                           [pins.check_layout_cases]),
    # experts: SwiGLU applied to the up projection instead of the gate
    "gate_up_swapped": ([("a[i] = silu(g) * u;", "a[i] = silu(u) * g;")],
                        [pins.check_structured_closed_form, pins.check_dense_swiglu_reduction]),
    # experts: sign error inside silu
    "silu_sign": ([("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));")],
                  [pins.check_dense_swiglu_reduction]),
    # experts: down projection read transposed
    "down_transposed": ([("y += a[i] * bf(Wd[(int64_t)c * I + i]);",
                          "y += a[i] * bf(Wd[(int64_t)i * H + c]);")],
                        [pins.check_structured_closed_form]),
    # combine: every route weighted by the top weight
    "combine_wrong_weight": ([("acc[c] += w[j] * y;", "acc[c] += w[0] * y;")],
                             [lambda o: pins.check_dense_masked(o, gen.CONFIGS["tiny"])]),
    # combine step: a dropped route in the gather-sum
    "combine_drops_route": ([("for (int32_t j = 0; j < k; ++j)\n                s += topk_w",
                              "for (int32_t j = 1; j < k; ++j)\n                s += topk_w")],
                            [pins.check_identity_experts]),
    # fp8: ties rounded away from zero instead of to even
    "fp8_ties_away": ([("return fmod(f, 2.0) == 0.0 ? f : f + 1.0;", "return f + 1.0;")],
                      [pins.check_fp8_encode]),
    # fp8: exponent bias off by one in the decoding
    "fp8_bias_off_by_one": ([("else v = ldexp((double)(8 + m), e - 10);",
                              "else v = ldexp((double)(8 + m), e - 11);")], [pins.check_fp8_decode]),
    # fp8: subnormal step taken as 2^-8
    "fp8_subnormal_step": ([("const double n = rne(a * 512.0);", "const double n = rne(a * 256.0);")],
                           [pins.check_fp8_encode]),
    # fp8: block absmax over the first 32 rows of each block only
    "fp8_short_block_amax": ([("for (int64_t i = 0; i < (int64_t)64 * K; ++i) {\n                const float a",
                               "for (int64_t i = 0; i < (int64_t)32 * K; ++i) {\n                const float a")],
                             [pins.check_fp8_quantize]),
    # fp8: dequantization takes the wrong block's scale
    "fp8_dequant_wrong_block": ([("const double s = (double)scale[e * nb + r / 64];",
                                  "const double s = (double)scale[e * nb + r % nb];")],
                                [pins.check_fp8_quantize]),
    # fp8 weights: gate rows read from the up half
    "w64_gate_from_up": ([("const double *wg = W + (int64_t)i * H;", "const double *wg = W + (int64_t)(I + i) * H;")],
                         [pins.check_glu_down_w64]),
    # backward: silu' loses its second term (used by both the loop and the steps)
    "bwd_silu_grad_first_term_only": ([("return s * (1.0 + g * (1.0 - s));", "return s;")],
                                      [pins.check_backward_finite_differences,
                                       pins.check_swiglu_bwd_derivative]),
    # backward loop: dy without the routing weight
    "bwd_dy_unweighted": ([("sdh += (w[j] * gr[c]) * bf(Wd[(int64_t)c * I + i]);",
                            "sdh += gr[c] * bf(Wd[(int64_t)c * I + i]);")],
                          [pins.check_backward_finite_differences]),
    # backward loop: W_down gradient written transposed
    "bwd_dwd_transposed": ([("dWd[(int64_t)c * I + i] += (w[j] * gr[c]) * a[j * I + i];",
                             "dWd[(int64_t)i * H + c] += (w[j] * gr[c]) * a[j * I + i];")],
                           [pins.check_backward_finite_differences]),
    # backward loop: dx misses the up projection's share
    "bwd_dx_drops_up": ([("const double d = i < I ? g[j * I + i] : u[j * I + i - I];",
                          "const double d = i < I ? g[j * I + i] : 0.0;")],
                        [pins.check_backward_finite_differences]),
    # backward loop: softmax gradient without the mean term
    "bwd_loop_softmax_no_mean": ([("dlogits[t * E + idx[j]] = w[j] * (dwt[j] - sw);",
                                   "dlogits[t * E + idx[j]] = w[j] * dwt[j];")],
                                 [pins.check_backward_finite_differences, pins.check_backward_invariants]),
    # backward steps: softmax gradient without the mean term
    "bwd_step_softmax_no_mean": ([("= topk_w[t * k + j] * (dw[t * k + j] - s);",
                                   "= topk_w[t * k + j] * dw[t * k + j];")],
                                 [pins.check_backward_steps_compose]),
    # backward steps: gate and up gradients swapped
    "bwd_step_swiglu_swapped": ([("dgu[p * 2 * I + i] = d * u * silu_grad(g);\n            dgu[p * 2 * I + I + i] = d * silu(g);",
                                  "dgu[p * 2 * I + I + i] = d * u * silu_grad(g);\n            dgu[p * 2 * I + i] = d * silu(g);")],
                                [pins.check_backward_steps_compose, pins.check_swiglu_bwd_derivative]),
    # backward steps: permute backward drops the first route of each token
    "bwd_step_permute_drops_route": ([("for (int32_t j = 0; j < k; ++j) s += dx_perm[",
                                       "for (int32_t j = 1; j < k; ++j) s += dx_perm[")],
                                     [pins.check_backward_steps_compose, pins.check_backward_invariants]),
    # backward steps: wgrad sums one row short per expert
    "bwd_step_wgrad_short": ([("for (int64_t p = p0; p < p0 + n; ++p) s += A[p * M + m] * B[p * N + c];",
                               "for (int64_t p = p0; p + 1 < p0 + n; ++p) s += A[p * M + m] * B[p * N + c];")],
                             [pins.check_backward_steps_compose, pins.check_backward_invariants]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    edits, checks = MUTANTS[name]
    mutant = oracle.Oracle(build_variant(edits, str(tmp_path)))
    for check in checks:
        with pytest.raises(AssertionError):
            check(mutant)


def test_unmutated_copy_passes(tmp_path):
    """The variant build itself (no edits) passes the same checks."""
    same = oracle.Oracle(build_variant([], str(tmp_path)))
    for _, checks in MUTANTS.values():
        for check in checks:
            check(same)
