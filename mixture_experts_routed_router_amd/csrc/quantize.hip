// quantize.hip -- block-scaled FP8 expert weights (OCP E4M3, gfx950 conversions).
//
// Expert weights are quantized once per weight update, not per layer call
// [prime-rl, Changes: FP8 expert weights quantized once per optimizer step], so
// the grouped GEMMs read half the weight bytes [Halo "Performance", Levers that
// do not help here: fine-grained experts are bound by weight bytes].
//
// W [E, R, K] bf16 is cut into blocks of 64 consecutive rows over all of K (one
// expert's rows never share a block with another's, R % 64 == 0). Per block:
//   scale = max |w| / 448 in fp32 (1 for an all-zero block),
//   code  = E4M3 nearest-even of clamp(w / scale, -448, 448)   (fp32 division)
// A scale constant along K multiplies whole dot products, so a GEMM applies it
// once to its fp32 accumulator. One workgroup per block: a max-reduction pass,
// then an encode pass over the same 64 * K elements (re-read from L2).
#include "common.hpp"

namespace moe {

constexpr int kQuantThreads = 256;

// Two fp32 values -> two E4M3 codes in the low (HI = false) or high half of `old`:
// v_cvt_pk_fp8_f32 rounds to nearest even; the inputs are already within +-448.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2_fp8(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

__device__ __forceinline__ float clamp448(float q) { return fminf(fmaxf(q, -448.0f), 448.0f); }

__global__ __launch_bounds__(kQuantThreads) void quantize_fp8_kernel(const uint16_t* __restrict__ w,
                                                                     int64_t block_elems,
                                                                     uint8_t* __restrict__ w8,
                                                                     float* __restrict__ scale) {
    MOE_DEBUG_GUARD();
    const int64_t blk = blockIdx.x;
    const uint16_t* src = w + blk * block_elems;
    uint8_t* dst = w8 + blk * block_elems;
    const int64_t pieces = block_elems / 8;  // 16 bytes of bf16 in, 8 bytes of codes out

    float amax = 0.0f;
    for (int64_t p = threadIdx.x; p < pieces; p += kQuantThreads) {
        const u32x4_t v = *(const u32x4_t*)(src + p * 8);
#pragma unroll
        for (int d = 0; d < 4; ++d)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[d])), fabsf(bf16_hi(v[d]))));
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    __shared__ float wave_max[kQuantThreads / kWave];
    if (lane_id() == 0) wave_max[threadIdx.x / kWave] = amax;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQuantThreads / kWave; ++i) amax = fmaxf(amax, wave_max[i]);

    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;  // IEEE division (hipcc's default)
    if (threadIdx.x == 0) scale[blk] = s;
    for (int64_t p = threadIdx.x; p < pieces; p += kQuantThreads) {
        const u32x4_t v = *(const u32x4_t*)(src + p * 8);
        uint32_t out[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t d0 = v[2 * h], d1 = v[2 * h + 1];
            const uint32_t lo = cvt2_fp8<false>(clamp448(bf16_lo(d0) / s), clamp448(bf16_hi(d0) / s), 0u);
            out[h] = cvt2_fp8<true>(clamp448(bf16_lo(d1) / s), clamp448(bf16_hi(d1) / s), lo);
        }
        *(uint2*)(dst + p * 8) = make_uint2(out[0], out[1]);
    }
}

hipError_t launch_quantize_fp8(const uint16_t* w, int64_t E, int R, int K, uint8_t* w8, float* scale,
                               hipStream_t stream) {
    const int64_t blocks = E * (R / 64);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, w,
                       (int64_t)64 * K, w8, scale);
    return hipGetLastError();
}

}  // namespace moe
