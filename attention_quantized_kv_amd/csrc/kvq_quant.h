// kvq_quant.h -- the block quantizers of the cache on the GPU: K as Q8_0 and
// V as Q4_0, 32-value blocks of one (token, KV head) row with one fp16 scale
// per block ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070 XT at 262k
// context, via adaptive KV streaming", first paragraph; "OSCAR2 KV Cache
// benchmark", compression-ratio table).  The block rules are the ones stated
// in include/kvq.h.
//
// One value per lane: a block is 32 consecutive lanes (an aligned half
// wavefront), so block reductions are five xor-shuffles.  Every product,
// quotient and sum is IEEE fp32 rounded on its own (no contraction), so codes
// and scales are bit-reproducible wherever these functions run.
#pragma once

#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {

// Round half away from zero.  t - trunc(t) is exact in fp32.
__device__ inline float round_half_away(float t) {
    float r = truncf(t);
    if (fabsf(t - r) >= 0.5f) r += copysignf(1.0f, t);
    return r;
}

__device__ inline float block_max32(float x) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// Largest magnitude of the block and the lowest index holding it.
__device__ inline void block_argmax_abs32(float ax, int idx, float* amax, int* aidx) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
        float oax = __shfl_xor(ax, o, 64);
        int oidx = __shfl_xor(idx, o, 64);
        if (oax > ax || (oax == ax && oidx < idx)) { ax = oax; idx = oidx; }
    }
    *amax = ax;
    *aidx = idx;
}

__device__ inline uint16_t f16_bits(float x) { return __half_as_ushort(__float2half_rn(x)); }

// x * y rounded to fp32 on its own.  The empty asm hides the product from the
// optimizer, which otherwise fuses it with a following add into one FMA
// (single rounding) regardless of contraction pragmas.
__device__ inline float mul_rounded(float x, float y) {
    float p = x * y;
    asm volatile("" : "+v"(p));
    return p;
}

// A quantized value: the code and the block's fp32 scale before its rounding
// to the stored fp16.
struct QCode {
    int code;
    float d;
};

// Q8_0: d = amax / 127, code = round-half-away(x / d) in [-127, 127]
// (x * (1/d), both rounded; an all-zero block has d = 0 and codes 0).
__device__ inline QCode quant_q8_0(float x) {
#pragma clang fp contract(off)
    const float amax = block_max32(fabsf(x));
    const float d = __fdiv_rn(amax, 127.0f);
    const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
    return {(int)round_half_away(mul_rounded(x, id)), d};
}

// Q4_0: m = the value of largest magnitude (lowest index on ties), d = m / -8,
// code = min(15, trunc(x * (1/d) + 8.5)) in [0, 15].  lane_in_wave picks the
// shuffle source: the block is lanes (lane & ~31) .. +31.
__device__ inline QCode quant_q4_0(float x, int lane_in_wave) {
#pragma clang fp contract(off)
    float amax;
    int aidx;
    block_argmax_abs32(fabsf(x), lane_in_wave & (kBlock - 1), &amax, &aidx);
    float m = __shfl(x, (lane_in_wave & ~(kBlock - 1)) + aidx, 64);
    if (amax == 0.0f) m = 0.0f;                        // all-zero block: m = +0
    const float d = __fdiv_rn(m, -8.0f);
    const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
    const float t = mul_rounded(x, id) + 8.5f;
    return {min(15, __float2int_rz(t)), d};
}

}  // namespace kvq
