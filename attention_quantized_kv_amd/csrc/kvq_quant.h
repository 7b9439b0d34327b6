// kvq_quant.h -- the block quantizers of the cache on the GPU: K as Q8_0 and
// V as Q4_0, 32-value blocks of one (token, KV head) row with one fp16 scale
// per block ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070 XT at 262k
// context, via adaptive KV streaming", first paragraph; "OSCAR2 KV Cache
// benchmark", compression-ratio table).  The block rules are the ones stated
// in include/kvq.h.
//
// One value per lane: a block is 32 consecutive lanes (an aligned half
// wavefront), reduced in five lane exchanges (DPP inside 16-lane rows, a
// permlane swap across them).  Every product,
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

// Lane exchanges without LDS round trips: DPP within a 16-lane row, and the
// gfx950 permlane swaps across rows (a 32-lane half and the whole wave).
template <int CTRL>
__device__ inline int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float x) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, x)));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i inside each 8 lanes
constexpr int kDppMirror = 0x140;       // lane i <-> 15-i inside each 16 lanes

// The value of lane ^ 16 (the other 16-lane row of the 32-lane half).
// v_permlane16_swap a, b swaps a's odd rows with b's even rows: with a = b =
// x, an even row finds its partner in b and an odd row in a.  Inline asm: the
// builtin's second result is folded into the first by the optimiser.
__device__ inline int xor16_i(int x, int lane) {
    int a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return (lane & 16) ? a : b;
}
// The value of lane ^ 32 (the other half of the wave), likewise.
__device__ inline int xor32_i(int x, int lane) {
    int a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return (lane & 32) ? a : b;
}
__device__ inline float xor16_f(float x, int lane) {
    return __builtin_bit_cast(float, xor16_i(__builtin_bit_cast(int, x), lane));
}
__device__ inline float xor32_f(float x, int lane) {
    return __builtin_bit_cast(float, xor32_i(__builtin_bit_cast(int, x), lane));
}

// Maximum over the 32-lane half holding this lane (every lane gets it).
__device__ inline float block_max32(float x, int lane) {
    x = fmaxf(x, dpp_f<kDppXor1>(x));
    x = fmaxf(x, dpp_f<kDppXor2>(x));
    x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_f<kDppMirror>(x));
    return fmaxf(x, xor16_f(x, lane));
}

// Sum over the whole wave (every lane gets it; the order is fixed).
__device__ inline float wave_sum(float x, int lane) {
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    x += dpp_f<kDppMirror>(x);
    x += xor16_f(x, lane);
    return x + xor32_f(x, lane);
}

// Maximum over the whole wave.
__device__ inline float wave_max(float x, int lane) {
    x = fmaxf(x, dpp_f<kDppXor1>(x));
    x = fmaxf(x, dpp_f<kDppXor2>(x));
    x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_f<kDppMirror>(x));
    x = fmaxf(x, xor16_f(x, lane));
    return fmaxf(x, xor32_f(x, lane));
}

// Over the 32-lane half: the value of largest magnitude, lowest index on ties
// (idx = position in the block).  The pair rule is symmetric, so both lanes
// of every exchange keep the same winner and the order of the steps does not
// matter.
struct ArgMax {
    float ax;   // |x|
    float x;    // the signed value
    int idx;
};
__device__ inline ArgMax pick(ArgMax a, ArgMax b) {
    return (b.ax > a.ax || (b.ax == a.ax && b.idx < a.idx)) ? b : a;
}
template <int CTRL>
__device__ inline ArgMax dpp_am(ArgMax a) {
    return {dpp_f<CTRL>(a.ax), dpp_f<CTRL>(a.x), dpp_i<CTRL>(a.idx)};
}
__device__ inline ArgMax block_argmax_abs32(float x, int lane) {
    ArgMax a{fabsf(x), x, lane & (kBlock - 1)};
    a = pick(a, dpp_am<kDppXor1>(a));
    a = pick(a, dpp_am<kDppXor2>(a));
    a = pick(a, dpp_am<kDppHalfMirror>(a));
    a = pick(a, dpp_am<kDppMirror>(a));
    return pick(a, ArgMax{xor16_f(a.ax, lane), xor16_f(a.x, lane), xor16_i(a.idx, lane)});
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
__device__ inline QCode quant_q8_0(float x, int lane_in_wave) {
#pragma clang fp contract(off)
    const float amax = block_max32(fabsf(x), lane_in_wave);
    const float d = __fdiv_rn(amax, 127.0f);
    const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
    return {(int)round_half_away(mul_rounded(x, id)), d};
}

// Q4_0: m = the value of largest magnitude (lowest index on ties), d = m / -8,
// code = min(15, trunc(x * (1/d) + 8.5)) in [0, 15].
__device__ inline QCode quant_q4_0(float x, int lane_in_wave) {
#pragma clang fp contract(off)
    const ArgMax am = block_argmax_abs32(x, lane_in_wave);
    const float m = am.ax == 0.0f ? 0.0f : am.x;        // all-zero block: m = +0
    const float d = __fdiv_rn(m, -8.0f);
    const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
    const float t = mul_rounded(x, id) + 8.5f;
    return {min(15, __float2int_rz(t)), d};
}

// INT2 (128-value blocks, value = zero + scale * code): from the block's
// minimum mn and maximum mx, d = (mx - mn) / 3 and its reciprocal id (0 when
// d = 0), and the code of x, min(3, trunc((x - mn) * id + 0.5)) -- the
// nearest of the four levels, ties upward.  The minimum and maximum are exact
// whatever the reduction order, so every kernel that quantizes a block gets
// the same codes and fp16 (scale, zero) = (fp16(d), fp16(mn)).
struct Int2Par {
    float d;
    float id;
};
__device__ inline Int2Par int2_params(float mn, float mx) {
#pragma clang fp contract(off)
    const float d = __fdiv_rn(mx - mn, 3.0f);
    return {d, d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f};
}
__device__ inline int int2_code(float x, float mn, float id) {
#pragma clang fp contract(off)
    return min(3, (int)(mul_rounded(x - mn, id) + 0.5f));
}

}  // namespace kvq
