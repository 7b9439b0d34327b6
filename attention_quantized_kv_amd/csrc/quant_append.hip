// quant_append.hip -- quantize new K/V rows into the paged pool (gfx950).
//
// K is encoded as Q8_0 and V as Q4_0, blocks of 32 values of one (token, KV
// head) row, one fp16 scale per block ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB
// RX 9070 XT at 262k context, via adaptive KV streaming", first paragraph;
// "OSCAR2 KV Cache benchmark", compression-ratio table).  The block rules are
// the ones stated in include/kvq.h; all arithmetic is IEEE fp32 with every
// product, quotient and sum rounded on its own (no contraction), so the codes
// and scales are bit-reproducible.
//
// One workgroup of D threads handles one pair of consecutive positions
// (2k, 2k+1) of one KV head: thread d owns dimension d of both rows.  A
// 32-value block is an aligned half-wavefront, so block reductions are five
// xor-shuffles.  The two rows of a pair share every V byte (their nibbles sit
// side by side in the chunk layout), so one thread writes that byte, merging
// with the old nibble when only one row of the pair is new.
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

// Every product and sum below is rounded on its own.
#pragma clang fp contract(off)

namespace kvq {
namespace {

// Round half away from zero.  t - trunc(t) is exact in fp32.
__device__ inline float round_half_away(float t) {
    float r = truncf(t);
    if (fabsf(t - r) >= 0.5f) r += copysignf(1.0f, t);
    return r;
}

__device__ inline float block_max(float x) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// Largest magnitude of the block and the lowest index holding it.
__device__ inline void block_argmax_abs(float ax, int idx, float* amax, int* aidx) {
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

template <int D>
__global__ __launch_bounds__(D) void append_kernel(Geom g, uint8_t* __restrict__ pool,
                                                   const int32_t* __restrict__ page_table,
                                                   int pos0, int n_new,
                                                   const float* __restrict__ k,
                                                   const float* __restrict__ v) {
    const int kvh = blockIdx.y;
    const int pos_a = 2 * (blockIdx.x + (pos0 >> 1));       // even position of the pair
    const int d = threadIdx.x;
    const int lane = threadIdx.x & 63;
    const int nb = D / kBlock;

    const int phys = page_table[pos_a / g.P];
    if (phys < 0 || phys >= g.n_pages) return;             // never touch a page outside the pool
    uint8_t* unit = pool + g.unit_index(phys, kvh) * g.unit_bytes();
    uint16_t* k_scales = reinterpret_cast<uint16_t*>(unit + g.k_scales_off());
    uint16_t* v_scales = reinterpret_cast<uint16_t*>(unit + g.v_scales_off());

    int vcode[2] = {0, 0};
    bool has[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int pos = pos_a + r;
        has[r] = pos >= pos0 && pos < pos0 + n_new;        // uniform over the workgroup
        if (!has[r]) continue;
        const int slot = pos % g.P;
        const size_t src = ((size_t)(pos - pos0) * g.n_kv + kvh) * D + d;

        // K: Q8_0
        const float xk = k[src];
        const float amax_k = block_max(fabsf(xk));
        const float dk = __fdiv_rn(amax_k, 127.0f);
        const float idk = dk != 0.0f ? __fdiv_rn(1.0f, dk) : 0.0f;
        const int ck = (int)round_half_away(mul_rounded(xk, idk));
        unit[k_code_pos(g, slot, d)] = (uint8_t)(int8_t)ck;
        if ((d & (kBlock - 1)) == 0) k_scales[slot * nb + d / kBlock] = f16_bits(dk);

        // V: Q4_0
        const float xv = v[src];
        float amax_v;
        int aidx;
        block_argmax_abs(fabsf(xv), d & (kBlock - 1), &amax_v, &aidx);
        float m = __shfl(xv, (lane & ~(kBlock - 1)) + aidx, 64);
        if (amax_v == 0.0f) m = 0.0f;                       // all-zero block: m = +0
        const float dv = __fdiv_rn(m, -8.0f);
        const float idv = dv != 0.0f ? __fdiv_rn(1.0f, dv) : 0.0f;
        const float t = mul_rounded(xv, idv) + 8.5f;
        vcode[r] = min(15, __float2int_rz(t));
        if ((d & (kBlock - 1)) == 0) v_scales[v_scale_idx(g, slot, d / kBlock)] = f16_bits(dv);
    }

    int nib;
    const int64_t off = v_code_pos(g, pos_a % g.P, d, &nib);   // even slot: low nibble
    const uint8_t old = (has[0] && has[1]) ? 0 : unit[off];
    const int lo = has[0] ? vcode[0] : (old & 15);
    const int hi = has[1] ? vcode[1] : (old >> 4);
    unit[off] = (uint8_t)(lo | (hi << 4));
}

}  // namespace

hipError_t launch_append(const Geom& g, uint8_t* pool, const int32_t* page_table, int pos0,
                         int n_new, const float* k, const float* v, hipStream_t stream) {
    const int pairs = ((pos0 + n_new - 1) >> 1) - (pos0 >> 1) + 1;
    dim3 grid(pairs, g.n_kv);
    switch (g.D) {
        case 64:  hipLaunchKernelGGL(append_kernel<64>, grid, dim3(64), 0, stream, g, pool, page_table, pos0, n_new, k, v); break;
        case 128: hipLaunchKernelGGL(append_kernel<128>, grid, dim3(128), 0, stream, g, pool, page_table, pos0, n_new, k, v); break;
        case 256: hipLaunchKernelGGL(append_kernel<256>, grid, dim3(256), 0, stream, g, pool, page_table, pos0, n_new, k, v); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
