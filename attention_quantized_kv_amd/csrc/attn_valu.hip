// attn_valu.hip -- portable split-K attention over the paged Q8_0/Q4_0 cache
// on plain vector ALUs (gfx950).  Correct for every supported shape; the MFMA
// kernels are the fast paths.
//
// One wavefront per (split, KV head, query): the split is a run of 32-token
// chunks, the wave serves all G query heads that share the KV head
// ("Context window and KV cache", GQA section), so each key is dequantized
// once for G heads.  Lane L owns dims L*D/64 .. +D/64.  For every key the G
// scores are reduced across the wave with an xor butterfly (every lane ends
// with the same bits), then each head's online-softmax state is updated.
// The partial (m, l, acc) of each row is merged later by online
// log-sum-exp ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070 XT at 262k
// context, via adaptive KV streaming", second paragraph).  Scores are kept in
// the log2 domain: q is pre-multiplied by scale*log2(e), so p = exp2(s - m).
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kMaxGroup = 16;

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ inline float f16_val(const uint8_t* p) {
    return __half2float(__ushort_as_half(*reinterpret_cast<const uint16_t*>(p)));
}

template <int D>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a, int cps, int n_splits, int group) {
    constexpr int DPL = D / 64;
    const int s = blockIdx.x, kvh = blockIdx.y, qi = blockIdx.z;
    const int lane = threadIdx.x;
    const Geom& g = a.g;
    const int nb = D / kBlock;
    const int last = a.ctx - a.n_q + qi;                       // last visible key
    const int j0 = s * cps * kChunk;
    const int j1 = min((s + 1) * cps * kChunk, last + 1);
    const float qscale = a.scale * 1.4426950408889634f;

    float q[kMaxGroup][DPL];
    float m[kMaxGroup], l[kMaxGroup], acc[kMaxGroup][DPL];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            acc[h][e] = 0.0f;
            q[h][e] = h < group
                ? a.q[((size_t)qi * a.n_heads + kvh * group + h) * D + lane * DPL + e] * qscale
                : 0.0f;
        }
    }

    bool bad = false;
    for (int j = j0; j < j1; ++j) {
        const int phys = a.page_table[j / g.P];
        if (phys < 0 || phys >= g.n_pages) { bad = true; break; }
        const uint8_t* unit = a.pool + g.unit_index(phys, kvh) * g.unit_bytes();
        const int slot = j % g.P;
        float kh[DPL], vh[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const int d = lane * DPL + e;
            const float ks = f16_val(unit + g.k_scales_off() + (slot * nb + d / kBlock) * 2);
            const float vs = f16_val(unit + g.v_scales_off() + v_scale_idx(g, slot, d / kBlock) * 2);
            kh[e] = ks * (float)(int8_t)unit[k_code_pos(g, slot, d)];
            int nib;
            const uint8_t byte = unit[v_code_pos(g, slot, d, &nib)];
            vh[e] = vs * (float)(((byte >> (4 * nib)) & 15) - 8);
        }
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            if (h >= group) continue;
            float part = 0.0f;
#pragma unroll
            for (int e = 0; e < DPL; ++e) part = fmaf(q[h][e], kh[e], part);
            const float sc = wave_sum(part);
            const float mn = fmaxf(m[h], sc);
            const float alpha = exp2f(m[h] - mn);
            const float p = exp2f(sc - mn);
            l[h] = l[h] * alpha + p;
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] = fmaf(acc[h][e], alpha, p * vh[e]);
            m[h] = mn;
        }
    }

#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
        if (h >= group) continue;
        const size_t row = (size_t)qi * a.n_heads + kvh * group + h;
        const size_t ps = row * n_splits + s;
        if (lane == 0) {
            a.ws_m[ps] = bad ? NAN : m[h];
            a.ws_l[ps] = bad ? NAN : l[h];
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e) a.ws_acc[ps * D + lane * DPL + e] = bad ? NAN : acc[h][e];
    }
}

}  // namespace

hipError_t launch_attn_valu(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    dim3 grid(pl.n_splits, a.g.n_kv, a.n_q);
    switch (a.g.D) {
        case 64:  hipLaunchKernelGGL(attn_valu_kernel<64>, grid, dim3(64), 0, stream, a, pl.chunks_per_split, pl.n_splits, pl.group); break;
        case 128: hipLaunchKernelGGL(attn_valu_kernel<128>, grid, dim3(64), 0, stream, a, pl.chunks_per_split, pl.n_splits, pl.group); break;
        case 256: hipLaunchKernelGGL(attn_valu_kernel<256>, grid, dim3(64), 0, stream, a, pl.chunks_per_split, pl.n_splits, pl.group); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
