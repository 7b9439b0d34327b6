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
#include "kvq_quant.h"

namespace kvq {
namespace {

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
        const QCode qk = quant_q8_0(k[src], lane);
        unit[k_code_pos(g, slot, d)] = (uint8_t)(int8_t)qk.code;
        if ((d & (kBlock - 1)) == 0) k_scales[slot * nb + d / kBlock] = f16_bits(qk.d);

        // V: Q4_0
        const QCode qv = quant_q4_0(v[src], lane);
        vcode[r] = qv.code;
        if ((d & (kBlock - 1)) == 0) v_scales[v_scale_idx(g, slot, d / kBlock)] = f16_bits(qv.d);
    }

    int nib;
    const int64_t off = v_code_pos(g, pos_a % g.P, d, &nib);   // even slot: low nibble
    const uint8_t old = (has[0] && has[1]) ? 0 : unit[off];
    const int lo = has[0] ? vcode[0] : (old & 15);
    const int hi = has[1] ? vcode[1] : (old >> 4);
    unit[off] = (uint8_t)(lo | (hi << 4));
}

// INT2 codec (K and V alike; "OSCAR2 KV Cache benchmark", compression-ratio
// table: 36 bytes per 128 values with fp16 zero-point metadata): per block of
// 128 values mn = min, mx = max, d = (mx - mn) / 3, code = min(3,
// floor((x - mn) * (1/d) + 0.5)), every operation rounded to fp32 on its own;
// stored fp16(d) and fp16(mn).
//
// One workgroup per (group of 8 consecutive positions, KV head, block): the
// 8 tokens of a group share every V code dword (a dword holds two dims of 8
// tokens), so the group is written by one workgroup and needs no atomics.
// Wave e quantizes token e of the group, two values per lane, writes its
// scale/zero pairs and leaves its codes in LDS; after a barrier 64 threads
// pack the tokens' K dwords (8 per token) and 64 threads the group's V
// dwords, keeping the old codes of the group's tokens that are not being
// appended.
__global__ __launch_bounds__(512) void append_int2_kernel(Geom g, uint8_t* __restrict__ pool,
                                                          const int32_t* __restrict__ page_table, int pos0,
                                                          int n_new, const float* __restrict__ k,
                                                          const float* __restrict__ v) {
#pragma clang fp contract(off)
    __shared__ uint8_t kcodes[8][kBlock2];
    __shared__ uint8_t vcodes[8][kBlock2];
    const int kvh = blockIdx.y, b = blockIdx.z;
    const int base = 8 * (blockIdx.x + (pos0 >> 3));         // first position of the group
    const int e = threadIdx.x >> 6, lane = threadIdx.x & 63;
    auto mine = [&](int t) { return base + t >= pos0 && base + t < pos0 + n_new; };
    const int phys = page_table[base / g.P];
    if (phys < 0 || phys >= g.n_pages) return;               // never touch a page outside the pool
    uint8_t* unit = pool + g.unit_index(phys, kvh) * g.unit_bytes();
    const int nb2 = g.nb2();
    if (mine(e)) {                                           // uniform per wave
        const int pos = base + e, slot = pos % g.P;
        const size_t src = ((size_t)(pos - pos0) * g.n_kv + kvh) * g.D + kBlock2 * b + 2 * lane;
        auto quant = [&](const float* x, uint8_t (&codes)[8][kBlock2], uint16_t& hs, uint16_t& hz) {
            const float x0 = x[src], x1 = x[src + 1];
            const float mn = -wave_max(-fminf(x0, x1), lane);  // exact: negation and max
            const float mx = wave_max(fmaxf(x0, x1), lane);
            const Int2Par pr = int2_params(mn, mx);
            codes[e][2 * lane] = (uint8_t)int2_code(x0, mn, pr.id);
            codes[e][2 * lane + 1] = (uint8_t)int2_code(x1, mn, pr.id);
            hs = f16_bits(pr.d);
            hz = f16_bits(mn);
        };
        uint16_t hs, hz;
        quant(k, kcodes, hs, hz);
        if (lane == 0) {
            uint16_t* kp = reinterpret_cast<uint16_t*>(unit + g.i2_k_params_off()) + ((size_t)slot * nb2 + b) * 2;
            kp[0] = hs;
            kp[1] = hz;
        }
        quant(v, vcodes, hs, hz);
        if (lane == 0) {
            const size_t i = ((size_t)(slot / kChunk) * nb2 + b) * kChunk + slot % kChunk;
            reinterpret_cast<uint16_t*>(unit + g.i2_v_scales_off())[i] = hs;
            reinterpret_cast<uint16_t*>(unit + g.i2_v_zeros_off())[i] = hz;
        }
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < 64) {
        // K dword (grp, i) of token te: words 2i, 2i+1 = 32-dim steps of this block
        const int te = t >> 3, grp = (t >> 1) & 3, i = 2 * b + (t & 1);
        if (mine(te)) {
            uint32_t w = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ee = 0; ee < 8; ++ee)
                    w |= (uint32_t)kcodes[te][32 * (2 * i + h) - kBlock2 * b + 8 * grp + ee] << i2_bit(h, ee);
            int bit;
            const int64_t off = i2_k_dword(g, (base + te) % g.P, 32 * (2 * i) + 8 * grp, &bit);
            *reinterpret_cast<uint32_t*>(unit + off) = w;
        }
    } else if (t < 128) {
        // V dword (n, i) of the group: words 2i, 2i+1 = dims 16 (2i + h) + n, tokens 0..7
        const int q = t - 64, n = q & 15, i = 4 * b + (q >> 4);
        int bit;
        const int64_t off = i2_v_dword(g, base % g.P, 16 * (2 * i) + n, &bit);
        uint32_t* dw = reinterpret_cast<uint32_t*>(unit + off);
        const bool all = base >= pos0 && base + 8 <= pos0 + n_new;
        const uint32_t old = all ? 0u : *dw;
        uint32_t w = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) {
                const int sh = i2_bit(h, ee);
                const uint32_t c = mine(ee) ? vcodes[ee][16 * (2 * i + h) + n - kBlock2 * b] : (old >> sh) & 3u;
                w |= c << sh;
            }
        *dw = w;
    }
}

}  // namespace

hipError_t launch_append(const Geom& g, uint8_t* pool, const int32_t* page_table, int pos0,
                         int n_new, const float* k, const float* v, hipStream_t stream) {
    if (g.codec == 1) {
        const int groups = ((pos0 + n_new - 1) >> 3) - (pos0 >> 3) + 1;
        hipLaunchKernelGGL(append_int2_kernel, dim3(groups, g.n_kv, g.nb2()), dim3(512), 0, stream, g, pool,
                           page_table, pos0, n_new, k, v);
        return hipGetLastError();
    }
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
