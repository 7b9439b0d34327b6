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
