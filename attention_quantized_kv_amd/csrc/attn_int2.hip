// attn_int2.hip -- paged decode attention over the INT2 cache (K and V both
// 2-bit, 128-value blocks with an fp16 scale d and zero-point z: value =
// z + d * code; "OSCAR2 KV Cache benchmark", compression-ratio table) on
// gfx950 matrix cores, streaming the cache once.
//
// What it computes: for each query row (query i, head h) and a split of the
// keys, the online-softmax state (m, l, acc) of exact attention over the
// dequantized cache, in the partial format that lse_merge.hip combines
// ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070 XT at 262k context, via
// adaptive KV streaming", third paragraph: paged decode attention; second
// paragraph: online log-sum-exp across pages).
//
// The zero-point splits off both products, so the matrix cores only ever see
// the small integer codes:
//   q . k  = sum_b d_b (q_b . c_b) + z_b sum(q_b)       (b: the 128-dim blocks)
//   p V    = sum_t (p_t d_t) c_t + sum_t p_t z_t         (per V block of dims)
// q_b . c_b is an MFMA over the codes as exact fp16 (q split into fp16 hi +
// lo, so every product is exact in fp32); sum(q_b) is a per-row constant.  On
// the V side P' = p d (fp32) multiplies the codes, and the zero-point term is
// one more MFMA per chunk, p times the chunk's V zero-points, whose output
// column b is the row's term for block b.  Both weights enter as fp16 hi +
// lo: the two terms can be much larger than the value they sum to, so a
// single fp16 rounding of the weights would not do.
//
// Work split as in the Q8_0/Q4_0 streaming kernel: a workgroup of W waves per
// (KV head, split), the split's 32-token chunks dealt round-robin to its
// waves, every query row of the KV head served from one read of each byte.
// A wave streams its chunks global -> LDS directly (global_load_lds_dwordx4:
// no registers held by data in flight) into a ring of NSLOT chunk slots,
// NSLOT - 1 chunks ahead of the one it computes.  A chunk is 2 x 8D/1024
// code requests of 1 KiB (K then V, contiguous in the pool thanks to its
// layout) and one full-wave request for its parameters: K (scale, zero) per
// token and block, V scales and V zero-points per block and token.
#include <hip/hip_fp16.h>

#include <type_traits>

#include "kvq_internal.h"
#include "kvq_mfma.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

template <int D>
struct I2Cfg {
    static constexpr int NB2 = D / kBlock2;   // 128-value blocks per row
    static constexpr int STEPS = D / 32;      // 32-dim MFMA steps of q . k
    static constexpr int NT = D / 16;         // 16-dim output tiles
};

// One chunk in a wave's LDS ring (bytes).
template <int D>
struct I2Slot {
    static constexpr int NB2 = D / kBlock2;
    static constexpr int CODE = 8 * D;                 // 32 tokens x D/4 bytes of K (or V) codes
    static constexpr int K_OFF = 0, V_OFF = CODE, P_OFF = 2 * CODE;
    static constexpr int VS_OFF = P_OFF + 128 * NB2;   // after the K (scale, zero) pairs [32][NB2][2]
    static constexpr int VZ_OFF = VS_OFF + 64 * NB2;   // V scales [NB2][32], then V zeros [NB2][32]
    static constexpr int BYTES = 2 * CODE + 1024;      // the parameter request lands a full 1 KiB
    static constexpr int CODE_REQS = CODE / 1024;      // 1 KiB requests per code region
    static constexpr int REQS = 2 * CODE_REQS + 1;     // requests per chunk
    static constexpr int PLANES = 16 * NB2;            // lanes whose parameter bytes are distinct
    static_assert(CODE % 1024 == 0, "whole wave requests");
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 32-bit LDS address of a pointer into shared memory.
__device__ inline uint32_t lds_off(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Reads of a ring slot.  They are written as LDS reads in asm blocks that wait
// for their own results: the compiler, unable to tell ring slots apart, would
// otherwise guard a read with a wait for every direct-to-LDS load in flight
// (the next chunks'), which takes away the prefetch.  The slot's own data has
// landed by then (an explicit vmcnt wait).
//
// K: the codes of the lane's token in both 16-token tiles and its (scale,
// zero) pairs (at D = 128 the upper half of each code vector is unused).
template <int D>
__device__ inline void read_k(const uint8_t* sl, int lane, int n16, u32x4 (&kc)[2], u32x2 (&kp)[2]) {
    using S = I2Slot<D>;
    const uint32_t ak = lds_off(sl + S::K_OFF + lane * (D / 16));
    const uint32_t ap = lds_off(sl + S::P_OFF + n16 * (S::NB2 * 4));
    if constexpr (D == 256) {
        asm volatile(
            "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
            "ds_read_b64 %2, %5\n\tds_read_b64 %3, %5 offset:128\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(kc[0]), "=&v"(kc[1]), "=&v"(kp[0]), "=&v"(kp[1])
            : "v"(ak), "v"(ap)
            : "memory");
    } else {
        static_assert(D == 128, "head_dim 128 or 256");
        u32x2 k0, k1;
        uint32_t p0, p1;
        asm volatile(
            "ds_read_b64 %0, %4\n\tds_read_b64 %1, %4 offset:512\n\t"
            "ds_read_b32 %2, %5\n\tds_read_b32 %3, %5 offset:64\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(k0), "=&v"(k1), "=&v"(p0), "=&v"(p1)
            : "v"(ak), "v"(ap)
            : "memory");
        kc[0] = u32x4{k0.x, k0.y, 0u, 0u};
        kc[1] = u32x4{k1.x, k1.y, 0u, 0u};
        kp[0] = u32x2{p0, 0u};
        kp[1] = u32x2{p1, 0u};
    }
}
// V: the lane's code dwords, its 8 tokens' zero-points for block n16 % NB2
// and their scales per block (at D = 128 the second halves are unused).
template <int D>
__device__ inline void read_v(const uint8_t* sl, int lane, int n16, int g4, u32x4 (&vc)[2], u32x4& vz,
                              u32x4 (&vs)[2]) {
    using S = I2Slot<D>;
    const uint32_t av = lds_off(sl + S::V_OFF + lane * (D / 8));
    const uint32_t az = lds_off(sl + S::VZ_OFF + (n16 % S::NB2) * 64 + 16 * g4);
    const uint32_t as = lds_off(sl + S::VS_OFF + 16 * g4);
    if constexpr (D == 256) {
        asm volatile(
            "ds_read_b128 %0, %5\n\tds_read_b128 %1, %5 offset:16\n\tds_read_b128 %2, %6\n\t"
            "ds_read_b128 %3, %7\n\tds_read_b128 %4, %7 offset:64\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(vc[0]), "=&v"(vc[1]), "=&v"(vz), "=&v"(vs[0]), "=&v"(vs[1])
            : "v"(av), "v"(az), "v"(as)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(vc[0]), "=&v"(vz), "=&v"(vs[0])
            : "v"(av), "v"(az), "v"(as)
            : "memory");
        vc[1] = vc[0];
        vs[1] = vs[0];
    }
}

// s_waitcnt vmcnt(n * REQS) for a run-time n in [0, NMAX].
template <int REQS, int NMAX, int I = 0>
__device__ inline void wait_chunks(int n) {
    if constexpr (I <= NMAX) {
        if (n == I) { vm_wait<I * REQS>(); return; }
        wait_chunks<REQS, NMAX, I + 1>(n);
    }
}

// The 8 codes of word H of dword x as fp16 MUL * code, exactly, in the
// order (c0, c2, c1, c3, c4, c6, c5, c7) (index bits 0 and 1 swapped: see
// code_slot).  The dword is spread into nibbles, n0 = x & 0x33333333 and n1 =
// (x >> 2) & 0x33333333; with the codes' interleave (code e of word h at bit
// 16 (e/4) + 8h + 2 (e%4)) byte 2k + h of n0 holds codes 4k, 4k+2 of word h
// and the same byte of n1 codes 4k+1, 4k+3.  A 2-bit code zero-extended to a
// nibble is the e2m1 (fp4) value code/2, and gfx950 converts two fp4 values
// with a scale into two fp16 at once: 2 MUL gives MUL * code exactly.  Both
// words of a dword share n0 and n1: 11 operations per 16 codes.
//
// (Masked into an fp16 with a zero exponent instead, a code reads as the
// subnormal c 4^j 2^-24 and needs no conversion, but the matrix cores
// truncate such tiny products toward zero in a sum, about 16 bits down: a
// bias that rotated caches turn into visible output errors.  The fp16
// operands here are normal, and their sums are as exact as fp32.)
template <int H, int MUL>
__device__ inline half8 i2_word(uint32_t x) {
    const uint32_t n0 = x & 0x33333333u, n1 = (x >> 2) & 0x33333333u;
    constexpr float sc = 2.0f * MUL;
    const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n0, sc, H);
    const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n1, sc, H);
    const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n0, sc, 2 + H);
    const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n1, sc, 2 + H);
    return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}
// The code (of a word) in operand element s.
__host__ __device__ constexpr int code_slot(int s) { return (s & 4) | ((s & 1) << 1) | ((s >> 1) & 1); }

// ---- Rows appended by a fused decode step (kvq_append_attn over the INT2
// cache).  The workgroup of the last split of each KV head takes every new
// row, after its waves have streamed their chunks: the 8 tokens of a group
// share each V code dword, so a single workgroup writes each such dword once,
// with no atomics.  Its inputs (the new rows' first blocks, the query rows,
// the page entries, the old V code dwords of the new rows' 8-token groups)
// are requested when the kernel starts and arrive with the first round trip.
// At the end the eight waves share the work:
//  1. wave w quantizes 128-value blocks w, w + 8, ... of the new rows (K and
//     V) with the append kernel's arithmetic -- two values per lane, the
//     block minimum and maximum over the wave -- so codes, scales and
//     zero-points are those kvq_append writes, bit for bit; it writes the
//     block's (scale, zero) into the pool and leaves codes and dequantized
//     values in LDS;
//  2. wave r scores query rows r and r + 8 (those below rows) against each
//     new key and leaves the key's softmax state as partial n_splits + j of
//     the row: m = the score, l = 1, acc = the dequantized V row (an empty
//     partial, l = 0, for rows of earlier queries, which do not see it; NaN
//     when the row's page entry lies outside the pool); wave W - 1 packs the
//     new rows' K code dwords and wave W - 2 rewrites the groups' V code
//     dwords (the other tokens' codes as they were).
// This launch reads the bytes written here only within the last cached
// chunk, when the new positions share it: there they are masked keys, whose
// values do not count (weights 0, scores -inf, zero-points replaced by 0),
// and the other tokens' codes of a shared V dword are written back unchanged.
constexpr int kI2NewRows = 8;                   // rows one fused call appends
template <int D, int QW>
struct I2NewIn {
    static constexpr int NV = D / 64;           // a lane holds dims NV lane .. NV lane + NV - 1 of a row
    static constexpr int GW = D / 128;          // V code dwords of an 8-token group per lane
    float x[2];                                 // this wave's first block: dims 128 b + 2 lane, + 1
    float q[QW][NV];                            // query rows `wave` (and `wave` + 8, QW = 2); row rows - 1 past the last
    int e[2];                                   // page entries of the first and last new 8-token group
    uint32_t old[2][GW];                        // those groups' V code dwords (wave W - 2)
};
// LDS of the end phase: codes [2][8][D] bytes (K, V), dequantized values
// [2][8][D] floats
template <int D>
struct I2NewLds {
    static constexpr int CODES = 0;
    static constexpr int XHAT = 2 * kI2NewRows * D;
    static constexpr int BYTES = XHAT + 2 * kI2NewRows * D * 4;
};

template <int NV>
__device__ inline void load_row(const float* src, float (&x)[NV]) {
    if constexpr (NV == 4) {
        const floatx4 t = *reinterpret_cast<const floatx4*>(src);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = t[i];
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) x[i] = src[i];
    }
}

// Block `it` of the new rows: row j, tensor t (0 K, 1 V), block b.
template <int D>
__device__ inline const float* new_block_src(const NewRows& nr, int n_kv, int kvh, int it, int lane, int& j, int& t,
                                             int& b) {
    constexpr int NB2 = D / kBlock2;
    j = it / (2 * NB2);
    t = (it / NB2) % 2;
    b = it % NB2;
    return (t == 0 ? nr.k : nr.v) + ((size_t)j * n_kv + kvh) * D + kBlock2 * b + 2 * lane;
}

// Requests the inputs that need no page entry (the first round trip).
template <int D, int W, int QW>
__device__ inline void new_rows_load(const AttnArgs& a, const NewRows& nr, int kvh, int group, int rows, int wave,
                                     int lane, I2NewIn<D, QW>& in) {
    constexpr int NV = I2NewIn<D, QW>::NV;
    const Geom& g = a.g;
    if (wave < nr.n_new * 2 * (D / kBlock2)) {
        int j, t, b;
        const float* src = new_block_src<D>(nr, g.n_kv, kvh, wave, lane, j, t, b);
        in.x[0] = src[0];
        in.x[1] = src[1];
    }
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        const int r = min(wave + 8 * i, rows - 1), qi = r / group, h = kvh * group + r % group;
        load_row<NV>(a.q + ((size_t)qi * a.n_heads + h) * D + NV * lane, in.q[i]);
    }
    const int g0 = nr.pos0 >> 3, g1 = (nr.pos0 + nr.n_new - 1) >> 3;
    in.e[0] = a.page_table[(8 * g0) / g.P];
    in.e[1] = a.page_table[(8 * g1) / g.P];
}

// Requests the old V code dwords of the new rows' groups (after the page
// entries have arrived).  Dword u of a group, u = lane + 64 i: dims
// 32 (u / 16) + u % 16 and 32 (u / 16) + 16 + u % 16 of its 8 tokens.
template <int D, int QW>
__device__ inline void new_rows_load_old(const AttnArgs& a, const NewRows& nr, int kvh, int lane,
                                         I2NewIn<D, QW>& in) {
    const Geom& g = a.g;
    const int g0 = nr.pos0 >> 3, g1 = (nr.pos0 + nr.n_new - 1) >> 3;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int grp = t == 0 ? g0 : g1;
        const bool ok = in.e[t] >= 0 && in.e[t] < g.n_pages && (t == 0 || g1 != g0);
        const uint8_t* unit = a.pool + g.unit_index(ok ? in.e[t] : 0, kvh) * g.unit_bytes();
#pragma unroll
        for (int i = 0; i < I2NewIn<D, QW>::GW; ++i) {
            const int u = lane + 64 * i;
            int bit;
            const int64_t off = i2_v_dword(g, (8 * grp) % g.P, 32 * (u / 16) + u % 16, &bit);
            in.old[t][i] = ok ? *reinterpret_cast<const uint32_t*>(unit + off) : 0u;
        }
    }
}

// The end phase of the new rows (every wave of the workgroup; starts and
// ends at a workgroup barrier).  lds: I2NewLds<D>::BYTES of scratch no longer
// read by the stream.
template <int D, int W, int QW>
__device__ inline void new_rows_finish(const AttnArgs& a, const NewRows& nr, int kvh, int group, int rows,
                                       int n_splits, int part_stride, int wave, int lane, const I2NewIn<D, QW>& in,
                                       uint8_t* lds) {
#pragma clang fp contract(off)
    constexpr int NV = I2NewIn<D, QW>::NV;
    constexpr int NB2 = D / kBlock2;
    using NL = I2NewLds<D>;
    const Geom& g = a.g;
    const int g0 = nr.pos0 >> 3, g1 = (nr.pos0 + nr.n_new - 1) >> 3;
    auto entry = [&](int j) { return ((nr.pos0 + j) >> 3) == g0 ? in.e[0] : in.e[1]; };
    auto valid = [&](int e) { return e >= 0 && e < g.n_pages; };
    uint8_t* codes = lds + NL::CODES;                                // [t][j][D]
    float* xhat = reinterpret_cast<float*>(lds + NL::XHAT);          // [t][j][D]
    __syncthreads();                           // every wave has streamed its chunks: the scratch is free

    // 1. the blocks: quantize, (scale, zero) into the pool, codes and values to LDS
    const int n_items = nr.n_new * 2 * NB2;
    for (int it = wave; it < n_items; it += W) {
        int j, t, b;
        const float* src = new_block_src<D>(nr, g.n_kv, kvh, it, lane, j, t, b);
        const float x0 = it == wave ? in.x[0] : src[0];
        const float x1 = it == wave ? in.x[1] : src[1];
        const float mn = -wave_max(-fminf(x0, x1), lane);   // exact: negation and max
        const float mx = wave_max(fmaxf(x0, x1), lane);
        const Int2Par pr = int2_params(mn, mx);
        const int c0 = int2_code(x0, mn, pr.id), c1 = int2_code(x1, mn, pr.id);
        const uint16_t hs = f16_bits(pr.d), hz = f16_bits(mn);
        const float d = __half2float(__ushort_as_half(hs)), z = __half2float(__ushort_as_half(hz));
        const int dim = kBlock2 * b + 2 * lane;
        *reinterpret_cast<uint16_t*>(codes + (t * kI2NewRows + j) * D + dim) = (uint16_t)(c0 | (c1 << 8));
        // d c is exact: one rounding, as z + d c
        *reinterpret_cast<float2*>(xhat + (t * kI2NewRows + j) * D + dim) =
            float2{fmaf(d, (float)c0, z), fmaf(d, (float)c1, z)};
        const int e = entry(j), slot = (nr.pos0 + j) % g.P;
        if (lane == 0 && valid(e)) {
            uint8_t* unit = nr.pool + g.unit_index(e, kvh) * g.unit_bytes();
            if (t == 0) {
                uint16_t* kp = reinterpret_cast<uint16_t*>(unit + g.i2_k_params_off()) + ((size_t)slot * NB2 + b) * 2;
                kp[0] = hs;
                kp[1] = hz;
            } else {
                const size_t vi = ((size_t)(slot / kChunk) * NB2 + b) * kChunk + slot % kChunk;
                reinterpret_cast<uint16_t*>(unit + g.i2_v_scales_off())[vi] = hs;
                reinterpret_cast<uint16_t*>(unit + g.i2_v_zeros_off())[vi] = hz;
            }
        }
    }
    __syncthreads();                           // codes and values visible to every wave

    // 2a. wave w: query rows w and w + 8, each row's partial for every new key
    const float qscale = a.scale * kLog2e;
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        const int r = wave + 8 * i;
        if (r >= rows) break;                  // uniform
        const int qi = r / group, h = kvh * group + r % group;
        for (int j = 0; j < nr.n_new; ++j) {
            float kh[NV], vh[NV];
            load_row<NV>(xhat + j * D + NV * lane, kh);
            load_row<NV>(xhat + (kI2NewRows + j) * D + NV * lane, vh);
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < NV; ++e) dot = fmaf(in.q[i][e] * qscale, kh[e], dot);
            const float sc = wave_sum(dot, lane);
            const bool sees = qi >= j, ok = valid(entry(j));
            const size_t ps = ((size_t)qi * a.n_heads + h) * part_stride + n_splits + j;
            if (lane == 0) {
                a.ws_m[ps] = !sees ? -INFINITY : ok ? sc : NAN;
                a.ws_l[ps] = !sees ? 0.0f : ok ? 1.0f : NAN;
            }
            float* dst = a.ws_acc + ps * D + NV * lane;
#pragma unroll
            for (int e = 0; e < NV; ++e) dst[e] = sees ? vh[e] : 0.0f;
        }
    }
    // 2b. wave W - 1: the K code dwords (each token's own); lane l packs dword
    // w = l % (D/16) of row j: dims 32 (2 k + h) + 8 grp + e, h < 2, e < 8,
    // for grp = w / (D/64), k = w % (D/64)
    if (wave == W - 1) {
        constexpr int PER = D / 16;            // dwords per row
        for (int j = lane / PER; j < nr.n_new; j += 64 / PER) {
            const int e = entry(j);
            if (!valid(e)) continue;
            const int w = lane % PER, grp = w / (D / 64), k = w % (D / 64);
            uint32_t word = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t* src = reinterpret_cast<const uint32_t*>(codes + j * D + 32 * (2 * k + h) + 8 * grp);
                const uint32_t c0 = src[0], c1 = src[1];   // dims e = 0..3 and 4..7, one code per byte
#pragma unroll
                for (int ee = 0; ee < 4; ++ee) {
                    word |= ((c0 >> (8 * ee)) & 3u) << i2_bit(h, ee);
                    word |= ((c1 >> (8 * ee)) & 3u) << i2_bit(h, ee + 4);
                }
            }
            uint8_t* unit = nr.pool + g.unit_index(e, kvh) * g.unit_bytes();
            int bit;
            *reinterpret_cast<uint32_t*>(unit + i2_k_dword(g, (nr.pos0 + j) % g.P, 32 * (2 * k) + 8 * grp, &bit)) =
                word;
        }
    }
    // 2c. wave W - 2: the V code dwords of the new rows' groups, the new rows'
    // two codes in each, the other tokens' codes as they were
    if (wave == W - 2) {
        const uint8_t* vcodes = codes + kI2NewRows * D;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int grp = t == 0 ? g0 : g1;
            const bool ok = valid(in.e[t]) && (t == 0 || g1 != g0);
            if (!ok) continue;
            uint8_t* unit = nr.pool + g.unit_index(in.e[t], kvh) * g.unit_bytes();
            const int j_lo = max(8 * grp, nr.pos0) - nr.pos0;
            const int j_hi = min(8 * grp + 8, nr.pos0 + nr.n_new) - nr.pos0;
#pragma unroll
            for (int i = 0; i < I2NewIn<D, QW>::GW; ++i) {
                const int u = lane + 64 * i, n = u % 16, wi = u / 16;
                uint32_t keep = in.old[t][i], put = 0;
                for (int j = j_lo; j < j_hi; ++j) {
                    const int ee = (nr.pos0 + j) & 7;
                    const uint8_t* src = vcodes + j * D + 32 * wi + n;
                    put |= ((uint32_t)src[0] << i2_bit(0, ee)) | ((uint32_t)src[16] << i2_bit(1, ee));
                    keep &= ~((3u << i2_bit(0, ee)) | (3u << i2_bit(1, ee)));
                }
                int bit;
                *reinterpret_cast<uint32_t*>(unit + i2_v_dword(g, (8 * grp) % g.P, 32 * wi + n, &bit)) = keep | put;
            }
        }
    }
}

template <int D, int JJ, int W, int NSLOT>
struct I2Lds {
    using C = I2Cfg<D>;
    using S = I2Slot<D>;
    // per wave: a ring of NSLOT chunk slots
    static constexpr int RING = NSLOT * S::BYTES;
    // q per 32-dim step, MFMA A layout: up to 8 rows carry fp16 hi in MFMA
    // rows {0,1,4,5,..} and lo two rows further down (one operand); up to 16
    // rows a hi and a lo operand
    static constexpr int QSTEP = JJ == 2 ? 1024 : 2048;
    static constexpr int Q_OFF = W * RING;
    static constexpr int QS_OFF = Q_OFF + C::STEPS * QSTEP;    // sum of q per (row, block): [16][NB2] floats
    static constexpr int PB_OFF = QS_OFF + 16 * C::NB2 * 4;
    static constexpr int PBUF = 16 * kPStride * 4;              // per wave: P transpose buffer
    static constexpr int LOOP_BYTES = PB_OFF + W * PBUF;
    // end: every wave's rows [wave][4 jj + g4][D], then (m, l) per row and wave
    static constexpr int CB_BYTES = W * JJ * 4 * D * 4;
    static constexpr int ML_OFF = LOOP_BYTES > CB_BYTES ? LOOP_BYTES : CB_BYTES;
    static constexpr int BYTES = ML_OFF + JJ * 4 * W * 2 * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int D, int JJ, int W, int NSLOT, class Batch, bool NEWR>
__global__ __launch_bounds__(W * 64) void attn_int2_kernel(AttnArgs a, int n_splits, int group, int rows, Batch sb,
                                                           NewRows nr, int part_stride) {
    using C = I2Cfg<D>;
    using S = I2Slot<D>;
    using L = I2Lds<D, JJ, W, NSLOT>;
    extern __shared__ __align__(16) uint8_t smem[];
    const Geom& g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g4 = lane >> 4, n16 = lane & 15;
    int wg = blockIdx.x;
    if constexpr (!std::is_same_v<Batch, NoBatch>) {
        // batched decode: this workgroup serves sequence b, whose keys, page
        // table row, queries and partials start where the table says
        const int b = seq_of(sb.wg0, sb.n, wg);
        wg -= sb.wg0[b];
        n_splits = sb.n_splits[b];
        part_stride = n_splits;
        a.ctx = sb.ctx[b];
        a.page_table += (size_t)b * sb.n_table;
        a.q += (size_t)b * a.n_q * a.n_heads * D;
        a.ws_m += sb.part0[b];
        a.ws_l += sb.part0[b];
        a.ws_acc += (size_t)sb.part0[b] * D;
    }
    const int split = wg % n_splits, kvh = wg / n_splits;
    const int c1 = (a.ctx + kChunk - 1) / kChunk;
    const int first_last = a.causal ? a.ctx - a.n_q : a.ctx - 1;   // last key of query 0
    const int mask_group = a.causal ? group : 0x7fffffff;
    // wave w of split s takes chunks s W + w, then every stride-th
    const int stride = n_splits * W, c0 = split * W + wave;
    // page-table entries of the wave's chunks kb .. kb+63, one per lane
    auto load_ents = [&](int kb) -> int {
        const int ck = c0 + (kb + lane) * stride;
        return ck < c1 ? a.page_table[(ck * kChunk) / g.P] : -1;
    };
    // fused decode step: this wave appends the new rows (after its chunks);
    // their inputs are requested now
    static_assert(!NEWR || W == 8, "new rows: eight waves, each with query rows w and w + 8");
    const bool helper = NEWR && split == n_splits - 1;   // uniform over the workgroup
    constexpr int QW = JJ == 4 ? 2 : 1;        // query rows per wave: up to 8 or up to 16 in all
    I2NewIn<D, QW> nin;
    if constexpr (NEWR) {
        if (helper) new_rows_load<D, W, QW>(a, nr, kvh, group, rows, wave, lane, nin);
    }
    int ents = load_ents(0);

    // ---- q: A operands and per-block sums in LDS.  Thread (r, b, i) takes
    // dims 128 b + 8 i .. +7 of row r, pre-scaled by scale * log2(e), in the
    // codes' element order (d0, d2, d1, d3, ...), split into fp16 hi + lo; the
    // 16 threads of (r, b) sum the block.
    const float qscale = a.scale * kLog2e;
    float* qsum = reinterpret_cast<float*>(smem + L::QS_OFF);
    {
        const int t = threadIdx.x, i = t & 15, r = (t >> 4) & 15, b = t >> 8;
        constexpr int NROW = JJ == 2 ? 8 : 16;
        static_assert(W * 64 >= 16 * 16 * C::NB2, "one thread per (row, block, 8 dims)");
        if (b < C::NB2 && r < NROW) {           // uniform per 16 lanes
            const bool ok = r < rows;
            const int qi = ok ? r / group : 0, h = kvh * group + (ok ? r % group : 0);
            // rows past the end read row 0 (a valid address), so the loads
            // are unconditional: all in flight at once, no wait per element
            const float* src = a.q + ((size_t)qi * a.n_heads + h) * D + kBlock2 * b + 8 * i;
            const floatx4 x0 = *reinterpret_cast<const floatx4*>(src);
            const floatx4 x1 = *reinterpret_cast<const floatx4*>(src + 4);
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = ok ? x0[e] * qscale : 0.0f;
                x[e + 4] = ok ? x1[e] * qscale : 0.0f;
            }
            half8 hi, lo;
            float sum = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = x[code_slot(e)];
                hi[e] = (_Float16)v;
                lo[e] = (_Float16)(v - (float)hi[e]);
                sum += v;
            }
            const int step = 4 * b + i / 4, gq = i % 4;
            uint8_t* qd = smem + L::Q_OFF + step * L::QSTEP;
            if constexpr (JJ == 2) {
                const int n = 4 * (r / 2) + r % 2;     // MFMA row of row r (logical_row<2> inverse)
                *reinterpret_cast<half8*>(qd + (gq * 16 + n) * 16) = hi;
                *reinterpret_cast<half8*>(qd + (gq * 16 + n + 2) * 16) = lo;
            } else {
                *reinterpret_cast<half8*>(qd + (gq * 16 + r) * 16) = hi;
                *reinterpret_cast<half8*>(qd + 1024 + (gq * 16 + r) * 16) = lo;
            }
            sum = row16_sum(sum);
            if (i == 0) qsum[r * C::NB2 + b] = sum;
        }
    }
    __syncthreads();
    float qs[C::NB2][JJ];
#pragma unroll
    for (int b = 0; b < C::NB2; ++b)
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) qs[b][jj] = qsum[logical_row<JJ>(0, 4 * g4 + jj) * C::NB2 + b];
    // up to 8 rows the q operands stay in registers (one per 32-dim step):
    // an LDS read before each step's products would put its latency on the
    // path of every chunk
    half8 qreg[JJ == 2 ? C::STEPS : 1];
    if constexpr (JJ == 2) {
#pragma unroll
        for (int st = 0; st < C::STEPS; ++st)
            qreg[st] = *reinterpret_cast<const half8*>(smem + L::Q_OFF + st * L::QSTEP + lane * 16);
    }

    float* plds = reinterpret_cast<float*>(smem + L::PB_OFF + wave * L::PBUF);
    floatx4 o[C::NT];
    floatx4 corr = {0.f, 0.f, 0.f, 0.f};     // sum p z: column b = V block b
    float m[4], l[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) { m[jj] = -INFINITY; l[jj] = 0.0f; }
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) o[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // chunks wholly visible to every row come first
    const int c_mask = first_last >= kChunk - 1 ? (first_last - (kChunk - 1)) / kChunk + 1 : 0;

    // One chunk: S = q K^T, online softmax, O += P' V, corr += p z.
    // MASK: some key of the chunk lies past the last key of some row.
    auto process = [&](const uint8_t* sl, int c, auto mask_tag) {
        constexpr bool mask = decltype(mask_tag)::value;
        const int j0 = c * kChunk;
        // K codes of the lane's token in each tile, and its (scale, zero) pairs
        u32x4 kcode[2];
        u32x2 kpar[2];
        read_k<D>(sl, lane, n16, kcode, kpar);
        floatx4 s[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int b = 0; b < C::NB2; ++b) {
            floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int step = 4 * b + st;
                const uint8_t* qp = smem + L::Q_OFF + step * L::QSTEP + lane * 16;
                half8 qa;
                if constexpr (JJ == 2) qa = qreg[step];
                else qa = *reinterpret_cast<const half8*>(qp);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const half8 kb = (step & 1) ? i2_word<1, 1>(kcode[tt][step / 2]) : i2_word<0, 1>(kcode[tt][step / 2]);
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa, kb, acc[tt], 0, 0, 0);
                    if constexpr (JJ == 4) {
                        const half8 ql = *reinterpret_cast<const half8*>(qp + 1024);
                        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, kb, acc[tt], 0, 0, 0);
                    }
                }
                SCHED_FENCE();
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const half2v dz = as_h2(kpar[tt][b]);
                const float d = (float)dz.x, z = (float)dz.y;
#pragma unroll
                for (int jj = 0; jj < JJ; ++jj) {
                    const float qc = JJ == 2 ? acc[tt][jj] + acc[tt][jj + 2] : acc[tt][jj];
                    s[tt][jj] = fmaf(z, qs[b][jj], fmaf(d, qc, s[tt][jj]));
                }
            }
            SCHED_FENCE();
        }
        // causal / tail mask: key j visible to row r iff j <= first_last + r / group
        if constexpr (mask) {
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) {
                const int row = logical_row<JJ>(0, 4 * g4 + jj);
                const int last = row >= 0 && row < rows ? first_last + row / mask_group : -1;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    if (j0 + tt * kTile + n16 > last) s[tt][jj] = -INFINITY;
            }
        }
        // online softmax (lazy rescaling by kTau; weights 2^(s - m - kTau) <= 1)
        // The row maxima only when some score of the wave passes its row's
        // reference by more than kTau: a row's maximum does iff one of its
        // scores does, so the test needs no cross-lane step.
        float smax[4];
        bool grow = false;
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            smax[jj] = max2(s[0][jj], s[1][jj]);
            grow |= smax[jj] > m[jj] + kTau;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            // rows whose maximum did not move get alpha = 1: one straight pass
            // over the accumulators, no per-row branches
            floatx4 alpha = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) {
                const float mnew = row16_max(smax[jj]);
                const bool up = mnew > m[jj];
                alpha[jj] = up ? fast_exp2(m[jj] - mnew) : 1.0f;
                l[jj] *= alpha[jj];
                m[jj] = up ? mnew : m[jj];
            }
            if constexpr (JJ == 2) {             // the lo rows follow their rows
                alpha[2] = alpha[0];
                alpha[3] = alpha[1];
            }
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) o[nt] *= alpha;
            corr *= alpha;
        }
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            const float mref = (m[jj] == -INFINITY ? 0.0f : m[jj]) + kTau;
            const float p0 = fast_exp2(s[0][jj] - mref);
            const float p1 = fast_exp2(s[1][jj] - mref);
            l[jj] += p0 + p1;
            float* prow = plds + (4 * g4 + jj) * kPStride;
            prow[n16] = p0;
            prow[kTile + n16] = p1;
        }
        lds_fence();
        // P in the A layout: row n16, tokens 8 g4 .. 8 g4 + 7.  The weights
        // enter the products as fp16 hi + lo: v = z + d c splits into terms
        // larger than v itself (large zero-points after a rotation), so one
        // fp16 rounding of the weights would cost too much.  Up to 8 rows
        // (JJ = 2) the lo halves sit in the spare MFMA rows 4 g + {2, 3} (the
        // rows' own lanes read row n16 - 2 and keep what fp16 missed); up to
        // 16 rows a second MFMA takes them.
        constexpr bool LO_ROWS = JJ == 2;
        const bool lo_lane = LO_ROWS && (n16 & 2) != 0;
        const int prow = LO_ROWS ? (n16 & ~2) : n16;
        float pf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = plds[prow * kPStride + 8 * g4 + e];
        // fp16 of x, or in a lo lane the part of x below it: x - s h with s =
        // 0 or 1 (one mixed-precision FMA; x - 0 h is x itself, x <= 65504)
        const float s_lo = lo_lane ? 1.0f : 0.0f;
        auto part = [&](float x) -> _Float16 { return (_Float16)fmaf(-s_lo, (float)(_Float16)x, x); };
        auto rest = [](float x) -> _Float16 { return (_Float16)fmaf(-1.0f, (float)(_Float16)x, x); };
        // zero-point term: p times the zero-points (keys past the context may
        // hold unwritten zero-points: they get 0)
        u32x4 vcode[2], vzr, vsr[2];
        read_v<D>(sl, lane, n16, g4, vcode, vzr, vsr);
        half8 az, bz = __builtin_bit_cast(half8, vzr);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            az[e] = part(pf[e]);
            if (mask && j0 + 8 * g4 + e >= a.ctx) bz[e] = (_Float16)0.0f;
        }
        corr = __builtin_amdgcn_mfma_f32_16x16x32_f16(az, bz, corr, 0, 0, 0);
        if constexpr (!LO_ROWS) {
            half8 azl;
#pragma unroll
            for (int e = 0; e < 8; ++e) azl[e] = rest(pf[e]);
            corr = __builtin_amdgcn_mfma_f32_16x16x32_f16(azl, bz, corr, 0, 0, 0);
        }
#pragma unroll
        for (int b = 0; b < C::NB2; ++b) {
            // P' = p * d_v in the codes' token order, one fp32 product, then
            // fp16 hi + lo
            const half8 sc = __builtin_bit_cast(half8, vsr[b]);
            half8 ap, apl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = code_slot(e);
                float x = fmaf(pf[t], (float)sc[t], 0.0f);
                if constexpr (mask) x = pf[t] == 0.0f ? 0.0f : x;   // masked keys may hold unwritten scales
                ap[e] = part(x);
                if constexpr (!LO_ROWS) apl[e] = rest(x);
            }
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int nt = 8 * b + w;
                // codes carry 2^kTau = 16 (the weights carry 2^-kTau)
                const half8 bv = (nt & 1) ? i2_word<1, 16>(vcode[nt / 8][(nt / 2) % 4])
                                          : i2_word<0, 16>(vcode[nt / 8][(nt / 2) % 4]);
                o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, bv, o[nt], 0, 0, 0);
                if constexpr (!LO_ROWS) o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(apl, bv, o[nt], 0, 0, 0);
                if (w & 1) SCHED_FENCE();       // a few B operands live at a time
            }
            SCHED_FENCE();
        }
    };

    // ---- stream.  Chunk i of the wave (global chunk c0 + i stride) lands in
    // ring slot i % NSLOT; computing chunk i first requests chunk
    // i + NSLOT - 1 into the slot chunk i - 1 used.  A page-table entry
    // outside the pool stops the requests there; the wave stops when it gets
    // to that chunk and its partial turns into NaN.
    uint8_t* const ring = smem + wave * L::RING;
    const int n_mine = c0 < c1 ? (c1 - 1 - c0) / stride + 1 : 0;   // chunks of this wave
    // the parameter request: lane l carries K (scale, zero) pairs, V scales
    // or V zeros, 16 bytes at pbase + slot0 * pmul of the unit
    int pbase, pmul;
    {
        const int pl = lane % S::PLANES;
        if (pl < 8 * C::NB2) {
            pbase = (int)g.i2_k_params_off() + 16 * pl;
            pmul = 4 * C::NB2;
        } else if (pl < 12 * C::NB2) {
            pbase = (int)g.i2_v_scales_off() + 16 * (pl - 8 * C::NB2);
            pmul = 2 * C::NB2;
        } else {
            pbase = (int)g.i2_v_zeros_off() + 16 * (pl - 12 * C::NB2);
            pmul = 2 * C::NB2;
        }
    }
    int n_req = 0;         // chunks requested so far
    int stop = n_mine;     // first chunk not requested (a bad page), else n_mine
    auto request = [&]() {
        if (n_req >= stop) return;
        if ((n_req & 63) == 0 && n_req > 0) {
            // the next 64 entries; a load that waits for itself (and for the
            // requests in flight), so no pending register outlives the branch
            const int ck = c0 + (n_req + lane) * stride;
            const int32_t* pe = a.page_table + (ck < c1 ? (ck * kChunk) / g.P : 0);
            int v;
            asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(pe) : "memory");
            ents = ck < c1 ? v : -1;
        }
        const int phys = __builtin_amdgcn_readlane(ents, n_req & 63);
        if (phys < 0 || phys >= g.n_pages) { stop = n_req; return; }
        const uint8_t* unit = a.pool + g.unit_index(phys, kvh) * g.unit_bytes();
        const uint32_t s0 = (uint32_t)(((c0 + n_req * stride) * kChunk) % g.P);
        uint8_t* sl = ring + (n_req % NSLOT) * S::BYTES;
        const uint8_t* kc = unit + s0 * (D / 4) + lane * 16;
        const uint8_t* vc = unit + g.i2_v_codes_off() + s0 * (D / 4) + lane * 16;
#pragma unroll
        for (int i = 0; i < S::CODE_REQS; ++i) dma16<kLoadNT>(kc + i * 1024, sl + S::K_OFF + i * 1024);
#pragma unroll
        for (int i = 0; i < S::CODE_REQS; ++i) dma16<kLoadNT>(vc + i * 1024, sl + S::V_OFF + i * 1024);
        dma16<kLoadNT>(unit + pbase + s0 * pmul, sl + S::P_OFF);
        ++n_req;
    };
    // the page entries are in by now, but their waits sat in the q staging's
    // branch: use them here, so that no wait before the first chunk request
    // (the first readlane) also waits for loads issued after this point
    asm volatile("" : "+v"(ents));
    if constexpr (NEWR) {
        // older than every chunk request, so the chunk waits count as before
        if (helper && wave == W - 2) new_rows_load_old<D, QW>(a, nr, kvh, lane, nin);
    }
#pragma unroll
    for (int i = 0; i + 1 < NSLOT; ++i) request();

    bool bad = false;
    int ci = 0;            // the wave's chunk being computed
    auto step = [&](auto mask_tag) {
        request();         // chunk ci + NSLOT - 1, into the slot chunk ci - 1 has left
        wait_chunks<S::REQS, NSLOT - 1>(n_req - ci - 1);   // chunk ci has landed
        process(ring + (ci % NSLOT) * S::BYTES, c0 + ci * stride, mask_tag);
        lds_fence();       // the slot is read out before it is requested again
        ++ci;
    };
    const int n_full = c0 < c_mask ? min((c_mask - 1 - c0) / stride + 1, n_mine) : 0;
    while (ci < n_full && ci < stop) step(std::false_type{});
    while (ci < n_mine && ci < stop) step(std::true_type{});
    bad = ci < n_mine;
    vm_wait<0>();          // nothing in flight into LDS past this point
    if constexpr (NEWR) {
        static_assert(!NEWR || L::CB_BYTES + I2NewLds<D>::BYTES <= L::LOOP_BYTES, "end-phase scratch");
        // (scratch past the combine's buffer: rings, q and P buffers, dead by now)
        if (helper)
            new_rows_finish<D, W, QW>(a, nr, kvh, group, rows, n_splits, part_stride, wave, lane, nin,
                                  smem + L::CB_BYTES);
    }

    // ---- finish: row sums, the zero-point term into o, then the W waves'
    // partials combined in wave order into one per workgroup
#pragma unroll
    for (int jj = 0; jj < JJ; ++jj) {
        l[jj] = row16_sum(l[jj]) * 16.0f;               // weights carried 2^-kTau
        if (bad) { m[jj] = NAN; l[jj] = NAN; }
    }
    if constexpr (JJ == 2) {
        // fold the lo rows into their rows
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
            o[nt][0] += o[nt][2];
            o[nt][1] += o[nt][3];
        }
        corr[0] += corr[2];
        corr[1] += corr[3];
    }
    {
        // the weights carry 2^-kTau (o has it made up by the codes); corr
        // column b (lane 16 g4 + b) times 2^kTau goes to the dims of block b
        float cz[C::NB2][JJ];
#pragma unroll
        for (int b = 0; b < C::NB2; ++b)
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) cz[b][jj] = 16.0f * __shfl(corr[jj], 16 * g4 + b);
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) o[nt][jj] += cz[nt / 8][jj];
    }
    __syncthreads();                                    // q and P buffers no longer read
    constexpr int SLOTW = JJ * 4 * D;                   // floats per wave
    float* cb = reinterpret_cast<float*>(smem);
    float* mls = reinterpret_cast<float*>(smem + L::ML_OFF);
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) cb[wave * SLOTW + (4 * jj + g4) * D + 16 * nt + n16] = o[nt][jj];
    if (n16 == 0) {
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            float* d = mls + ((4 * jj + g4) * W + wave) * 2;
            d[0] = m[jj];
            d[1] = l[jj];
        }
    }
    __syncthreads();
    for (int unit = threadIdx.x; unit < JJ * 4 * (D / 4); unit += W * 64) {
        const int slot = unit / (D / 4), dim = 4 * (unit % (D / 4));
        const int jj = slot / 4, gg = slot % 4;
        const int row = logical_row<JJ>(0, 4 * gg + jj);
        if (row < 0 || row >= rows) continue;
        float mw[W], lw[W];
#pragma unroll
        for (int w = 0; w < W; ++w) {
            mw[w] = mls[(slot * W + w) * 2];
            lw[w] = mls[(slot * W + w) * 2 + 1];
        }
        float mm = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) mm = fmaxf(mm, mw[w]);
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        float lt = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            // NaN (a bad page) propagates; a wave without keys (l = 0) adds nothing
            const float f = lw[w] == 0.0f ? 0.0f : fast_exp2(mw[w] - mm);
            lt += lw[w] * f;
            acc += f * *reinterpret_cast<const floatx4*>(cb + w * SLOTW + slot * D + dim);
        }
        const size_t ps = ((size_t)(row / group) * a.n_heads + kvh * group + row % group) * part_stride + split;
        *reinterpret_cast<floatx4*>(a.ws_acc + ps * D + dim) = acc;
        if (dim == 0) {
            a.ws_m[ps] = mm;
            a.ws_l[ps] = lt;
        }
    }
}

constexpr int kInt2Waves = 8;   // two per SIMD, one workgroup per CU
constexpr int kInt2Slots = 3;   // chunks in a wave's ring: two in flight while one is computed

template <int D, int JJ, bool NEWR, class Batch>
hipError_t launch_dj(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg,
                     const NewRows& nr, int part_stride) {
    constexpr int W = kInt2Waves, NS = kInt2Slots;
    using L = I2Lds<D, JJ, W, NS>;
    if (L::BYTES > 64 * 1024) {
        hipError_t e = allow_lds<attn_int2_kernel<D, JJ, W, NS, Batch, NEWR>>(L::BYTES);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((attn_int2_kernel<D, JJ, W, NS, Batch, NEWR>), dim3(n_wg), dim3(W * 64), L::BYTES, stream,
                       a, pl.n_splits, pl.group, pl.rows, sb, nr, part_stride);
    return hipGetLastError();
}

template <int D, bool NEWR, class Batch>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg,
                    const NewRows& nr, int part_stride) {
    if (pl.rows <= 8) return launch_dj<D, 2, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
    if (pl.rows <= 16) return launch_dj<D, 4, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
    return hipErrorInvalidValue;
}

template <bool NEWR, class Batch>
hipError_t launch_any(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg,
                      const NewRows& nr, int part_stride) {
    switch (a.g.D) {
        case 128: return launch_d<128, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
        case 256: return launch_d<256, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int int2_waves() { return kInt2Waves; }
int int2_max_new_rows() { return kI2NewRows; }

hipError_t launch_attn_int2(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const SeqBatch* batch) {
    const NewRows none{nullptr, nullptr, nullptr, 0, 0};
    if (batch != nullptr && batch->n > 0)
        return launch_any<false>(a, pl, stream, *batch, batch->wg0[batch->n], none, 0);
    return launch_any<false>(a, pl, stream, NoBatch{}, pl.n_splits * a.g.n_kv, none, pl.n_splits);
}

hipError_t launch_attn_int2_new(const AttnArgs& a, const AttnPlan& pl, const NewRows& nr, hipStream_t stream) {
    if (nr.n_new < 1 || nr.n_new > kI2NewRows || pl.rows > 16 || pl.n_splits < 1) return hipErrorInvalidValue;
    return launch_any<true>(a, pl, stream, NoBatch{}, pl.n_splits * a.g.n_kv, nr, pl.n_splits + nr.n_new);
}

}  // namespace kvq
