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

template <int D, int JJ, int W, int NSLOT, class Batch>
__global__ __launch_bounds__(W * 64) void attn_int2_kernel(AttnArgs a, int n_splits, int group, int rows, Batch sb) {
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
            const float* src = a.q + ((size_t)qi * a.n_heads + h) * D + kBlock2 * b + 8 * i;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = ok ? src[e] * qscale : 0.0f;
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
        const size_t ps = ((size_t)(row / group) * a.n_heads + kvh * group + row % group) * n_splits + split;
        *reinterpret_cast<floatx4*>(a.ws_acc + ps * D + dim) = acc;
        if (dim == 0) {
            a.ws_m[ps] = mm;
            a.ws_l[ps] = lt;
        }
    }
}

constexpr int kInt2Waves = 8;   // two per SIMD, one workgroup per CU
constexpr int kInt2Slots = 3;   // chunks in a wave's ring: two in flight while one is computed

template <int D, int JJ, class Batch>
hipError_t launch_dj(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg) {
    constexpr int W = kInt2Waves, NS = kInt2Slots;
    using L = I2Lds<D, JJ, W, NS>;
    if (L::BYTES > 64 * 1024) {
        hipError_t e = allow_lds<attn_int2_kernel<D, JJ, W, NS, Batch>>(L::BYTES);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((attn_int2_kernel<D, JJ, W, NS, Batch>), dim3(n_wg), dim3(W * 64), L::BYTES, stream, a,
                       pl.n_splits, pl.group, pl.rows, sb);
    return hipGetLastError();
}

template <int D, class Batch>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg) {
    if (pl.rows <= 8) return launch_dj<D, 2>(a, pl, stream, sb, n_wg);
    if (pl.rows <= 16) return launch_dj<D, 4>(a, pl, stream, sb, n_wg);
    return hipErrorInvalidValue;
}

template <class Batch>
hipError_t launch_any(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg) {
    switch (a.g.D) {
        case 128: return launch_d<128>(a, pl, stream, sb, n_wg);
        case 256: return launch_d<256>(a, pl, stream, sb, n_wg);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int int2_waves() { return kInt2Waves; }

hipError_t launch_attn_int2(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const SeqBatch* batch) {
    if (batch != nullptr && batch->n > 0) return launch_any(a, pl, stream, *batch, batch->wg0[batch->n]);
    return launch_any(a, pl, stream, NoBatch{}, pl.n_splits * a.g.n_kv);
}

}  // namespace kvq
