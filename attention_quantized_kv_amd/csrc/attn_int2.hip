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
// q_b . c_b is an MFMA over exact fp16 codes (q split into fp16 hi + lo, so
// every product is exact in fp32); sum(q_b) is a per-row constant.  On the V
// side P' = p d (fp32, rounded once to fp16) multiplies the codes, and the
// zero-point term is one more MFMA per chunk, fp16(p) times the chunk's V
// zero-points, whose output column b is the row's term for block b.
//
// Work split as in the Q8_0/Q4_0 streaming kernel: a workgroup of W waves per
// (KV head, split), the split's 32-token chunks dealt round-robin to its
// waves, every query row of the KV head served from one read of each byte.
// Per chunk a lane loads its share straight into registers (two chunk
// buffers: chunk c+1 is requested before chunk c is computed):
//   K codes  2 tiles x D/16 bytes   V codes  D/8 bytes
//   K (scale, zero) of its token, per tile: 4 bytes per block
//   V scales of its 8 tokens (MFMA A layout), 16 bytes per block
//   V zero-points of its 8 tokens for block n16 % NB2: 16 bytes
// Each code load is one contiguous 1 KiB (D = 256) wave request thanks to
// the pool layout.
#include <hip/hip_fp16.h>

#include "kvq_internal.h"
#include "kvq_mfma.h"

namespace kvq {
namespace {

template <int D>
struct I2Cfg {
    static constexpr int NB2 = D / kBlock2;   // 128-value blocks per row
    static constexpr int STEPS = D / 32;      // 32-dim MFMA steps of q . k
    static constexpr int KD = D / 64;         // K code dwords per lane and 16-token tile
    static constexpr int VD = D / 32;         // V code dwords per lane and 32-token chunk
    static constexpr int NT = D / 16;         // 16-dim output tiles
};

// One chunk's loads of one lane.
template <int D>
struct I2Chunk {
    uint32_t k[2][I2Cfg<D>::KD];
    uint32_t v[I2Cfg<D>::VD];
    uint32_t kp[2][I2Cfg<D>::NB2];   // (scale, zero) fp16 pair per block, token n16 of each tile
    u32x4 vs[I2Cfg<D>::NB2];         // V scales of tokens 8 g4 .. 8 g4 + 7, per block
    u32x4 vz;                        // V zero-points of the same tokens, block n16 % NB2
};

template <int N>
__device__ inline void load_dwords(uint32_t (&d)[N], const uint8_t* p) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const u32x4 x = reinterpret_cast<const u32x4*>(p)[i];
            d[4 * i] = x.x;
            d[4 * i + 1] = x.y;
            d[4 * i + 2] = x.z;
            d[4 * i + 3] = x.w;
        }
    } else if constexpr (N == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        d[0] = x.x;
        d[1] = x.y;
    } else {
        static_assert(N == 1, "1, 2 or a multiple of 4 dwords");
        d[0] = *reinterpret_cast<const uint32_t*>(p);
    }
}

// Requests chunk slot0 .. slot0 + 31 of a unit (slot0 a multiple of 32).
template <int D>
__device__ inline void load_chunk(I2Chunk<D>& r, const uint8_t* unit, const Geom& g, int slot0, int lane) {
    using C = I2Cfg<D>;
    const int g4 = lane >> 4, n16 = lane & 15;
    const uint32_t s0 = (uint32_t)slot0;
    // K tile t covers tokens 16t .. 16t+15 in 16 * D/4 bytes, lane l at l * D/16
    const uint8_t* kc = unit + s0 * (D / 4) + lane * (D / 16);
    load_dwords(r.k[0], kc);
    load_dwords(r.k[1], kc + kTile * (D / 4));
    // V chunk c covers tokens 32c .. 32c+31 in 32 * D/4 bytes, lane l at l * D/8
    load_dwords(r.v, unit + g.i2_v_codes_off() + s0 * (D / 4) + lane * (D / 8));
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
        load_dwords(r.kp[tt], unit + g.i2_k_params_off() + (s0 + kTile * tt + n16) * (C::NB2 * 4));
    const uint8_t* vsb = unit + g.i2_v_scales_off() + (s0 / kChunk) * (C::NB2 * kChunk * 2) + 16 * g4;
#pragma unroll
    for (int b = 0; b < C::NB2; ++b) r.vs[b] = *reinterpret_cast<const u32x4*>(vsb + b * (kChunk * 2));
    r.vz = *reinterpret_cast<const u32x4*>(unit + g.i2_v_zeros_off() + (s0 / kChunk) * (C::NB2 * kChunk * 2) +
                                           (n16 % C::NB2) * (kChunk * 2) + 16 * g4);
}

// The 8 codes of word H (0: low, 1: high byte of each half) of dword x as
// fp16 MUL * code, exactly, in the order (c0, c4, c1, c5, c2, c6, c3, c7).
// Code j sits at bits 2j (and code 4+j at bits 16+2j): masked in place under
// the fp16 exponent of 2^(10-2j), whose mantissa step is then 1, it reads
// 2^(10-2j) + code; one FMA per pair removes the offset.  The offsets live in
// registers (magic), so each pair costs one v_and_or_b32 and one
// v_pk_fma_f16.
template <int H, int MUL>
__device__ inline half8 i2_word_to_half(uint32_t x, const uint32_t (&magic)[4]) {
    const uint32_t y = H ? x >> 8 : x;
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (y & (0x00030003u << (2 * j))) | magic[j];
    const half8 h = __builtin_bit_cast(half8, w);
    const _Float16 m = (_Float16)MUL;
    const _Float16 a0 = (_Float16)(-1024.0f * MUL), a1 = (_Float16)(-256.0f * MUL);
    const _Float16 a2 = (_Float16)(-64.0f * MUL), a3 = (_Float16)(-16.0f * MUL);
    const half8 add = {a0, a0, a1, a1, a2, a2, a3, a3};
    return h * half8{m, m, m, m, m, m, m, m} + add;
}

template <int D, int JJ, int W>
struct I2Lds {
    using C = I2Cfg<D>;
    // q per 32-dim step, MFMA A layout: up to 8 rows carry fp16 hi in MFMA
    // rows {0,1,4,5,..} and lo two rows further down (one operand); up to 16
    // rows a hi and a lo operand
    static constexpr int QSTEP = JJ == 2 ? 1024 : 2048;
    static constexpr int QS_OFF = C::STEPS * QSTEP;            // sum of q per (row, block): [16][NB2] floats
    static constexpr int PB_OFF = QS_OFF + 16 * C::NB2 * 4;
    static constexpr int PBUF = 16 * kPStride * 4;              // per wave: P transpose buffer
    static constexpr int LOOP_BYTES = PB_OFF + W * PBUF;
    // end: every wave's rows [wave][4 jj + g4][D], then (m, l) per row and wave
    static constexpr int CB_BYTES = W * JJ * 4 * D * 4;
    static constexpr int ML_OFF = LOOP_BYTES > CB_BYTES ? LOOP_BYTES : CB_BYTES;
    static constexpr int BYTES = ML_OFF + JJ * 4 * W * 2 * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int D, int JJ, int W>
__global__ __launch_bounds__(W * 64) void attn_int2_kernel(AttnArgs a, int n_splits, int group, int rows) {
    using C = I2Cfg<D>;
    using L = I2Lds<D, JJ, W>;
    extern __shared__ __align__(16) uint8_t smem[];
    const Geom& g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g4 = lane >> 4, n16 = lane & 15;
    const int split = blockIdx.x % n_splits, kvh = blockIdx.x / n_splits;
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
    // dims 128 b + 8 i .. +7 of row r, pre-scaled by scale * log2(e), split
    // into fp16 hi + lo, stored in the codes' element order (d0, d4, d1, d5,
    // ...); the 16 threads of (r, b) sum hi + lo over the block.
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
                const float v = x[(e & 1) ? 4 + e / 2 : e / 2];
                hi[e] = (_Float16)v;
                lo[e] = (_Float16)(v - (float)hi[e]);
                sum += (float)hi[e] + (float)lo[e];
            }
            const int step = 4 * b + i / 4, gq = i % 4;
            uint8_t* qd = smem + step * L::QSTEP;
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

    float* plds = reinterpret_cast<float*>(smem + L::PB_OFF + wave * L::PBUF);
    floatx4 o[C::NT];
    floatx4 corr = {0.f, 0.f, 0.f, 0.f};     // sum p z: column b = V block b
    float m[4], l[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) { m[jj] = -INFINITY; l[jj] = 0.0f; }
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) o[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    uint32_t magic[4] = {0x64006400u, 0x5C005C00u, 0x54005400u, 0x4C004C00u};   // fp16 2^10, 2^8, 2^6, 2^4
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(magic[j]));              // keep them in VGPRs

    // chunks wholly visible to every row come first
    const int c_mask = first_last >= kChunk - 1 ? (first_last - (kChunk - 1)) / kChunk + 1 : 0;

    // One chunk: S = q K^T, online softmax, O += P' V, corr += p z.
    auto process = [&](const I2Chunk<D>& cur, int c) {
        const int j0 = c * kChunk;
        const bool mask = c >= c_mask;
        floatx4 s[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int b = 0; b < C::NB2; ++b) {
            floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int step = 4 * b + st;
                const uint8_t* qp = smem + step * L::QSTEP + lane * 16;
                const half8 qa = *reinterpret_cast<const half8*>(qp);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const half8 kb = (step & 1) ? i2_word_to_half<1, 1>(cur.k[tt][step / 2], magic)
                                                : i2_word_to_half<0, 1>(cur.k[tt][step / 2], magic);
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa, kb, acc[tt], 0, 0, 0);
                    if constexpr (JJ == 4) {
                        const half8 ql = *reinterpret_cast<const half8*>(qp + 1024);
                        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, kb, acc[tt], 0, 0, 0);
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const half2v dz = as_h2(cur.kp[tt][b]);
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
        if (mask) {
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
        float mnew[4];
        bool grow = false;
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            mnew[jj] = row16_max(fmaxf(s[0][jj], s[1][jj]));
            grow |= mnew[jj] > m[jj] + kTau;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            floatx4 alpha = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) {
                const bool up = mnew[jj] > m[jj];
                alpha[jj] = up ? fast_exp2(m[jj] - mnew[jj]) : 1.0f;
                l[jj] *= alpha[jj];
                m[jj] = up ? mnew[jj] : m[jj];
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
        // P in the A layout: row n16, tokens 8 g4 .. 8 g4 + 7
        float pf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = plds[n16 * kPStride + 8 * g4 + e];
        // zero-point term: fp16(p) times the zero-points (keys past the
        // context may hold unwritten zero-points: they get 0)
        half8 az, bz = __builtin_bit_cast(half8, cur.vz);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            az[e] = (_Float16)pf[e];
            if (mask && j0 + 8 * g4 + e >= a.ctx) bz[e] = (_Float16)0.0f;
        }
        corr = __builtin_amdgcn_mfma_f32_16x16x32_f16(az, bz, corr, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < C::NB2; ++b) {
            // P' = p * d_v, rounded once to fp16, in the codes' token order
            const half8 sc = __builtin_bit_cast(half8, cur.vs[b]);
            half8 ap;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x0 = pf[j] * (float)sc[j];
                float x1 = pf[4 + j] * (float)sc[4 + j];
                if (mask) {                      // masked keys may hold unwritten scales
                    x0 = pf[j] == 0.0f ? 0.0f : x0;
                    x1 = pf[4 + j] == 0.0f ? 0.0f : x1;
                }
                ap[2 * j] = (_Float16)x0;
                ap[2 * j + 1] = (_Float16)x1;
            }
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int nt = 8 * b + w;
                // codes carry 2^kTau = 16 (the weights carry 2^-kTau)
                const half8 bv = (nt & 1) ? i2_word_to_half<1, 16>(cur.v[nt / 2], magic)
                                          : i2_word_to_half<0, 16>(cur.v[nt / 2], magic);
                o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, bv, o[nt], 0, 0, 0);
            }
            SCHED_FENCE();
        }
    };

    // ---- stream, two chunk buffers.  A page-table entry outside the pool
    // stops the wave (nothing is loaded from it) and turns its partial into NaN.
    I2Chunk<D> buf0, buf1;
    bool bad = false;
    int c = c0, k = 0;
    auto request = [&](I2Chunk<D>& r, int kk, int cc) {
        const int phys = __builtin_amdgcn_readlane(ents, kk & 63);
        if (phys < 0 || phys >= g.n_pages) return false;
        load_chunk<D>(r, a.pool + g.unit_index(phys, kvh) * g.unit_bytes(), g, (cc * kChunk) % g.P, lane);
        return true;
    };
    if (c < c1) bad = !request(buf0, 0, c);
    // processes chunk c from cur after requesting the wave's next chunk into nxt
    auto advance = [&](const I2Chunk<D>& cur, I2Chunk<D>& nxt) {
        const int cn = c + stride;
        bool ok = true;
        if (cn < c1) {
            if (((k + 1) & 63) == 0) {
                ents = load_ents(k + 1);
                asm volatile("" : "+v"(ents));
            }
            ok = request(nxt, k + 1, cn);
        }
        process(cur, c);
        c = cn;
        ++k;
        bad = !ok;
    };
    while (c < c1 && !bad) {
        advance(buf0, buf1);
        if (c >= c1 || bad) break;
        advance(buf1, buf0);
    }

    // ---- finish: row sums, the zero-point term into o, then the W waves'
    // partials combined in wave order into one per workgroup
#pragma unroll
    for (int jj = 0; jj < JJ; ++jj) {
        l[jj] = row16_sum(l[jj]) * 16.0f;               // weights carried 2^-kTau
        if (bad) { m[jj] = NAN; l[jj] = NAN; }
    }
    {
        // corr column b (lane 16 g4 + b) times 2^kTau goes to the dims of block b
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

template <int D, int JJ>
hipError_t launch_dj(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    constexpr int W = kInt2Waves;
    using L = I2Lds<D, JJ, W>;
    if (L::BYTES > 64 * 1024) {
        hipError_t e = allow_lds<attn_int2_kernel<D, JJ, W>>(L::BYTES);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((attn_int2_kernel<D, JJ, W>), dim3(pl.n_splits * a.g.n_kv), dim3(W * 64), L::BYTES, stream, a,
                       pl.n_splits, pl.group, pl.rows);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    if (pl.rows <= 8) return launch_dj<D, 2>(a, pl, stream);
    if (pl.rows <= 16) return launch_dj<D, 4>(a, pl, stream);
    return hipErrorInvalidValue;
}

}  // namespace

int int2_waves() { return kInt2Waves; }

hipError_t launch_attn_int2(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    switch (a.g.D) {
        case 128: return launch_d<128>(a, pl, stream);
        case 256: return launch_d<256>(a, pl, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
