// attn_mfma_stream.hip -- paged decode / verify-batch attention over the
// Q8_0-K / Q4_0-V cache on gfx950 matrix cores, streaming the cache once.
//
// What it computes: for each query row (query i, head h) and a split of the
// keys, the online-softmax state (m, l, acc) of exact attention over the
// dequantized cache; lse_merge.hip combines the splits ("Qwen 27B (IQ4_XS,
// Q8/Q4 KV) on a 16GB RX 9070 XT at 262k context, via adaptive KV streaming",
// third paragraph: paged decode attention, extended to the verify batch;
// second paragraph: online log-sum-exp across pages).
//
// Work split.  A workgroup (4 wavefronts) owns one KV head and a contiguous
// run of 4*cps 32-token chunks; each wave streams cps of them.  All query
// rows that use this KV head -- the G heads of the group ("Context window and
// KV cache", GQA section) times n_q queries -- are served from one read of
// every K/V byte, so the cache is read once per KV head.
//
// Per 32-token chunk and wave (D = head_dim, NB = D/32 blocks):
//  * loads: two 16-token K tiles (D/64 x 16 B per lane each), their K scales,
//    the V chunk (D/64 x 16 B per lane) and its V scales; every instruction
//    is one contiguous 1 KiB request thanks to the pool layout, and chunk c+1
//    is in flight while chunk c is computed;
//  * S = Q K^T on v_mfma_f32_16x16x32_f16: K = 32 is exactly one quant block,
//    so the int8 codes go in unscaled (exact in fp16) and the block's fp16
//    scale multiplies the fp32 result.  q is split into fp16 hi + lo parts
//    (two MFMAs into one accumulator), so every product is exact in fp32;
//  * softmax: row max over the 16 tokens of a tile with DPP row rotations,
//    running max m, exp2 in the log2 domain (q carries scale*log2 e), the
//    accumulator is rescaled only when some row's max grows;
//  * P goes through a per-wave LDS buffer from the S layout (lane = token) to
//    the MFMA A layout (lane = row), is multiplied by the V scale of its
//    (token, block) in fp32 and rounded once to fp16; O += P' Vcodes on MFMA
//    with the 4-bit codes converted exactly to fp16 (c - 8).
// At the end the 4 waves are combined in LDS in a fixed order (deterministic)
// and one partial per workgroup is written.
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kPStride = 36;   // floats per row of the P transpose buffer (32 + padding)
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Cfg {
    static constexpr int NB = D / kBlock;       // quant blocks per row
    static constexpr int KL = D / 64;           // 16-byte loads per lane: K tile, V chunk
    static constexpr int NT = D / 16;           // 16-wide output tiles
    static constexpr int KSW = NB / 2;          // K-scale dwords per token
    static constexpr int VSD = 16 * NB;         // V-scale dwords per chunk (32 tokens)
    static constexpr int VSW = (VSD + 63) / 64; // V-scale dwords per lane
};

template <int D>
struct ChunkRegs {
    u32x4 k[2][Cfg<D>::KL];
    uint32_t ks[2][Cfg<D>::KSW];
    u32x4 v[Cfg<D>::KL];
    uint32_t vs[Cfg<D>::VSW];
};

template <int CTRL>
__device__ inline float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Reductions over the 16 lanes of a DPP row (rotate by 8, by 4, then swap
// pairs inside quads): every lane ends with the row's result.
__device__ inline float row16_max(float x) {
    x = fmaxf(x, dpp<0x128>(x));
    x = fmaxf(x, dpp<0x124>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0xB1>(x));
    return x;
}
__device__ inline float row16_sum(float x) {
    x += dpp<0x128>(x);
    x += dpp<0x124>(x);
    x += dpp<0x4E>(x);
    x += dpp<0xB1>(x);
    return x;
}

// Keeps the scheduler from hoisting later blocks' LDS reads and conversions
// above this point (which would raise register pressure past the budget).
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

__device__ inline void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 2^x on the hardware exp unit (results below the normal range flush to 0,
// which only drops weights far below the row maximum).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }

// 8 int8 codes -> 8 fp16 values, exactly: flip the sign bit to get c + 128,
// place each byte under the fp16 exponent of 1024 (0x64xx = 1024 + byte),
// subtract 1152.
__device__ inline half8 k_codes_to_half(uint32_t x0, uint32_t x1) {
    x0 ^= 0x80808080u;
    x1 ^= 0x80808080u;
    const half2v off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const u32x4 w = {__builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u),
                     __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)};
    half8 h = __builtin_bit_cast(half8, w);
    return h - half8{off.x, off.x, off.x, off.x, off.x, off.x, off.x, off.x};
}

// 8 four-bit codes (nibble i = token i of the lane's group) -> fp16 (c - 8),
// exactly, in the order (t0, t4, t1, t5, t2, t6, t3, t7).  Nibbles at bits
// 0-3 of a half become 1024 + n; at bits 4-7, 1024 + 16n.
__device__ inline half8 v_codes_to_half(uint32_t x) {
    const uint32_t magic = 0x64006400u;
    const uint32_t y = x >> 8;
    const u32x4 w = {(x & 0x000F000Fu) | magic, (x & 0x00F000F0u) | magic,
                     (y & 0x000F000Fu) | magic, (y & 0x00F000F0u) | magic};
    const half8 h = __builtin_bit_cast(half8, w);
    const _Float16 one = 1.0f, sixteenth = 0.0625f, o0 = -1032.0f, o1 = -72.0f;
    const half8 mul = {one, one, sixteenth, sixteenth, one, one, sixteenth, sixteenth};
    const half8 add = {o0, o0, o1, o1, o0, o0, o1, o1};
    return h * mul + add;
}

__device__ inline float half_lo(uint32_t w) { return (float)__builtin_bit_cast(half2v, w).x; }
__device__ inline float half_hi(uint32_t w) { return (float)__builtin_bit_cast(half2v, w).y; }

template <int D>
__device__ inline void load_chunk(ChunkRegs<D>& r, const uint8_t* unit, const Geom& g, int slot0, int lane) {
    using C = Cfg<D>;
    const uint8_t* kbase = unit + (int64_t)(slot0 / kTile) * kTile * D + lane * 16;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int p = 0; p < C::KL; ++p)
            r.k[tt][p] = *reinterpret_cast<const u32x4*>(kbase + tt * kTile * D + p * 1024);
    const uint32_t* ks = reinterpret_cast<const uint32_t*>(unit + g.k_scales_off());
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int tok = slot0 + tt * kTile + (lane & 15);
#pragma unroll
        for (int w = 0; w < C::KSW; ++w) r.ks[tt][w] = ks[tok * C::KSW + w];
    }
    const uint8_t* vbase = unit + g.v_codes_off() + (int64_t)(slot0 / kChunk) * kChunk * D / 2 + lane * 16;
#pragma unroll
    for (int u = 0; u < C::KL; ++u) r.v[u] = *reinterpret_cast<const u32x4*>(vbase + u * 1024);
    const uint32_t* vs = reinterpret_cast<const uint32_t*>(unit + g.v_scales_off()) + slot0 * C::NB / 2;
#pragma unroll
    for (int w = 0; w < C::VSW; ++w) {
        const int i = lane + 64 * w;
        r.vs[w] = i < C::VSD ? vs[i] : 0u;
    }
}

template <int D, int RT>
struct WaveState {
    floatx4 o[RT][Cfg<D>::NT];   // unnormalized output, MFMA C layout
    float m[RT][4];              // running max of each of the lane's 4 rows per tile
    float l[RT][4];              // this lane's share of the row sums
};

// Phase 1 of a 32-token chunk: S = (q_hi + q_lo) K^T for both 16-token tiles,
// plus staging of the chunk's V scales.  MASK: some key of the chunk lies
// beyond the last key of some row (causal edge, or positions past ctx_len).
template <int D, int RT, bool MASK>
__device__ inline void qk_phase(floatx4 (&s)[RT][2], const ChunkRegs<D>& r, const half8* __restrict__ qlds,
                                uint32_t* __restrict__ vslds, int lane, int j0, int first_last, int group,
                                int rows) {
    using C = Cfg<D>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    // stage this chunk's V scales block-major ([block][32 tokens] halves) for
    // the P' products below: dword i of the chunk holds blocks 2w, 2w+1 of
    // token i / (NB/2)
    {
        uint16_t* vsh = reinterpret_cast<uint16_t*>(vslds);
#pragma unroll
        for (int w = 0; w < C::VSW; ++w) {
            const int i = lane + 64 * w;
            if (i < C::VSD) {
                const int tok = i / (C::NB / 2), blk = 2 * (i % (C::NB / 2));
                vsh[blk * kChunk + tok] = (uint16_t)(r.vs[w] & 0xFFFFu);
                vsh[(blk + 1) * kChunk + tok] = (uint16_t)(r.vs[w] >> 16);
            }
        }
    }

    // ---- S = (q_hi + q_lo) K^T, one 32-value block per MFMA K step
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) s[rt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
        half8 kb[2];
        float ksc[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const u32x4 kr = r.k[tt][b / 2];
            kb[tt] = (b & 1) ? k_codes_to_half(kr.z, kr.w) : k_codes_to_half(kr.x, kr.y);
            const uint32_t sw = r.ks[tt][b / 2];
            ksc[tt] = (b & 1) ? half_hi(sw) : half_lo(sw);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const half8 qh = qlds[((rt * C::NB + b) * 2 + 0) * 64 + lane];
            const half8 ql = qlds[((rt * C::NB + b) * 2 + 1) * 64 + lane];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh, kb[tt], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, kb[tt], c, 0, 0, 0);
                s[rt][tt] += ksc[tt] * c;
            }
        }
        SCHED_FENCE();
    }

    // ---- causal / tail mask: key j visible to row r iff j <= first_last + r / group
    if (MASK) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * g4 + jj;
                const int last = row < rows ? first_last + row / group : -1;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    if (j0 + tt * kTile + n16 > last) s[rt][tt][jj] = -INFINITY;
            }
    }

}

// Phase 2: online softmax over the chunk's scores, then O += (P * vscale) V.
template <int D, int RT, bool MASK>
__device__ inline void pv_phase(WaveState<D, RT>& st, floatx4 (&s)[RT][2], const u32x4 (&v)[Cfg<D>::KL],
                                float* __restrict__ plds, const uint32_t* __restrict__ vslds, int lane) {
    using C = Cfg<D>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    // ---- online softmax (log2 domain)
    float mnew[RT][4];
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float mx = row16_max(fmaxf(s[rt][0][jj], s[rt][1][jj]));
            mnew[rt][jj] = fmaxf(st.m[rt][jj], mx);
            grow |= mnew[rt][jj] > st.m[rt][jj];
        }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float alpha = mnew[rt][jj] > st.m[rt][jj] ? fast_exp2(st.m[rt][jj] - mnew[rt][jj]) : 1.0f;
                st.l[rt][jj] *= alpha;
#pragma unroll
                for (int nt = 0; nt < C::NT; ++nt) st.o[rt][nt][jj] *= alpha;
                st.m[rt][jj] = mnew[rt][jj];
            }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float mref = st.m[rt][jj] == -INFINITY ? 0.0f : st.m[rt][jj];
            const float p0 = fast_exp2(s[rt][0][jj] - mref);
            const float p1 = fast_exp2(s[rt][1][jj] - mref);
            st.l[rt][jj] += p0 + p1;
            float* prow = plds + (rt * 16 + 4 * g4 + jj) * kPStride;
            prow[n16] = p0;
            prow[kTile + n16] = p1;
        }
    lds_fence();

    // ---- O += (P * vscale) Vcodes
    float pf[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float* prow = plds + (rt * 16 + n16) * kPStride + 8 * g4;
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[rt][i] = prow[i];
    }
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
        // V scales of the lane's 8 tokens (8*g4 .. 8*g4+7) for block b
        const u32x4 sw = reinterpret_cast<const u32x4*>(vslds)[(b * kChunk + 8 * g4) / 8];
        const float sc[8] = {half_lo(sw.x), half_hi(sw.x), half_lo(sw.y), half_hi(sw.y),
                             half_lo(sw.z), half_hi(sw.z), half_lo(sw.w), half_hi(sw.w)};
        half8 a[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float x0 = pf[rt][k] * sc[k], x1 = pf[rt][k + 4] * sc[k + 4];
                if (MASK) {             // masked keys may hold unwritten scales
                    x0 = pf[rt][k] == 0.0f ? 0.0f : x0;
                    x1 = pf[rt][k + 4] == 0.0f ? 0.0f : x1;
                }
                a[rt][2 * k] = (_Float16)x0;
                a[rt][2 * k + 1] = (_Float16)x1;
            }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int nt = 2 * b + h;
            const half8 bv = v_codes_to_half(v[nt / 4][nt % 4]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                st.o[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[rt], bv, st.o[rt][nt], 0, 0, 0);
        }
        SCHED_FENCE();
    }
}

template <int D, int RT>
__global__ __launch_bounds__(256, 1) void attn_mfma_stream_kernel(AttnArgs a, int cps, int n_splits,
                                                                                 int group, int rows) {
    using C = Cfg<D>;
    extern __shared__ __align__(16) uint8_t smem[];
    const Geom& g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave: scalar
    const int split = blockIdx.x % n_splits;
    const int kvh = blockIdx.x / n_splits;
    const int total_chunks = (a.ctx + kChunk - 1) / kChunk;
    const int first_last = a.ctx - a.n_q;             // last key of query 0

    // LDS carve-up: [Q hi/lo | P per wave | V scales per wave], reused for the
    // final combine; [m, l per wave and row] kept apart.
    const int q_bytes = RT * C::NB * 2 * 64 * 16;
    const int p_bytes = kWaves * RT * 16 * kPStride * 4;
    const int vs_bytes = kWaves * C::VSD * 4;
    const int comb_bytes = 2 * RT * 16 * D * 4;
    const int main_bytes = max(q_bytes + p_bytes + vs_bytes, comb_bytes);
    half8* qlds = reinterpret_cast<half8*>(smem);
    float* plds = reinterpret_cast<float*>(smem + q_bytes) + wave * RT * 16 * kPStride;
    uint32_t* vslds = reinterpret_cast<uint32_t*>(smem + q_bytes + p_bytes) + wave * C::VSD;
    float* mls = reinterpret_cast<float*>(smem + main_bytes);     // [wave][RT*16][2]

    // ---- stage q rows as fp16 hi/lo in the MFMA A layout, pre-scaled by scale*log2(e)
    const float qscale = a.scale * kLog2e;
    for (int e = threadIdx.x; e < RT * C::NB * 64; e += 256) {
        const int l = e & 63, rb = e >> 6, b = rb % C::NB, rt = rb / C::NB;
        const int row = 16 * rt + (l & 15);
        half8 hi, lo;
        if (row < rows) {
            const int qi = row / group, h = kvh * group + row % group;
            const float* src = a.q + ((size_t)qi * a.n_heads + h) * D + b * kBlock + 8 * (l >> 4);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = src[i] * qscale;
                hi[i] = (_Float16)x;
                lo[i] = (_Float16)(x - (float)hi[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) { hi[i] = (_Float16)0.0f; lo[i] = (_Float16)0.0f; }
        }
        qlds[(rb * 2 + 0) * 64 + l] = hi;
        qlds[(rb * 2 + 1) * 64 + l] = lo;
    }
    __syncthreads();

    WaveState<D, RT> st;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) { st.m[rt][jj] = -INFINITY; st.l[rt][jj] = 0.0f; }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) st.o[rt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- stream this wave's chunks, chunk c+1 in flight while c is computed
    const int c0 = split * kWaves * cps + wave * cps;
    const int c1 = min(c0 + cps, total_chunks);
    bool bad = false;
    auto unit_of = [&](int c, bool& ok) -> const uint8_t* {
        const int phys = a.page_table[(c * kChunk) / g.P];
        ok = phys >= 0 && phys < g.n_pages;
        return a.pool + g.unit_index(ok ? phys : 0, kvh) * g.unit_bytes();
    };
    // Chunk c's K registers die after its QK phase, so chunk c+1's loads are
    // issued there: they fly during chunk c's softmax and P*V work.
    auto phase1 = [&](floatx4 (&s)[RT][2], const ChunkRegs<D>& r, int c) {
        const int j0 = c * kChunk;
        if (j0 + kChunk - 1 > first_last)
            qk_phase<D, RT, true>(s, r, qlds, vslds, lane, j0, first_last, group, rows);
        else
            qk_phase<D, RT, false>(s, r, qlds, vslds, lane, j0, first_last, group, rows);
    };
    auto phase2 = [&](floatx4 (&s)[RT][2], const ChunkRegs<D>& r, int c) {
        if (c * kChunk + kChunk - 1 > first_last)
            pv_phase<D, RT, true>(st, s, r.v, plds, vslds, lane);
        else
            pv_phase<D, RT, false>(st, s, r.v, plds, vslds, lane);
    };
    if (c0 < c1) {
        ChunkRegs<D> ra, rb;
        floatx4 s[RT][2];
        bool oka, okb = true;
        const uint8_t* ua = unit_of(c0, oka);
        if (oka) load_chunk<D>(ra, ua, g, (c0 * kChunk) % g.P, lane);
        for (int c = c0; c < c1; c += 2) {
            if (oka) phase1(s, ra, c);
            if (c + 1 < c1) {
                const uint8_t* ub = unit_of(c + 1, okb);
                if (okb) load_chunk<D>(rb, ub, g, ((c + 1) * kChunk) % g.P, lane);
            }
            if (oka) phase2(s, ra, c); else bad = true;
            if (c + 1 >= c1) break;
            if (okb) phase1(s, rb, c + 1);
            if (c + 2 < c1) {
                ua = unit_of(c + 2, oka);
                if (oka) load_chunk<D>(ra, ua, g, ((c + 2) * kChunk) % g.P, lane);
            }
            if (okb) phase2(s, rb, c + 1); else bad = true;
        }
    }

    // ---- finish the row sums, combine the 4 waves in a fixed order
    const int g4 = lane >> 4, n16 = lane & 15;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            st.l[rt][jj] = row16_sum(st.l[rt][jj]);
            if (bad) { st.m[rt][jj] = NAN; st.l[rt][jj] = NAN; }
            if (n16 == 0) {
                const int row = 16 * rt + 4 * g4 + jj;
                mls[(wave * RT * 16 + row) * 2 + 0] = st.m[rt][jj];
                mls[(wave * RT * 16 + row) * 2 + 1] = st.l[rt][jj];
            }
        }
    __syncthreads();
    float M[RT][4], Ltot[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int row = 16 * rt + 4 * g4 + jj;
            float mm = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, mls[(w * RT * 16 + row) * 2]);
            float lt = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = mls[(w * RT * 16 + row) * 2], lw = mls[(w * RT * 16 + row) * 2 + 1];
                lt += lw == 0.0f ? 0.0f : lw * exp2f(mw - mm);
            }
            M[rt][jj] = mm;
            Ltot[rt][jj] = lt;
            const float f = st.l[rt][jj] == 0.0f ? 0.0f : exp2f(st.m[rt][jj] - mm);
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) st.o[rt][nt][jj] *= f;
        }
    float* ob = reinterpret_cast<float*>(smem);          // [2][RT*16][D]
    auto put = [&](int slot) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    ob[((size_t)slot * RT * 16 + 16 * rt + 4 * g4 + jj) * D + 16 * nt + n16] = st.o[rt][nt][jj];
    };
    auto add = [&](int slot) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    st.o[rt][nt][jj] += ob[((size_t)slot * RT * 16 + 16 * rt + 4 * g4 + jj) * D + 16 * nt + n16];
    };
    __syncthreads();                       // every wave is done with Q / P / V-scale LDS
    if (wave >= 2) put(wave - 2);
    __syncthreads();
    if (wave < 2) add(wave);
    __syncthreads();
    if (wave == 1) put(0);
    __syncthreads();
    if (wave != 0) return;
    add(0);

    // ---- write the partial of each row this workgroup serves
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int row = 16 * rt + 4 * g4 + jj;
            if (row >= rows) continue;
            const int qi = row / group, h = kvh * group + row % group;
            const size_t ps = ((size_t)qi * a.n_heads + h) * n_splits + split;
            if (n16 == 0) {
                a.ws_m[ps] = M[rt][jj];
                a.ws_l[ps] = Ltot[rt][jj];
            }
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) a.ws_acc[ps * D + 16 * nt + n16] = st.o[rt][nt][jj];
        }
}

template <int D, int RT>
hipError_t launch_dr(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    using C = Cfg<D>;
    const int q_bytes = RT * C::NB * 2 * 64 * 16;
    const int p_bytes = kWaves * RT * 16 * kPStride * 4;
    const int vs_bytes = kWaves * C::VSD * 4;
    const int comb_bytes = 2 * RT * 16 * D * 4;
    const int main_bytes = q_bytes + p_bytes + vs_bytes > comb_bytes ? q_bytes + p_bytes + vs_bytes : comb_bytes;
    const int lds = main_bytes + kWaves * RT * 16 * 2 * 4;
    auto kern = attn_mfma_stream_kernel<D, RT>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid(pl.n_splits * a.g.n_kv);
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, a, pl.chunks_per_split, pl.n_splits, pl.group, pl.rows);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    const int rt = (pl.rows + 15) / 16;
    switch (rt) {
        case 1: return launch_dr<D, 1>(a, pl, stream);
        case 2: return launch_dr<D, 2>(a, pl, stream);
        case 3: return launch_dr<D, 3>(a, pl, stream);
        case 4: return launch_dr<D, 4>(a, pl, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attn_mfma_stream(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    switch (a.g.D) {
        case 64: return launch_d<64>(a, pl, stream);
        case 128: return launch_d<128>(a, pl, stream);
        case 256: return launch_d<256>(a, pl, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
