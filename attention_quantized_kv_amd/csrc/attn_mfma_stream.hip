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
// Work split.  A workgroup of W wavefronts belongs to one KV head; the
// head's chunks are dealt round-robin to its waves (about cps each).  All query
// rows that use this KV head -- the G heads of the group ("Context window and
// KV cache", GQA section) times n_q queries -- are served from one read of
// every K/V byte, so the cache is read once per KV head.
//
// Data path per 32-token chunk and wave (D = head_dim, NB = D/32 blocks):
//  * global -> LDS directly (global_load_lds_dwordx4), one contiguous 1 KiB
//    wave request (16 bytes per lane) per piece thanks to the pool layout,
//    so data in flight costs no VGPRs.  A chunk is 3*KL code pieces (K tile
//    0/1 of each 64-dim slice, then the V slices) plus a K-scale and a
//    V-scale piece.  The code pieces stream through a per-wave ring of R
//    slots in the order they are consumed: as soon as a piece has been read
//    out of LDS, the piece R places further on is requested into its slot.
//    The HBM system delivers the most when each wave keeps only a few KiB in
//    flight (more outstanding requests lower the throughput), so the ring is
//    kept short; the scale pieces of chunk c+1 are requested once chunk c's
//    have been used.  The wait counts are computed at compile time from the
//    fixed request order (Waits below).
//  * S = Q K^T on v_mfma_f32_16x16x32_f16: K = 32 is exactly one quant block,
//    so the int8 codes go in unscaled (exact in fp16) and the block's fp16
//    scale multiplies the fp32 result.  q is split into fp16 hi + lo parts
//    (two MFMAs into one accumulator), so every product is exact in fp32.
//  * softmax: row max over the 16 tokens of a tile with DPP row rotations,
//    log2 domain (q carries scale*log2 e), lazy rescaling (below).
//  * P goes through a per-wave LDS buffer from the S layout (lane = token) to
//    the MFMA A layout (lane = row), is multiplied by the V scale of its
//    (token, block) in fp32 and rounded once to fp16; O += P' Vcodes on MFMA
//    with the 4-bit codes converted exactly to fp16.
// At the end the W waves are combined in LDS in a fixed order (deterministic)
// and one partial per workgroup is written.
#include <hip/hip_fp16.h>

#include <type_traits>

#include "kvq_internal.h"
#include "kvq_mfma.h"
#include "kvq_quant.h"
#include "kvq_waits.h"

namespace kvq {
namespace {

// 8 int8 codes -> 8 fp16 values, exactly: flip the sign bit to get c + 128,
// place each byte under the fp16 exponent of 1024 (0x64xx = 1024 + byte),
// subtract 1152.
__device__ inline half8 k_codes_to_half(uint32_t x0, uint32_t x1) {
    x0 ^= 0x80808080u;
    x1 ^= 0x80808080u;
    const u32x4 w = {__builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u),
                     __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)};
    const _Float16 off = 1152.0f;
    return __builtin_bit_cast(half8, w) - half8{off, off, off, off, off, off, off, off};
}

// 8 four-bit codes (nibble i = token i of the lane's group) -> fp16
// (c - 8) * 2^kTau, exactly, in the order (t0, t4, t1, t5, t2, t6, t3, t7).
// Nibbles at bits 0-3 of a half become 1024 + n, at bits 4-7 1024 + 16n;
// one FMA per half then gives (n - 8) * 16 (a small integer, exact).  The
// magic exponent lives in a register so that mask-and-insert is one
// v_and_or_b32 (gfx9 VOP3 takes no literal).
__device__ inline half8 v_codes_to_half(uint32_t x, uint32_t magic) {
    const uint32_t y = x >> 8;
    const u32x4 w = {(x & 0x000F000Fu) | magic, (x & 0x00F000F0u) | magic,
                     (y & 0x000F000Fu) | magic, (y & 0x00F000F0u) | magic};
    const half8 h = __builtin_bit_cast(half8, w);
    const _Float16 m0 = 16.0f, m1 = 1.0f, a0 = -16512.0f, a1 = -1152.0f;
    const half8 mul = {m0, m0, m1, m1, m0, m0, m1, m1};
    const half8 add = {a0, a0, a1, a1, a0, a0, a1, a1};
    return h * mul + add;
}

template <int D, int R, int RT = 1>
struct Cfg {
    static constexpr int NB = D / kBlock;       // quant blocks per row
    static constexpr int KL = D / 64;           // 64-dim slices (1 KiB pieces per K tile / V chunk)
    static constexpr int NT = D / 16;           // 16-wide output tiles
    static constexpr int NP = 3 * KL;           // code pieces per chunk: K(t0,p), K(t1,p) for each p, then V(u)
    static_assert(NP % R == 0 && R <= NP, "ring slots must divide the pieces of a chunk");
    // per-wave LDS: code ring, K scales, V scales, P transpose buffer (bytes)
    static constexpr int RING = R * 1024;
    static constexpr int LAND_KS = 1024;        // 32 x NB fp16, padded to one full-wave request
    static constexpr int LAND_VS = 1024;        // NB x 32 fp16, padded likewise
    static constexpr int PBUF = 16 * kPStride * 4;  // one row tile's P
    static constexpr int WAVE_BYTES = RING + LAND_KS + LAND_VS + RT * PBUF;
    static constexpr int Q_BYTES = NB * 2 * 1024;   // one row tile's q, fp16 hi/lo, MFMA A layout
};

// Workgroup LDS: W per-wave areas | q of each of the RG row groups (both
// reused by the final combine; up to 8 rows q's area grows to hold the small
// combine's rows) | (m, l) per wave, row tile and row | the chunk list (one
// row group) | the partial index of every row.
template <int D, int R, int W, int RG, int JJ, int RT = 1>
struct WgLds {
    using C = Cfg<D, R, RT>;
    static constexpr int WPG = W / RG;
    // up to 8 rows (JJ = 2): the waves' rows for the one-barrier combine, in
    // a region of their own so that a wave can store them while others still
    // stream -- q's region, which is dead once every wave holds q in
    // registers (a barrier after those reads)
    static constexpr bool SMALL_COMBINE = JJ == 2 && RG == 1 && RT == 1;
    static constexpr int CB_BYTES = SMALL_COMBINE ? W * 8 * D * 4 : 0;
    // otherwise every wave's sums of one row tile, [W][NT][64] float4, over
    // the rings and q (dead by then)
    static constexpr int COMB_BYTES = SMALL_COMBINE ? 0 : W * C::NT * 64 * 16;
    static constexpr int Q_ALL = RG * RT * C::Q_BYTES;
    static constexpr int MAIN_BYTES = W * C::WAVE_BYTES > COMB_BYTES - Q_ALL ? W * C::WAVE_BYTES : COMB_BYTES - Q_ALL;
    static constexpr int Q_OFF = MAIN_BYTES;
    static constexpr int CB_OFF = Q_OFF;
    static constexpr int ML_OFF = Q_OFF + (CB_BYTES > Q_ALL ? CB_BYTES : Q_ALL);
    // one row group: the workgroup's chunk list (page entries) and the index
    // of the next chunk to hand out
    static constexpr int LIST = 256;
    static constexpr int LIST_OFF = ML_OFF + W * RT * 16 * 2 * 4;
    // the partial index of every row of every tile (-1: no row there)
    static constexpr int PS_OFF = LIST_OFF + (RG == 1 ? (LIST + 4) * 4 : 0);
    static constexpr int BYTES = PS_OFF + RG * RT * 16 * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Per-wave LDS of the stream.
struct Land {
    uint8_t* ring;  // [R][1 KiB] code pieces
    uint8_t* ks;    // [32 tokens][NB] fp16 (then repeats)
    uint8_t* vs;    // [NB][32 tokens] fp16 (then repeats)
};

// Where one chunk's data sits in the pool: the start of its K code tiles, V
// code chunk, K scales and V scales (unit base + region offset + the chunk's
// first slot times the bytes per slot of that region).
struct ChunkPtr {
    const uint8_t* k;
    const uint8_t* v;
    const uint8_t* ks;
    const uint8_t* vs;
};
template <int D>
__device__ inline ChunkPtr chunk_ptr(const uint8_t* unit, const Geom& g, int slot0) {
    constexpr int NB = D / kBlock;
    return {unit + (uint32_t)slot0 * D, unit + g.v_codes_off() + (uint32_t)slot0 * (D / 2),
            unit + g.k_scales_off() + (uint32_t)slot0 * (2 * NB), unit + g.v_scales_off() + (uint32_t)slot0 * (2 * NB)};
}

// Requests code piece j of a chunk into ring slot j % R.  Full-wave request
// (see the scale pieces below).
template <int D, int R, int POL>
__device__ inline void issue_piece(const Land& L, const ChunkPtr& cp, int j, int lane) {
    using C = Cfg<D, R>;
    const uint8_t* src;
    if (j < 2 * C::KL) src = cp.k + (j % 2) * kTile * D + (j / 2) * 1024 + lane * 16;
    else src = cp.v + (j - 2 * C::KL) * 1024 + lane * 16;
    dma16<POL>(src, L.ring + (j % R) * 1024);
}

// 32 tokens x NB scales = 4*NB pieces of 16 bytes.  Every lane takes part
// (lanes past 4*NB repeat a piece): a direct-to-LDS load under a
// lane-dependent branch can get its LDS base merged with a neighbouring one's.
template <int D, int R, int POL>
__device__ inline void issue_kscales(const Land& L, const ChunkPtr& cp, int lane) {
    using C = Cfg<D, R>;
    dma16<POL>(cp.ks + (lane % (4 * C::NB)) * 16, L.ks);
}
template <int D, int R, int POL>
__device__ inline void issue_vscales(const Land& L, const ChunkPtr& cp, int lane) {
    using C = Cfg<D, R>;
    dma16<POL>(cp.vs + (lane % (4 * C::NB)) * 16, L.vs);
}

template <int D, int R>
struct TileState {
    floatx4 o[Cfg<D, R>::NT];   // unnormalized output of the tile, MFMA C layout
    float m[4];                 // reference max of each of the lane's 4 rows
    float l[4];                 // this lane's share of the row sums
};
template <int D, int R, int RT = 1>
struct WaveState {
    TileState<D, R> t[RT];      // one per row tile
};

// Row layout of tile rt of a wave with RT tiles.  JJ = 3 (17-24 rows): the
// last tile holds at most 8 rows in the JJ = 2 layout -- one MFMA per block
// for q's hi and lo halves, half the softmax -- and the others JJ = 4.
template <int JJ, int RT>
__device__ constexpr int tile_jj(int rt) { return JJ == 3 ? (rt == RT - 1 ? 2 : 4) : JJ; }
// The query row at MFMA row prow of tile t (the group's tile index), which is
// tile rt of its wave, or -1.
template <int JJ, int RT>
__device__ inline int tile_row(int t, int rt, int prow) {
    return tile_jj<JJ, RT>(rt) == 4 ? logical_row<4>(t, prow) : logical_row<2>(t, prow);
}

// S = (q_hi + q_lo) K^T for the chunk's two 16-token tiles.  MASK: some key
// of the chunk lies beyond the last key of some row (causal edge, or
// positions past ctx_len).  wait(p) runs before slice p's pieces are read,
// done(p) after they have been read out of LDS.  q(i) gives q's operand i
// (block i / 2, hi for even i, lo for odd).
template <int D, int R, int JJ, int RT, bool MASK, class QSrc, class Wait, class Done>
__device__ inline void qk_step(floatx4 (&s)[RT][2], const Land& L, QSrc q, int lane,
                               int j0, int first_last, int group, int rows, int rt0, Wait wait, Done done) {
    using C = Cfg<D, R>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    wait(0);
    // K scales of the lane's token in each tile (NB halves)
    uint32_t ksw[2][C::NB / 2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(L.ks + (tt * kTile + n16) * C::NB * 2);
#pragma unroll
        for (int w = 0; w < C::NB / 2; ++w) ksw[tt][w] = src[w];
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) s[rt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
    u32x4 kr[2];
    // The products are scaled by the K scales and added to s in the block
    // that made them (several row tiles: the other tiles' MFMAs cover the
    // latency) or one block later (one tile), and pinned there: left alone,
    // the compiler sinks every scaling to the end and keeps all the blocks'
    // raw products live, 64 VGPRs per row tile at head_dim 256.
    constexpr bool LAG = RT == 1;
    floatx4 cp[RT][2];
    float kscp[2];
    auto fold = [&]() {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                s[rt][tt] += kscp[tt] * cp[rt][tt];
                asm volatile("" :: "v"(s[rt][tt]));
            }
    };
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
        if ((b & 1) == 0) {
            const int p = b / 2;
            if (p > 0) wait(p);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                kr[tt] = *reinterpret_cast<const u32x4*>(L.ring + ((2 * p + tt) % R) * 1024 + lane * 16);
            done(p);
        }
        half8 kb[2];
        float ksc[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            kb[tt] = (b & 1) ? k_codes_to_half(kr[tt].z, kr[tt].w) : k_codes_to_half(kr[tt].x, kr[tt].y);
            const half2v sw = as_h2(ksw[tt][b / 2]);
            ksc[tt] = (b & 1) ? (float)sw.y : (float)sw.x;
        }
        // the converted codes serve every row tile of the wave
        floatx4 c[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const half8 qh = q(rt, 2 * b);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                c[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh, kb[tt], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
        if constexpr (JJ != 2) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (tile_jj<JJ, RT>(rt) != 4) continue;      // (hi and lo in one operand)
                const half8 ql = q(rt, 2 * b + 1);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    c[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, kb[tt], c[rt][tt], 0, 0, 0);
            }
        }
        if (LAG && b > 0) fold();
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            kscp[tt] = ksc[tt];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) cp[rt][tt] = c[rt][tt];
        }
        if (!LAG) fold();
        SCHED_FENCE();
    }
    if (LAG) fold();
    // in a tile of up to 8 rows the lo halves' products sit two rows down:
    // fold them in
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (tile_jj<JJ, RT>(rt) != 2) continue;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            s[rt][tt][0] += s[rt][tt][2];
            s[rt][tt][1] += s[rt][tt][3];
        }
    }
    // causal / tail mask: key j visible to row r iff j <= first_last + r / group
    // (group is huge when every row sees all keys)
    if (MASK) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int jj = 0; jj < tile_jj<JJ, RT>(rt); ++jj) {
                const int row = tile_row<JJ, RT>(rt0 + rt, rt, 4 * g4 + jj);
                const int last = row >= 0 && row < rows ? first_last + row / group : -1;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    if (j0 + tt * kTile + n16 > last) s[rt][tt][jj] = -INFINITY;
            }
    }
}

// Online softmax over the chunk's scores of row tile rt; writes P to the
// tile's LDS buffer.
template <int D, int R, int JJ>
__device__ inline void softmax_step(TileState<D, R>& st, floatx4 (&s)[2], float* __restrict__ plds, int lane) {
    using C = Cfg<D, R>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    // The row maxima only when some score of the wave passes its row's
    // reference by more than kTau: a row's maximum does iff one of its
    // scores does, so the test needs no cross-lane step.
    float smax[4];
    bool grow = false;
#pragma unroll
    for (int jj = 0; jj < JJ; ++jj) {
        smax[jj] = max2(s[0][jj], s[1][jj]);
        grow |= smax[jj] > st.m[jj] + kTau;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        // rows whose maximum did not move get alpha = 1: one straight pass
        // over the accumulators, no per-row branches
        floatx4 alpha = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            const float mnew = row16_max(smax[jj]);
            const bool up = mnew > st.m[jj];
            alpha[jj] = up ? fast_exp2(st.m[jj] - mnew) : 1.0f;
            st.l[jj] *= alpha[jj];
            st.m[jj] = up ? mnew : st.m[jj];
        }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) st.o[nt] *= alpha;
    }
#pragma unroll
    for (int jj = 0; jj < JJ; ++jj) {
        const float mref = (st.m[jj] == -INFINITY ? 0.0f : st.m[jj]) + kTau;
        const float p0 = fast_exp2(s[0][jj] - mref);
        const float p1 = fast_exp2(s[1][jj] - mref);
        st.l[jj] += p0 + p1;
        float* prow = plds + (4 * g4 + jj) * kPStride;
        prow[n16] = p0;
        prow[kTile + n16] = p1;
    }
    lds_fence();
}

// O += (P * vscale) Vcodes for the chunk.  wait(u) / done(u) around the
// read of V slice u.
template <int D, int R, int RT, bool MASK, class Wait, class Done>
__device__ inline void pv_step(WaveState<D, R, RT>& st, const Land& L, const float* __restrict__ plds, int lane,
                               Wait wait, Done done) {
    using C = Cfg<D, R, RT>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    uint32_t magic = 0x64006400u;
    asm volatile("" : "+v"(magic));          // keep the constant in a VGPR
    float pf[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float* prow = plds + rt * (C::PBUF / 4) + n16 * kPStride + 8 * g4;
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[rt][i] = prow[i];
    }
    u32x4 vr;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
        if ((b & 1) == 0) {
            const int u = b / 2;
            wait(u);
            vr = *reinterpret_cast<const u32x4*>(L.ring + ((2 * C::KL + u) % R) * 1024 + lane * 16);
            done(u);
        }
        // V scales of the lane's 8 tokens (8*g4 .. 8*g4+7) for block b
        const half8 sc = *reinterpret_cast<const half8*>(L.vs + (b * kChunk + 8 * g4) * 2);
        // P' = p * vscale: one fused fp32 multiply rounded once to fp16
        half8 a[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float x0 = fmaf(pf[rt][k], (float)sc[k], 0.0f);
                float x1 = fmaf(pf[rt][k + 4], (float)sc[k + 4], 0.0f);
                if (MASK) {             // masked keys may hold unwritten scales
                    x0 = pf[rt][k] == 0.0f ? 0.0f : x0;
                    x1 = pf[rt][k + 4] == 0.0f ? 0.0f : x1;
                }
                a[rt][2 * k] = (_Float16)x0;
                a[rt][2 * k + 1] = (_Float16)x1;
            }
        // the converted V codes serve every row tile of the wave
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int nt = 2 * b + h;
            const half8 bv = v_codes_to_half(vr[nt % 4], magic);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                st.t[rt].o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[rt], bv, st.t[rt].o[nt], 0, 0, 0);
        }
        SCHED_FENCE();
    }
}

// Runs vm_wait<Waits::qk(p)> (or pv) for a p known only after unrolling.
template <class WT, int P = 0>
__device__ inline void wait_qk(int p) {
    if constexpr (P < WT::NP / 3) {
        if (p == P) { vm_wait<WT::qk(P)>(); return; }
        wait_qk<WT, P + 1>(p);
    }
}
template <class WT, int P = 0>
__device__ inline void wait_pv(int p) {
    if constexpr (P < WT::NP / 3) {
        if (p == P) { vm_wait<WT::pv(P)>(); return; }
        wait_pv<WT, P + 1>(p);
    }
}

// A row appended by a fused decode step (kvq_append_attn), handled by one
// wave of one workgroup while the rest of the chip streams the cached keys.
// New row j (position pos0 + j) of KV head kvh is quantized with the append
// kernel's block code (the values the pool will hold, bit for bit) and
// written into the pool; then every query row r of the KV head (query i =
// r / group) gets the softmax state of this one key as partial part_idx:
// m = its score, l = 1, acc = its dequantized value when i >= j (causal
// among the new rows), an empty partial (l = 0) otherwise.  A new row whose
// page entry lies outside the pool is not written and its partials are NaN.
// Lane owns dims 64 p + lane (p < D/64): every 32-lane half is one
// quantization block.  Every pool byte is written by one thread: a V byte
// holds slots (2k, 2k+1) and is written by the wave of the odd slot's row,
// or of the even slot's row when the odd slot is not a new row; the other
// nibble is then the old one, or the partner new row's code, quantized here
// as well.
constexpr int kMaxNewRows = 8;
template <int D>
__device__ inline void new_row_partials(const AttnArgs& a, const NewRows& nr, int kvh, int group, int rows, int j,
                                        int part_stride, int part_idx, int lane) {
    constexpr int NP = D / 64;
    const Geom& g = a.g;
    const int pos = nr.pos0 + j, slot = pos % g.P;
    const bool odd = (pos & 1) != 0;
    const bool partner_new = odd ? j >= 1 : j + 1 < nr.n_new;   // the other slot of the V byte is a new row
    const bool own_byte = odd || !partner_new;
    const size_t src = ((size_t)j * g.n_kv + kvh) * D + lane;
    const size_t psrc = odd && partner_new ? src - (size_t)g.n_kv * D : src;   // row j - 1
    float kh[NP], vh[NP], vp[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        kh[p] = nr.k[src + 64 * p];
        vh[p] = nr.v[src + 64 * p];
        vp[p] = nr.v[psrc + 64 * p];
    }
    const int e = a.page_table[pos / g.P];
    // the query rows' q (scaled), 8 rows per batch, each batch's loads in
    // flight together; the first batch is requested before the quantization
    constexpr int QB = 8;
    const float qscale = a.scale * kLog2e;
    float qv[QB][NP];
    auto load_q = [&](int r0) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const int r = min(r0 + b, rows - 1), qi = r / group, h = kvh * group + r % group;
#pragma unroll
            for (int p = 0; p < NP; ++p) qv[b][p] = a.q[((size_t)qi * a.n_heads + h) * D + 64 * p + lane];
        }
    };
    load_q(0);
    const bool ok = e >= 0 && e < g.n_pages;
    uint8_t* unit = nr.pool + g.unit_index(ok ? e : 0, kvh) * g.unit_bytes();
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int d = 64 * p + lane;
        const QCode ck = quant_q8_0(kh[p], lane);
        const QCode cv = quant_q4_0(vh[p], lane);
        kh[p] = (float)ck.code * __half2float(__float2half_rn(ck.d));
        vh[p] = (float)(cv.code - 8) * __half2float(__float2half_rn(cv.d));
        if (ok) {
            unit[k_code_pos(g, slot, d)] = (uint8_t)(int8_t)ck.code;
            if ((lane & (kBlock - 1)) == 0) {
                reinterpret_cast<uint16_t*>(unit + g.k_scales_off())[slot * g.nb() + d / kBlock] = f16_bits(ck.d);
                reinterpret_cast<uint16_t*>(unit + g.v_scales_off())[v_scale_idx(g, slot, d / kBlock)] = f16_bits(cv.d);
            }
            if (own_byte) {
                int nib;
                const int64_t off = v_code_pos(g, slot, d, &nib);
                const int other = partner_new ? quant_q4_0(vp[p], lane).code : (odd ? unit[off] & 15 : unit[off] >> 4);
                unit[off] = (uint8_t)(odd ? other | (cv.code << 4) : cv.code | (other << 4));
            }
        }
    }
    // one partial per query row; rows of queries before j see no new key here
    for (int r0 = 0; r0 < rows; r0 += QB) {
        if (r0 > 0) load_q(r0);
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const int r = r0 + b;
            if (r >= rows) break;                          // uniform
            const int qi = r / group, h = kvh * group + r % group;
            const size_t ps = ((size_t)qi * a.n_heads + h) * part_stride + part_idx;
            const bool sees = qi >= j;
            float dot = 0.0f;
#pragma unroll
            for (int p = 0; p < NP; ++p) dot = fmaf(qv[b][p] * qscale, kh[p], dot);
            const float sc = wave_sum(dot, lane);
            if (lane == 0) {
                a.ws_m[ps] = !sees ? -INFINITY : ok ? sc : NAN;
                a.ws_l[ps] = !sees ? 0.0f : ok ? 1.0f : NAN;
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) a.ws_acc[ps * D + 64 * p + lane] = sees ? vh[p] : 0.0f;
        }
    }
}

template <int D, int JJ, int RG, int R, int W, int RT, class Batch, bool NEWR>
__global__ __launch_bounds__(W * 64) void attn_mfma_stream_kernel(AttnArgs a, int cps, int n_splits, int group,
                                                                  int rows, Batch sb, NewRows nr, int part_stride) {
    using C = Cfg<D, R, RT>;
    using WT = Waits<C::KL, R>;
    using WL = WgLds<D, R, W, RG, JJ, RT>;
    // RG row groups of 16 RT rows; the WPG waves of group gi share its rows
    // and deal its chunks among themselves.  Every group streams the same
    // chunks, so a chunk read by a second group mostly comes from L2.  A wave
    // holds RT row tiles of 16 rows: it converts every code of its chunks
    // once and feeds the result to the MFMAs of all its tiles.
    constexpr int WPG = W / RG;
    // the cache is read once: non-temporal loads, except where several row
    // groups read each chunk and the later ones hit in L2
    constexpr int POL = RG == 1 ? kLoadNT : kLoadPlain;
    extern __shared__ __align__(16) uint8_t smem[];
    const Geom& g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave: scalar
    int wg = blockIdx.x;
    if constexpr (!std::is_same_v<Batch, NoBatch>) {
        // batched decode: this workgroup serves sequence b, whose keys, page
        // table row, queries and partials start where the table says
        const int b = seq_of(sb.wg0, sb.n, wg);
        wg -= sb.wg0[b];
        n_splits = sb.n_splits[b];
        part_stride = n_splits;                 // the sequence's own partials per row
        a.ctx = sb.ctx[b];
        a.page_table += (size_t)b * sb.n_table;
        a.q += (size_t)b * a.n_q * a.n_heads * D;
        a.ws_m += sb.part0[b];
        a.ws_l += sb.part0[b];
        a.ws_acc += (size_t)sb.part0[b] * D;
    }
    const int split = wg % n_splits;
    const int kvh = wg / n_splits;
    const int total_chunks = (a.ctx + kChunk - 1) / kChunk;
    // last key of query 0; query i sees i keys more (causal), or all keys
    const int first_last = a.causal ? a.ctx - a.n_q : a.ctx - 1;
    const int mask_group = a.causal ? group : 0x7fffffff;

    // LDS: [per wave: ring + scales + P buffer] (reused by the final combine)
    // | [q of each row group] | [m, l per wave and row]
    uint8_t* wbase = smem + wave * C::WAVE_BYTES;
    const Land land = {wbase, wbase + C::RING, wbase + C::RING + C::LAND_KS};
    float* plds = reinterpret_cast<float*>(wbase + C::RING + C::LAND_KS + C::LAND_VS);
    float* mls = reinterpret_cast<float*>(smem + WL::ML_OFF);        // [wave][RT][16][2]

    // ---- this wave's chunks: wave g of a row group takes the group's chunks
    // g, g + N, g + 2N, ... (N waves per group and KV head), so all waves
    // sweep the context together and the addresses in flight at any time
    // stay close.
    const int gi = wave / WPG, wig = wave % WPG;
    const int stride = n_splits * WPG;
    const int c0 = split * WPG + wig;
    const int c1 = total_chunks;
    (void)cps;
    // One row group: the workgroup's chunks -- list entry p is chunk
    // split * W + p % W + (p / W) * stride, the chunks its waves would take
    // round-robin -- are handed out in list order from an LDS counter as the
    // waves ask for their next chunk, so a wave that falls behind (the second
    // wave of a SIMD, mostly) takes fewer.  Each wave starts with entry `wave`.
    const int n_list = W * (c1 / stride) + min(max(c1 % stride - split * W, 0), W);
    // (Several row groups keep the fixed round-robin: handed out per group,
    // the groups drift apart and lose the L2 hits of reading the same chunks
    // at about the same time.)
    const bool dyn = RG == 1 && n_list <= WL::LIST;
    int* const lst = reinterpret_cast<int*>(smem + WL::LIST_OFF);     // [LIST] page entries
    int* const lctr = lst + WL::LIST;                                   // next list entry to hand out
    auto list_chunk = [&](int p) { return split * W + p % W + (p / W) * stride; };
    // one list entry for the whole wave: a single lane takes it
    auto pop = [&]() {
        int v = 0;
        if (lane == 0) v = atomicAdd(lctr, 1);
        return __builtin_amdgcn_readlane(v, 0);
    };
    // Page-table entries: lane k of `ents` holds the entry of the wave's
    // chunk number kb + k (batches of 64, one gather load per batch), and the
    // loop picks them out with readlane -- no memory access, hence no wait,
    // between the requests in flight.
    auto load_ents = [&](int kb) -> int {
        const int ck = c0 + (kb + lane) * stride;
        return ck < c1 ? a.page_table[(ck * kChunk) / g.P] : -1;
    };
    auto unit_at = [&](int phys, bool& ok) -> const uint8_t* {
        ok = phys >= 0 && phys < g.n_pages;
        return a.pool + g.unit_index(ok ? phys : 0, kvh) * g.unit_bytes();
    };
    // ---- q as fp16 hi/lo in the MFMA A layout, pre-scaled by scale*log2(e),
    // once per row group in LDS: 1 KiB per (block, hi/lo), lane l's 16 bytes
    // = the row at MFMA row l % 16, dims 8 (l / 16) .. +7 of the block.  The
    // group's waves take the blocks round-robin.  The loads go out before the
    // page-table gather, so both arrive in one round trip.
    const float qscale = a.scale * kLog2e;
    const uint8_t* qlds = smem + WL::Q_OFF + gi * RT * C::Q_BYTES;   // tile rt at + rt * Q_BYTES
    constexpr int QB = (C::NB + WPG - 1) / WPG;      // blocks per wave
    float qv[RT][QB][8];
    bool q_ok[RT];
    if constexpr (RT == 1) {
        // (straight-line for one tile: the loop form below, even of one
        // trip, made the register allocator spill the decode kernel)
        const int q_row = logical_row<JJ>(gi, lane & 15);
        q_ok[0] = q_row >= 0 && q_row < rows;
        const bool ok = q_ok[0];
        const int qi = ok ? q_row / group : 0, h = kvh * group + (ok ? q_row % group : 0);
        const float* src = a.q + ((size_t)qi * a.n_heads + h) * D + 8 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < QB; ++i) {
            const int b = wig + i * WPG < C::NB ? wig + i * WPG : 0;   // waves with no block left reload block 0
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[0][i][e] = src[b * kBlock + e];   // rows past the end read row 0
        }
    } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int q_row = tile_row<JJ, RT>(gi * RT + rt, rt, lane & 15);
            q_ok[rt] = q_row >= 0 && q_row < rows;
            const int qi = q_ok[rt] ? q_row / group : 0, h = kvh * group + (q_ok[rt] ? q_row % group : 0);
            const float* src = a.q + ((size_t)qi * a.n_heads + h) * D + 8 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < QB; ++i) {
                const int b = wig + i * WPG < C::NB ? wig + i * WPG : 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) qv[rt][i][e] = src[b * kBlock + e];
            }
        }
    }

    // the wave's own entries go out before the list gather, whose stores
    // into LDS wait for their loads: all of them arrive in one round trip
    int ents = load_ents(0);
    if (dyn) {
        for (int p = threadIdx.x; p < n_list; p += W * 64) lst[p] = a.page_table[(list_chunk(p) * kChunk) / g.P];
        if (threadIdx.x == 0) lctr[0] = W;
    }
    asm volatile("" : "+v"(ents));             // wait for it (and q) here, before any chunk request
    // first slot of the current chunk in its page; it advances by dslot (mod P)
    // from one chunk of the wave to the next
    int slot_cur = (c0 * kChunk) % g.P;
    const int dslot = (stride * kChunk) % g.P;
    bool ok_cur = false;
    const uint8_t* u_cur = nullptr;
    if (c0 < c1) {
        u_cur = unit_at(__builtin_amdgcn_readlane(ents, 0), ok_cur);
        if (ok_cur) {
            // the first chunk's requests in the order a previous chunk would
            // have issued them (refills of pieces NP-R.., K scales after the QK
            // slices, V scales last), so the steady-state wait counts hold
            const ChunkPtr cp = chunk_ptr<D>(u_cur, g, slot_cur);
#pragma unroll
            for (int J = 0; J < 2 * C::KL; ++J)
                if (J + R >= C::NP) issue_piece<D, R, POL>(land, cp, J + R - C::NP, lane);
            issue_kscales<D, R, POL>(land, cp, lane);
#pragma unroll
            for (int J = 2 * C::KL; J < C::NP; ++J)
                if (J + R >= C::NP) issue_piece<D, R, POL>(land, cp, J + R - C::NP, lane);
            issue_vscales<D, R, POL>(land, cp, lane);
        }
    }

    // q into LDS (hi + lo fp16 halves; rows past the end are zero)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < QB; ++i) {
        const int b = wig + i * WPG;
        if (b >= C::NB) break;
        half8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = q_ok[rt] ? qv[rt][i][e] * qscale : 0.0f;
            hi[e] = (_Float16)x;
            lo[e] = (_Float16)(x - (float)hi[e]);
        }
        uint8_t* dst = smem + WL::Q_OFF + (gi * RT + rt) * C::Q_BYTES + (2 * b) * 1024 + lane * 16;
        if (tile_jj<JJ, RT>(rt) == 2) {
            // up to 8 rows one operand holds both halves: the lo half of MFMA
            // row n goes to row n + 2, a row no query uses (same k group)
            if ((lane & 2) == 0) {
                *reinterpret_cast<half8*>(dst) = hi;
                *reinterpret_cast<half8*>(dst + 32) = lo;
            }
        } else {
            *reinterpret_cast<half8*>(dst) = hi;
            *reinterpret_cast<half8*>(dst + 1024) = lo;
        }
    }
    lds_barrier();                             // q visible to the group; the first chunk stays in flight
    // up to 8 rows the operands of q (hi and lo in one per block) stay in
    // registers, 32 VGPRs at head_dim 256: LDS reads per 32-dim block would
    // add more LDS traffic per chunk and wave than the chunk itself
    constexpr bool QREG = JJ == 2;
    half8 qreg[QREG ? C::NB : 1];
    if constexpr (QREG) {
#pragma unroll
        for (int i = 0; i < C::NB; ++i) qreg[i] = *reinterpret_cast<const half8*>(qlds + (2 * i) * 1024 + lane * 16);
        static_assert(!QREG || WL::SMALL_COMBINE, "the small combine reuses q's LDS");
        lds_barrier();                         // every wave holds q: its LDS is free for the small combine
    }
    auto qop = [&](int rt, int i) -> half8 {
        if constexpr (QREG) return qreg[i / 2];       // (one row tile)
        else return *reinterpret_cast<const half8*>(qlds + rt * C::Q_BYTES + i * 1024 + lane * 16);
    };
    // fused decode step: appended row j is handled by the last wave of split
    // n_splits - 1 - j of each KV head -- the last splits hold the fewest
    // chunks -- before its loop (its first chunk's requests stay in flight;
    // in list mode the other waves take its share)
    if constexpr (NEWR) {
        if (wave == W - 1)
            for (int j = n_splits - 1 - split; j < nr.n_new; j += n_splits)
                new_row_partials<D>(a, nr, kvh, group, rows, j, part_stride, n_splits + j, lane);
    }

    WaveState<D, R, RT> st;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) { st.t[rt].m[jj] = -INFINITY; st.t[rt].l[jj] = 0.0f; }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) st.t[rt].o[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- stream.  A page-table entry outside the pool stops the wave
    // (nothing is loaded from it) and turns its partial into NaN.
    bool bad = c0 < c1 && !ok_cur;
    int c = c0, k = 0;
    // list mode: the wave's next list entry (handed out one chunk ahead)
    int p_next = dyn && c0 < c1 ? pop() : 0;
    // one chunk: MASK when some key of it lies past the last key of some row
    auto chunk = [&](auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int j0 = c * kChunk;
        // The two waves of a SIMD (w and w + W/2) take turns at the higher
        // issue priority, chunk by chunk.  With the hardware's oldest-first
        // choice alone, the second wave of every SIMD ends several percent
        // later than the first (and, with two row groups, the groups drift
        // apart and lose their shared L2 reads).
        if (((k ^ (wave >= W / 2 ? 1 : 0)) & 1) != 0) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        bool has_next, ok_next = false;
        const uint8_t* u_next = u_cur;
        int slot_next = slot_cur, cn = c1, p_nn = 0;
        if (dyn) {
            has_next = p_next < n_list;
            if (has_next) {
                cn = list_chunk(p_next);
                u_next = unit_at(lst[p_next], ok_next);
                slot_next = (cn * kChunk) % g.P;
                p_nn = pop();                   // the entry after it
            }
        } else {
            has_next = c + stride < c1;
            if (has_next && ((k + 1) & 63) == 0) {  // every 64 chunks
                ents = load_ents(k + 1);
                asm volatile("" : "+v"(ents));      // consume it here, so the loop's other path has nothing to wait for
            }
            if (has_next) {
                cn = c + stride;
                u_next = unit_at(__builtin_amdgcn_readlane(ents, (k + 1) & 63), ok_next);
                slot_next = slot_cur + dslot >= g.P ? slot_cur + dslot - g.P : slot_cur + dslot;
            }
        }
        const bool more = has_next && ok_next;  // requests for the next chunk go out in this iteration
        const ChunkPtr cp = chunk_ptr<D>(u_cur, g, slot_cur), np = chunk_ptr<D>(u_next, g, slot_next);
        // consuming piece J requests piece J + R: of this chunk, or of the next
        auto refill = [&](int J) {
            const int jn = J + R;
            if (jn < C::NP) issue_piece<D, R, POL>(land, cp, jn, lane);
            else if (more) issue_piece<D, R, POL>(land, np, jn - C::NP, lane);
        };
        auto qk_wait = [&](int p) {
            if (!more) vm_wait<0>();
            else wait_qk<WT>(p);
        };
        auto qk_done = [&](int p) {
            lds_fence();                        // slice p read out: its slots are free
            refill(2 * p);
            refill(2 * p + 1);
        };
        auto pv_wait = [&](int u) {
            if (!more) vm_wait<0>();
            else wait_pv<WT>(u);
        };
        auto pv_done = [&](int u) {
            lds_fence();
            refill(2 * C::KL + u);
        };
        floatx4 s[RT][2];
        qk_step<D, R, JJ, RT, MASK>(s, land, qop, lane, j0, first_last, mask_group, rows, gi * RT, qk_wait, qk_done);
        lds_fence();                            // K scales read out
        if (more) issue_kscales<D, R, POL>(land, np, lane);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (tile_jj<JJ, RT>(rt) == 2) softmax_step<D, R, 2>(st.t[rt], s[rt], plds + rt * (C::PBUF / 4), lane);
            else softmax_step<D, R, 4>(st.t[rt], s[rt], plds + rt * (C::PBUF / 4), lane);
        }
        pv_step<D, R, RT, MASK>(st, land, plds, lane, pv_wait, pv_done);
        lds_fence();                            // V scales read out
        if (more) issue_vscales<D, R, POL>(land, np, lane);
        if (has_next && !ok_next) bad = true;
        u_cur = u_next;
        slot_cur = slot_next;
        c = cn;
        p_next = p_nn;
        ++k;
    };
    // chunks wholly visible to every row first, then the masked ones
    const int c_mask = first_last >= kChunk - 1 ? (first_last - (kChunk - 1)) / kChunk + 1 : 0;
    while (c < c1 && c < c_mask && !bad) chunk(std::false_type{});
    while (c < c1 && !bad) chunk(std::true_type{});
    vm_wait<0>();

    // ---- finish the row sums, combine the group's waves in a fixed order
    const int g4 = lane >> 4, n16 = lane & 15;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < tile_jj<JJ, RT>(rt); ++jj) {
            st.t[rt].l[jj] = row16_sum(st.t[rt].l[jj]) * 16.0f;        // weights carried 2^-kTau
            if (bad) { st.t[rt].m[jj] = NAN; st.t[rt].l[jj] = NAN; }
        }
    if constexpr (WL::SMALL_COMBINE) {
        // At most 8 rows: every wave stores its unscaled rows ([wave][row
        // slot][dim], row slot = 4 jj + g4) and their (m, l) ([row slot][wave]);
        // after one barrier each thread takes 4 consecutive dims of one row:
        // it forms the row's wave factors 2^(m_w - M) and sums the waves in
        // wave order.
        constexpr int SLOTW = JJ * 4 * D;             // floats per wave
        float* cb = reinterpret_cast<float*>(smem + WL::CB_OFF);
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) cb[wave * SLOTW + (4 * jj + g4) * D + 16 * nt + n16] = st.t[0].o[nt][jj];
        if (n16 == 0) {
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) {
                float* d = mls + ((4 * jj + g4) * W + wave) * 2;
                d[0] = st.t[0].m[jj];
                d[1] = st.t[0].l[jj];
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
                const floatx4 o = *reinterpret_cast<const floatx4*>(cb + w * SLOTW + slot * D + dim);
                acc += f * o;
            }
            const size_t ps = ((size_t)(row / group) * a.n_heads + kvh * group + row % group) * part_stride + split;
            *reinterpret_cast<floatx4*>(a.ws_acc + ps * D + dim) = acc;
            if (dim == 0) {
                a.ws_m[ps] = mm;
                a.ws_l[ps] = lt;
            }
        }
        return;
    }
    // 16-row tiles: every wave's (m, l) per row of each tile; then per tile
    // each wave scales its sums to the group's maximum and stores them
    // ([wave][nt][lane] float4: the MFMA layout, conflict-free), and after a
    // barrier all threads of the workgroup sum the group's waves in wave
    // order and write the partial.  The buffer covers the rings and q, which
    // are dead once every wave has left its loop (the first barrier).
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < tile_jj<JJ, RT>(rt); ++jj)
            if (n16 == 0) {
                float* d = mls + ((wave * RT + rt) * 16 + 4 * g4 + jj) * 2;
                d[0] = st.t[rt].m[jj];
                d[1] = st.t[rt].l[jj];
            }
    int* const pst = reinterpret_cast<int*>(smem + WL::PS_OFF);      // [RG * RT tiles][16 rows]
    if (threadIdx.x < RG * RT * 16) {
        const int lrow = tile_row<JJ, RT>(threadIdx.x / 16, (threadIdx.x / 16) % RT, threadIdx.x % 16);
        pst[threadIdx.x] = lrow >= 0 && lrow < rows
                               ? ((lrow / group) * a.n_heads + kvh * group + lrow % group) * part_stride + split
                               : -1;
    }
    __syncthreads();
    floatx4* const cb = reinterpret_cast<floatx4*>(smem);          // [W][NT][64]
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (rt > 0) __syncthreads();                // the tile before has been read out
        {
            // lane L looks after row L % 16 of the tile and waves L / 16,
            // L / 16 + 4, ... of the group: the group's maximum and weight
            // sum of the row, and this wave's factor for it
            const int r = lane & 15;
            const float* mrow = mls + ((gi * WPG * RT + rt) * 16 + r) * 2;     // + wave-in-group * RT * 32
            float mm = -INFINITY;
#pragma unroll
            for (int j = g4; j < WPG; j += 4) mm = fmaxf(mm, mrow[j * RT * 32]);
            mm = fmaxf(mm, xor16_f(mm, lane));
            mm = fmaxf(mm, xor32_f(mm, lane));
            float lt = 0.0f;
#pragma unroll
            for (int j = g4; j < WPG; j += 4) {
                const float mw = mrow[j * RT * 32], lw = mrow[j * RT * 32 + 1];
                // NaN (a bad page) propagates; a wave without keys adds nothing
                lt += lw == 0.0f ? 0.0f : lw * fast_exp2(mw - mm);
            }
            lt += xor16_f(lt, lane);
            lt += xor32_f(lt, lane);
            const float ms = mrow[wig * RT * 32], ls = mrow[wig * RT * 32 + 1];
            const float fr = ls == 0.0f ? 0.0f : fast_exp2(ms - mm);
            // lane (g4, n16) holds rows 4 g4 + jj: their factors sit in lanes 4 g4 + jj
#pragma unroll
            for (int jj = 0; jj < tile_jj<JJ, RT>(rt); ++jj) {
                const float f = __shfl(fr, 4 * g4 + jj);
#pragma unroll
                for (int nt = 0; nt < C::NT; ++nt) st.t[rt].o[nt][jj] *= f;
            }
            // (m, l) of the partial: the group's first wave
            const int ps = pst[(gi * RT + rt) * 16 + r];
            if (wig == 0 && lane < 16 && ps >= 0) {
                a.ws_m[ps] = mm;
                a.ws_l[ps] = lt;
            }
        }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) cb[(wave * C::NT + nt) * 64 + lane] = st.t[rt].o[nt];
        __syncthreads();
        // element e = (group, nt, lane of the MFMA layout): rows 4 (lane / 16)
        // + jj of the group's tile rt, column 16 nt + lane % 16
        for (int e = threadIdx.x; e < RG * C::NT * 64; e += W * 64) {
            const int eg = e / (C::NT * 64), ent = (e / 64) % C::NT, el = e % 64;
            floatx4 acc = cb[((eg * WPG) * C::NT + ent) * 64 + el];
#pragma unroll
            for (int j = 1; j < WPG; ++j) acc += cb[((eg * WPG + j) * C::NT + ent) * 64 + el];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {                  // (rows a tile does not hold have ps = -1)
                const int ps = pst[(eg * RT + rt) * 16 + 4 * (el >> 4) + jj];
                if (ps >= 0) a.ws_acc[(size_t)ps * D + 16 * ent + (el & 15)] = acc[jj];
            }
        }
    }
}

// Waves per workgroup: two per SIMD, one workgroup per CU.  (With at most 8
// rows three waves per SIMD would fit in the registers, but 12 waves with
// 4 KiB in flight each read HBM more slowly than 8.)
template <int JJ>
constexpr int stream_waves() { return 8; }

template <int D, int JJ, int RG, int RT, bool NEWR, class Batch>
hipError_t launch_dr(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg,
                     const NewRows& nr, int part_stride) {
    constexpr int R = stream_ring_slots(D, JJ == 2 || (RT == 2 && RG == 1));   // ring slots: a few KiB in flight per wave
    constexpr int W = stream_waves<JJ>();
    using WL = WgLds<D, R, W, RG, JJ, RT>;
    auto kern = attn_mfma_stream_kernel<D, JJ, RG, R, W, RT, Batch, NEWR>;
    if (WL::BYTES > 64 * 1024) {
        hipError_t e = allow_lds<attn_mfma_stream_kernel<D, JJ, RG, R, W, RT, Batch, NEWR>>(WL::BYTES);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_wg), dim3(W * 64), WL::BYTES, stream, a, pl.chunks_per_split, pl.n_splits,
                       pl.group, pl.rows, sb, nr, part_stride);
    return hipGetLastError();
}

// Up to 8 rows two per lane group (JJ = 2), up to 16 rows one per MFMA row,
// up to 32 rows two row tiles per wave (every code converted once for both;
// up to 24 the second tile in the 8-row layout, JJ = 3), more rows in 2 row
// groups of two tiles.
template <int D, bool NEWR, class Batch>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg,
                    const NewRows& nr, int part_stride) {
    if (pl.rows <= 8) return launch_dr<D, 2, 1, 1, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
    if (pl.rows <= 16) return launch_dr<D, 4, 1, 1, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
    if (pl.rows <= 24) return launch_dr<D, 3, 1, 2, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
    if (pl.rows <= 32) return launch_dr<D, 4, 1, 2, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
    if (pl.rows <= 64) return launch_dr<D, 4, 2, 2, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
    return hipErrorInvalidValue;
}

template <bool NEWR, class Batch>
hipError_t launch_any(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg,
                      const NewRows& nr, int part_stride) {
    switch (a.g.D) {
        case 64: return launch_d<64, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
        case 128: return launch_d<128, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
        case 256: return launch_d<256, NEWR>(a, pl, stream, sb, n_wg, nr, part_stride);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int mfma_stream_row_groups(int rows) { return rows <= 32 ? 1 : 2; }
int mfma_stream_waves(int rows) {
    return (rows <= 8 ? stream_waves<2>() : stream_waves<4>()) / mfma_stream_row_groups(rows);
}

hipError_t launch_attn_mfma_stream(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const SeqBatch* batch) {
    const NewRows none{nullptr, nullptr, nullptr, 0, 0};
    if (batch != nullptr && batch->n > 0)
        return launch_any<false>(a, pl, stream, *batch, batch->wg0[batch->n], none, pl.n_splits);
    return launch_any<false>(a, pl, stream, NoBatch{}, pl.n_splits * a.g.n_kv, none, pl.n_splits);
}

hipError_t launch_attn_mfma_stream_new(const AttnArgs& a, const AttnPlan& pl, const NewRows& nr, hipStream_t stream) {
    if (nr.n_new < 1 || nr.n_new > kMaxNewRows || pl.n_splits < 1) return hipErrorInvalidValue;
    return launch_any<true>(a, pl, stream, NoBatch{}, pl.n_splits * a.g.n_kv, nr, pl.n_splits + nr.n_new);
}

}  // namespace kvq
