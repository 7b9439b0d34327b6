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

template <int D, int R>
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
    static constexpr int PBUF = 16 * kPStride * 4;
    static constexpr int WAVE_BYTES = RING + LAND_KS + LAND_VS + PBUF;
    static constexpr int Q_BYTES = NB * 2 * 1024;   // one row group's q, fp16 hi/lo, MFMA A layout
};

// Workgroup LDS: W per-wave areas (reused by the final combine) | q of each
// of the RG row groups | (m, l) per wave and row.  The combine first folds the
// waves past the largest power of two P2 <= WPG into the first ones, then
// halves P2 down to one wave; SLOTS partial sums per group are in flight.
template <int D, int R, int W, int RG, int JJ>
struct WgLds {
    using C = Cfg<D, R>;
    static constexpr int WPG = W / RG;
    static constexpr int P2 = WPG >= 8 ? 8 : WPG >= 4 ? 4 : WPG >= 2 ? 2 : 1;
    static_assert(WPG < 16, "power-of-two fold");
    static constexpr int SLOTS = (P2 / 2 > WPG - P2 ? P2 / 2 : WPG - P2) > 0 ? (P2 / 2 > WPG - P2 ? P2 / 2 : WPG - P2) : 1;
    static constexpr int COMB_BYTES = RG * SLOTS * 16 * D * 4;
    static constexpr int MAIN_BYTES = W * C::WAVE_BYTES > COMB_BYTES ? W * C::WAVE_BYTES : COMB_BYTES;
    static constexpr int Q_OFF = MAIN_BYTES;
    static constexpr int ML_OFF = Q_OFF + RG * C::Q_BYTES;
    // one row group: the workgroup's chunk list (page entries) and the index
    // of the next chunk to hand out
    static constexpr int LIST = 256;
    static constexpr int LIST_OFF = ML_OFF + W * 16 * 2 * 4;
    // up to 8 rows (JJ = 2): the waves' rows for the one-barrier combine, in
    // a region of their own so that a wave can store them while others still
    // stream
    static constexpr bool SMALL_COMBINE = JJ == 2 && RG == 1;
    static constexpr int CB_OFF = LIST_OFF + (RG == 1 ? (LIST + 4) * 4 : 0);
    static constexpr int BYTES = CB_OFF + (SMALL_COMBINE ? W * 8 * D * 4 : 0);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Wait counts.  Per chunk a wave issues its requests in a fixed order: the
// QK step consumes code pieces 2p, 2p+1 (slice p, both tiles) and requests
// the pieces R places further on; then the next chunk's K scales; the PV
// step consumes piece 2KL+u and requests the one R further on; then the next
// chunk's V scales.  Piece J of chunk k was requested when piece J-R was
// consumed, so the number of requests issued after it by the time it is
// consumed is fixed; s_waitcnt vmcnt(that count) guarantees it has landed
// (requests complete in order).  The first chunk's requests go out in the
// same order before the loop, so it uses the same counts; the last chunk
// (nothing further requested) waits with 0.
template <int KL, int R>
struct Waits {
    static constexpr int NP = 3 * KL, NI = 3 * KL + 2;
    static constexpr int issue_pos(int j) { return j < 2 * KL ? j : j + 1; }          // slot of "consume j" in a chunk's requests
    static constexpr int event_pos(int J) { return J < 2 * KL ? 2 * (J / 2) : 2 * KL + 1 + (J - 2 * KL); }
    static constexpr int after(int J) {
        const int m = ((J - R) % NP + NP) % NP;
        return event_pos(J) - issue_pos(m) - 1 + (J < R ? NI : 0);
    }
    static constexpr int mn(int a, int b) { return a < b ? a : b; }
    // QK slice p (and, for p = 0, this chunk's K scales, issued at 2KL of the
    // chunk before)
    static constexpr int qk(int p) { return p == 0 ? mn(mn(after(0), after(1)), NI - 2 * KL - 1) : mn(after(2 * p), after(2 * p + 1)); }
    // PV slice u (and, for u = 0, this chunk's V scales, issued last in the chunk before)
    static constexpr int pv(int u) { return u == 0 ? mn(after(2 * KL), NI - KL - 1) : after(2 * KL + u); }
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
template <int D, int R>
__device__ inline void issue_piece(const Land& L, const ChunkPtr& cp, int j, int lane) {
    using C = Cfg<D, R>;
    const uint8_t* src;
    if (j < 2 * C::KL) src = cp.k + (j % 2) * kTile * D + (j / 2) * 1024 + lane * 16;
    else src = cp.v + (j - 2 * C::KL) * 1024 + lane * 16;
    dma16(src, L.ring + (j % R) * 1024);
}

// 32 tokens x NB scales = 4*NB pieces of 16 bytes.  Every lane takes part
// (lanes past 4*NB repeat a piece): a direct-to-LDS load under a
// lane-dependent branch can get its LDS base merged with a neighbouring one's.
template <int D, int R>
__device__ inline void issue_kscales(const Land& L, const ChunkPtr& cp, int lane) {
    using C = Cfg<D, R>;
    dma16(cp.ks + (lane % (4 * C::NB)) * 16, L.ks);
}
template <int D, int R>
__device__ inline void issue_vscales(const Land& L, const ChunkPtr& cp, int lane) {
    using C = Cfg<D, R>;
    dma16(cp.vs + (lane % (4 * C::NB)) * 16, L.vs);
}

template <int D, int R>
struct WaveState {
    floatx4 o[Cfg<D, R>::NT];   // unnormalized output, MFMA C layout
    float m[4];                 // reference max of each of the lane's 4 rows
    float l[4];                 // this lane's share of the row sums
};

// S = (q_hi + q_lo) K^T for the chunk's two 16-token tiles.  MASK: some key
// of the chunk lies beyond the last key of some row (causal edge, or
// positions past ctx_len).  wait(p) runs before slice p's pieces are read,
// done(p) after they have been read out of LDS.  q(i) gives q's operand i
// (block i / 2, hi for even i, lo for odd).
template <int D, int R, int JJ, bool MASK, class QSrc, class Wait, class Done>
__device__ inline void qk_step(floatx4 (&s)[2], const Land& L, QSrc q, int lane,
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
    for (int tt = 0; tt < 2; ++tt) s[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
    u32x4 kr[2];
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
        const half8 qh = q(2 * b);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh, kb[tt], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            if constexpr (JJ == 4) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(q(2 * b + 1), kb[tt], c, 0, 0, 0);
            s[tt] += ksc[tt] * c;
        }
        SCHED_FENCE();
    }
    // up to 8 rows the lo halves' products sit two rows down: fold them in
    if constexpr (JJ == 2) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            s[tt][0] += s[tt][2];
            s[tt][1] += s[tt][3];
        }
    }
    // causal / tail mask: key j visible to row r iff j <= first_last + r / group
    // (group is huge when every row sees all keys)
    if (MASK) {
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            const int row = logical_row<JJ>(rt0, 4 * g4 + jj);
            const int last = row >= 0 && row < rows ? first_last + row / group : -1;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                if (j0 + tt * kTile + n16 > last) s[tt][jj] = -INFINITY;
        }
    }
}

// Online softmax over the chunk's scores; writes P to the wave's LDS buffer.
template <int D, int R, int JJ>
__device__ inline void softmax_step(WaveState<D, R>& st, floatx4 (&s)[2], float* __restrict__ plds, int lane) {
    using C = Cfg<D, R>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    float mnew[4];
    bool grow = false;
#pragma unroll
    for (int jj = 0; jj < JJ; ++jj) {
        mnew[jj] = row16_max(fmaxf(s[0][jj], s[1][jj]));
        grow |= mnew[jj] > st.m[jj] + kTau;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        // rows whose maximum did not move get alpha = 1: one straight pass
        // over the accumulators, no per-row branches
        floatx4 alpha = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            const bool up = mnew[jj] > st.m[jj];
            alpha[jj] = up ? fast_exp2(st.m[jj] - mnew[jj]) : 1.0f;
            st.l[jj] *= alpha[jj];
            st.m[jj] = up ? mnew[jj] : st.m[jj];
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
template <int D, int R, bool MASK, class Wait, class Done>
__device__ inline void pv_step(WaveState<D, R>& st, const Land& L, const float* __restrict__ plds, int lane,
                               Wait wait, Done done) {
    using C = Cfg<D, R>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    uint32_t magic = 0x64006400u;
    asm volatile("" : "+v"(magic));          // keep the constant in a VGPR
    float pf[8];
    {
        const float* prow = plds + n16 * kPStride + 8 * g4;
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[i] = prow[i];
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
        half8 a;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float x0 = fmaf(pf[k], (float)sc[k], 0.0f);
            float x1 = fmaf(pf[k + 4], (float)sc[k + 4], 0.0f);
            if (MASK) {             // masked keys may hold unwritten scales
                x0 = pf[k] == 0.0f ? 0.0f : x0;
                x1 = pf[k + 4] == 0.0f ? 0.0f : x1;
            }
            a[2 * k] = (_Float16)x0;
            a[2 * k + 1] = (_Float16)x1;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int nt = 2 * b + h;
            const half8 bv = v_codes_to_half(vr[nt % 4], magic);
            st.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bv, st.o[nt], 0, 0, 0);
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

template <int D, int JJ, int RG, int R, int W, class Batch>
__global__ __launch_bounds__(W * 64) void attn_mfma_stream_kernel(AttnArgs a, int cps, int n_splits, int group,
                                                                  int rows, Batch sb) {
    using C = Cfg<D, R>;
    using WT = Waits<C::KL, R>;
    using WL = WgLds<D, R, W, RG, JJ>;
    // RG row groups of 16 rows; the WPG waves of group gi share its rows and
    // deal its chunks among themselves.  Every group streams the same
    // chunks, so a chunk read by a second group mostly comes from L2.
    constexpr int WPG = W / RG;
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
    float* mls = reinterpret_cast<float*>(smem + WL::ML_OFF);        // [wave][16][2]

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
    const uint8_t* qlds = smem + WL::Q_OFF + gi * C::Q_BYTES;
    constexpr int QB = (C::NB + WPG - 1) / WPG;      // blocks per wave
    float qv[QB][8];
    const int q_row = logical_row<JJ>(gi, lane & 15);
    const bool q_ok = q_row >= 0 && q_row < rows;
    {
        const int qi = q_ok ? q_row / group : 0, h = kvh * group + (q_ok ? q_row % group : 0);
        const float* src = a.q + ((size_t)qi * a.n_heads + h) * D + 8 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < QB; ++i) {
            const int b = wig + i * WPG < C::NB ? wig + i * WPG : 0;   // waves with no block left reload block 0
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[i][e] = src[b * kBlock + e];   // rows past the end read row 0
        }
    }

    if (dyn) {
        for (int p = threadIdx.x; p < n_list; p += W * 64) lst[p] = a.page_table[(list_chunk(p) * kChunk) / g.P];
        if (threadIdx.x == 0) lctr[0] = W;
    }
    int ents = load_ents(0);
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
                if (J + R >= C::NP) issue_piece<D, R>(land, cp, J + R - C::NP, lane);
            issue_kscales<D, R>(land, cp, lane);
#pragma unroll
            for (int J = 2 * C::KL; J < C::NP; ++J)
                if (J + R >= C::NP) issue_piece<D, R>(land, cp, J + R - C::NP, lane);
            issue_vscales<D, R>(land, cp, lane);
        }
    }

    // q into LDS (hi + lo fp16 halves; rows past the end are zero)
#pragma unroll
    for (int i = 0; i < QB; ++i) {
        const int b = wig + i * WPG;
        if (b >= C::NB) break;
        half8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = q_ok ? qv[i][e] * qscale : 0.0f;
            hi[e] = (_Float16)x;
            lo[e] = (_Float16)(x - (float)hi[e]);
        }
        uint8_t* dst = smem + WL::Q_OFF + gi * C::Q_BYTES + (2 * b) * 1024 + lane * 16;
        if constexpr (JJ == 2) {
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
    }
    auto qop = [&](int i) -> half8 {
        if constexpr (QREG) return qreg[i / 2];
        else return *reinterpret_cast<const half8*>(qlds + i * 1024 + lane * 16);
    };

    WaveState<D, R> st;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) { st.m[jj] = -INFINITY; st.l[jj] = 0.0f; }
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) st.o[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

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
            if (jn < C::NP) issue_piece<D, R>(land, cp, jn, lane);
            else if (more) issue_piece<D, R>(land, np, jn - C::NP, lane);
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
        floatx4 s[2];
        qk_step<D, R, JJ, MASK>(s, land, qop, lane, j0, first_last, mask_group, rows, gi, qk_wait, qk_done);
        lds_fence();                            // K scales read out
        if (more) issue_kscales<D, R>(land, np, lane);
        softmax_step<D, R, JJ>(st, s, plds, lane);
        pv_step<D, R, MASK>(st, land, plds, lane, pv_wait, pv_done);
        lds_fence();                            // V scales read out
        if (more) issue_vscales<D, R>(land, np, lane);
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
    for (int jj = 0; jj < JJ; ++jj) {
        st.l[jj] = row16_sum(st.l[jj]) * 16.0f;        // weights carried 2^-kTau
        if (bad) { st.m[jj] = NAN; st.l[jj] = NAN; }
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
            for (int jj = 0; jj < JJ; ++jj) cb[wave * SLOTW + (4 * jj + g4) * D + 16 * nt + n16] = st.o[nt][jj];
        if (n16 == 0) {
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) {
                float* d = mls + ((4 * jj + g4) * W + wave) * 2;
                d[0] = st.m[jj];
                d[1] = st.l[jj];
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
            const size_t ps = ((size_t)(row / group) * a.n_heads + kvh * group + row % group) * n_splits + split;
            *reinterpret_cast<floatx4*>(a.ws_acc + ps * D + dim) = acc;
            if (dim == 0) {
                a.ws_m[ps] = mm;
                a.ws_l[ps] = lt;
            }
        }
        return;
    }
#pragma unroll
    for (int jj = 0; jj < JJ; ++jj) {
        if (n16 == 0) {
            const int row = 4 * g4 + jj;
            mls[(wave * 16 + row) * 2 + 0] = st.m[jj];
            mls[(wave * 16 + row) * 2 + 1] = st.l[jj];
        }
    }
    __syncthreads();                       // every wave is done with its landing zone
    float M[4], Ltot[4];
#pragma unroll
    for (int jj = 0; jj < JJ; ++jj) {
        const int row = 4 * g4 + jj;
        float mm = -INFINITY;
#pragma unroll
        for (int j = 0; j < WPG; ++j) mm = fmaxf(mm, mls[((gi * WPG + j) * 16 + row) * 2]);
        float lt = 0.0f;
#pragma unroll
        for (int j = 0; j < WPG; ++j) {
            const int w = gi * WPG + j;
            const float mw = mls[(w * 16 + row) * 2], lw = mls[(w * 16 + row) * 2 + 1];
            lt += lw == 0.0f ? 0.0f : lw * exp2f(mw - mm);
        }
        M[jj] = mm;
        Ltot[jj] = lt;
        const float f = st.l[jj] == 0.0f ? 0.0f : exp2f(st.m[jj] - mm);
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) st.o[nt][jj] *= f;
    }
    float* ob = reinterpret_cast<float*>(smem);          // [RG * SLOTS][16][D]
    auto put = [&](int slot) {
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj)
                ob[((size_t)slot * 16 + 4 * g4 + jj) * D + 16 * nt + n16] = st.o[nt][jj];
    };
    auto add = [&](int slot) {
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj)
                st.o[nt][jj] += ob[((size_t)slot * 16 + 4 * g4 + jj) * D + 16 * nt + n16];
    };
    // inside each row group: waves [P2, WPG) first hand their sums to waves
    // [0, WPG - P2), then waves [h, 2h) to waves [0, h) for h = P2/2 .. 1;
    // group gi uses buffer slots gi*SLOTS .. (gi+1)*SLOTS - 1
    constexpr int P2 = WL::P2;
    if constexpr (WPG > P2) {
        if (wig >= P2) put(gi * WL::SLOTS + wig - P2);
        __syncthreads();
        if (wig < WPG - P2) add(gi * WL::SLOTS + wig);
        __syncthreads();
    }
#pragma unroll
    for (int h = P2 / 2; h >= 1; h /= 2) {
        if (wig >= h && wig < 2 * h) put(gi * WL::SLOTS + wig - h);
        __syncthreads();
        if (wig < h) add(gi * WL::SLOTS + wig);
        __syncthreads();
    }
    if (wig != 0) return;

    // ---- write the partial of each row this row group serves
#pragma unroll
    for (int jj = 0; jj < JJ; ++jj) {
        const int row = logical_row<JJ>(gi, 4 * g4 + jj);
        if (row < 0 || row >= rows) continue;
        const int qi = row / group, h = kvh * group + row % group;
        const size_t ps = ((size_t)qi * a.n_heads + h) * n_splits + split;
        if (n16 == 0) {
            a.ws_m[ps] = M[jj];
            a.ws_l[ps] = Ltot[jj];
        }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) a.ws_acc[ps * D + 16 * nt + n16] = st.o[nt][jj];
    }
}

// Waves per workgroup: two per SIMD, one workgroup per CU.  (With at most 8
// rows three waves per SIMD would fit in the registers, but 12 waves with
// 4 KiB in flight each read HBM more slowly than 8.)
template <int JJ>
constexpr int stream_waves() { return 8; }

template <int D, int JJ, int RG, class Batch>
hipError_t launch_dr(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg) {
    constexpr int R = D == 64 ? 3 : D == 128 ? 3 : 4;   // ring slots: a few KiB in flight per wave
    constexpr int W = stream_waves<JJ>();
    using WL = WgLds<D, R, W, RG, JJ>;
    auto kern = attn_mfma_stream_kernel<D, JJ, RG, R, W, Batch>;
    if (WL::BYTES > 64 * 1024) {
        hipError_t e = allow_lds<attn_mfma_stream_kernel<D, JJ, RG, R, W, Batch>>(WL::BYTES);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_wg), dim3(W * 64), WL::BYTES, stream, a, pl.chunks_per_split, pl.n_splits,
                       pl.group, pl.rows, sb);
    return hipGetLastError();
}

// Up to 8 rows two per lane group (JJ = 2), up to 16 rows one per MFMA row,
// more rows in 2 or 4 row groups of 16.
template <int D, class Batch>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg) {
    if (pl.rows <= 8) return launch_dr<D, 2, 1>(a, pl, stream, sb, n_wg);
    if (pl.rows <= 16) return launch_dr<D, 4, 1>(a, pl, stream, sb, n_wg);
    if (pl.rows <= 32) return launch_dr<D, 4, 2>(a, pl, stream, sb, n_wg);
    if (pl.rows <= 64) return launch_dr<D, 4, 4>(a, pl, stream, sb, n_wg);
    return hipErrorInvalidValue;
}

template <class Batch>
hipError_t launch_any(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const Batch& sb, int n_wg) {
    switch (a.g.D) {
        case 64: return launch_d<64>(a, pl, stream, sb, n_wg);
        case 128: return launch_d<128>(a, pl, stream, sb, n_wg);
        case 256: return launch_d<256>(a, pl, stream, sb, n_wg);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int mfma_stream_row_groups(int rows) { return rows <= 16 ? 1 : rows <= 32 ? 2 : 4; }
int mfma_stream_waves(int rows) {
    return (rows <= 8 ? stream_waves<2>() : stream_waves<4>()) / mfma_stream_row_groups(rows);
}

hipError_t launch_attn_mfma_stream(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const SeqBatch* batch) {
    if (batch != nullptr && batch->n > 0) return launch_any(a, pl, stream, *batch, batch->wg0[batch->n]);
    return launch_any(a, pl, stream, NoBatch{}, pl.n_splits * a.g.n_kv);
}

}  // namespace kvq
