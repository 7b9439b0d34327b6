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
//  * global -> LDS directly (global_load_lds_dwordx4) into the wave's own
//    landing zone: two 16-token K tiles, their K scales, the V chunk and its
//    V scales.  Each instruction moves one contiguous 1 KiB (16 bytes per
//    lane) thanks to the pool layout, and data in flight costs no VGPRs.
//    K of chunk c+1 is requested as soon as chunk c's K has been read out of
//    LDS (after its QK step), V of chunk c+1 as soon as chunk c's V has been
//    read (after its PV step), so each load has about a chunk of work to hide
//    behind, plus the other wave on the SIMD.
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

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kPStride = 36;   // floats per row of the P transpose buffer (32 + padding)
constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescaling: a row's reference maximum m moves only when a chunk's
// maximum exceeds it by more than kTau (log2 units).  Weights are formed as
// 2^(s - m - kTau) <= 1 and the V codes carry the compensating 2^kTau
// exactly, so fp16 operands never overflow; the row sum is scaled by 2^kTau
// at the end.
constexpr float kTau = 4.0f;

template <int D, int RT>
struct Cfg {
    static constexpr int NB = D / kBlock;       // quant blocks per row
    static constexpr int KL = D / 64;           // 1 KiB loads: per K tile, per V chunk
    static constexpr int NT = D / 16;           // 16-wide output tiles
    static constexpr int W = RT == 1 ? 8 : 4;   // waves per workgroup (kThreadsFor / 64)
    // per-wave landing zone and P buffer (bytes)
    static constexpr int LAND_K = 2 * KL * 1024;
    static constexpr int LAND_KS = 1024;        // 32 x NB fp16, padded to one full-wave DMA
    static constexpr int LAND_V = KL * 1024;
    static constexpr int LAND_VS = 1024;        // NB x 32 fp16, padded likewise
    static constexpr int PBUF = RT * 16 * kPStride * 4;
    static constexpr int WAVE_BYTES = LAND_K + LAND_KS + LAND_V + LAND_VS + PBUF;
    static constexpr int Q_BYTES = RT == 1 ? 0 : RT * NB * 2 * 64 * 16;   // q staged in LDS only for RT > 1
    static constexpr int COMB_BYTES = (W / 2) * RT * 16 * D * 4;
    static constexpr int MAIN_BYTES = Q_BYTES + W * WAVE_BYTES > COMB_BYTES ? Q_BYTES + W * WAVE_BYTES : COMB_BYTES;
    static constexpr int ML_BYTES = W * RT * 16 * 2 * 4;
    static constexpr int LDS_BYTES = MAIN_BYTES + ML_BYTES;
    // vector-memory instructions per request
    static constexpr int K_ISSUES = 2 * KL + 1;
    static constexpr int V_ISSUES = KL + 1;
};

// MFMA row placement.  Row tile rt holds MFMA rows 0..15; lane group g4 of the
// S / O layouts owns rows 4*g4 .. 4*g4+3.  With at most 8 query rows (JJ = 2)
// the rows go to MFMA rows {0,1, 4,5, 8,9, 12,13}, so each lane holds 2 real
// rows and the softmax work per lane halves; otherwise (JJ = 4) row i sits at
// MFMA row i.  Returns the query row at MFMA row prow of tile rt, or -1.
template <int JJ>
__device__ inline int logical_row(int rt, int prow) {
    if (JJ == 4) return 16 * rt + prow;
    return (prow & 3) < 2 ? 8 * rt + 2 * (prow >> 2) + (prow & 3) : -1;
}

template <int RT>
constexpr int kThreadsFor = (RT == 1 ? 8 : 4) * 64;   // workgroup size (must match Cfg::W)

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

// Keeps the scheduler from moving work across a block boundary (which would
// lengthen live ranges past the register budget).
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Waits for this wave's outstanding LDS reads; also a compiler memory fence.
__device__ inline void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Waits until at most N vector-memory requests of this wave are outstanding
// (direct-to-LDS loads count); also a compiler memory fence, since the
// compiler cannot see that later LDS reads depend on those loads.
template <int N>
__device__ inline void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// 16 bytes per lane, global -> LDS: lane i's bytes land at lds + 16 i.
__device__ inline void dma16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds, 16, 0, 0);
}

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

// Per-wave LDS landing zone of one chunk.
struct Land {
    uint8_t* k;     // [2 tiles][KL][1 KiB]
    uint8_t* ks;    // [32 tokens][NB] fp16 (then repeats)
    uint8_t* v;     // [KL][1 KiB]
    uint8_t* vs;    // [NB][32 tokens] fp16 (then repeats)
};

template <int D, int RT>
__device__ inline void issue_k(const Land& L, const uint8_t* unit, const Geom& g, int slot0, int lane) {
    using C = Cfg<D, RT>;
    const uint8_t* src = unit + (int64_t)(slot0 / kTile) * kTile * D + lane * 16;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int p = 0; p < C::KL; ++p) dma16(src + tt * kTile * D + p * 1024, L.k + (tt * C::KL + p) * 1024);
    // 32 tokens x NB scales = 4*NB pieces of 16 bytes.  Every lane takes part
    // (lanes past 4*NB repeat a piece): a DMA under a lane-dependent branch
    // can get its LDS base merged with a neighbouring DMA's by the compiler.
    dma16(unit + g.k_scales_off() + (int64_t)slot0 * C::NB * 2 + (lane % (4 * C::NB)) * 16, L.ks);
}

template <int D, int RT>
__device__ inline void issue_v(const Land& L, const uint8_t* unit, const Geom& g, int slot0, int lane) {
    using C = Cfg<D, RT>;
    const uint8_t* src = unit + g.v_codes_off() + (int64_t)(slot0 / kChunk) * kChunk * D / 2 + lane * 16;
#pragma unroll
    for (int u = 0; u < C::KL; ++u) dma16(src + u * 1024, L.v + u * 1024);
    dma16(unit + g.v_scales_off() + (int64_t)(slot0 / kChunk) * C::NB * kChunk * 2 + (lane % (4 * C::NB)) * 16,
          L.vs);
}

template <int D, int RT>
struct WaveState {
    floatx4 o[RT][Cfg<D, RT>::NT];   // unnormalized output, MFMA C layout
    float m[RT][4];                  // reference max of each of the lane's 4 rows per tile
    float l[RT][4];                  // this lane's share of the row sums
};

// S = (q_hi + q_lo) K^T for the chunk's two 16-token tiles.  MASK: some key
// of the chunk lies beyond the last key of some row (causal edge, or
// positions past ctx_len).
template <int D, int RT, int JJ, bool MASK>
__device__ inline void qk_step(floatx4 (&s)[RT][2], const Land& L, const half8* __restrict__ qlds,
                               const half8 (&qreg)[Cfg<D, RT>::NB][2], int lane, int j0, int first_last, int group,
                               int rows, int rt0) {
    using C = Cfg<D, RT>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    // With several row tiles q is read from LDS per block.  The offset is
    // made opaque so that the compiler does not hoist those loop-invariant
    // reads out of the chunk loop (which would pin all of q in registers).
    int qoff = lane;
    if (RT > 1) asm volatile("" : "+v"(qoff));
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
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
        if ((b & 1) == 0) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                kr[tt] = *reinterpret_cast<const u32x4*>(L.k + (tt * C::KL + b / 2) * 1024 + lane * 16);
        }
        half8 kb[2];
        float ksc[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            kb[tt] = (b & 1) ? k_codes_to_half(kr[tt].z, kr[tt].w) : k_codes_to_half(kr[tt].x, kr[tt].y);
            const half2v sw = as_h2(ksw[tt][b / 2]);
            ksc[tt] = (b & 1) ? (float)sw.y : (float)sw.x;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            // one row tile: q lives in registers; more: read it from LDS
            const half8 qh = RT == 1 ? qreg[b][0] : qlds[((rt * C::NB + b) * 2 + 0) * 64 + qoff];
            const half8 ql = RT == 1 ? qreg[b][1] : qlds[((rt * C::NB + b) * 2 + 1) * 64 + qoff];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh, kb[tt], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, kb[tt], c, 0, 0, 0);
                s[rt][tt] += ksc[tt] * c;
            }
        }
        SCHED_FENCE();
    }
    // causal / tail mask: key j visible to row r iff j <= first_last + r / group
    if (MASK) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) {
                const int row = logical_row<JJ>(rt0 + rt, 4 * g4 + jj);
                const int last = row >= 0 && row < rows ? first_last + row / group : -1;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    if (j0 + tt * kTile + n16 > last) s[rt][tt][jj] = -INFINITY;
            }
    }
}

// Online softmax over the chunk's scores; writes P to the wave's LDS buffer.
template <int D, int RT, int JJ>
__device__ inline void softmax_step(WaveState<D, RT>& st, floatx4 (&s)[RT][2], float* __restrict__ plds, int lane) {
    using C = Cfg<D, RT>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    float mnew[RT][4];
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            mnew[rt][jj] = row16_max(fmaxf(s[rt][0][jj], s[rt][1][jj]));
            grow |= mnew[rt][jj] > st.m[rt][jj] + kTau;
        }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        // rows whose maximum did not move get alpha = 1: one straight pass
        // over the accumulators per row tile, no per-row branches
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            floatx4 alpha = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
            for (int jj = 0; jj < JJ; ++jj) {
                const bool up = mnew[rt][jj] > st.m[rt][jj];
                alpha[jj] = up ? fast_exp2(st.m[rt][jj] - mnew[rt][jj]) : 1.0f;
                st.l[rt][jj] *= alpha[jj];
                st.m[rt][jj] = up ? mnew[rt][jj] : st.m[rt][jj];
            }
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) st.o[rt][nt] *= alpha;
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            const float mref = (st.m[rt][jj] == -INFINITY ? 0.0f : st.m[rt][jj]) + kTau;
            const float p0 = fast_exp2(s[rt][0][jj] - mref);
            const float p1 = fast_exp2(s[rt][1][jj] - mref);
            st.l[rt][jj] += p0 + p1;
            float* prow = plds + (rt * 16 + 4 * g4 + jj) * kPStride;
            prow[n16] = p0;
            prow[kTile + n16] = p1;
        }
    lds_fence();
}

// O += (P * vscale) Vcodes for the chunk.
template <int D, int RT, bool MASK>
__device__ inline void pv_step(WaveState<D, RT>& st, const Land& L, const float* __restrict__ plds, int lane) {
    using C = Cfg<D, RT>;
    const int g4 = lane >> 4;
    const int n16 = lane & 15;
    uint32_t magic = 0x64006400u;
    asm volatile("" : "+v"(magic));          // keep the constant in a VGPR
    float pf[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float* prow = plds + (rt * 16 + n16) * kPStride + 8 * g4;
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[rt][i] = prow[i];
    }
    u32x4 vr;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
        if ((b & 1) == 0) vr = *reinterpret_cast<const u32x4*>(L.v + (b / 2) * 1024 + lane * 16);
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
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int nt = 2 * b + h;
            const half8 bv = v_codes_to_half(vr[nt % 4], magic);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                st.o[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[rt], bv, st.o[rt][nt], 0, 0, 0);
        }
        SCHED_FENCE();
    }
}

template <int D, int RT, int JJ, int RG>
__global__ __launch_bounds__(kThreadsFor<RT>) void attn_mfma_stream_kernel(AttnArgs a, int cps, int n_splits,
                                                                           int group, int rows) {
    using C = Cfg<D, RT>;
    constexpr int W = C::W;
    // RG row groups of RT*16 rows; the WPG waves of group gi share its rows
    // and deal its chunks among themselves.  Every group streams the same
    // chunks, so a chunk read by a second group mostly comes from L2.
    constexpr int WPG = W / RG;
    static_assert(RG == 1 || RT == 1, "row groups take one row tile per wave");
    extern __shared__ __align__(16) uint8_t smem[];
    const Geom& g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave: scalar
    const int split = blockIdx.x % n_splits;
    const int kvh = blockIdx.x / n_splits;
    const int total_chunks = (a.ctx + kChunk - 1) / kChunk;
    const int first_last = a.ctx - a.n_q;             // last key of query 0

    // LDS: [Q hi/lo | per wave: landing zone + P buffer] (reused by the final
    // combine) | [m, l per wave and row]
    half8* qlds = reinterpret_cast<half8*>(smem);
    uint8_t* wbase = smem + C::Q_BYTES + wave * C::WAVE_BYTES;
    const Land land = {wbase, wbase + C::LAND_K, wbase + C::LAND_K + C::LAND_KS,
                       wbase + C::LAND_K + C::LAND_KS + C::LAND_V};
    float* plds = reinterpret_cast<float*>(wbase + C::LAND_K + C::LAND_KS + C::LAND_V + C::LAND_VS);
    float* mls = reinterpret_cast<float*>(smem + C::MAIN_BYTES);     // [wave][RT*16][2]

    // ---- this wave's chunks: wave g of the KV head takes chunks g, g + N,
    // g + 2N, ... (N waves per head), so all waves sweep the context together
    // and the addresses in flight at any time stay close (better DRAM and
    // translation locality than one contiguous run per wave).  Start the
    // first loads before staging q.
    const int gi = wave / WPG, wig = wave % WPG;
    const int stride = n_splits * WPG;
    const int c0 = split * WPG + wig;
    const int c1 = total_chunks;
    (void)cps;
    // Page-table entries: lane k of `ents` holds the entry of the wave's
    // chunk number kb + k (batches of 64, one gather load per batch), and the
    // loop picks them out with readlane -- no memory access, hence no wait,
    // between the K/V requests in flight.
    auto load_ents = [&](int kb) -> int {
        const int ck = c0 + (kb + lane) * stride;
        return ck < c1 ? a.page_table[(ck * kChunk) / g.P] : -1;
    };
    auto unit_at = [&](int phys, bool& ok) -> const uint8_t* {
        ok = phys >= 0 && phys < g.n_pages;
        return a.pool + g.unit_index(ok ? phys : 0, kvh) * g.unit_bytes();
    };
    int ents = load_ents(0);
    bool ok_cur = false;
    if (c0 < c1) {
        const uint8_t* u0 = unit_at(__builtin_amdgcn_readlane(ents, 0), ok_cur);
        if (ok_cur) {
            issue_k<D, RT>(land, u0, g, (c0 * kChunk) % g.P, lane);
            issue_v<D, RT>(land, u0, g, (c0 * kChunk) % g.P, lane);
        }
    }

    // ---- q as fp16 hi/lo in the MFMA A layout, pre-scaled by scale*log2(e):
    // one row tile per wave is loaded straight into the wave's registers
    // (lane l: row of MFMA row l % 16, dims 8 (l / 16) .. +7 of each block);
    // several row tiles are staged in LDS and read per block.
    const float qscale = a.scale * kLog2e;
    half8 qreg[C::NB][2];
    if (RT == 1) {
        const int row = logical_row<JJ>(gi, lane & 15);
        const bool ok = row >= 0 && row < rows;
        const int qi = ok ? row / group : 0, h = kvh * group + (ok ? row % group : 0);
        const float* src = a.q + ((size_t)qi * a.n_heads + h) * D + 8 * (lane >> 4);
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = src[b * kBlock + i];          // in bounds: rows past the end read row 0
                const float x = ok ? v * qscale : 0.0f;
                qreg[b][0][i] = (_Float16)x;
                qreg[b][1][i] = (_Float16)(x - (float)qreg[b][0][i]);
            }
    } else {
        for (int e = threadIdx.x; e < RT * C::NB * 64; e += W * 64) {
            const int l = e & 63, rb = e >> 6, b = rb % C::NB, rt = rb / C::NB;
            const int row = logical_row<JJ>(rt, l & 15);
            half8 hi, lo;
            if (row >= 0 && row < rows) {
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
    }

    WaveState<D, RT> st;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) { st.m[rt][jj] = -INFINITY; st.l[rt][jj] = 0.0f; }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) st.o[rt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- stream: K(c+1) is requested after QK(c), V(c+1) after PV(c).  A
    // page-table entry outside the pool stops the wave (nothing is loaded
    // from it) and turns its partial into NaN.
    bool bad = c0 < c1 && !ok_cur;
    for (int c = c0, k = 0; c < c1 && !bad; c += stride, ++k) {
        const int j0 = c * kChunk;
        const bool mask = j0 + kChunk - 1 > first_last;
        const bool has_next = c + stride < c1;
        if (has_next && ((k + 1) & 63) == 0) {  // every 64 chunks
            ents = load_ents(k + 1);
            asm volatile("" : "+v"(ents));      // consume it here, so the loop's other path has nothing to wait for
        }
        bool ok_next = false;
        const uint8_t* u_next = has_next ? unit_at(__builtin_amdgcn_readlane(ents, (k + 1) & 63), ok_next) : nullptr;
        const int slot_next = ((c + stride) * kChunk) % g.P;
        floatx4 s[RT][2];
        vm_wait<C::V_ISSUES>();                 // K(c) landed (V(c) may still fly)
        if (mask) qk_step<D, RT, JJ, true>(s, land, qlds, qreg, lane, j0, first_last, group, rows, gi);
        else qk_step<D, RT, JJ, false>(s, land, qlds, qreg, lane, j0, first_last, group, rows, gi);
        lds_fence();                            // K(c) read out: the zone is free
        if (ok_next) issue_k<D, RT>(land, u_next, g, slot_next, lane);
        softmax_step<D, RT, JJ>(st, s, plds, lane);
        if (ok_next) vm_wait<C::K_ISSUES>(); else vm_wait<0>();   // V(c) landed
        if (mask) pv_step<D, RT, true>(st, land, plds, lane);
        else pv_step<D, RT, false>(st, land, plds, lane);
        lds_fence();                            // V(c) read out
        if (ok_next) issue_v<D, RT>(land, u_next, g, slot_next, lane);
        if (c + stride < c1 && !ok_next) bad = true;
    }
    vm_wait<0>();

    // ---- finish the row sums, combine the W waves in a fixed order
    const int g4 = lane >> 4, n16 = lane & 15;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            st.l[rt][jj] = row16_sum(st.l[rt][jj]) * 16.0f;        // weights carried 2^-kTau
            if (bad) { st.m[rt][jj] = NAN; st.l[rt][jj] = NAN; }
            if (n16 == 0) {
                const int row = 16 * rt + 4 * g4 + jj;
                mls[(wave * RT * 16 + row) * 2 + 0] = st.m[rt][jj];
                mls[(wave * RT * 16 + row) * 2 + 1] = st.l[rt][jj];
            }
        }
    __syncthreads();                       // every wave is done with its landing zone
    float M[RT][4], Ltot[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            const int row = 16 * rt + 4 * g4 + jj;
            float mm = -INFINITY;
#pragma unroll
            for (int j = 0; j < WPG; ++j) mm = fmaxf(mm, mls[((gi * WPG + j) * RT * 16 + row) * 2]);
            float lt = 0.0f;
#pragma unroll
            for (int j = 0; j < WPG; ++j) {
                const int w = gi * WPG + j;
                const float mw = mls[(w * RT * 16 + row) * 2], lw = mls[(w * RT * 16 + row) * 2 + 1];
                lt += lw == 0.0f ? 0.0f : lw * exp2f(mw - mm);
            }
            M[rt][jj] = mm;
            Ltot[rt][jj] = lt;
            const float f = st.l[rt][jj] == 0.0f ? 0.0f : exp2f(st.m[rt][jj] - mm);
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) st.o[rt][nt][jj] *= f;
        }
    float* ob = reinterpret_cast<float*>(smem);          // [W/2][RT*16][D]
    auto put = [&](int slot) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
                for (int jj = 0; jj < JJ; ++jj)
                    ob[((size_t)slot * RT * 16 + 16 * rt + 4 * g4 + jj) * D + 16 * nt + n16] = st.o[rt][nt][jj];
    };
    auto add = [&](int slot) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
                for (int jj = 0; jj < JJ; ++jj)
                    st.o[rt][nt][jj] += ob[((size_t)slot * RT * 16 + 16 * rt + 4 * g4 + jj) * D + 16 * nt + n16];
    };
    // tree inside each row group: waves [h, 2h) of the group hand their sums
    // to waves [0, h), h = WPG/2 .. 1; group gi uses buffer slots
    // gi*WPG/2 .. (gi+1)*WPG/2 - 1
#pragma unroll
    for (int h = WPG / 2; h >= 1; h /= 2) {
        if (wig >= h && wig < 2 * h) put(gi * (WPG / 2) + wig - h);
        __syncthreads();
        if (wig < h) add(gi * (WPG / 2) + wig);
        __syncthreads();
    }
    if (wig != 0) return;

    // ---- write the partial of each row this workgroup serves
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            const int row = logical_row<JJ>(gi + rt, 4 * g4 + jj);
            if (row < 0 || row >= rows) continue;
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

template <int D, int RT, int JJ, int RG>
hipError_t launch_dr(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    using C = Cfg<D, RT>;
    auto kern = attn_mfma_stream_kernel<D, RT, JJ, RG>;
    if (C::LDS_BYTES > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
        if (e != hipSuccess) return e;
    }
    dim3 grid(pl.n_splits * a.g.n_kv);
    hipLaunchKernelGGL(kern, grid, dim3(C::W * 64), C::LDS_BYTES, stream, a, pl.chunks_per_split, pl.n_splits,
                       pl.group, pl.rows);
    return hipGetLastError();
}

// One row tile per wave: up to 8 rows two per lane group (JJ = 2), up to
// 16 rows one per MFMA row, more rows in 2 or 4 row groups.
template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    if (pl.rows <= 8) return launch_dr<D, 1, 2, 1>(a, pl, stream);
    if (pl.rows <= 16) return launch_dr<D, 1, 4, 1>(a, pl, stream);
    if (pl.rows <= 32) return launch_dr<D, 1, 4, 2>(a, pl, stream);
    if (pl.rows <= 64) return launch_dr<D, 1, 4, 4>(a, pl, stream);
    return hipErrorInvalidValue;
}

}  // namespace

int mfma_stream_row_groups(int rows) { return rows <= 16 ? 1 : rows <= 32 ? 2 : 4; }
int mfma_stream_waves(int rows) { return 8 / mfma_stream_row_groups(rows); }

hipError_t launch_attn_mfma_stream(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    switch (a.g.D) {
        case 64: return launch_d<64>(a, pl, stream);
        case 128: return launch_d<128>(a, pl, stream);
        case 256: return launch_d<256>(a, pl, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
