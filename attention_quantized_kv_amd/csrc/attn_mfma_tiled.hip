// attn_mfma_tiled.hip -- chunked prefill attention over the Q8_0-K / Q4_0-V
// cache on gfx950 matrix cores ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070
// XT at 262k context, via adaptive KV streaming", second paragraph: chunked
// prefill over streamed pages with online log-sum-exp accumulation; "Context
// window and KV cache", GQA section: the q heads of a group share one KV head).
//
// Work split.  A workgroup owns 128 query rows of one KV head (row = query i
// times the G heads of the group, query-major) and one contiguous run of
// 32-token chunks; each of its 128 / (16 RT) wavefronts owns RT tiles of 16
// rows (RT = 1 is built: 8 waves, two per SIMD).  Every K/V fragment a wave
// reads from LDS serves all its RT row tiles.
// Splits of the key range are merged afterwards by lse_merge.hip (with a
// single split the kernel writes the normalised output itself).
//
// Per 32-token chunk, shared by the whole workgroup:
//  * the raw chunk arrives by direct-to-LDS loads (one contiguous 1 KiB wave
//    request each) in a ring of kRing slots, requested kRing chunks ahead so
//    that the loads of two chunks are in flight behind the math, at no VGPR
//    cost;
//  * the threads then convert it into one of two LDS stages (the math of the
//    chunk before reads the other): K codes exactly to fp16 (int8 -> fp16 is
//    exact, the scale stays apart), V to (c - 8) * scale as an exact fp16
//    hi + lo pair, laid out as the MFMA operand fragments the waves read with
//    one 16-byte LDS load.  A wave with rows runs its share of this between
//    its PV products of the chunk before (its raw inputs read one product
//    group ahead), so that the VALU work partly hides under the matrix core;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_f16, one K = 32 step per quant block:
//    the block's scale multiplies the fp32 result per key (fma_mix), and q is
//    split into fp16 hi + lo parts (two MFMAs), so every score is the exact
//    dot product up to fp32 accumulation.  With keys on the MFMA M axis each
//    lane owns one query row: the row max needs only two cross-row lane swaps
//    and P comes out already in the B-operand layout of O^T = V^T P^T;
//  * online softmax in the log2 domain (q carries scale * log2 e) with lazy
//    rescaling: the reference max moves only when a chunk beats it by more
//    than kTau, so weights stay <= 2^kTau and fp16 P cannot overflow;
//  * O^T += V^T P^T with P and V each split into fp16 hi + lo (three MFMAs per
//    tile; lo*lo is below 2^-22).  Rounding either factor to one fp16 leaves
//    errors of 2^-12 of |v| per weight, which the output tolerance does not
//    absorb when a few large values nearly cancel.
#include <hip/hip_fp16.h>

#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kRowsPerWg = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 4.0f;
constexpr int kRing = 4;         // raw chunks in flight per workgroup (direct-to-LDS ring); a power of 2

template <int RT>
constexpr int kThreadsFor = kRowsPerWg / (16 * RT) * 64;

template <int D, int RT, int CODEC>
struct TCfg {
    static constexpr int W = kRowsPerWg / (16 * RT);   // waves per workgroup
    static constexpr int THREADS = W * 64;
    static constexpr int NB = D / kBlock;       // 32-dim MFMA steps (quant blocks of Q8_0/Q4_0)
    static constexpr int NB2 = D / kBlock2;     // 128-value INT2 blocks
    static constexpr int NT = D / 16;           // 16-wide output dim tiles
    static constexpr int KL = D / 64;           // 1 KiB pieces per K tile / V chunk
    static constexpr int K_FRAG = 2 * NB * 64 * 16;   // [tile][step][lane] x 16 B
    static constexpr int KS = 2 * NB * 16 * 2;        // [tile][step][16 keys] fp16 (INT2: the 128-block's d per step)
    static constexpr int KZ = CODEC == 1 ? 2 * NB2 * 16 * 2 : 0;   // INT2: [tile][block][16 keys] fp16 zero-points
    static constexpr int V_FRAG = NT * 64 * 16;       // [dim tile][lane] x 16 B, hi then lo parts
    static constexpr int STAGE = K_FRAG + KS + KZ + 2 * V_FRAG;
    // raw chunk as it arrives by direct-to-LDS loads, one 1 KiB wave request
    // each.  Q8_0/Q4_0: [K tiles 2KL][K scales 1][V pieces KL][V scales 1].
    // INT2: [K codes 8D/1024][V codes 8D/1024][parameters 1]: K (scale, zero)
    // [32 tokens][NB2][2], V scales [NB2][32], V zeros [NB2][32] (fp16).
    static constexpr int CR = 8 * D / 1024;           // INT2: 1 KiB requests per code region
    static constexpr int N_DMA = CODEC == 1 ? 2 * CR + 1 : 3 * KL + 2;
    static constexpr int ND = (N_DMA + W - 1) / W;    // requests per wave and chunk
    static constexpr int SLOT = N_DMA * 1024;
    static constexpr int OFF_KS = 2 * KL * 1024, OFF_V = OFF_KS + 1024, OFF_VS = OFF_V + KL * 1024;
    static constexpr int I2_V = 8 * D, I2_P = 16 * D;                 // INT2 raw offsets: V codes, parameters
    static constexpr int I2_VS = I2_P + 128 * NB2, I2_VZ = I2_VS + 64 * NB2;
    static constexpr int LDS = 2 * STAGE + kRing * SLOT;
    static constexpr int K_ITEMS = 128 * KL;    // 16-byte K-code pieces per chunk
    static constexpr int KS_ITEMS = 4 * NB;     // 16-byte K-scale pieces per chunk
    static_assert(KS_ITEMS <= THREADS, "one K-scale piece per thread");
    static_assert(CODEC == 0 || (D % 128 == 0 && 32 * NB2 <= THREADS), "INT2: head_dim 128 or 256");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Reinterprets 32 bits as two fp16 values.  Takes the bits by value: hipcc's
// __builtin_bit_cast applied directly to a vector element (v.y, v[1]) reads
// element 0 instead.
__device__ inline half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }

// 8 int8 codes -> 8 fp16 values, exactly (bias by 128, put each byte under
// the fp16 exponent of 1024, subtract 1152).
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

// Byte M of x holds the codes of two consecutive tokens (low nibble first).
// Sets hi + lo = ((c_lo - 8) * s.x, (c_hi - 8) * s.y) exactly: the low
// nibble lands under the exponent of 1024 in the low half, the high nibble
// (times 16) in the high half, an exact FMA recovers c - 8; the product has at
// most 15 significant bits, so hi = fp16(product) and the FMA residual
// lo = product - hi are both exact.
template <int M>
__device__ inline void v_pair(uint32_t x, half2v s, uint32_t magic, half2v& hi, half2v& lo) {
    const uint32_t t = __builtin_amdgcn_perm(x, x, 0x01010101u * M);
    const half2v h = __builtin_bit_cast(half2v, (t & 0x00F0000Fu) | magic);
    const half2v mul = {(_Float16)1.0f, (_Float16)0.0625f};
    const half2v add = {(_Float16)-1032.0f, (_Float16)-72.0f};
    const half2v c = h * mul + add;
    hi = c * s;
    lo = __builtin_elementwise_fma(c, s, -hi);
}

// Lanes l, l^16, l^32, l^48 hold one query row.  v_permlane16_swap a, b
// swaps a's odd 16-lane rows with b's even rows; with a = b = x that leaves
// (x0 x0 x2 x2) in a and (x1 x1 x3 x3) in b, and v_permlane32_swap does the
// same for the 32-lane halves.  Written as inline asm: the compiler's
// optimiser folds the builtin's second result into its first.
__device__ inline void swap16(float x, float& r0, float& r1) {
    r0 = x;
    r1 = x;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(r0), "+v"(r1));
}
__device__ inline void swap32(float x, float& r0, float& r1) {
    r0 = x;
    r1 = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(r0), "+v"(r1));
}

// max / sum over the four lanes of a query row
__device__ inline float xmax4(float x) {
    float a, b;
    swap16(x, a, b);
    swap32(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}

__device__ inline float xsum4(float x) {
    float a, b;
    swap16(x, a, b);
    swap32(a + b, a, b);
    return a + b;
}

#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// 16 bytes per lane, global -> LDS: lane i's bytes land at lds + 16 i.
__device__ inline void dma16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds, 16, 0, 0);
}

// Waits until at most N vector-memory requests of this wave are outstanding
// (direct-to-LDS loads count); also a compiler memory fence.
template <int N>
__device__ inline void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Workgroup barrier for LDS data: waits for this wave's own LDS accesses,
// then s_barrier.  Unlike __syncthreads() it carries no release fence, which
// would also wait for every direct-to-LDS load still in flight (the ring's
// later chunks); each wave waits for the loads that must have landed with an
// explicit vm_wait before it.  The empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The raw chunk's N_DMA wave requests are dealt to the waves (wave w takes
// requests w, w + W, ...); waves left over repeat an earlier request, so
// every wave issues exactly ND of them and the wait counts are the same for
// all.  Every request runs on the full wave (a direct-to-LDS load under a
// lane-dependent branch can get its LDS base merged with another one's): the
// scale pieces, 4*NB of 16 bytes, are repeated across the remaining lanes.
// A request's source is unit + off + mul * slot0, with off and mul fixed per
// wave (computed once), slot0 = the chunk's first slot in its page.
template <int D, int RT, int CODEC>
struct Requests {
    using C = TCfg<D, RT, CODEC>;
    int64_t off[C::ND];
    int mul[C::ND];
    int dst[C::ND];

    __device__ Requests(const Geom& g, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < C::ND; ++j) {
            int item = j * C::W + wave;
            while (item >= C::N_DMA) item -= C::N_DMA;
            dst[j] = item * 1024;
            if constexpr (CODEC == 1) {
                if (item < C::CR) {                         // K codes, piece item (chunk-contiguous)
                    off[j] = (int64_t)item * 1024 + lane * 16;
                    mul[j] = D / 4;
                } else if (item < 2 * C::CR) {              // V codes
                    off[j] = g.i2_v_codes_off() + (int64_t)(item - C::CR) * 1024 + lane * 16;
                    mul[j] = D / 4;
                } else {                                    // parameters: lane pl of 16 NB2
                    const int pl = lane % (16 * C::NB2);
                    if (pl < 8 * C::NB2) {
                        off[j] = g.i2_k_params_off() + 16 * pl;
                        mul[j] = 4 * C::NB2;
                    } else if (pl < 12 * C::NB2) {
                        off[j] = g.i2_v_scales_off() + 16 * (pl - 8 * C::NB2);
                        mul[j] = 2 * C::NB2;
                    } else {
                        off[j] = g.i2_v_zeros_off() + 16 * (pl - 12 * C::NB2);
                        mul[j] = 2 * C::NB2;
                    }
                }
                continue;
            }
            if (item < 2 * C::KL) {                     // K codes: tile tt, piece p
                const int tt = item / C::KL, pc = item % C::KL;
                off[j] = (int64_t)tt * kTile * D + pc * 1024 + lane * 16;
                mul[j] = D;                             // (slot0 / 16) * 16 * D
            } else if (item == 2 * C::KL) {             // K scales [token][block]
                off[j] = g.k_scales_off() + (lane % (4 * C::NB)) * 16;
                mul[j] = C::NB * 2;
            } else if (item < 3 * C::KL + 1) {          // V codes: piece u
                off[j] = g.v_codes_off() + (item - 2 * C::KL - 1) * 1024 + lane * 16;
                mul[j] = D / 2;                         // (slot0 / 32) * 32 * D / 2
            } else {                                    // V scales [block][32]
                off[j] = g.v_scales_off() + (lane % (4 * C::NB)) * 16;
                mul[j] = C::NB * 2;                     // (slot0 / 32) * NB * 32 * 2
            }
        }
    }

    __device__ inline void issue(uint8_t* slot, const uint8_t* unit, int slot0) const {
#pragma unroll
        for (int j = 0; j < C::ND; ++j) dma16(unit + off[j] + (int64_t)mul[j] * slot0, slot + dst[j]);
    }
};

// Converts one raw chunk (ring slot) into a stage's operand fragments.
//  K: K piece (tile, p), lane L: 16 codes -> the fp16 fragments of blocks 2p
//     and 2p+1 at lane L (the raw layout already is the fragment layout).
//  V: V fragment (dim tile nt, lane fl = 16 G + n) holds dim 16 nt + n of the
//     keys {4G..4G+3, 16+4G..16+4G+3} (the key order of the P fragment), as
//     hi and lo fp16 parts; those keys are nibbles 4(G%2)..+3 of two raw
//     dwords.  Consecutive threads take consecutive fragments of a dim tile,
//     so the 16-byte stores are conflict-free.
//  K scales: thread t < 4*NB spreads 8 of them to [tile][block][16 keys].
// kvalid: tokens of the chunk that exist (< ctx); V of the others is zeroed so
// that a masked key (weight 0) cannot meet an unwritten, non-finite scale.
// The work is cut into parts, one pass of the threads over K items (it < KI),
// V items (KI <= it < KI + VI) or the scales (the last part), so that a wave
// can run the parts of the next chunk between the products of this one.
template <int D, int RT, int CODEC>
struct Parts {
    using C = TCfg<D, RT, CODEC>;
    static constexpr int K_N = CODEC == 1 ? 2 * C::NB * 64 : C::K_ITEMS;
    static constexpr int V_N = C::NT * 64;
    static constexpr int KI = (K_N + C::THREADS - 1) / C::THREADS;
    static constexpr int VI = (V_N + C::THREADS - 1) / C::THREADS;
    static constexpr int N = KI + VI + 1;
};

// Raw inputs of one part (read from the ring slot), kept in registers between
// the LDS reads and the arithmetic that consumes them.
struct PartRaw {
    uint32_t w[10];
};

template <int D, int RT, int CODEC, bool FULL = false>
__device__ inline void convert_part(int part, const uint8_t* slot, uint8_t* stage, int t, int kvalid);

// INT2 operands come out of the fp4 conversion (see part_store_int2) with
// elements 1 and 2 of every group of 4 swapped: operand element e holds item
// i2_slot(e) (an involution), for the dims of a K fragment (so q is staged in
// that order) and the keys of a V fragment (so P is too).
__host__ __device__ constexpr int i2_slot(int e) { return (e & ~3) | ((e & 1) << 1) | ((e >> 1) & 1); }

// INT2 (the same stage layout; K codes exact, the scale per 128-value block
// replicated over its four 32-dim steps, zero-points apart, V = z + d c).
// A 2-bit code zero-extended to a nibble is the fp4 (e2m1) value code/2, and
// gfx950 converts two fp4 values into two fp16 (times a scale) at once: a
// dword spread into nibbles (x & 0x33333333, (x >> 2) & 0x33333333) gives,
// byte by byte, codes in the order i2_slot.
//  K: fragment (tile tt, step s, lane L = 16 g + n) = dims 32 s + 8 g + i2_slot(e)
//     of token 16 tt + n: word s of lane L's raw K bytes (code e at bit
//     16 (e/4) + 8 (s%2) + 2 (e%4) of its dword), bytes s%2 and 2 + s%2 of the
//     nibbles.
//  V: fragment (dim tile nt, lane fl = 16 G + n): dim 16 nt + n of keys
//     4G + i2_slot(i) and 16 + 4G + i2_slot(i); the four codes of each key
//     group are one byte of one raw dword.  hi + lo of z + d c (fp32).
//  Scales and zero-points: thread t < 32 NB2 takes (token, block).
template <int D, int RT>
__device__ inline void part_load_int2(int part, const uint8_t* slot, int t, PartRaw& r) {
    using C = TCfg<D, RT, 1>;
    using PP = Parts<D, RT, 1>;
    if (part < PP::KI) {
        const int item = part * C::THREADS + t;
        if (PP::K_N % C::THREADS != 0 && item >= PP::K_N) return;
        const int tt = item / (C::NB * 64), st = (item / 64) % C::NB, L = item % 64;
        r.w[0] = *reinterpret_cast<const uint32_t*>(slot + tt * (kTile * D / 4) + L * (D / 16) + (st / 2) * 4);
    } else if (part < PP::KI + PP::VI) {
        const int item = (part - PP::KI) * C::THREADS + t;
        if (PP::V_N % C::THREADS != 0 && item >= PP::V_N) return;
        const int nt = item / 64, fl = item % 64, G = fl / 16, n = fl % 16, b = nt / 8;
        // keys 4G.. (raw lane group G/2), 16+4G.. (group 2+G/2)
        const uint8_t* vraw = slot + C::I2_V + n * (D / 8) + (nt / 2) * 4;
        r.w[0] = *reinterpret_cast<const uint32_t*>(vraw + (G / 2) * 16 * (D / 8));
        r.w[1] = *reinterpret_cast<const uint32_t*>(vraw + (2 + G / 2) * 16 * (D / 8));
        const uint8_t* vs = slot + C::I2_VS + b * kChunk * 2;
        const uint8_t* vz = slot + C::I2_VZ + b * kChunk * 2;
        const u32x2 s0 = *reinterpret_cast<const u32x2*>(vs + 8 * G), s1 = *reinterpret_cast<const u32x2*>(vs + 32 + 8 * G);
        const u32x2 z0 = *reinterpret_cast<const u32x2*>(vz + 8 * G), z1 = *reinterpret_cast<const u32x2*>(vz + 32 + 8 * G);
        r.w[2] = s0.x; r.w[3] = s0.y; r.w[4] = s1.x; r.w[5] = s1.y;
        r.w[6] = z0.x; r.w[7] = z0.y; r.w[8] = z1.x; r.w[9] = z1.y;
    } else if (t < kChunk * C::NB2) {
        const int tok = t / C::NB2, b = t % C::NB2;
        r.w[0] = *reinterpret_cast<const uint32_t*>(slot + C::I2_P + (tok * C::NB2 + b) * 4);
    }
}

template <int D, int RT, bool FULL>
__device__ inline void part_store_int2(int part, const PartRaw& r, uint8_t* stage, int t, int kvalid) {
    using C = TCfg<D, RT, 1>;
    using PP = Parts<D, RT, 1>;
    uint8_t* kf = stage;
    _Float16* ksl = reinterpret_cast<_Float16*>(stage + C::K_FRAG);
    _Float16* kzl = reinterpret_cast<_Float16*>(stage + C::K_FRAG + C::KS);
    uint8_t* vf = stage + C::K_FRAG + C::KS + C::KZ;
    if (part < PP::KI) {
        const int item = part * C::THREADS + t;
        if (PP::K_N % C::THREADS != 0 && item >= PP::K_N) return;
        const int tt = item / (C::NB * 64), st = (item / 64) % C::NB, L = item % 64;
        const uint32_t x = r.w[0];
        const uint32_t n0 = x & 0x33333333u, n1 = (x >> 2) & 0x33333333u;
        half2v a, b, c, d;
        if (st & 1) {                            // uniform: 64 items per wave share st
            a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n0, 2.0f, 1);
            b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n1, 2.0f, 1);
            c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n0, 2.0f, 3);
            d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n1, 2.0f, 3);
        } else {
            a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n0, 2.0f, 0);
            b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n1, 2.0f, 0);
            c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n0, 2.0f, 2);
            d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n1, 2.0f, 2);
        }
        *reinterpret_cast<half8*>(kf + ((tt * C::NB + st) * 64 + L) * 16) =
            half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
    } else if (part < PP::KI + PP::VI) {
        const int item = (part - PP::KI) * C::THREADS + t;
        if (PP::V_N % C::THREADS != 0 && item >= PP::V_N) return;
        const int nt = item / 64, fl = item % 64, G = fl / 16;
        const int sh = 16 * (G % 2) + 8 * (nt % 2);
        // keys 4G.. in byte 0, 16+4G.. in byte 1
        const uint32_t w = ((r.w[0] >> sh) & 0xFFu) | (((r.w[1] >> sh) & 0xFFu) << 8);
        const uint32_t n0 = w & 0x3333u, n1 = (w >> 2) & 0x3333u;
        const half2v c01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n0, 2.0f, 0);
        const half2v c23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n1, 2.0f, 0);
        const half2v c45 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n0, 2.0f, 1);
        const half2v c67 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n1, 2.0f, 1);
        const half8 code = {c01.x, c01.y, c23.x, c23.y, c45.x, c45.y, c67.x, c67.y};
        const half4 s0 = __builtin_bit_cast(half4, u32x2{r.w[2], r.w[3]}), s1 = __builtin_bit_cast(half4, u32x2{r.w[4], r.w[5]});
        const half4 z0 = __builtin_bit_cast(half4, u32x2{r.w[6], r.w[7]}), z1 = __builtin_bit_cast(half4, u32x2{r.w[8], r.w[9]});
        half8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ki = i2_slot(e % 4);
            const int key = (e < 4 ? 4 * G : 16 + 4 * G) + ki;
            const _Float16 sv = e < 4 ? s0[ki] : s1[ki], zv = e < 4 ? z0[ki] : z1[ki];
            const float v = FULL || key < kvalid ? fmaf((float)sv, (float)code[e], (float)zv) : 0.0f;
            hi[e] = (_Float16)v;
            lo[e] = (_Float16)(v - (float)hi[e]);
        }
        *reinterpret_cast<half8*>(vf + (nt * 64 + fl) * 16) = hi;
        *reinterpret_cast<half8*>(vf + C::V_FRAG + (nt * 64 + fl) * 16) = lo;
    } else if (t < kChunk * C::NB2) {
        const int tok = t / C::NB2, b = t % C::NB2;
        const half2v dz = as_h2(r.w[0]);
        const int tt = tok / kTile, key = tok % kTile;
#pragma unroll
        for (int st = 4 * b; st < 4 * b + 4; ++st) ksl[(tt * C::NB + st) * kTile + key] = dz.x;
        kzl[(tt * C::NB2 + b) * kTile + key] = dz.y;
    }
}

template <int D, int RT, int CODEC>
__device__ inline void part_load(int part, const uint8_t* slot, int t, PartRaw& r) {
    if constexpr (CODEC == 1) {
        part_load_int2<D, RT>(part, slot, t, r);
        return;
    }
    using C = TCfg<D, RT, CODEC>;
    using PP = Parts<D, RT, CODEC>;
    if (part < PP::KI) {
        const int item = part * C::THREADS + t;
        if (C::K_ITEMS % C::THREADS != 0 && item >= C::K_ITEMS) return;
        const int tt = item / (64 * C::KL), pc = (item / 64) % C::KL, L = item % 64;
        const u32x4 k = *reinterpret_cast<const u32x4*>(slot + (tt * C::KL + pc) * 1024 + L * 16);
        r.w[0] = k.x; r.w[1] = k.y; r.w[2] = k.z; r.w[3] = k.w;
    } else if (part < PP::KI + PP::VI) {
        const int item = (part - PP::KI) * C::THREADS + t;
        if (PP::V_N % C::THREADS != 0 && item >= PP::V_N) return;
        const int nt = item / 64, fl = item % 64, G = fl / 16, n = fl % 16;
        const int u = nt / 4, w = nt % 4, b = nt / 2;
        const uint8_t* vraw = slot + C::OFF_V + u * 1024 + n * 16 + w * 4;
        r.w[0] = *reinterpret_cast<const uint32_t*>(vraw + (G / 2) * 256);         // tokens 8(G/2)..
        r.w[1] = *reinterpret_cast<const uint32_t*>(vraw + (2 + G / 2) * 256);     // tokens 16+8(G/2)..
        const u32x2 s1 = *reinterpret_cast<const u32x2*>(slot + C::OFF_VS + (b * kChunk + 4 * G) * 2);
        const u32x2 s2 = *reinterpret_cast<const u32x2*>(slot + C::OFF_VS + (b * kChunk + 16 + 4 * G) * 2);
        r.w[2] = s1.x; r.w[3] = s1.y; r.w[4] = s2.x; r.w[5] = s2.y;
    } else if (t < C::KS_ITEMS) {
        const u32x4 h = *reinterpret_cast<const u32x4*>(slot + C::OFF_KS + t * 16);
        r.w[0] = h.x; r.w[1] = h.y; r.w[2] = h.z; r.w[3] = h.w;
    }
}

template <int D, int RT, int CODEC, bool FULL>
__device__ inline void part_store(int part, const PartRaw& r, uint8_t* stage, int t, int kvalid) {
    if constexpr (CODEC == 1) {
        part_store_int2<D, RT, FULL>(part, r, stage, t, kvalid);
        return;
    }
    using C = TCfg<D, RT, CODEC>;
    using PP = Parts<D, RT, CODEC>;
    uint8_t* kf = stage;
    _Float16* ksl = reinterpret_cast<_Float16*>(stage + C::K_FRAG);
    uint8_t* vf = stage + C::K_FRAG + C::KS;
    if (part < PP::KI) {
        const int item = part * C::THREADS + t;
        if (C::K_ITEMS % C::THREADS != 0 && item >= C::K_ITEMS) return;
        const int tt = item / (64 * C::KL), pc = (item / 64) % C::KL, L = item % 64;
        *reinterpret_cast<half8*>(kf + ((tt * C::NB + 2 * pc) * 64 + L) * 16) = k_codes_to_half(r.w[0], r.w[1]);
        *reinterpret_cast<half8*>(kf + ((tt * C::NB + 2 * pc + 1) * 64 + L) * 16) = k_codes_to_half(r.w[2], r.w[3]);
    } else if (part < PP::KI + PP::VI) {
        const int item = (part - PP::KI) * C::THREADS + t;
        if (PP::V_N % C::THREADS != 0 && item >= PP::V_N) return;
        uint32_t magic = 0x64006400u;
        asm volatile("" : "+v"(magic));
        const int nt = item / 64, fl = item % 64, G = fl / 16;
        const int sh = 16 * (G % 2);
        const uint32_t y1 = r.w[0] >> sh, y2 = r.w[1] >> sh;    // keys 4G..4G+3 / 16+4G.. in the low 16 bits
        half2v h0, h1, h2, h3, l0, l1, l2, l3;
        v_pair<0>(y1, as_h2(r.w[2]), magic, h0, l0);
        v_pair<1>(y1, as_h2(r.w[3]), magic, h1, l1);
        v_pair<0>(y2, as_h2(r.w[4]), magic, h2, l2);
        v_pair<1>(y2, as_h2(r.w[5]), magic, h3, l3);
        half8 hi = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
        half8 lo = {l0[0], l0[1], l1[0], l1[1], l2[0], l2[1], l3[0], l3[1]};
        if (!FULL && kvalid < kChunk) {
            const _Float16 z = (_Float16)0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (4 * G + i >= kvalid) { hi[i] = z; lo[i] = z; }
                if (16 + 4 * G + i >= kvalid) { hi[4 + i] = z; lo[4 + i] = z; }
            }
        }
        *reinterpret_cast<half8*>(vf + (nt * 64 + fl) * 16) = hi;
        *reinterpret_cast<half8*>(vf + C::V_FRAG + (nt * 64 + fl) * 16) = lo;
    } else if (t < C::KS_ITEMS) {
        const half8 h = __builtin_bit_cast(half8, u32x4{r.w[0], r.w[1], r.w[2], r.w[3]});
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = 8 * t + i, j = e / C::NB, bb = e % C::NB;
            ksl[((j / kTile) * C::NB + bb) * kTile + j % kTile] = h[i];
        }
    }
}

template <int D, int RT, int CODEC, bool FULL>
__device__ inline void convert_part(int part, const uint8_t* slot, uint8_t* stage, int t, int kvalid) {
    PartRaw r;
    part_load<D, RT, CODEC>(part, slot, t, r);
    part_store<D, RT, CODEC, FULL>(part, r, stage, t, kvalid);
}

template <int D, int RT, int CODEC>
__device__ inline void convert_chunk(const uint8_t* slot, uint8_t* stage, int t, int kvalid) {
#pragma unroll
    for (int part = 0; part < Parts<D, RT, CODEC>::N; ++part) convert_part<D, RT, CODEC>(part, slot, stage, t, kvalid);
}

template <int D, int RT>
struct Rows {
    floatx4 o[RT][D / 16];            // O^T: row tile rt, this lane's row, dims 16 nt + 4 (lane / 16) + i
    float m[RT];                      // reference max (log2 domain), equal on the row's 4 lanes
    float l[RT];                      // this lane's share of the row sum
};

// Orders the instructions of one scheduling region that holds NM matrix
// products and conversion work: two products, then one product per four VALU
// instructions (VALU work issues while independent products run on the
// matrix core), then the rest and the LDS writes.
template <int NM>
__device__ inline void interleave_products() {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // MFMA
#pragma unroll
    for (int i = 2; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 256, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, 32, 0);     // LDS writes
}

// One chunk: S^T = K Q^T, online softmax, O^T += V^T P^T for the wave's RT
// row tiles.  MASK: some key of the chunk lies beyond some row's last key.
// FUSE: the wave also converts the next raw chunk (cslot, whole) into the
// other stage (cstage), its parts spread over the PV products.
template <int D, int RT, int CODEC, bool MASK, bool FUSE>
__device__ inline void chunk_step(Rows<D, RT>& st, const uint8_t* __restrict__ stage,
                                  const half8 (&qh)[RT][D / kBlock], const half8 (&ql)[RT][D / kBlock],
                                  const float (&qsum)[RT][D / kBlock2 > 0 ? D / kBlock2 : 1], int lane, int j0,
                                  const int (&last)[RT], const uint8_t* cslot, uint8_t* cstage, int t) {
    using C = TCfg<D, RT, CODEC>;
    using PP = Parts<D, RT, CODEC>;
    const uint8_t* kf = stage;
    const _Float16* ksl = reinterpret_cast<const _Float16*>(stage + C::K_FRAG);
    const _Float16* kzl = reinterpret_cast<const _Float16*>(stage + C::K_FRAG + C::KS);
    const uint8_t* vf = stage + C::K_FRAG + C::KS + C::KZ;
    const int grp = lane >> 4;
    floatx4 s[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) s[rt][0] = s[rt][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    // Block b+1's fragments are read while block b's products run; hi and lo
    // products of the tiles alternate so that no MFMA waits on the one issued
    // right before it.  Each K fragment serves all RT row tiles.
    half8 ka[2], kn[2];
    half4 ks[2], ksn[2];
    auto load_block = [&](int b, half8 (&k)[2], half4 (&sc)[2]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            k[tt] = *reinterpret_cast<const half8*>(kf + ((tt * C::NB + b) * 64 + lane) * 16);
            sc[tt] = *reinterpret_cast<const half4*>(ksl + (tt * C::NB + b) * kTile + 4 * grp);
        }
    };
    load_block(0, ka, ks);
    // Q8_0/Q4_0: block b's products are scaled and added in block b + 1's
    // region, between that block's hi and lo products, so the lo product
    // issues well after the hi one it accumulates onto and the scaling reads
    // products that have completed (measured faster; over the 2-bit cache,
    // whose zero-point term follows, the same order measured slower).
    constexpr bool LAG = CODEC == 0;
    floatx4 cp[RT][2];
    half4 ksp[2];
    auto fold = [&]() {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[rt][tt][i] = fmaf(cp[rt][tt][i], (float)ksp[tt][i], s[rt][tt][i]);
    };
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
        if (b + 1 < C::NB) load_block(b + 1, kn, ksn);
        floatx4 c[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                c[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[tt], qh[rt][b], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        if (LAG && b > 0) fold();
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                c[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[tt], ql[rt][b], c[rt][tt], 0, 0, 0);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            ksp[tt] = ks[tt];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) cp[rt][tt] = c[rt][tt];
        }
        if (!LAG) fold();
        if (b + 1 < C::NB) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) { ka[tt] = kn[tt]; ks[tt] = ksn[tt]; }
        }
        SCHED_FENCE();      // one block of lookahead, no more (register budget)
    }
    if (LAG) fold();
    if constexpr (CODEC == 1) {
        // the zero-point term of the INT2 keys: z (key, block) times the
        // block's sum of this lane's q row
#pragma unroll
        for (int b = 0; b < C::NB2; ++b)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const half4 z = *reinterpret_cast<const half4*>(kzl + (tt * C::NB2 + b) * kTile + 4 * grp);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[rt][tt][i] = fmaf((float)z[i], qsum[rt][b], s[rt][tt][i]);
            }
    }
    if (MASK) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (j0 + tt * kTile + 4 * grp + i > last[rt]) s[rt][tt][i] = -INFINITY;
    }
    // online softmax (per row tile, this lane: one row, 8 keys)
    half8 ph[RT], pl[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float cm = fmaxf(fmaxf(fmaxf(s[rt][0][0], s[rt][0][1]), fmaxf(s[rt][0][2], s[rt][0][3])),
                         fmaxf(fmaxf(s[rt][1][0], s[rt][1][1]), fmaxf(s[rt][1][2], s[rt][1][3])));
        cm = xmax4(cm);
        const bool grow = cm > st.m[rt] + kTau;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            if (cm > st.m[rt]) {
                const float alpha = __builtin_amdgcn_exp2f(st.m[rt] - cm);
                st.l[rt] *= alpha;
#pragma unroll
                for (int nt = 0; nt < C::NT; ++nt) st.o[rt][nt] *= alpha;
                st.m[rt] = cm;
            }
        }
        const float mref = st.m[rt] == -INFINITY ? 0.0f : st.m[rt];
        // P = ph + pl to about 2^-22 relative (weights are <= 2^kTau)
        float lsum = 0.0f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(s[rt][tt][i] - mref);
                lsum += p;
                const _Float16 h = (_Float16)p;
                const int e = 4 * tt + (CODEC == 1 ? i2_slot(i) : i);   // the V fragment's key order
                ph[rt][e] = h;
                pl[rt][e] = (_Float16)(p - (float)h);
            }
        st.l[rt] += lsum;
    }
    // O^T += V^T P^T with both factors split: hi*hi + hi*lo + lo*hi, four
    // output tiles at a time so that dependent products are 4 RT apart; each
    // V fragment serves all RT row tiles
    constexpr int NG = 4;
    constexpr int NGR = C::NT / NG;                 // groups of output tiles
    constexpr int NP = PP::KI + PP::VI;             // conversion parts under the products
    if constexpr (FUSE) {
        // Registers for one group of fragments only: each is reloaded with
        // the next group's as soon as its last product has been issued.
        half8 vh[NG], vl[NG];
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            vh[i] = *reinterpret_cast<const half8*>(vf + (i * 64 + lane) * 16);
            vl[i] = *reinterpret_cast<const half8*>(vf + C::V_FRAG + (i * 64 + lane) * 16);
        }
        // the parts of group g are read in group g - 1's region (group 0's
        // own parts, if any, in its region)
        PartRaw raw[NP];
#pragma unroll
        for (int part = 0; part < 1 * NP / NGR; ++part) part_load<D, RT, CODEC>(part, cslot, t, raw[part]);
#pragma unroll
        for (int n0 = 0; n0 < C::NT; n0 += NG) {
            const int g = n0 / NG;
#pragma unroll
            for (int part = g * NP / NGR; part < (g + 1) * NP / NGR; ++part)
                part_store<D, RT, CODEC, true>(part, raw[part], cstage, t, kChunk);
#pragma unroll
            for (int part = (g + 1) * NP / NGR; part < (g + 2) * NP / NGR && part < NP; ++part)
                part_load<D, RT, CODEC>(part, cslot, t, raw[part]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < NG; ++i)
                    st.o[rt][n0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[i], ph[rt], st.o[rt][n0 + i], 0, 0, 0);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < NG; ++i)
                    st.o[rt][n0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[i], pl[rt], st.o[rt][n0 + i], 0, 0, 0);
            if (n0 + NG < C::NT) {
#pragma unroll
                for (int i = 0; i < NG; ++i)
                    vh[i] = *reinterpret_cast<const half8*>(vf + ((n0 + NG + i) * 64 + lane) * 16);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < NG; ++i)
                    st.o[rt][n0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl[i], ph[rt], st.o[rt][n0 + i], 0, 0, 0);
            if (n0 + NG < C::NT) {
#pragma unroll
                for (int i = 0; i < NG; ++i)
                    vl[i] = *reinterpret_cast<const half8*>(vf + C::V_FRAG + ((n0 + NG + i) * 64 + lane) * 16);
            }
            interleave_products<3 * NG * RT>();
            SCHED_FENCE();
        }
        convert_part<D, RT, CODEC, true>(PP::N - 1, cslot, cstage, t, kChunk);
        return;
    }
    half8 vh[NG], vl[NG], vhn[NG], vln[NG];
    auto load_group = [&](int n0, half8 (&h)[NG], half8 (&l)[NG]) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            h[i] = *reinterpret_cast<const half8*>(vf + ((n0 + i) * 64 + lane) * 16);
            l[i] = *reinterpret_cast<const half8*>(vf + C::V_FRAG + ((n0 + i) * 64 + lane) * 16);
        }
    };
    load_group(0, vh, vl);
#pragma unroll
    for (int n0 = 0; n0 < C::NT; n0 += NG) {
        if (n0 + NG < C::NT) load_group(n0 + NG, vhn, vln);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < NG; ++i)
                st.o[rt][n0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[i], ph[rt], st.o[rt][n0 + i], 0, 0, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < NG; ++i)
                st.o[rt][n0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[i], pl[rt], st.o[rt][n0 + i], 0, 0, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < NG; ++i)
                st.o[rt][n0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl[i], ph[rt], st.o[rt][n0 + i], 0, 0, 0);
        if (n0 + NG < C::NT) {
#pragma unroll
            for (int i = 0; i < NG; ++i) { vh[i] = vhn[i]; vl[i] = vln[i]; }
        }
        SCHED_FENCE();      // one group of lookahead
    }
}

template <int D, int RT, int CODEC>
__global__ __launch_bounds__(kThreadsFor<RT>) void attn_mfma_tiled_kernel(AttnArgs a, int cps, int n_splits,
                                                                          int group, int rows, int row_tiles) {
    using C = TCfg<D, RT, CODEC>;
    extern __shared__ __align__(16) uint8_t smem[];
    const Geom& g = a.g;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);

    // XCD-aware order: consecutive workgroup ids go to different XCDs, so the
    // ids an XCD receives are remapped to consecutive work items -- the row
    // tiles of one (KV head, split) -- which then share that XCD's L2.
    const int nwg = gridDim.x;
    int w = blockIdx.x;
    if (nwg % 8 == 0) w = (w % 8) * (nwg / 8) + w / 8;
    const int rtile = w % row_tiles;
    const int split = (w / row_tiles) % n_splits;
    const int kvh = w / (row_tiles * n_splits);

    const int total_chunks = (a.ctx + kChunk - 1) / kChunk;
    const int first_last = a.ctx - a.n_q;              // last key of query 0
    const int r0 = rtile * kRowsPerWg;
    const int rmax = min(r0 + kRowsPerWg, rows) - 1;
    const int c_begin = split * cps;
    const int c_end = min(min(total_chunks, c_begin + cps), (first_last + rmax / group) / kChunk + 1);
    const int min_last = first_last + r0 / group;      // chunks ending at or below it need no mask

    // this lane's query rows (one per row tile); a wave whose rows all lie
    // past the end (few rows, e.g. a verify batch) skips the math but still
    // stages chunks
    const int wrow0 = r0 + wave * 16 * RT;
    const bool wave_active = wrow0 < rows;
    int qi[RT], hh[RT], last[RT];
    bool row_ok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int row = wrow0 + 16 * rt + (lane & 15);
        row_ok[rt] = row < rows;
        qi[rt] = row_ok[rt] ? row / group : 0;
        hh[rt] = kvh * group + (row_ok[rt] ? row % group : 0);
        last[rt] = row_ok[rt] ? first_last + qi[rt] : -1;
    }

    // Page-table entries: lane k of `ents` holds the entry of page pb + k
    // (batches of 64 pages, one gather load per batch); the loop picks them
    // out with readlane, so no memory access sits between the loads in flight.
    int pb = (c_begin * kChunk) / g.P;
    const int pend = c_end > c_begin ? ((c_end - 1) * kChunk) / g.P + 1 : pb;
    auto load_ents = [&](int base) -> int { return base + lane < pend ? a.page_table[base + lane] : -1; };
    int ents = load_ents(pb);
    auto unit_of = [&](int page, bool& ok) -> const uint8_t* {
        if (page - pb >= 64) {                 // next batch of entries
            pb += 64;
            ents = load_ents(pb);
            asm volatile("" : "+v"(ents));
        }
        const int phys = __builtin_amdgcn_readlane(ents, page - pb);
        ok = phys >= 0 && phys < g.n_pages;
        return a.pool + g.unit_index(ok ? phys : 0, kvh) * g.unit_bytes();
    };

    bool bad = false;
    uint8_t* ring = smem + 2 * C::STAGE;
    const Requests<D, RT, CODEC> req(g, wave, lane);
    // position of the next chunk to request, advanced one chunk at a time
    int iss_c = c_begin, iss_page = (c_begin * kChunk) / g.P, iss_slot = (c_begin * kChunk) % g.P;
    auto issue_next = [&]() {
        bool ok;
        const uint8_t* u = unit_of(iss_page, ok);
        bad |= !ok;
        req.issue(ring + (iss_c & (kRing - 1)) * C::SLOT, u, iss_slot);
        ++iss_c;
        iss_slot += kChunk;
        if (iss_slot == g.P) { iss_slot = 0; ++iss_page; }
    };
    // raw chunks c_begin .. c_begin + kRing - 1 in flight before q is staged
    for (int i = 0; i < kRing; ++i)
        if (c_begin + i < c_end) issue_next();

    // q of this lane's rows as fp16 hi + lo, pre-scaled by scale * log2(e), in
    // the B-operand layout (row = lane % 16, dims 8 (lane / 16) .. +7 per block)
    // (INT2: also the row's sum of the pre-scaled q over each 128-value
    // block, for the zero-point term: this lane's 32 dims of it, then the
    // row's 4 lanes)
    half8 qh[RT][C::NB], ql[RT][C::NB];
    float qsum[RT][C::NB2 > 0 ? C::NB2 : 1];
    {
        const float qscale = a.scale * kLog2e;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float* src = a.q + ((size_t)qi[rt] * a.n_heads + hh[rt]) * D + 8 * (lane >> 4);
#pragma unroll
            for (int b = 0; b < (C::NB2 > 0 ? C::NB2 : 1); ++b) qsum[rt][b] = 0.0f;
#pragma unroll
            for (int b = 0; b < C::NB; ++b)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    // in bounds: rows past the end read row 0 (INT2: the codes' dim order)
                    const float v = src[b * kBlock + (CODEC == 1 ? i2_slot(i) : i)];
                    const float x = row_ok[rt] ? v * qscale : 0.0f;
                    qh[rt][b][i] = (_Float16)x;
                    ql[rt][b][i] = (_Float16)(x - (float)qh[rt][b][i]);
                    if constexpr (CODEC == 1) qsum[rt][b / 4] += x;
                }
            if constexpr (CODEC == 1) {
#pragma unroll
                for (int b = 0; b < C::NB2; ++b) qsum[rt][b] = xsum4(qsum[rt][b]);
            }
        }
    }

    Rows<D, RT> st;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        st.m[rt] = -INFINITY;
        st.l[rt] = 0.0f;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) st.o[rt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    auto convert = [&](int c) {
        convert_chunk<D, RT, CODEC>(ring + (c & (kRing - 1)) * C::SLOT, smem + (c & 1) * C::STAGE, t,
                                    a.ctx - c * kChunk);
    };
    if (c_begin < c_end) {
        vm_wait<0>();
        lds_barrier();                         // chunks c_begin, c_begin + 1 have landed
        convert(c_begin);
        lds_barrier();
    }
    // Per chunk c: request c + kRing into the slot chunk c was converted
    // from, run the math on c, convert c + 1 (landed before the last barrier)
    // into the other stage, wait for this wave's requests of c + 2, barrier.
    // FUSE: the conversion runs under the products of c (a wave with rows,
    // a next chunk in the range that is whole); otherwise before the math.
    auto step = [&](int c, auto masked, auto fuse) {
        constexpr bool MASKED = decltype(masked)::value;
        const bool more = c + kRing < c_end;
        if (more) issue_next();
        SCHED_FENCE();
        if constexpr (decltype(fuse)::value) {
            chunk_step<D, RT, CODEC, MASKED, true>(st, smem + (c & 1) * C::STAGE, qh, ql, qsum, lane, c * kChunk,
                                                   last, ring + ((c + 1) & (kRing - 1)) * C::SLOT,
                                                   smem + ((c + 1) & 1) * C::STAGE, t);
        } else {
            if (c + 1 < c_end) convert(c + 1);
            SCHED_FENCE();
            if (wave_active)
                chunk_step<D, RT, CODEC, MASKED, false>(st, smem + (c & 1) * C::STAGE, qh, ql, qsum, lane,
                                                        c * kChunk, last, nullptr, nullptr, t);
        }
        SCHED_FENCE();
        if (more) vm_wait<(kRing - 2) * C::ND>(); else vm_wait<0>();
        lds_barrier();
    };
    // Chunks ending at or before min_last need no mask; chunks before c_fuse
    // have a whole next chunk in the range.  Each kind runs in a loop of its
    // own, in chunk order (the fused and plain steps in one loop would need
    // more registers than a wave has).
    const int c_mask = max(c_begin, min(c_end, (min_last + 1) / kChunk));
    const int c_fuse = wave_active ? min(c_end, a.ctx / kChunk) - 1 : c_begin;
    const std::false_type no{};
    const std::true_type yes{};
    int c = c_begin;
    for (const int e = max(c_begin, min(c_mask, c_fuse)); c < e; ++c) step(c, no, yes);
    for (; c < c_mask; ++c) step(c, no, no);
    for (const int e = max(c_mask, c_fuse); c < e; ++c) step(c, yes, yes);
    for (; c < c_end; ++c) step(c, yes, no);

    const int grp = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        // row sum over the row's 4 lanes; every lane then holds (m, L) of its row
        float L = xsum4(st.l[rt]);
        float M = st.m[rt];
        if (bad) { M = NAN; L = NAN; }
        if (!row_ok[rt]) continue;
        const size_t orow = (size_t)qi[rt] * a.n_heads + hh[rt];
        if (n_splits == 1) {
            const float inv = 1.0f / L;
            float* dst = a.out + orow * D + 4 * grp;
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) *reinterpret_cast<floatx4*>(dst + 16 * nt) = st.o[rt][nt] * inv;
            if (a.lse != nullptr && grp == 0) a.lse[orow] = (M + log2f(L)) * 0.69314718055994531f;
        } else {
            const size_t ps = orow * n_splits + split;
            if (grp == 0) {
                a.ws_m[ps] = M;
                a.ws_l[ps] = L;
            }
            float* dst = a.ws_acc + ps * D + 4 * grp;
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) *reinterpret_cast<floatx4*>(dst + 16 * nt) = st.o[rt][nt];
        }
    }
}

template <int D, int RT, int CODEC>
hipError_t launch_dr(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    using C = TCfg<D, RT, CODEC>;
    auto kern = attn_mfma_tiled_kernel<D, RT, CODEC>;
    if (C::LDS > 64 * 1024) {
        hipError_t e = allow_lds<attn_mfma_tiled_kernel<D, RT, CODEC>>(C::LDS);
        if (e != hipSuccess) return e;
    }
    const int row_tiles = (pl.rows + kRowsPerWg - 1) / kRowsPerWg;
    dim3 grid(row_tiles * pl.n_splits * a.g.n_kv);
    hipLaunchKernelGGL(kern, grid, dim3(C::THREADS), C::LDS, stream, a, pl.chunks_per_split, pl.n_splits, pl.group,
                       pl.rows, row_tiles);
    return hipGetLastError();
}

}  // namespace

int mfma_tiled_rows_per_wg() { return kRowsPerWg; }

hipError_t launch_attn_mfma_tiled(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    // one row tile per wave: at head_dim 256 two tiles per wave need more than
    // the 512 registers a wave can hold
    if (a.g.codec == 1) {
        switch (a.g.D) {
            case 128: return launch_dr<128, 1, 1>(a, pl, stream);
            case 256: return launch_dr<256, 1, 1>(a, pl, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.g.D) {
        case 64: return launch_dr<64, 1, 0>(a, pl, stream);
        case 128: return launch_dr<128, 1, 0>(a, pl, stream);
        case 256: return launch_dr<256, 1, 0>(a, pl, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
