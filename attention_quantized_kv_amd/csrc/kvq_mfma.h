// kvq_mfma.h -- device helpers shared by the matrix-core attention kernels
// (gfx950): fragment types, the query-row placement in an MFMA tile, DPP
// reductions over the 16 lanes of a row, and the online-softmax constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPStride = 36;   // floats per row of the P transpose buffer (32 + padding)
constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescaling: a row's reference maximum m moves only when a chunk's
// maximum exceeds it by more than kTau (log2 units).  Weights are formed as
// 2^(s - m - kTau) <= 1 and the V codes carry the compensating 2^kTau
// exactly, so fp16 operands never overflow; the row sum is scaled by 2^kTau
// at the end.
constexpr float kTau = 4.0f;

// MFMA row placement.  Row tile rt holds query rows 16 rt .. 16 rt + 15 in
// MFMA rows 0..15; lane group g4 of the S / O layouts owns rows 4*g4 ..
// 4*g4+3.  A tile with at most 8 query rows (JJ = 2) puts them in MFMA rows
// {0,1, 4,5, 8,9, 12,13}, so each lane holds 2 real rows and the softmax work
// per lane halves; otherwise (JJ = 4) row i sits at MFMA row i.  Returns the
// query row at MFMA row prow of tile rt, or -1.
template <int JJ>
__device__ inline int logical_row(int rt, int prow) {
    if (JJ == 4) return 16 * rt + prow;
    return (prow & 3) < 2 ? 16 * rt + 2 * (prow >> 2) + (prow & 3) : -1;
}

template <int CTRL>
__device__ inline float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// max(x, x of the lane that DPP control CTRL names), one v_max_f32_dpp (the
// builtin route adds a move and a NaN-quieting max per step).  s_nop 1 covers
// the two wait states a DPP read needs after the VALU write of its source.
// Volatile: the compiler would otherwise hoist the reductions out of the
// rarely taken branch that needs them.
#define KVQ_MAX_DPP(CTRL)                                                                  \
    __device__ inline float max_dpp_##CTRL(float x) {                                     \
        float r;                                                                          \
        asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 " KVQ_DPP_##CTRL                 \
                     " row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));                   \
        return r;                                                                         \
    }
#define KVQ_DPP_ror8 "row_ror:8"
#define KVQ_DPP_ror4 "row_ror:4"
#define KVQ_DPP_swap2 "quad_perm:[2,3,0,1]"
#define KVQ_DPP_swap1 "quad_perm:[1,0,3,2]"
KVQ_MAX_DPP(ror8)
KVQ_MAX_DPP(ror4)
KVQ_MAX_DPP(swap2)
KVQ_MAX_DPP(swap1)

// max(a, b) as one v_max_f32: fmaxf adds a NaN-quieting max per operand
// whenever the compiler cannot prove the operands canonical (values that
// reach the softmax from another basic block, here)
__device__ inline float max2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Reductions over the 16 lanes of a DPP row (rotate by 8, by 4, then swap
// pairs inside quads): every lane ends with the row's result.
__device__ inline float row16_max(float x) {
    return max_dpp_swap1(max_dpp_swap2(max_dpp_ror4(max_dpp_ror8(x))));
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

// 2^x on the hardware exp unit (results below the normal range flush to 0,
// which only drops weights far below the row maximum).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Workgroup barrier for LDS data only: unlike __syncthreads() it does not wait
// for the direct-to-LDS loads in flight (the release fence there would).
__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Waits until at most N vector-memory requests of this wave are outstanding
// (direct-to-LDS loads count); also a compiler memory fence, since the
// compiler cannot see that later LDS reads depend on those loads.
template <int N>
__device__ inline void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Cache policy of a global load: kLoadNT marks it non-temporal (the data is
// read once and should not displace other lines on its way).  Measured on a
// plain sweep of 436 MB with 8 waves per CU and 4 KiB in flight per wave:
// 7.17 TB/s with the hint against 6.35 TB/s without, for register loads and
// direct-to-LDS loads alike.
constexpr int kLoadPlain = 0;
constexpr int kLoadNT = 2;

// 16 bytes per lane, global -> LDS: lane i's bytes land at lds + 16 i.
template <int POLICY = kLoadPlain>
__device__ inline void dma16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds, 16, 0, POLICY);
}

}  // namespace
}  // namespace kvq
