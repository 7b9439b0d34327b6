// lse_merge.hip -- combine split-K partials into the exact softmax output.
//
// Each split s of a query row left (m_s, l_s, acc_s): the log2-domain maximum
// of its scores, the sum of exp2(score - m_s) and the matching unnormalized
// sum of values.  With M = max_s m_s:
//   L = sum_s l_s * 2^(m_s - M),  o = sum_s acc_s * 2^(m_s - M) / L,
//   lse = (M + log2 L) * ln 2     (natural-log convention of the ABI)
// This is the online log-sum-exp combination the pages use to accumulate
// over pages ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070 XT at 262k
// context, via adaptive KV streaming", second paragraph).
//
// One workgroup per (row, 64 output dims): its 4 wavefronts each fold every
// 4th split with a running maximum, loading 8 splits at a time so their loads
// overlap, then wave 0 folds the 4 wave results in a fixed order.
// Splits with no visible key (l = 0) are skipped; a NaN partial (a page-table
// entry outside the pool) propagates to the output.
#include "kvq_internal.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int n_splits, int D) {
    __shared__ float sm[4], sl[4], so[4][64];
    const int row = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int d = blockIdx.y * 64 + lane;
    const float* m = a.ws_m + (size_t)row * n_splits;
    const float* l = a.ws_l + (size_t)row * n_splits;
    const float* acc = a.ws_acc + (size_t)row * n_splits * D + d;

    // batches of 8 splits: all 24 loads of a batch are independent, so they
    // are in flight together; the batch is then folded in order
    float M = -INFINITY, L = 0.0f, o = 0.0f;
    constexpr int kBatch = 8;
    for (int s0 = wave; s0 < n_splits; s0 += 4 * kBatch) {
        float ms[kBatch], ls[kBatch], xs[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int s = s0 + 4 * k;
            const bool in = s < n_splits;
            ms[k] = in ? m[s] : -INFINITY;
            ls[k] = in ? l[s] : 0.0f;
            xs[k] = in ? acc[(size_t)s * D] : 0.0f;
        }
        float bm = M;
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (ls[k] != 0.0f) bm = fmaxf(bm, ms[k]);
        if (bm > M) {
            const float f = exp2f(M - bm);
            L *= f;
            o *= f;
            M = bm;
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (ls[k] == 0.0f) continue;
            const float w = exp2f(ms[k] - M);
            L = fmaf(ls[k], w, L);
            o = fmaf(xs[k], w, o);
        }
    }
    if (lane == 0) { sm[wave] = M; sl[wave] = L; }
    so[wave][lane] = o;
    __syncthreads();
    if (wave != 0) return;
    float Mt = -INFINITY;
    for (int w = 0; w < 4; ++w) Mt = fmaxf(Mt, sm[w]);
    float Lt = 0.0f, ot = 0.0f;
    for (int w = 0; w < 4; ++w) {
        if (sl[w] == 0.0f) continue;
        const float f = exp2f(sm[w] - Mt);
        Lt = fmaf(sl[w], f, Lt);
        ot = fmaf(so[w][lane], f, ot);
    }
    a.out[(size_t)row * D + d] = ot / Lt;
    if (a.lse != nullptr && blockIdx.y == 0 && lane == 0) a.lse[row] = (Mt + log2f(Lt)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_merge(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    dim3 grid(a.n_q * a.n_heads, a.g.D / 64);
    hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, stream, a, pl.n_splits, a.g.D);
    return hipGetLastError();
}

}  // namespace kvq
