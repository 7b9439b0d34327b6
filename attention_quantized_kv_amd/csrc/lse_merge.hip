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
// Splits with no visible key (l = 0) are skipped; a NaN partial (a page-table
// entry outside the pool) propagates to the output.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kBatch = 64;      // splits folded per round

// One workgroup per query row, one thread per output dim.  Per batch of 64
// splits every thread loads its dim of all 64 accumulators at once (one
// memory round trip), while wave 0 folds the batch's (m, l) into weights:
// M' = max(M, max_s m_s), w_s = 2^(m_s - M'), L' = L 2^(M - M') + sum w_s l_s;
// then o' = o 2^(M - M') + sum w_s acc_s.  The folding order is fixed.
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(AttnArgs a, int n_splits) {
    __shared__ float w_s[kBatch];
    __shared__ float alpha_s, l_s, m_s;
    const int row = blockIdx.x;
    const int t = threadIdx.x;
    const float* m = a.ws_m + (size_t)row * n_splits;
    const float* l = a.ws_l + (size_t)row * n_splits;
    const float* acc = a.ws_acc + (size_t)row * n_splits * D + t;
    float M = -INFINITY, L = 0.0f, o = 0.0f;       // wave 0 keeps M, L; every thread its o
    for (int s0 = 0; s0 < n_splits; s0 += kBatch) {
        const int nb = min(kBatch, n_splits - s0);
        float x[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) x[k] = k < nb ? acc[(size_t)(s0 + k) * D] : 0.0f;
        if (t < 64) {
            const float mk = t < nb ? m[s0 + t] : -INFINITY;
            const float lk = t < nb ? l[s0 + t] : 0.0f;
            // splits with no visible key (l = 0) do not count; a NaN partial
            // (page outside the pool) propagates through its weight
            float bm = lk != 0.0f ? mk : -INFINITY;
#pragma unroll
            for (int off = 32; off >= 1; off /= 2) bm = fmaxf(bm, __shfl_xor(bm, off));
            const float Mn = fmaxf(M, bm);
            const float wk = lk != 0.0f ? exp2f(mk - Mn) : 0.0f;
            float sl = wk * lk;
#pragma unroll
            for (int off = 32; off >= 1; off /= 2) sl += __shfl_xor(sl, off);
            const float al = M == -INFINITY ? 0.0f : exp2f(M - Mn);
            L = L * al + sl;
            M = Mn;
            w_s[t] = wk;
            if (t == 0) { alpha_s = al; l_s = L; m_s = M; }
        }
        __syncthreads();
        float sum = o * alpha_s;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) sum = fmaf(w_s[k], x[k], sum);
        o = sum;
        __syncthreads();                           // w_s is rewritten by the next batch
    }
    const float Lt = l_s, Mt = m_s;
    a.out[(size_t)row * D + t] = o / Lt;
    if (a.lse != nullptr && t == 0) a.lse[row] = (Mt + log2f(Lt)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_merge(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    dim3 grid(a.n_q * a.n_heads);
    switch (a.g.D) {
        case 64: hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, stream, a, pl.n_splits); break;
        case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(128), 0, stream, a, pl.n_splits); break;
        case 256: hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(256), 0, stream, a, pl.n_splits); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
