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
// One workgroup per query row, one thread per output dimension; every thread
// walks the row's partials in the same order, so the weights are identical.
// Splits with no visible key (l = 0) are skipped; a NaN partial (a page-table
// entry outside the pool) propagates to the output.
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int D>
__global__ __launch_bounds__(D) void merge_kernel(AttnArgs a, int n_splits) {
    const int row = blockIdx.x;
    const int d = threadIdx.x;
    const float* m = a.ws_m + (size_t)row * n_splits;
    const float* l = a.ws_l + (size_t)row * n_splits;
    const float* acc = a.ws_acc + (size_t)row * n_splits * D;

    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) M = fmaxf(M, m[s]);
    float L = 0.0f, o = 0.0f;
    for (int s = 0; s < n_splits; ++s) {
        const float ls = l[s];
        if (ls == 0.0f) continue;
        const float w = exp2f(m[s] - M);
        L = fmaf(ls, w, L);
        o = fmaf(acc[(size_t)s * D + d], w, o);
    }
    a.out[(size_t)row * D + d] = o / L;
    if (a.lse != nullptr && d == 0) a.lse[row] = (M + log2f(L)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_merge(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    dim3 grid(a.n_q * a.n_heads);
    switch (a.g.D) {
        case 64:  hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, stream, a, pl.n_splits); break;
        case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(128), 0, stream, a, pl.n_splits); break;
        case 256: hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(256), 0, stream, a, pl.n_splits); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
