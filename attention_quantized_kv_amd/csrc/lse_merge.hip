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
#include <type_traits>

#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kBatch = 64;      // splits folded per round
constexpr int kMaxNew = 8;      // rows appended by one fused call (the decode / verify limit)
constexpr float kLog2eM = 1.4426950408889634f;

// One workgroup per query row, one thread per output dim.  Per batch of 64
// splits every thread loads its dim of all 64 accumulators at once (one
// memory round trip), while wave 0 folds the batch's (m, l) into weights:
// M' = max(M, max_s m_s), w_s = 2^(m_s - M'), L' = L 2^(M - M') + sum w_s l_s;
// then o' = o 2^(M - M') + sum w_s acc_s.  The folding order is fixed.
// Batched launches: row b * n_q * n_heads + r is row r of sequence b, whose
// partials start at partial b.part0[b] and number n_splits[b] per row.
template <int D, class Batch>
__global__ __launch_bounds__(D) void merge_kernel(AttnArgs a, int n_splits, Batch sb) {
    __shared__ float w_s[kBatch];
    __shared__ float alpha_s, l_s, m_s;
    const int row = blockIdx.x;
    const int t = threadIdx.x;
    size_t p0 = (size_t)row * n_splits;            // this row's first partial
    if constexpr (!std::is_same_v<Batch, NoBatch>) {
        const int rps = a.n_q * a.n_heads;
        const int b = row / rps;
        n_splits = sb.n_splits[b];
        p0 = (size_t)sb.part0[b] + (size_t)(row - b * rps) * n_splits;
    }
    const float* m = a.ws_m + p0;
    const float* l = a.ws_l + p0;
    const float* acc = a.ws_acc + p0 * D + t;
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
            bm = wave_max(bm, t);
            const float Mn = fmaxf(M, bm);
            const float wk = lk != 0.0f ? exp2f(mk - Mn) : 0.0f;
            float sl = wk * lk;
            sl = wave_sum(sl, t);
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

// Fused append + attention, second half.  Row (i, h) -- query i at position
// pos0 + i -- has the split partials over the cached keys 0..pos0-1 and sees
// the new rows 0..i as well (causal among the new rows).  Each workgroup
// quantizes the new K/V rows of its KV head with the append kernel's block
// code (so the values are the ones the pool will hold, bit for bit), scores
// the dequantized keys, folds them in as one more partial after the splits,
// and writes out and lse.  The workgroup of (i, first head of the group)
// writes new row i of that KV head into the pool: K codes and both scales by
// plain stores, the V nibble (which shares a byte with its pair slot) by an
// atomic and-or on the containing dword.  One thread per output dim.
template <int D>
__global__ __launch_bounds__(D) void merge_new_kernel(AttnArgs a, NewRows nr, int n_splits, int group) {
    constexpr int NW = D / 64;
    __shared__ float w_s[kBatch];
    __shared__ float alpha_s, l_s, m_s;
    __shared__ float red_s[kMaxNew][NW];
    const Geom& g = a.g;
    const int row = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    const int qi = row / a.n_heads, h = row % a.n_heads, kvh = h / group;
    const int n_vis = qi + 1;                          // new rows visible to query qi (uniform)
    const bool writer = h % group == 0;
    const float* m = a.ws_m + (size_t)row * n_splits;
    const float* l = a.ws_l + (size_t)row * n_splits;
    const float* acc = a.ws_acc + (size_t)row * n_splits * D + t;

    // ---- every load up front: the first batch of split partials, the
    // visible new rows of this KV head, q, their page entries
    const int nb0 = min(kBatch, n_splits);
    float x[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) x[k] = k < nb0 ? acc[(size_t)k * D] : 0.0f;
    const float m0 = t < nb0 ? m[t] : -INFINITY;
    const float l0 = t < nb0 ? l[t] : 0.0f;
    float kx[kMaxNew], vx[kMaxNew];
#pragma unroll
    for (int j = 0; j < kMaxNew; ++j) {
        const size_t src = ((size_t)j * g.n_kv + kvh) * D + t;
        kx[j] = j < n_vis ? nr.k[src] : 0.0f;
        vx[j] = j < n_vis ? nr.v[src] : 0.0f;
    }
    const float xq = a.q[(size_t)row * D + t] * (a.scale * kLog2eM);
    const int pos = nr.pos0 + qi;
    // page entries of the visible new rows: one outside the pool makes the
    // row's result NaN (as a cached key on such a page does); a row whose own
    // entry lies outside the pool is not written
    int phys = -1;
    bool bad_page = false;
#pragma unroll
    for (int j = 0; j < kMaxNew; ++j) {
        if (j >= n_vis) break;
        const int e = a.page_table[(nr.pos0 + j) / g.P];
        bad_page |= e < 0 || e >= g.n_pages;
        if (j == qi) phys = e;
    }

    // ---- quantize; score the dequantized keys; this row's own new row goes to the pool
    float vhat[kMaxNew];
#pragma unroll
    for (int j = 0; j < kMaxNew; ++j) {
        if (j >= n_vis) break;                         // uniform
        const QCode ck = quant_q8_0(kx[j], lane);
        const QCode cv = quant_q4_0(vx[j], lane);
        const float kd = __half2float(__float2half_rn(ck.d)), vd = __half2float(__float2half_rn(cv.d));
        vhat[j] = (float)(cv.code - 8) * vd;
        const float p = wave_sum(xq * ((float)ck.code * kd), lane);
        if (lane == 0) red_s[j][wv] = p;
        if (writer && j == qi && phys >= 0 && phys < g.n_pages) {
            uint8_t* unit = nr.pool + g.unit_index(phys, kvh) * g.unit_bytes();
            const int slot = pos % g.P;
            unit[k_code_pos(g, slot, t)] = (uint8_t)(int8_t)ck.code;
            int nib;
            const int64_t off = v_code_pos(g, slot, t, &nib);
            unsigned int* dw = reinterpret_cast<unsigned int*>(unit + (off & ~(int64_t)3));
            const int shift = (int)(off & 3) * 8 + nib * 4;
            atomicAnd(dw, ~(0xFu << shift));
            atomicOr(dw, (unsigned int)cv.code << shift);
            if ((t & (kBlock - 1)) == 0) {
                reinterpret_cast<uint16_t*>(unit + g.k_scales_off())[slot * g.nb() + t / kBlock] = f16_bits(ck.d);
                reinterpret_cast<uint16_t*>(unit + g.v_scales_off())[v_scale_idx(g, slot, t / kBlock)] = f16_bits(cv.d);
            }
        }
    }

    // ---- the split partials over the cached keys (as merge_kernel); the
    // new rows' scores are summed over the waves after the first barrier
    float M = -INFINITY, L = 0.0f, o = 0.0f;
    for (int s0 = 0; s0 < n_splits; s0 += kBatch) {
        const int nb = min(kBatch, n_splits - s0);
        float mk = m0, lk = l0;
        if (s0 > 0) {
#pragma unroll
            for (int k = 0; k < kBatch; ++k) x[k] = k < nb ? acc[(size_t)(s0 + k) * D] : 0.0f;
            mk = t < nb ? m[s0 + t] : -INFINITY;
            lk = t < nb ? l[s0 + t] : 0.0f;
        }
        if (t < 64) {
            float bm = lk != 0.0f ? mk : -INFINITY;
            bm = wave_max(bm, t);
            const float Mn = fmaxf(M, bm);
            const float wk = lk != 0.0f ? exp2f(mk - Mn) : 0.0f;
            float sl = wk * lk;
            sl = wave_sum(sl, t);
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
        __syncthreads();
    }
    if (n_splits > 0) { M = m_s; L = l_s; }
    else __syncthreads();                              // red_s complete

    // ---- the new rows' keys, folded in after the splits
    float sj[kMaxNew];
    float m_new = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxNew; ++j) {
        if (j >= n_vis) break;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red_s[j][w];
        sj[j] = sum;
        m_new = fmaxf(m_new, sum);
    }
    float l_new = 0.0f, acc_new = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxNew; ++j) {
        if (j >= n_vis) break;
        const float w = exp2f(sj[j] - m_new);
        l_new += w;
        acc_new = fmaf(w, vhat[j], acc_new);
    }
    const float Mt = fmaxf(M, m_new);
    const float a_old = M == -INFINITY ? 0.0f : exp2f(M - Mt);
    const float a_new = exp2f(m_new - Mt);
    const float Lt = L * a_old + l_new * a_new;
    const float res = bad_page ? NAN : (o * a_old + acc_new * a_new) / Lt;
    a.out[(size_t)row * D + t] = res;
    if (a.lse != nullptr && t == 0) a.lse[row] = bad_page ? NAN : (Mt + log2f(Lt)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_merge_new(const AttnArgs& a, const NewRows& nr, int n_splits, hipStream_t stream) {
    if (nr.n_new < 1 || nr.n_new > kMaxNew) return hipErrorInvalidValue;
    const int group = a.n_heads / a.g.n_kv;
    dim3 grid(a.n_q * a.n_heads);
    switch (a.g.D) {
        case 64: hipLaunchKernelGGL(merge_new_kernel<64>, grid, dim3(64), 0, stream, a, nr, n_splits, group); break;
        case 128: hipLaunchKernelGGL(merge_new_kernel<128>, grid, dim3(128), 0, stream, a, nr, n_splits, group); break;
        case 256: hipLaunchKernelGGL(merge_new_kernel<256>, grid, dim3(256), 0, stream, a, nr, n_splits, group); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class Batch>
hipError_t launch_merge_b(const AttnArgs& a, int n_splits, int n_rows, hipStream_t stream, const Batch& sb) {
    dim3 grid(n_rows);
    switch (a.g.D) {
        case 64: hipLaunchKernelGGL((merge_kernel<64, Batch>), grid, dim3(64), 0, stream, a, n_splits, sb); break;
        case 128: hipLaunchKernelGGL((merge_kernel<128, Batch>), grid, dim3(128), 0, stream, a, n_splits, sb); break;
        case 256: hipLaunchKernelGGL((merge_kernel<256, Batch>), grid, dim3(256), 0, stream, a, n_splits, sb); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const SeqBatch* batch) {
    if (batch != nullptr && batch->n > 0)
        return launch_merge_b(a, 0, batch->n * a.n_q * a.n_heads, stream, *batch);
    return launch_merge_b(a, pl.n_splits, a.n_q * a.n_heads, stream, NoBatch{});
}

}  // namespace kvq
