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
//
// The merge runs after the split kernel, on the same stream, so its duration
// adds straight to every decode step: it is built for latency.  One wavefront
// per (query row, 64-dim slice) -- D/64 times more workgroups than rows, so
// the work spreads over the chip -- loads everything it needs in one memory
// round trip (a batch of 64 splits' accumulators for its 64 dims, one split
// per lane for (m, l), the new rows), folds the (m, l) of the batch across
// lanes and broadcasts each split's weight with readlane.
#include <type_traits>

#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kBatch = 64;      // splits folded per round (one per lane)
constexpr int kMaxNew = 8;      // rows appended by one fused call (the decode / verify limit)
constexpr int kSlice = 64;      // output dims per workgroup (one per lane)
constexpr float kLog2eM = 1.4426950408889634f;

__device__ inline float readlane_f(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Workgroup = one wavefront: query row `row` (all rows are n_q * n_heads, in
// (query, head) order; a batched launch stacks its sequences), output dims
// 64 z .. 64 z + 63 (lane = dim).
//
// NEW (the second half of the fused append + attention call): row (i, h) --
// query i at position pos0 + i -- has the split partials over the cached
// keys 0..pos0-1 and sees the new rows 0..i as well (causal among the new
// rows).  Each workgroup quantizes the visible new K rows of its KV head over
// all D dims and the V rows over its own dims, with the append kernel's block
// code (so the values are the ones the pool will hold, bit for bit), scores
// the dequantized keys, and folds them in as one more partial after the
// splits.  The workgroups of (i, first head of the group) write new row i of
// that KV head into the pool, each its own dims: K codes and both scales by
// plain stores, the V nibble (which shares a byte with its pair slot) by an
// atomic and-or on the containing dword.
template <int D, bool NEW, class Batch>
__global__ __launch_bounds__(64) void merge_rows_kernel(AttnArgs a, NewRows nr, int n_splits, int group, Batch sb) {
    constexpr int NS = D / kSlice;          // slices per row
    const Geom& g = a.g;
    const int lane = threadIdx.x;
    const int row = blockIdx.x / NS, z = blockIdx.x % NS;
    const int d = kSlice * z + lane;
    size_t p0 = (size_t)row * n_splits;     // this row's first partial
    if constexpr (!std::is_same_v<Batch, NoBatch>) {
        const int rps = a.n_q * a.n_heads;
        const int b = row / rps;
        n_splits = sb.n_splits[b];
        p0 = (size_t)sb.part0[b] + (size_t)(row - b * rps) * n_splits;
    }
    const float* m = a.ws_m + p0;
    const float* l = a.ws_l + p0;
    const float* acc = a.ws_acc + p0 * D + d;

    // ---- every load up front: the first batch of partials and, for NEW, q,
    // the visible new K rows (all dims) and V rows (this slice), their page
    // entries
    const int nb0 = min(kBatch, n_splits);
    float x[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) x[k] = k < nb0 ? acc[(size_t)k * D] : 0.0f;
    float mk = lane < nb0 ? m[lane] : -INFINITY;
    float lk = lane < nb0 ? l[lane] : 0.0f;

    const int qi = row / a.n_heads, h = row % a.n_heads, kvh = h / group;
    const int n_vis = NEW ? qi + 1 : 0;     // new rows visible to query qi (uniform)
    float qx[NS], kx[NEW ? kMaxNew : 1][NS], vx[NEW ? kMaxNew : 1];
    int phys = -1;
    bool bad_page = false;
    if constexpr (NEW) {
#pragma unroll
        for (int s = 0; s < NS; ++s) qx[s] = a.q[(size_t)row * D + kSlice * s + lane] * (a.scale * kLog2eM);
#pragma unroll
        for (int j = 0; j < kMaxNew; ++j) {
            const size_t src = ((size_t)j * g.n_kv + kvh) * D;
#pragma unroll
            for (int s = 0; s < NS; ++s) kx[j][s] = j < n_vis ? nr.k[src + kSlice * s + lane] : 0.0f;
            vx[j] = j < n_vis ? nr.v[src + d] : 0.0f;
        }
        // a visible new row whose page entry lies outside the pool makes the
        // row's result NaN (as a cached key on such a page does); a row whose
        // own entry lies outside the pool is not written
#pragma unroll
        for (int j = 0; j < kMaxNew; ++j) {
            if (j >= n_vis) break;
            const int e = a.page_table[(nr.pos0 + j) / g.P];
            bad_page |= e < 0 || e >= g.n_pages;
            if (j == qi) phys = e;
        }
    }

    // ---- fold the split partials, 64 per round
    float M = -INFINITY, L = 0.0f, o = 0.0f;
    for (int s0 = 0; s0 < n_splits; s0 += kBatch) {
        const int nb = min(kBatch, n_splits - s0);
        if (s0 > 0) {
#pragma unroll
            for (int k = 0; k < kBatch; ++k) x[k] = k < nb ? acc[(size_t)(s0 + k) * D] : 0.0f;
            mk = lane < nb ? m[s0 + lane] : -INFINITY;
            lk = lane < nb ? l[s0 + lane] : 0.0f;
        }
        // splits with no visible key (l = 0) do not count; a NaN partial
        // (page outside the pool) propagates through its weight
        const float bm = wave_max(lk != 0.0f ? mk : -INFINITY, lane);
        const float Mn = fmaxf(M, bm);
        const float wk = lk != 0.0f ? exp2f(mk - Mn) : 0.0f;
        const float sl = wave_sum(wk * lk, lane);
        const float al = M == -INFINITY ? 0.0f : exp2f(M - Mn);
        L = L * al + sl;
        M = Mn;
        float sum = o * al;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) sum = fmaf(readlane_f(wk, k), x[k], sum);
        o = sum;
    }

    if constexpr (!NEW) {
        a.out[(size_t)row * D + d] = o / L;
        if (a.lse != nullptr && z == 0 && lane == 0) a.lse[row] = (M + log2f(L)) * 0.69314718055994531f;
        return;
    } else {
        // ---- the new rows: quantize, score, fold in after the splits; this
        // row's own new row goes to the pool
        const bool writer = h % group == 0 && phys >= 0 && phys < g.n_pages;
        uint8_t* unit = nr.pool + g.unit_index(writer ? phys : 0, kvh) * g.unit_bytes();
        const int slot = (nr.pos0 + qi) % g.P;
        float sj[kMaxNew], vhat[kMaxNew];
        float m_new = -INFINITY;
#pragma unroll
        for (int j = 0; j < kMaxNew; ++j) {
            if (j >= n_vis) break;                         // uniform
            float dot = 0.0f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const QCode ck = quant_q8_0(kx[j][s], lane);
                const float kd = __half2float(__float2half_rn(ck.d));
                dot = fmaf(qx[s], (float)ck.code * kd, dot);
                if (s == z && writer && j == qi) {
                    unit[k_code_pos(g, slot, d)] = (uint8_t)(int8_t)ck.code;
                    if ((lane & (kBlock - 1)) == 0)
                        reinterpret_cast<uint16_t*>(unit + g.k_scales_off())[slot * g.nb() + d / kBlock] = f16_bits(ck.d);
                }
            }
            sj[j] = wave_sum(dot, lane);
            m_new = fmaxf(m_new, sj[j]);
            const QCode cv = quant_q4_0(vx[j], lane);
            vhat[j] = (float)(cv.code - 8) * __half2float(__float2half_rn(cv.d));
            if (writer && j == qi) {
                int nib;
                const int64_t off = v_code_pos(g, slot, d, &nib);
                unsigned int* dw = reinterpret_cast<unsigned int*>(unit + (off & ~(int64_t)3));
                const int shift = (int)(off & 3) * 8 + nib * 4;
                atomicAnd(dw, ~(0xFu << shift));
                atomicOr(dw, (unsigned int)cv.code << shift);
                if ((lane & (kBlock - 1)) == 0)
                    reinterpret_cast<uint16_t*>(unit + g.v_scales_off())[v_scale_idx(g, slot, d / kBlock)] = f16_bits(cv.d);
            }
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
        a.out[(size_t)row * D + d] = bad_page ? NAN : (o * a_old + acc_new * a_new) / Lt;
        if (a.lse != nullptr && z == 0 && lane == 0)
            a.lse[row] = bad_page ? NAN : (Mt + log2f(Lt)) * 0.69314718055994531f;
    }
}

template <bool NEW, class Batch>
hipError_t launch_rows(const AttnArgs& a, const NewRows& nr, int n_splits, int n_rows, hipStream_t stream,
                       const Batch& sb) {
    const int group = a.n_heads / a.g.n_kv;
    switch (a.g.D) {
        case 64:
            hipLaunchKernelGGL((merge_rows_kernel<64, NEW, Batch>), dim3(n_rows), dim3(64), 0, stream, a, nr, n_splits,
                               group, sb);
            break;
        case 128:
            hipLaunchKernelGGL((merge_rows_kernel<128, NEW, Batch>), dim3(n_rows * 2), dim3(64), 0, stream, a, nr,
                               n_splits, group, sb);
            break;
        case 256:
            hipLaunchKernelGGL((merge_rows_kernel<256, NEW, Batch>), dim3(n_rows * 4), dim3(64), 0, stream, a, nr,
                               n_splits, group, sb);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_new(const AttnArgs& a, const NewRows& nr, int n_splits, hipStream_t stream) {
    if (nr.n_new < 1 || nr.n_new > kMaxNew) return hipErrorInvalidValue;
    return launch_rows<true>(a, nr, n_splits, a.n_q * a.n_heads, stream, NoBatch{});
}

hipError_t launch_merge(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const SeqBatch* batch) {
    const NewRows none{nullptr, nullptr, nullptr, 0, 0};
    if (batch != nullptr && batch->n > 0)
        return launch_rows<false>(a, none, 0, batch->n * a.n_q * a.n_heads, stream, *batch);
    return launch_rows<false>(a, none, pl.n_splits, a.n_q * a.n_heads, stream, NoBatch{});
}

}  // namespace kvq
