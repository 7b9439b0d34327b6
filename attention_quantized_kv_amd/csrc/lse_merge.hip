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
// adds straight to every decode step: it is built for latency.  A workgroup
// per (query row, 64-dim slice) -- D/64 times more workgroups than rows, so
// the partials' bytes spread over the chip -- issues every load it needs at
// once (a few 16-byte loads per thread), so the merge costs one memory round
// trip plus a few hundred instructions.
#include <type_traits>

#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kBatch = 64;      // splits folded per round (one per lane)
constexpr int kMaxNew = 8;      // rows appended by one fused call (the decode / verify limit)
constexpr int kSlice = 64;      // output dims per workgroup (one per lane)
constexpr float kLog2eM = 1.4426950408889634f;

// Workgroup = 4 wavefronts for query row `row` (all rows are n_q * n_heads,
// in (query, head) order; a batched launch stacks its sequences) and output
// dims 64 z .. 64 z + 63.  Partials: per round of 64 splits, thread (wave w,
// lane = 16 si + dq) reads 16 bytes (dims 4 dq .. 4 dq + 3 of the slice) of
// splits 16 p + 4 w + si, p < 4: four 16-byte loads, no branches (addresses
// past the last split are clamped and weighted 0).  Every wave folds the
// round's (m, l) itself (lane = split), so M, L and the weights are the same
// in all of them; a thread takes its splits' weights with a lane shuffle,
// the 4 split groups of a wave are summed with permlane swaps, and the 4
// waves through 1 KiB of LDS; wave 0 then owns dim 64 z + lane.
//
// NEW (the second half of the fused append + attention call): row (i, h) --
// query i at position pos0 + i -- has the split partials over the cached
// keys 0..pos0-1 and sees the new rows 0..i as well (causal among the new
// rows).  Thread t quantizes dim t of the visible new K rows of its KV head
// (all D dims over the workgroup) and wave 0 dim 64 z + lane of the V rows,
// with the append kernel's block code (so the values are the ones the pool
// will hold, bit for bit); the scores of the dequantized keys are summed over
// the waves with the partials, and the new keys are folded in as one more
// partial after the splits.  The workgroups of (i, first head of the group)
// write new row i of that KV head into the pool, each its own 64 dims, with
// plain stores: K codes and both scales.  Two slots (2k, 2k+1) share every V
// byte, so the byte is written once, by the workgroup of the later new row
// of the pair, which sees both rows (the other nibble is either new row i-1
// or a slot no new row touches, kept as it was).  No byte of the pool is
// written by two workgroups, so no atomics are needed and no L2 of another
// XCD can hold a stale copy of a byte being changed.
template <int D, bool NEW, class Batch>
__global__ __launch_bounds__(256) void merge_rows_kernel(AttnArgs a, NewRows nr, int n_splits, int group, Batch sb) {
    constexpr int NS = D / kSlice;          // slices per row
    __shared__ float4 red4[4][16];          // per wave: the 64 dims' sums of its splits
    __shared__ float dots[kMaxNew][4];      // per wave: its part of each new key's score
    const Geom& g = a.g;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int si = lane >> 4, dq = lane & 15;
    const int row = blockIdx.x / NS, z = blockIdx.x % NS;
    size_t p0 = (size_t)row * n_splits;     // this row's first partial
    if constexpr (!std::is_same_v<Batch, NoBatch>) {
        const int rps = a.n_q * a.n_heads;
        const int b = row / rps;
        n_splits = sb.n_splits[b];
        p0 = (size_t)sb.part0[b] + (size_t)(row - b * rps) * n_splits;
    }
    const float* m = a.ws_m + p0;
    const float* l = a.ws_l + p0;
    const float* acc = a.ws_acc + p0 * D + kSlice * z + 4 * dq;

    // ---- every load up front: the first round of partials and, for NEW, q,
    // the visible new K rows (dim t) and V rows (wave 0: dim 64 z + lane), and
    // their page entries
    auto load_round = [&](int s0, float4 (&x)[4], float& mk, float& lk) {
        const int last = n_splits - 1;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int s = min(s0 + 16 * p + 4 * wv + si, last);
            x[p] = *reinterpret_cast<const float4*>(acc + (size_t)s * D);
        }
        const int s = min(s0 + lane, last);
        mk = m[s];
        lk = l[s];
    };
    float4 x[4];
    float mk = -INFINITY, lk = 0.0f;
    if (n_splits > 0) load_round(0, x, mk, lk);

    const int qi = row / a.n_heads, h = row % a.n_heads, kvh = h / group;
    const int n_vis = NEW ? qi + 1 : 0;     // new rows visible to query qi (uniform)
    const bool kdim = t < D;                // threads that quantize a K dim
    float qx = 0.0f, kx[NEW ? kMaxNew : 1], vx[NEW ? kMaxNew : 1];
    int phys = -1;
    bool bad_page = false;
    if constexpr (NEW) {
        if (kdim) qx = a.q[(size_t)row * D + t] * (a.scale * kLog2eM);
#pragma unroll
        for (int j = 0; j < kMaxNew; ++j) {
            const size_t src = ((size_t)j * g.n_kv + kvh) * D;
            kx[j] = j < n_vis && kdim ? nr.k[src + t] : 0.0f;
            vx[j] = j < n_vis && wv == 0 ? nr.v[src + kSlice * z + lane] : 0.0f;
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

    // ---- the new keys: quantize, score (this thread's dim), write this
    // slice's dims of the row's own new key into the pool
    float vhat[NEW ? kMaxNew : 1];
    int vc_self = 0, vc_prev = 0;           // V codes (this lane's dim) of new rows qi and qi - 1
    const bool writer = NEW && h % group == 0 && phys >= 0 && phys < g.n_pages;
    uint8_t* unit = NEW ? nr.pool + g.unit_index(writer ? phys : 0, kvh) * g.unit_bytes() : nullptr;
    const int slot = NEW ? (nr.pos0 + qi) % g.P : 0;
    if constexpr (NEW) {
#pragma unroll
        for (int j = 0; j < kMaxNew; ++j) {
            if (j >= n_vis) break;                         // uniform
            if (kdim) {                                    // uniform per wave
                const QCode ck = quant_q8_0(kx[j], lane);
                const float kd = __half2float(__float2half_rn(ck.d));
                const float part = wave_sum(qx * ((float)ck.code * kd), lane);
                if (lane == 0) dots[j][wv] = part;
                if (writer && j == qi && wv == z) {
                    unit[k_code_pos(g, slot, t)] = (uint8_t)(int8_t)ck.code;
                    if ((lane & (kBlock - 1)) == 0)
                        reinterpret_cast<uint16_t*>(unit + g.k_scales_off())[slot * g.nb() + t / kBlock] = f16_bits(ck.d);
                }
            }
            if (wv == 0) {
                const QCode cv = quant_q4_0(vx[j], lane);
                vhat[j] = (float)(cv.code - 8) * __half2float(__float2half_rn(cv.d));
                if (j == qi) vc_self = cv.code;
                if (j == qi - 1) vc_prev = cv.code;
                if (writer && j == qi && (lane & (kBlock - 1)) == 0)
                    reinterpret_cast<uint16_t*>(unit + g.v_scales_off())[v_scale_idx(g, slot, (kSlice * z + lane) / kBlock)] =
                        f16_bits(cv.d);
            }
        }
        // the V byte of the pair holding slot (pos0 + qi): written here when
        // qi is the pair's odd slot, or its even slot with no new row after it
        if (writer && wv == 0) {
            const bool odd = ((nr.pos0 + qi) & 1) != 0;
            if (odd || qi == nr.n_new - 1) {
                int nib;
                const int64_t off = v_code_pos(g, slot, kSlice * z + lane, &nib);
                const int old = unit[off];
                const int lo = odd ? (qi >= 1 ? vc_prev : (old & 15)) : vc_self;
                const int hi = odd ? vc_self : (old >> 4);
                unit[off] = (uint8_t)(lo | (hi << 4));
            }
        }
    }

    // ---- fold the split partials, 64 per round
    float M = -INFINITY, L = 0.0f;
    float4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < n_splits; s0 += kBatch) {
        if (s0 > 0) load_round(s0, x, mk, lk);
        const bool in = s0 + lane < n_splits;
        // splits with no visible key (l = 0) do not count; a NaN partial
        // (page outside the pool) propagates through its weight
        const bool live = in && lk != 0.0f;
        const float bm = wave_max(live ? mk : -INFINITY, lane);
        const float Mn = fmaxf(M, bm);
        const float wk = live ? exp2f(mk - Mn) : 0.0f;
        const float sl = wave_sum(wk * lk, lane);
        const float al = M == -INFINITY ? 0.0f : exp2f(M - Mn);
        L = L * al + sl;
        M = Mn;
        o *= al;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float w = __shfl(wk, 16 * p + 4 * wv + si);
            o += w * x[p];
        }
    }
    // sum the 4 split groups of the wave (lanes dq, dq + 16, dq + 32, dq + 48)
    o.x += xor16_f(o.x, lane);
    o.y += xor16_f(o.y, lane);
    o.z += xor16_f(o.z, lane);
    o.w += xor16_f(o.w, lane);
    o.x += xor32_f(o.x, lane);
    o.y += xor32_f(o.y, lane);
    o.z += xor32_f(o.z, lane);
    o.w += xor32_f(o.w, lane);
    if (lane < 16) red4[wv][lane] = o;
    __syncthreads();
    if (wv != 0) return;
    // wave 0: dim 64 z + lane
    const float* r = reinterpret_cast<const float*>(red4);
    const float od = r[lane] + r[64 + lane] + r[128 + lane] + r[192 + lane];
    const size_t oi = (size_t)row * D + kSlice * z + lane;
    if constexpr (!NEW) {
        a.out[oi] = od / L;
        if (a.lse != nullptr && z == 0 && lane == 0) a.lse[row] = (M + log2f(L)) * 0.69314718055994531f;
    } else {
        float sj[kMaxNew];
        float m_new = -INFINITY;
#pragma unroll
        for (int j = 0; j < kMaxNew; ++j) {
            if (j >= n_vis) break;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < D / 64; ++w) sum += dots[j][w];
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
        a.out[oi] = bad_page ? NAN : (od * a_old + acc_new * a_new) / Lt;
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
            hipLaunchKernelGGL((merge_rows_kernel<64, NEW, Batch>), dim3(n_rows), dim3(256), 0, stream, a, nr, n_splits,
                               group, sb);
            break;
        case 128:
            hipLaunchKernelGGL((merge_rows_kernel<128, NEW, Batch>), dim3(n_rows * 2), dim3(256), 0, stream, a, nr,
                               n_splits, group, sb);
            break;
        case 256:
            hipLaunchKernelGGL((merge_rows_kernel<256, NEW, Batch>), dim3(n_rows * 4), dim3(256), 0, stream, a, nr,
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
