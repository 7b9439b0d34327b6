// kvq_internal.h -- page-pool layout, launch plans and kernel entry points of
// libkvq (gfx950).  Internal to the library; the public ABI is include/kvq.h.
//
// Layout of one unit (one page of one KV head; P = page_size, D = head_dim):
//   K codes  [P*D]        int8, 16-token tiles, each tile D/64 wave-loads of
//                         1 KiB; lane (g, n) of load p holds token n's dims
//                         64p+8g..+7 and 64p+32+8g..+7 (the MFMA B operand of
//                         two consecutive 32-value blocks)
//   K scales [P][D/32]    fp16 bits
//   V codes  [P*D/2]      4-bit, 32-token chunks, each chunk D/64 wave-loads of
//                         1 KiB; lane (g, n) of load u holds, in dword w, dim
//                         16(4u+w)+n of the 8 tokens 8g..8g+7 of the chunk
//                         (the MFMA B operand of the P*V product)
//   V scales [P/32][D/32][32]  fp16 bits, block-major inside each 32-token chunk
// Every wave-level load of the streaming kernels is therefore one contiguous,
// 16-byte-per-lane, 1 KiB request.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kBlock = 32;       // values per quantization block
constexpr int kTile = 16;        // tokens per K tile (MFMA N/M = 16)
constexpr int kChunk = 32;       // tokens per V chunk (MFMA K = 32)

constexpr int kBlock2 = 128;     // values per INT2 block

struct Geom {
    int D;          // head_dim
    int P;          // page_size
    int n_kv;       // KV heads
    int n_pages;    // physical pages
    int codec = 0;  // 0: K Q8_0 + V Q4_0; 1: K and V INT2
    __host__ __device__ int nb() const { return D / kBlock; }
    __host__ __device__ int64_t k_codes_off() const { return 0; }
    __host__ __device__ int64_t k_scales_off() const { return (int64_t)P * D; }
    __host__ __device__ int64_t v_codes_off() const { return (int64_t)P * D + (int64_t)P * nb() * 2; }
    __host__ __device__ int64_t v_scales_off() const { return v_codes_off() + (int64_t)P * D / 2; }
    __host__ __device__ int64_t unit_bytes() const {
        return codec == 1 ? i2_v_zeros_off() + (int64_t)P * nb2() * 2 : v_scales_off() + (int64_t)P * nb() * 2;
    }
    __host__ __device__ int64_t unit_index(int page, int kvh) const { return (int64_t)page * n_kv + kvh; }
    // INT2 unit: K codes, V codes, K (scale, zero), V scales, V zeros
    __host__ __device__ int nb2() const { return D / kBlock2; }
    __host__ __device__ int64_t i2_v_codes_off() const { return (int64_t)P * D / 4; }
    __host__ __device__ int64_t i2_k_params_off() const { return (int64_t)P * D / 2; }
    __host__ __device__ int64_t i2_v_scales_off() const { return i2_k_params_off() + (int64_t)P * nb2() * 4; }
    __host__ __device__ int64_t i2_v_zeros_off() const { return i2_v_scales_off() + (int64_t)P * nb2() * 2; }
};

// INT2 code words: 8 codes each, two words per dword -- code e of word h
// (0: the even word, 1: the odd one) at bit 16 (e / 4) + 8 h + 2 (e % 4).
// Spread into nibbles (x & 0x33333333, (x >> 2) & 0x33333333), every byte
// then holds two codes of one word as two fp4 values, ready for the gfx950
// fp4 -> fp16 conversion.
__host__ __device__ inline int i2_bit(int h, int e) { return 16 * (e / 4) + 8 * h + 2 * (e % 4); }
// INT2 unit: byte offset of the dword holding K code (slot s, dim d), and
// the code's bit in it.
__host__ __device__ inline int64_t i2_k_dword(const Geom& g, int s, int d, int* bit) {
    const int t = s / kTile, n = s % kTile, step = d / 32, grp = (d % 32) / 8;
    *bit = i2_bit(step & 1, d % 8);
    return (int64_t)t * kTile * g.D / 4 + (int64_t)(grp * 16 + n) * (g.D / 16) + (step / 2) * 4;
}
// INT2 unit: the same for V code (slot s, dim d).
__host__ __device__ inline int64_t i2_v_dword(const Geom& g, int s, int d, int* bit) {
    const int c = s / kChunk, grp = (s % kChunk) / 8, w = d / 16, n = d % 16;
    *bit = i2_bit(w & 1, s % 8);
    return g.i2_v_codes_off() + (int64_t)c * kChunk * g.D / 4 + (int64_t)(grp * 16 + n) * (g.D / 8) + (w / 2) * 4;
}

// Byte offset (within a unit) of K code (slot s, dim d).
__host__ __device__ inline int64_t k_code_pos(const Geom& g, int s, int d) {
    int t = s / kTile, n = s % kTile;
    int p = d / 64, r = d % 64, half = r / 32, w = r % 32, grp = w / 8, e = w % 8;
    return (int64_t)t * kTile * g.D + ((int64_t)(p * 64 + grp * 16 + n) * 16) + half * 8 + e;
}

// Byte offset (within a unit) of the byte holding V code (slot s, dim d), and
// the nibble (0 = low) inside it.  Slots 2k and 2k+1 share a byte.
__host__ __device__ inline int64_t v_code_pos(const Geom& g, int s, int d, int* nibble) {
    int c = s / kChunk, jj = s % kChunk, grp = jj / 8, i = jj % 8;
    int tau = d / 16, n = d % 16, u = tau / 4, w = tau % 4;
    *nibble = i & 1;
    return g.v_codes_off() + (int64_t)c * kChunk * g.D / 2 +
           (int64_t)(u * 64 + grp * 16 + n) * 16 + w * 4 + i / 2;
}

// Index (in fp16 elements, within the V-scale array) of V scale (slot s, block b).
__host__ __device__ inline int v_scale_idx(const Geom& g, int s, int b) {
    return ((s / kChunk) * g.nb() + b) * kChunk + s % kChunk;
}

// Launch plan for attention: which kernel and how the keys are split.
struct AttnPlan {
    int kernel;            // 1 VALU, 2 MFMA streaming, 3 MFMA LDS-tiled, 4 INT2 streaming
    int chunks_per_split;  // 32-token chunks per merged partial
    int n_splits;          // partials per query row
    int group;             // q heads per KV head
    int rows;              // n_q * group: query rows per KV head
};

struct AttnArgs {
    Geom g;
    const uint8_t* pool;
    const int32_t* page_table;
    int ctx;
    int n_heads;
    int n_q;
    const float* q;
    float scale;
    float* out;
    float* lse;
    float* ws_acc;   // [n_q*n_heads][n_splits][D]
    float* ws_m;     // [n_q*n_heads][n_splits]   log2-domain running max
    float* ws_l;     // [n_q*n_heads][n_splits]   sum of exp2(s - m)
    // 1: the n_q query rows are the last n_q positions of the ctx keys (key j
    // visible to query i iff j <= ctx - n_q + i).  0: every row sees all ctx
    // keys (the cached part of a fused append + attention call).
    int causal = 1;
};

// Rows appended by the fused append + attention call.  The merge kernel
// quantizes them, writes their codes into the pool and adds their keys
// (causally among themselves) to the split partials over the cached keys.
struct NewRows {
    uint8_t* pool;   // the pool, writable
    const float* k;  // [n_new][n_kv][D]
    const float* v;  // [n_new][n_kv][D]
    int pos0;        // position of the first new row (= cached keys)
    int n_new;       // = n_q
};

// Several sequences in one launch (batched decode): each has its own context
// length, page-table row and split count; the streaming kernel's workgroups
// and the merge kernel's rows are dealt to the sequences in order.  n = 0: a
// single-sequence call, where AttnArgs and the plan say everything.
constexpr int kMaxSeqs = 64;
struct SeqBatch {
    int n = 0;                 // sequences in the launch
    int n_table = 0;           // page-table entries per sequence (row stride of the page tables)
    int wg0[kMaxSeqs + 1];     // first streaming workgroup of sequence b; wg0[n] = the grid
    int ctx[kMaxSeqs];         // keys of sequence b
    int n_splits[kMaxSeqs];    // partials per query row of sequence b
    int part0[kMaxSeqs];       // first partial of sequence b (rows of all sequences are n_q * n_heads)
};
struct NoBatch {};             // the kernel argument of single-sequence launches

// Index of the sequence that owns item `i` of a launch, given each sequence's
// first item (first[0] = 0, first[n] = the total); uniform across the wave.
__device__ inline int seq_of(const int* first, int n, int i) {
    int b = 0;
    while (b + 1 < n && i >= first[b + 1]) ++b;
    return b;
}

// Workspace bytes for a plan.
inline size_t ws_bytes_for(const AttnPlan& pl, int n_q, int n_heads, int D) {
    if (pl.n_splits <= 1 && pl.kernel == 3) return 0;
    size_t rows = (size_t)n_q * n_heads;
    size_t acc = rows * pl.n_splits * D * sizeof(float);
    size_t ml = rows * pl.n_splits * sizeof(float);
    return acc + 2 * ((ml + 255) / 256 * 256);
}

// Raises kernel Kern's dynamic LDS limit to `bytes`, once per kernel and
// device (so that a launch inside a stream capture makes no such call).
template <auto Kern>
inline hipError_t allow_lds(int bytes) {
    static unsigned int done = 0;   // bit d: set on device d
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned int bit = dev < 32 ? 1u << dev : 0u;
    if (bit != 0 && (__atomic_load_n(&done, __ATOMIC_ACQUIRE) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit != 0) __atomic_fetch_or(&done, bit, __ATOMIC_RELEASE);
    return e;
}

// Kernel launchers (each returns the hipError_t of its launch).
hipError_t launch_append(const Geom& g, uint8_t* pool, const int32_t* page_table, int pos0,
                         int n_new, const float* k, const float* v, hipStream_t stream);
hipError_t launch_attn_valu(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream);
hipError_t launch_attn_mfma_stream(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream,
                                   const SeqBatch* batch = nullptr);
hipError_t launch_attn_mfma_tiled(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream);
hipError_t launch_merge(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream, const SeqBatch* batch = nullptr);
// Merge of n_splits partials (0: none) with the new rows' keys, and the
// rows' quantized write into the pool.
hipError_t launch_merge_new(const AttnArgs& a, const NewRows& nr, int n_splits, hipStream_t stream);
// The streaming MFMA kernel of a fused decode step (pl.n_splits >= 1 over the
// cached keys): it also quantizes the nr.n_new appended rows into the pool
// and leaves new row j's softmax state as partial n_splits + j of every row
// (n_splits + n_new partials per row, folded by launch_merge with that count).
hipError_t launch_attn_mfma_stream_new(const AttnArgs& a, const AttnPlan& pl, const NewRows& nr, hipStream_t stream);
// Streaming MFMA kernel: row groups per workgroup, and waves sharing one row
// group (each partial folds that many waves' chunks), for a given row count.
int mfma_stream_row_groups(int rows);
int mfma_stream_waves(int rows);
// In-place normalized Hadamard rotation of n_rows rows of dim floats (dim a
// power of two in [2, 1024], n_rows in [1, 2^31 - 1]).
hipError_t launch_hadamard(float* x, int64_t n_rows, int dim, hipStream_t stream);
// Decode over the INT2 codec (rows <= 16) and its waves per workgroup.
hipError_t launch_attn_int2(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream,
                            const SeqBatch* batch = nullptr);
int int2_waves();
// The INT2 streaming kernel of a fused decode step (rows <= 16, pl.n_splits
// >= 1 over the cached keys, 1 <= nr.n_new <= int2_max_new_rows()): it also
// quantizes the appended rows into the pool and leaves new row j's softmax
// state as partial n_splits + j of every row, like
// launch_attn_mfma_stream_new.
hipError_t launch_attn_int2_new(const AttnArgs& a, const AttnPlan& pl, const NewRows& nr, hipStream_t stream);
int int2_max_new_rows();
// Query rows per workgroup of the LDS-tiled MFMA kernel.
int mfma_tiled_rows_per_wg();

}  // namespace kvq
