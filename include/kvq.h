/*
 * kvq.h -- C ABI of libkvq: attention over a block-quantized, paged KV cache
 * on one AMD Instinct MI355X (gfx950).
 *
 * K is stored as Q8_0 and V as Q4_0: blocks of 32 consecutive values of one
 * (token, KV head) row, each block with one fp16 scale
 *   ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070 XT at 262k context, via
 *    adaptive KV streaming", first paragraph;
 *    "Adaptive KV streaming lands on ROCm: Qwen3.8-27B at full 262k context on
 *    a 16 GB RX 9070 XT", "What shipped";
 *    "OSCAR2 KV Cache benchmark", compression-ratio table: Q8_0 = 136 bytes
 *    per 128 values).
 * The cache lives in fixed-size pages of tokens reached through a page table;
 * decode attention is computed split over pages and the per-split results are
 * merged with an online log-sum-exp ("Qwen 27B ... RX 9070 XT", second and
 * third paragraphs: per-page online-LSE accumulation for chunked prefill, and
 * paged decode attention extended to the speculative verify batch).
 *
 * Conventions for every call:
 *  - Pointers named d_* are device pointers (HIP, same device as the stream);
 *    the library never dereferences them on the host and never copies them.
 *  - The caller owns every buffer.  The library allocates nothing, keeps no
 *    state between calls and may be called from several host threads.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and is asynchronous; a returned KVQ_OK means "validated and enqueued".
 *  - Every condition that can be checked on the host is checked before any
 *    launch; on failure nothing is enqueued, a negative kvq_status is
 *    returned and kvq_last_error() describes it (thread-local).
 *  - Page-table entries outside [0, n_pages) are never dereferenced: append
 *    skips such rows, attention writes NaN for rows that would read them.
 *  - Inputs must be finite; behaviour for NaN/Inf inputs is unspecified.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_BLOCK 32          /* values per quantization block */
#define KVQ_MAX_NQ_DECODE 8   /* largest n_q accepted by kvq_decode_attn */
#define KVQ_MAX_SEQS 64       /* largest n_seqs accepted by kvq_decode_attn_batch */

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = -1,   /* null pointer, negative size, inconsistent shapes */
    KVQ_ERR_UNSUPPORTED = -2,   /* head_dim / page_size / group size outside the built set */
    KVQ_ERR_WORKSPACE = -3,     /* workspace missing or smaller than kvq_workspace_bytes() */
    KVQ_ERR_CAPACITY = -4,      /* positions beyond what the page table covers */
    KVQ_ERR_HIP = -5            /* the HIP runtime reported an error at launch */
} kvq_status;

/*
 * Shape of one layer's page pool.
 *   n_kv_heads  KV heads of the layer, >= 1
 *   head_dim    D, one of 64, 128, 256 (128 or 256 for KVQ_CODEC_INT2)
 *   page_size   tokens per page, a multiple of 32 in [32, 1024]
 *   n_pages     physical pages in the pool, >= 1
 *   codec       how K and V are stored: KVQ_CODEC_Q8K_Q4V (0, the default
 *               of a zero-initialised layout) or KVQ_CODEC_INT2
 */
#define KVQ_CODEC_Q8K_Q4V 0   /* K Q8_0, V Q4_0, 32-value blocks */
#define KVQ_CODEC_INT2 1      /* K and V INT2, 128-value blocks with an fp16 scale and zero-point */
typedef struct {
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t n_pages;
    int32_t codec;
} kvq_layout;

/*
 * Pool memory.  The pool is one device allocation of kvq_pool_bytes() bytes,
 * 256-byte aligned, made of n_pages * n_kv_heads units; unit (page p, KV head
 * g) starts at (p * n_kv_heads + g) * kvq_unit_bytes().  A unit holds the
 * page_size tokens of one KV head (P = page_size, D = head_dim, nb = D/32):
 *
 *   [0, P*D)                 K codes, int8 two's complement, tile order:
 *                            16-token tiles t; inside a tile, 16-byte pieces
 *                            (p, lane) with p < D/64 and lane = g*16 + n
 *                            (g < 4, n < 16) hold token 16t+n, bytes 0..7 =
 *                            dims 64p+8g+(0..7) (block 2p), bytes 8..15 =
 *                            dims 64p+32+8g+(0..7) (block 2p+1).
 *   [P*D, P*D + 2*P*nb)      K scales, fp16 bits, [token][block].
 *   next P*D/2 bytes         V codes, 4 bits each, chunk order: 32-token
 *                            chunks c; inside a chunk, 16-byte pieces
 *                            (u, lane) with u < D/64, lane = g*16 + n; dword
 *                            w < 4 of a piece holds dim 16(4u+w)+n of tokens
 *                            32c+8g+i (i < 8) in bits 4i..4i+3.
 *   next 2*P*nb bytes        V scales, fp16 bits, [chunk][block][32 tokens]
 *                            (block-major inside each 32-token chunk).
 *
 * A value is scale * code for K and scale * (code - 8) for V.  The unit is
 * 26*P*D/16 bytes: 416 bytes per token at D = 256, matching Q8_0 (34 B) +
 * Q4_0 (18 B) per 32-value block ("Adaptive KV streaming lands on ROCm ...",
 * "Why it matters": 26,624 bytes per token over 16 layers).
 *
 * KVQ_CODEC_INT2 ("OSCAR2 KV Cache benchmark", compression-ratio table: a
 * 2-bit cache of 36 bytes per 128 values with fp16 zero-point metadata, the
 * same codec for K and V).  Per block of 128 values of one row: mn = min,
 * mx = max, d = (mx - mn) / 3 (fp32), code = min(3, floor((x - mn) * (1/d)
 * + 0.5)) (0 when d = 0; each operation rounded to fp32), stored scale =
 * fp16(d) and zero = fp16(mn); the value is zero + scale * code.  Unit
 * layout (nb2 = D/128).  Codes come in words of 8 codes, two words per
 * dword: code e (< 8) of word 2i+h (h < 2) sits at bit
 * 16*(e/4) + 8*h + 2*(e%4) of dword i.
 *   [0, P*D/4)               K codes, 16-token tiles t; inside a tile lane
 *                            L = g*16 + n (g < 4, n < 16) has D/16 bytes:
 *                            word s < D/32 holds dims 32s+8g+e of token
 *                            16t+n.
 *   next P*D/4 bytes         V codes, 32-token chunks c; inside a chunk lane
 *                            L = g*16 + n has D/8 bytes: word w < D/16 holds
 *                            dim 16w+n of tokens 32c+8g+e.
 *   next 4*P*nb2 bytes       K scale and zero, fp16 bits, [token][block][2].
 *   next 2*P*nb2 bytes       V scales, fp16 bits, [chunk][block][32 tokens].
 *   next 2*P*nb2 bytes       V zeros, fp16 bits, [chunk][block][32 tokens].
 * The unit is 9*P*D/16 bytes: 144 bytes per token at D = 256.
 * Attention over this codec: kernel 4 (its streaming kernel: decode, verify
 * and kvq_decode_attn_batch with n_q * group <= 16) and kernel 3 (the
 * LDS-tiled kernel: kvq_prefill_attn, and decode or verify with more rows);
 * kernel 0 picks 4 where it applies, else 3.  kvq_append_attn runs
 * kvq_append and then the attention call.
 */
int kvq_unit_bytes(const kvq_layout *layout, size_t *bytes);
int kvq_pool_bytes(const kvq_layout *layout, size_t *bytes);

/*
 * kvq_append -- quantize n_new new K/V rows into the pool.
 *
 * Row r (0 <= r < n_new) is token position pos0 + r; it goes to physical page
 * d_page_table[(pos0 + r) / page_size], slot (pos0 + r) % page_size.
 *   d_k, d_v      fp32 [n_new][n_kv_heads][head_dim], device
 *   d_page_table  int32 [n_table], device; logical page -> physical page
 *   n_table       entries in the page table; (pos0 + n_new) <= n_table * page_size
 * Per block of 32 values (IEEE fp32 arithmetic, bit-reproducible):
 *   K (Q8_0): d = max|x| / 127; code = round-half-away-from-zero(x * (1/d))
 *             (0 when d = 0); scale = fp16(d), nearest-even.
 *   V (Q4_0): m = the first value of largest magnitude (+0 if all are zero);
 *             d = m / -8; code = min(15, floor(x * (1/d) + 8.5)) with the
 *             product and the sum rounded separately (code 8 when d = 0);
 *             scale = fp16(d).
 * Other slots of the touched pages are left as they were.  Rows that share a
 * pool byte are written by one thread; calls on one stream are ordered, and
 * calls on different streams must not touch the same page concurrently.
 * Errors: INVALID_ARG (null pointers, n_new < 0, pos0 < 0), UNSUPPORTED,
 * CAPACITY, HIP.  n_new == 0 is a no-op.
 */
int kvq_append(const kvq_layout *layout, void *d_pool,
               const int32_t *d_page_table, int32_t n_table,
               int32_t pos0, int32_t n_new,
               const float *d_k, const float *d_v, void *stream);

/*
 * Attention.  Keys are the token positions [0, ctx_len).  Query i (0 <= i <
 * n_q) sits at position ctx_len - n_q + i and attends to every key at a
 * position <= its own (its own key included, so append first).  Query head h
 * uses KV head h / (n_heads / n_kv_heads) ("Context window and KV cache", GQA
 * section: several query heads share one KV head).  Attention reads the
 * quantized values:
 *   s_j = scale * sum_d q[d] * Khat_j[d],  o = sum_j softmax(s)_j * Vhat_j,
 *   lse = log(sum_j exp(s_j))              (natural log)
 * i.e. exact softmax attention ("Context window and KV cache", flash-attention
 * lever) over the dequantized cache.
 *   d_q    fp32 [n_q][n_heads][head_dim]
 *   d_out  fp32 [n_q][n_heads][head_dim]
 *   d_lse  fp32 [n_q][n_heads], may be NULL
 *   d_ws   workspace of at least kvq_workspace_bytes() bytes (NULL if that is 0)
 * The result does not depend on how the cache is split internally beyond
 * fp32 rounding.  Errors: INVALID_ARG (nulls, n_q < 1, ctx_len < n_q,
 * n_heads % n_kv_heads != 0), UNSUPPORTED (n_heads / n_kv_heads > 16 or
 * n_q * group > 64 for decode; a kernel choice that does not read the
 * layout's codec), CAPACITY (ctx_len > n_table * page_size), WORKSPACE, HIP.
 */

/* Workspace bytes kvq_decode_attn / kvq_prefill_attn need for this shape. */
int kvq_workspace_bytes(const kvq_layout *layout, int32_t n_heads, int32_t ctx_len,
                        int32_t n_q, int32_t prefill, size_t *bytes);

/* kvq_decode_attn -- one decode query (n_q = 1) or a speculative verify batch
 * (2 <= n_q <= KVQ_MAX_NQ_DECODE): split over pages, merged by online LSE. */
int kvq_decode_attn(const kvq_layout *layout, const void *d_pool,
                    const int32_t *d_page_table, int32_t n_table,
                    int32_t ctx_len, int32_t n_heads, int32_t n_q,
                    const float *d_q, float scale,
                    float *d_out, float *d_lse,
                    void *d_ws, size_t ws_bytes, void *stream);

/* kvq_prefill_attn -- a causal chunk of n_q >= 1 queries (chunked prefill). */
int kvq_prefill_attn(const kvq_layout *layout, const void *d_pool,
                     const int32_t *d_page_table, int32_t n_table,
                     int32_t ctx_len, int32_t n_heads, int32_t n_q,
                     const float *d_q, float scale,
                     float *d_out, float *d_lse,
                     void *d_ws, size_t ws_bytes, void *stream);

/*
 * Explicit kernel and split choice, for tests and tuning.  Same semantics and
 * errors as kvq_decode_attn / kvq_prefill_attn.
 *   kernel: 0 = automatic, 1 = portable VALU kernel (any supported shape),
 *           2 = MFMA streaming kernel (n_q * group <= 64),
 *           3 = MFMA LDS-tiled chunk kernel (both codecs),
 *           4 = MFMA streaming kernel of KVQ_CODEC_INT2 (decode, n_q * group <= 16);
 *           1 and 2 read KVQ_CODEC_Q8K_Q4V only
 *   chunks_per_split: 0 = automatic.  Kernels 1 and 3: 32-token chunks per
 *           merged partial.  Kernels 2 and 4: 32-token chunks per wave of a
 *           split; a merged partial covers the split's waves (the 8 waves of
 *           a workgroup, or the 4 of a row group above 32 rows) times this.
 *   kernel_begin_event, kernel_end_event: optional hipEvent_t handles (or
 *           NULL), recorded on `stream` immediately before and after the
 *           attention kernel itself (not the split merge), so a caller can time
 *           that kernel alone.  Owned by the caller.
 */
typedef struct {
    int32_t kernel;
    int32_t chunks_per_split;
    void *kernel_begin_event;
    void *kernel_end_event;
} kvq_attn_opts;

int kvq_workspace_bytes_ex(const kvq_layout *layout, int32_t n_heads, int32_t ctx_len,
                           int32_t n_q, const kvq_attn_opts *opts, size_t *bytes);

int kvq_attn_ex(const kvq_layout *layout, const void *d_pool,
                const int32_t *d_page_table, int32_t n_table,
                int32_t ctx_len, int32_t n_heads, int32_t n_q,
                const float *d_q, float scale,
                float *d_out, float *d_lse,
                void *d_ws, size_t ws_bytes, const kvq_attn_opts *opts, void *stream);

/*
 * One decode step: kvq_append of n_new rows at pos0, then attention of the
 * n_new queries over the pos0 + n_new keys -- exactly kvq_append followed by
 * kvq_attn_ex(ctx_len = pos0 + n_new, n_q = n_new), in two launches instead
 * of three ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070 XT at 262k
 * context, via adaptive KV streaming": quantize on append, paged decode
 * attention, online log-sum-exp across pages).  Over the Q8_0/Q4_0 cache
 * with the streaming kernel (opts->kernel 0 or 2, n_new * group <= 64), and
 * over the INT2 cache with its streaming kernel (opts->kernel 0 or 4,
 * n_new * group <= 16, pos0 >= 1), the split pass reads the pos0 cached keys
 * only; the new rows are quantized (the same codes and scales kvq_append
 * writes), written into the pool and scored by the split pass (or, over
 * Q8_0/Q4_0 with more than 32 query rows or no cached keys, by the merge
 * pass), and the merge pass folds them into the softmax.  Other choices run
 * kvq_append and the attention one after the other.
 *   pos0, n_new, d_k, d_v  as for kvq_append (1 <= n_new <= KVQ_MAX_NQ_DECODE)
 *   d_q, d_out, d_lse      as for attention with n_q = n_new
 *   d_ws   workspace of at least kvq_append_attn_workspace_bytes() bytes
 *          (NULL if that is 0); opts as for kvq_attn_ex, may be NULL.
 * Every pool byte the call changes is written by one thread (the two slots
 * of a V byte together); the same ordering rules as kvq_append apply.  Errors: as kvq_append and
 * kvq_attn_ex (INVALID_ARG also for n_new outside [1, KVQ_MAX_NQ_DECODE]).
 */
int kvq_append_attn_workspace_bytes(const kvq_layout *layout, int32_t n_heads, int32_t pos0,
                                    int32_t n_new, const kvq_attn_opts *opts, size_t *bytes);

int kvq_append_attn(const kvq_layout *layout, void *d_pool,
                    const int32_t *d_page_table, int32_t n_table,
                    int32_t pos0, int32_t n_new,
                    const float *d_k, const float *d_v,
                    int32_t n_heads, const float *d_q, float scale,
                    float *d_out, float *d_lse,
                    void *d_ws, size_t ws_bytes, const kvq_attn_opts *opts, void *stream);

/*
 * kvq_append_attn_noalloc -- kvq_append_attn without a workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The split partials live in
 * a static device array of kvq_noalloc_scratch_bytes() bytes (8 MiB) that the
 * library holds on every GPU it runs on until the process ends; the call
 * itself allocates nothing.  Arguments, results and errors are those of
 * kvq_append_attn with d_ws / ws_bytes left out, plus WORKSPACE when the step
 * needs more scratch than the array holds (kvq_append_attn_workspace_bytes()
 * tells; e.g. 24 heads over 4 KV heads at head_dim 256 fit up to n_new = 4).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (several host threads, or several streams) race and give wrong
 * results.  Nothing in the array needs to start at any value.
 */
size_t kvq_noalloc_scratch_bytes(void);

int kvq_append_attn_noalloc(const kvq_layout *layout, void *d_pool,
                            const int32_t *d_page_table, int32_t n_table,
                            int32_t pos0, int32_t n_new,
                            const float *d_k, const float *d_v,
                            int32_t n_heads, const float *d_q, float scale,
                            float *d_out, float *d_lse, const kvq_attn_opts *opts, void *stream);

/*
 * Batched decode: n_seqs independent sequences in one call, each with its own
 * context length and page-table row, all in one page pool (sequences normally
 * own disjoint pages).  For every sequence b it computes exactly what
 * kvq_decode_attn computes for that sequence alone ("Qwen 27B (IQ4_XS, Q8/Q4
 * KV) on a 16GB RX 9070 XT at 262k context, via adaptive KV streaming", third
 * paragraph: paged decode attention; the server there answers several
 * requests at once): query i of b sits at position ctx_lens[b] - n_q + i.
 *   d_page_tables  int32 [n_seqs][n_table], device; row b is sequence b's table
 *   ctx_lens       int32 [n_seqs], HOST memory (the split plan is made on the
 *                  host); n_q <= ctx_lens[b] <= n_table * page_size
 *   d_q            fp32 [n_seqs][n_q][n_heads][head_dim]
 *   d_out          fp32 [n_seqs][n_q][n_heads][head_dim]
 *   d_lse          fp32 [n_seqs][n_q][n_heads], may be NULL
 *   d_ws           workspace of at least kvq_decode_attn_batch_workspace_bytes()
 *                  bytes for the same n_seqs, ctx_lens, n_heads and n_q
 *   opts           may be NULL; as for kvq_attn_ex, except that kernel must be
 *                  0 or the codec's streaming kernel (2 for
 *                  KVQ_CODEC_Q8K_Q4V, 4 for KVQ_CODEC_INT2) and
 *                  chunks_per_split is ignored (the events bracket the
 *                  streaming kernel of all sequences)
 * 1 <= n_seqs <= KVQ_MAX_SEQS, 1 <= n_q <= KVQ_MAX_NQ_DECODE, and
 * n_q * (n_heads / n_kv_heads) <= 64 (16 for KVQ_CODEC_INT2; the streaming
 * kernel runs every sequence; a sequence's share of the workgroups follows
 * its context length).
 * Errors: INVALID_ARG (nulls, n_seqs or n_q out of range, a ctx_lens[b] <
 * n_q, opts->kernel other than 0, 2 or 4), UNSUPPORTED (the other codec's
 * kernel, too many rows), CAPACITY (a ctx_lens[b] > n_table * page_size),
 * WORKSPACE, HIP.
 */
int kvq_decode_attn_batch_workspace_bytes(const kvq_layout *layout, int32_t n_seqs, const int32_t *ctx_lens,
                                          int32_t n_heads, int32_t n_q, size_t *bytes);

int kvq_decode_attn_batch(const kvq_layout *layout, const void *d_pool,
                          const int32_t *d_page_tables, int32_t n_table,
                          int32_t n_seqs, const int32_t *ctx_lens,
                          int32_t n_heads, int32_t n_q,
                          const float *d_q, float scale,
                          float *d_out, float *d_lse,
                          void *d_ws, size_t ws_bytes, const kvq_attn_opts *opts, void *stream);

/*
 * Host-resident KV streaming ("Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070
 * XT at 262k context, via adaptive KV streaming", first paragraph: the cache
 * lives in host memory and its pages stream to the GPU as attention needs
 * them).  Copies logical pages 0 .. n_copy-1 of a sequence, whose physical
 * pages in a host pool are h_page_table[0 .. n_copy-1], to consecutive
 * physical pages dst_first .. dst_first + n_copy - 1 of a device pool, as
 * asynchronous copies on `stream` (runs of consecutive host pages go as one
 * copy).  Attention then reads the device pool with the page table
 * dst_first + i.
 *   host_layout, h_pool   the host pool (pinned memory for copies that overlap
 *                         the GPU's work; pageable memory also works, with
 *                         copies the runtime may serialize)
 *   h_page_table          int32 [n_copy], HOST memory
 *   dev_layout, d_pool    the device pool; n_kv_heads, head_dim, page_size
 *                         and codec must equal the host pool's
 * The source pages must not change until the copies are done (an event
 * recorded on `stream` after this call tells when).  Errors: INVALID_ARG
 * (nulls, n_copy < 0, layouts that differ, a host page outside the host pool,
 * destination pages past the device pool), HIP.  n_copy == 0 is a no-op.
 */
int kvq_stage_pages(const kvq_layout *host_layout, const void *h_pool, const int32_t *h_page_table,
                    int32_t n_copy, const kvq_layout *dev_layout, void *d_pool, int32_t dst_first,
                    void *stream);

/*
 * kvq_hadamard -- rotate rows in place: x_r <- x_r H / sqrt(dim), H the dim x
 * dim Hadamard matrix of Sylvester's construction (H_1 = [1], H_2m =
 * [[H_m, H_m], [H_m, -H_m]]).  The 2-bit cache is meant to hold rotated K and
 * V ("OSCAR2 KV Cache benchmark", rotation model conversion: a Hadamard
 * rotation per head baked into the model), which spreads outlier channels
 * over the whole row.  H / sqrt(dim) is orthogonal and its own inverse, so a
 * caller that rotates k and v before kvq_append and q before the attention
 * call gets the same scores and the rotated output, which one more
 * kvq_hadamard turns back.
 *   d_x     fp32 [n_rows][dim], device, contiguous rows; read and written
 *   dim     a power of two in [2, 1024] (head_dim)
 * fp32 butterflies in a fixed order, then one product by fp32(1/sqrt(dim)).
 * Errors: INVALID_ARG (dim not such a power of two, n_rows < 0 or > 2^31 - 1,
 * n_rows * dim / 2 >= 2^32 (one thread per pair of values: larger inputs go
 * in several calls), NULL or misaligned x), HIP.  n_rows == 0 is a no-op.
 */
int kvq_hadamard(float *d_x, int64_t n_rows, int32_t dim, void *stream);

/* Status name, and the detail of the last failure on this thread. */
const char *kvq_status_str(int status);
const char *kvq_last_error(void);

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH. */
int kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
