// kvq_api.hip -- the C ABI of libkvq: argument validation, launch planning and
// dispatch onto the caller's HIP stream.  Declarations and semantics are in
// include/kvq.h.  Nothing here allocates device memory or synchronizes.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>

#include "../../include/kvq.h"
#include "kvq_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return KVQ_OK;
}

// The current detail, copied (for a message that wraps it).
const char* kvq_last_error_copy() {
    thread_local char copy[512];
    snprintf(copy, sizeof(copy), "%s", g_err);
    return copy;
}

int check_layout(const kvq_layout* L, kvq::Geom* g) {
    if (L == nullptr) return fail(KVQ_ERR_INVALID_ARG, "layout is NULL");
    if (L->n_kv_heads < 1 || L->head_dim < 1 || L->page_size < 1 || L->n_pages < 1)
        return fail(KVQ_ERR_INVALID_ARG, "layout fields must be >= 1 (n_kv_heads=%d head_dim=%d page_size=%d n_pages=%d)",
                    L->n_kv_heads, L->head_dim, L->page_size, L->n_pages);
    if (L->head_dim != 64 && L->head_dim != 128 && L->head_dim != 256)
        return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d not built (64, 128, 256)", L->head_dim);
    if (L->page_size % kvq::kChunk != 0 || L->page_size > 1024)
        return fail(KVQ_ERR_UNSUPPORTED, "page_size %d must be a multiple of 32 in [32, 1024]", L->page_size);
    if (L->codec != KVQ_CODEC_Q8K_Q4V && L->codec != KVQ_CODEC_INT2)
        return fail(KVQ_ERR_INVALID_ARG, "unknown codec %d", L->codec);
    if (L->codec == KVQ_CODEC_INT2 && L->head_dim % kvq::kBlock2 != 0)
        return fail(KVQ_ERR_UNSUPPORTED, "the INT2 codec takes head_dim 128 or 256 (got %d)", L->head_dim);
    *g = kvq::Geom{L->head_dim, L->page_size, L->n_kv_heads, L->n_pages, L->codec};
    const double total = (double)g->unit_bytes() * L->n_kv_heads * L->n_pages;
    if (total > 9.0e18) return fail(KVQ_ERR_INVALID_ARG, "pool size overflows");
    return KVQ_OK;
}

// Compute units of the current device (256 on an MI355X).
int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    return cus;
}

// Split heuristic: enough independent wavefronts to cover the CUs, with
// partials small next to the cache bytes.
int auto_chunks_per_split(int kernel, int total_chunks, int n_kv, int n_q, int rows) {
    long units = (long)total_chunks * n_kv;
    if (kernel == 1) {
        // one wave per (split, KV head, query); aim for ~4096 waves
        long per = units * n_q / 4096;
        return (int)(per < 1 ? 1 : per);
    }
    if (kernel == 2 || kernel == 4) {
        // one 8-wave workgroup fits a CU (registers): at most one workgroup
        // per CU and KV head-split, so that all run in a single round; each
        // wave of a row group takes cps chunks of its split
        const long cus = device_cus();
        long splits = cus / n_kv;
        if (splits < 1) splits = 1;
        const long wpg = kernel == 4 ? kvq::int2_waves() : kvq::mfma_stream_waves(rows);
        long per = ((long)total_chunks + wpg * splits - 1) / (wpg * splits);
        return (int)(per < 1 ? 1 : per);
    }
    // LDS-tiled chunk kernel: a workgroup per (row tile, KV head, split);
    // split the keys until about three workgroups per CU exist, keeping at
    // least 16 chunks per split
    (void)units;
    const int rpw = kvq::mfma_tiled_rows_per_wg();
    const long tiles = (long)((rows + rpw - 1) / rpw) * n_kv;
    long splits = (768 + tiles - 1) / tiles;
    long max_splits = total_chunks / 16;
    if (max_splits < 1) max_splits = 1;
    if (splits > max_splits) splits = max_splits;
    return (int)((total_chunks + splits - 1) / splits);
}

int make_plan(const kvq_layout* L, int n_heads, int ctx, int n_q, bool prefill,
              const kvq_attn_opts* opts, kvq::AttnPlan* pl) {
    const int group = n_heads / L->n_kv_heads;
    const int rows = n_q * group;
    int kernel = opts ? opts->kernel : 0;
    if (kernel < 0 || kernel > 4) return fail(KVQ_ERR_INVALID_ARG, "unknown kernel %d", kernel);
    if (L->codec == KVQ_CODEC_INT2) {
        // kernel 4: the INT2 streaming kernel (decode and verify, up to 16
        // rows per KV head); kernel 3: the LDS-tiled kernel (prefill, more rows)
        if (kernel == 1 || kernel == 2)
            return fail(KVQ_ERR_UNSUPPORTED, "the INT2 codec runs kernel 3 or 4 (got kernel %d)", kernel);
        if (kernel == 4 && (prefill || rows > 16))
            return fail(KVQ_ERR_UNSUPPORTED, "kernel 4 takes decode with n_q*group <= 16 (got %d rows%s)", rows,
                        prefill ? ", prefill" : "");
        if (kernel == 0) kernel = (!prefill && rows <= 16) ? 4 : 3;
    } else if (kernel == 4) {
        return fail(KVQ_ERR_INVALID_ARG, "kernel 4 reads the INT2 codec only");
    }
    if (kernel == 0) kernel = (!prefill && rows <= 64) ? 2 : 3;
    if (group > 16) return fail(KVQ_ERR_UNSUPPORTED, "group size %d > 16", group);
    if (kernel == 2 && rows > 64) return fail(KVQ_ERR_UNSUPPORTED, "streaming MFMA kernel takes n_q*group <= 64 (got %d)", rows);
    const int total_chunks = (ctx + kvq::kChunk - 1) / kvq::kChunk;
    int cps = opts ? opts->chunks_per_split : 0;
    if (cps < 0) return fail(KVQ_ERR_INVALID_ARG, "chunks_per_split %d < 0", cps);
    if (cps == 0) cps = auto_chunks_per_split(kernel, total_chunks, L->n_kv_heads, n_q, rows);
    if (cps > total_chunks) cps = total_chunks;
    pl->kernel = kernel;
    pl->chunks_per_split = cps;
    // the streaming MFMA kernel folds the waves of a workgroup into one partial
    const int per_partial = kernel == 2 ? kvq::mfma_stream_waves(rows) * cps
                            : kernel == 4 ? kvq::int2_waves() * cps : cps;
    pl->n_splits = (total_chunks + per_partial - 1) / per_partial;
    pl->group = group;
    pl->rows = rows;
    return KVQ_OK;
}

int check_attn_shape(const kvq_layout* L, int32_t n_table, int32_t ctx, int32_t n_heads, int32_t n_q,
                     bool prefill) {
    if (n_heads < 1 || n_heads % L->n_kv_heads != 0)
        return fail(KVQ_ERR_INVALID_ARG, "n_heads %d must be a positive multiple of n_kv_heads %d", n_heads, L->n_kv_heads);
    if (n_q < 1) return fail(KVQ_ERR_INVALID_ARG, "n_q %d < 1", n_q);
    if (!prefill && n_q > KVQ_MAX_NQ_DECODE)
        return fail(KVQ_ERR_INVALID_ARG, "decode takes n_q <= %d (got %d); use kvq_prefill_attn", KVQ_MAX_NQ_DECODE, n_q);
    if (ctx < n_q) return fail(KVQ_ERR_INVALID_ARG, "ctx_len %d < n_q %d", ctx, n_q);
    if (n_table < 1) return fail(KVQ_ERR_INVALID_ARG, "n_table %d < 1", n_table);
    if ((int64_t)ctx > (int64_t)n_table * L->page_size)
        return fail(KVQ_ERR_CAPACITY, "ctx_len %d exceeds the page table (%d pages of %d)", ctx, n_table, L->page_size);
    return KVQ_OK;
}

int workspace_impl(const kvq_layout* L, int32_t n_heads, int32_t ctx, int32_t n_q, bool prefill,
                   const kvq_attn_opts* opts, size_t* bytes) {
    kvq::Geom g;
    int st = check_layout(L, &g);
    if (st) return st;
    if (bytes == nullptr) return fail(KVQ_ERR_INVALID_ARG, "bytes is NULL");
    if (n_heads < 1 || n_heads % L->n_kv_heads != 0)
        return fail(KVQ_ERR_INVALID_ARG, "n_heads %d must be a positive multiple of n_kv_heads %d", n_heads, L->n_kv_heads);
    if (n_q < 1 || ctx < n_q) return fail(KVQ_ERR_INVALID_ARG, "need 1 <= n_q <= ctx_len (n_q=%d ctx_len=%d)", n_q, ctx);
    kvq::AttnPlan pl;
    st = make_plan(L, n_heads, ctx, n_q, prefill, opts, &pl);
    if (st) return st;
    *bytes = kvq::ws_bytes_for(pl, n_q, n_heads, L->head_dim);
    return ok();
}

int attn_impl(const kvq_layout* L, const void* d_pool, const int32_t* d_page_table, int32_t n_table,
              int32_t ctx, int32_t n_heads, int32_t n_q, const float* d_q, float scale,
              float* d_out, float* d_lse, void* d_ws, size_t ws_bytes, bool prefill,
              const kvq_attn_opts* opts, void* stream) {
    kvq::Geom g;
    int st = check_layout(L, &g);
    if (st) return st;
    if (d_pool == nullptr || d_page_table == nullptr || d_q == nullptr || d_out == nullptr)
        return fail(KVQ_ERR_INVALID_ARG, "pool, page_table, q and out must be non-NULL");
    st = check_attn_shape(L, n_table, ctx, n_heads, n_q, prefill);
    if (st) return st;
    kvq::AttnPlan pl;
    st = make_plan(L, n_heads, ctx, n_q, prefill, opts, &pl);
    if (st) return st;
    const size_t need = kvq::ws_bytes_for(pl, n_q, n_heads, L->head_dim);
    if (need > 0 && (d_ws == nullptr || ws_bytes < need))
        return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, ws_bytes,
                    d_ws == nullptr ? " (NULL)" : "");
    if (((uintptr_t)d_pool & 255) != 0) return fail(KVQ_ERR_INVALID_ARG, "pool must be 256-byte aligned");
    if (((uintptr_t)d_ws & 15) != 0) return fail(KVQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

    kvq::AttnArgs a;
    a.g = g;
    a.pool = static_cast<const uint8_t*>(d_pool);
    a.page_table = d_page_table;
    a.ctx = ctx;
    a.n_heads = n_heads;
    a.n_q = n_q;
    a.q = d_q;
    a.scale = scale;
    a.out = d_out;
    a.lse = d_lse;
    const size_t rows = (size_t)n_q * n_heads;
    const size_t ml = (rows * pl.n_splits * sizeof(float) + 255) / 256 * 256;
    uint8_t* ws = static_cast<uint8_t*>(d_ws);
    a.ws_m = reinterpret_cast<float*>(ws);
    a.ws_l = reinterpret_cast<float*>(ws + ml);
    a.ws_acc = reinterpret_cast<float*>(ws + 2 * ml);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (opts != nullptr && opts->kernel_begin_event != nullptr)
        e = hipEventRecord(static_cast<hipEvent_t>(opts->kernel_begin_event), s);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
    switch (pl.kernel) {
        case 1: e = kvq::launch_attn_valu(a, pl, s); break;
        case 2: e = kvq::launch_attn_mfma_stream(a, pl, s); break;
        case 3: e = kvq::launch_attn_mfma_tiled(a, pl, s); break;
        case 4: e = kvq::launch_attn_int2(a, pl, s); break;
    }
    if (e == hipSuccess && opts != nullptr && opts->kernel_end_event != nullptr)
        e = hipEventRecord(static_cast<hipEvent_t>(opts->kernel_end_event), s);
    if (e == hipSuccess && !(pl.kernel == 3 && need == 0)) e = kvq::launch_merge(a, pl, s);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Fused append + attention.  The streaming kernel can take the cached keys
// alone (every new row sees all of them) and the merge kernel adds the new
// rows; other kernel choices run kvq_append and then the attention call.
// Over the INT2 cache the INT2 streaming kernel appends and scores the new
// rows itself, up to 16 query rows per KV head (its range) and with cached
// keys before them; other INT2 steps run kvq_append and then the attention
// call.
bool append_attn_fused(const kvq_layout* L, int32_t n_heads, int32_t pos0, int32_t n_new, const kvq_attn_opts* opts) {
    const int kernel = opts ? opts->kernel : 0;
    const int rows = n_new * (n_heads / L->n_kv_heads);
    if (L->codec == KVQ_CODEC_INT2)
        return (kernel == 0 || kernel == 4) && pos0 > 0 && rows <= 16 && n_new <= kvq::int2_max_new_rows();
    return L->codec == KVQ_CODEC_Q8K_Q4V && (kernel == 0 || kernel == 2) && rows <= 64;
}

// Where a fused step's new rows are quantized and scored.  With one row
// group the split kernel does it: one wave per new row, whose share of the
// cached chunks the other waves of its workgroup take over from the LDS list.
// With several row groups (the verify batch's fixed chunk order) that wave
// would hold up its workgroup's end, so the merge kernel does it instead.
// The INT2 streaming kernel always does it (one wave per KV head, after its
// chunks).
bool new_rows_in_split(const kvq::AttnPlan& pl) {
    if (pl.kernel == 4) return pl.n_splits > 0;
    return pl.n_splits > 0 && kvq::mfma_stream_row_groups(pl.rows) == 1;
}

// Partials per row of a fused step: the splits over the cached keys, and one
// per new row when the split kernel handles them.
int fused_parts(const kvq::AttnPlan& pl, int n_new) { return pl.n_splits + (new_rows_in_split(pl) ? n_new : 0); }

size_t fused_ws_bytes(const kvq::AttnPlan& pl, int n_new, int n_heads, int D) {
    if (pl.n_splits <= 0) return 0;
    kvq::AttnPlan pw = pl;
    pw.n_splits = fused_parts(pl, n_new);
    return kvq::ws_bytes_for(pw, n_new, n_heads, D);
}

// Plan of the cached part (fused) or of the whole attention (otherwise).
int append_attn_plan(const kvq_layout* L, int32_t n_heads, int32_t pos0, int32_t n_new, const kvq_attn_opts* opts,
                     bool fused, kvq::AttnPlan* pl) {
    if (!fused) return make_plan(L, n_heads, pos0 + n_new, n_new, false, opts, pl);
    kvq_attn_opts o = opts ? *opts : kvq_attn_opts{0, 0, nullptr, nullptr};
    o.kernel = L->codec == KVQ_CODEC_INT2 ? 4 : 2;
    if (pos0 > 0) return make_plan(L, n_heads, pos0, n_new, false, &o, pl);
    int st = make_plan(L, n_heads, kvq::kChunk, n_new, false, &o, pl);   // checks only: no cached keys
    pl->n_splits = 0;
    return st;
}

int check_append_attn(const kvq_layout* L, int32_t n_table, int32_t pos0, int32_t n_new, int32_t n_heads) {
    if (n_heads < 1 || n_heads % L->n_kv_heads != 0)
        return fail(KVQ_ERR_INVALID_ARG, "n_heads %d must be a positive multiple of n_kv_heads %d", n_heads, L->n_kv_heads);
    if (n_new < 1 || n_new > KVQ_MAX_NQ_DECODE)
        return fail(KVQ_ERR_INVALID_ARG, "n_new %d must be in [1, %d]", n_new, KVQ_MAX_NQ_DECODE);
    if (pos0 < 0) return fail(KVQ_ERR_INVALID_ARG, "pos0 %d < 0", pos0);
    if (n_table < 1) return fail(KVQ_ERR_INVALID_ARG, "n_table %d < 1", n_table);
    if ((int64_t)pos0 + n_new > (int64_t)n_table * L->page_size)
        return fail(KVQ_ERR_CAPACITY, "positions up to %lld exceed the page table (%d pages of %d)",
                    (long long)pos0 + n_new, n_table, L->page_size);
    if ((int64_t)pos0 + n_new > INT32_MAX) return fail(KVQ_ERR_CAPACITY, "positions overflow int32");
    return KVQ_OK;
}

// Batched decode plan: every sequence's split count from its share of the
// context (about one workgroup per CU and KV head in all), the workgroup and
// partial offsets of each, and the partials in all (for the workspace).
int batch_plan(const kvq_layout* L, int32_t n_table, int32_t n_seqs, const int32_t* ctx_lens, int32_t n_heads,
               int32_t n_q, kvq::AttnPlan* pl, kvq::SeqBatch* sb, size_t* parts) {
    kvq::Geom g;
    int st = check_layout(L, &g);
    if (st) return st;
    if (n_seqs < 1 || n_seqs > KVQ_MAX_SEQS)
        return fail(KVQ_ERR_INVALID_ARG, "n_seqs %d outside [1, %d]", n_seqs, KVQ_MAX_SEQS);
    if (ctx_lens == nullptr) return fail(KVQ_ERR_INVALID_ARG, "ctx_lens is NULL");
    if (n_q < 1 || n_q > KVQ_MAX_NQ_DECODE)
        return fail(KVQ_ERR_INVALID_ARG, "batched decode takes 1 <= n_q <= %d (got %d)", KVQ_MAX_NQ_DECODE, n_q);
    long total = 0;
    for (int b = 0; b < n_seqs; ++b) {
        st = check_attn_shape(L, n_table, ctx_lens[b], n_heads, n_q, false);
        if (st) return fail(st, "sequence %d: %s", b, kvq_last_error_copy());
        total += (ctx_lens[b] + kvq::kChunk - 1) / kvq::kChunk;
    }
    // the streaming kernel of the codec: 2 (Q8_0/Q4_0) or 4 (INT2)
    kvq_attn_opts opts{L->codec == KVQ_CODEC_INT2 ? 4 : 2, 1, nullptr, nullptr};
    st = make_plan(L, n_heads, ctx_lens[0], n_q, false, &opts, pl);   // kernel, group, rows
    if (st) return st;
    const int wpg = pl->kernel == 4 ? kvq::int2_waves() : kvq::mfma_stream_waves(pl->rows);
    long per_head = device_cus() / L->n_kv_heads;
    if (per_head < 1) per_head = 1;
    sb->n = n_seqs;
    sb->n_table = n_table;
    long wg = 0, part = 0;
    for (int b = 0; b < n_seqs; ++b) {
        const long chunks = (ctx_lens[b] + kvq::kChunk - 1) / kvq::kChunk;
        long want = (per_head * chunks + total / 2) / total;
        if (want < 1) want = 1;
        const long cps = (chunks + wpg * want - 1) / (wpg * want);
        const long splits = (chunks + wpg * cps - 1) / (wpg * cps);
        sb->wg0[b] = (int)wg;
        sb->ctx[b] = ctx_lens[b];
        sb->n_splits[b] = (int)splits;
        sb->part0[b] = (int)part;
        wg += splits * L->n_kv_heads;
        part += (long)n_q * n_heads * splits;
    }
    sb->wg0[n_seqs] = (int)wg;
    *parts = (size_t)part;
    return KVQ_OK;
}

size_t batch_ws_bytes(size_t parts, int D) {
    return 2 * ((parts * sizeof(float) + 255) / 256 * 256) + parts * (size_t)D * sizeof(float);
}

}  // namespace

extern "C" {

int kvq_version(void) { return 10000; }

const char* kvq_status_str(int status) {
    switch (status) {
        case KVQ_OK: return "KVQ_OK";
        case KVQ_ERR_INVALID_ARG: return "KVQ_ERR_INVALID_ARG";
        case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
        case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE";
        case KVQ_ERR_CAPACITY: return "KVQ_ERR_CAPACITY";
        case KVQ_ERR_HIP: return "KVQ_ERR_HIP";
        default: return "KVQ_ERR_UNKNOWN";
    }
}

const char* kvq_last_error(void) { return g_err; }

int kvq_unit_bytes(const kvq_layout* layout, size_t* bytes) {
    kvq::Geom g;
    int st = check_layout(layout, &g);
    if (st) return st;
    if (bytes == nullptr) return fail(KVQ_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = (size_t)g.unit_bytes();
    return ok();
}

int kvq_pool_bytes(const kvq_layout* layout, size_t* bytes) {
    kvq::Geom g;
    int st = check_layout(layout, &g);
    if (st) return st;
    if (bytes == nullptr) return fail(KVQ_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = (size_t)g.unit_bytes() * layout->n_kv_heads * layout->n_pages;
    return ok();
}

int kvq_append(const kvq_layout* layout, void* d_pool, const int32_t* d_page_table, int32_t n_table,
               int32_t pos0, int32_t n_new, const float* d_k, const float* d_v, void* stream) {
    kvq::Geom g;
    int st = check_layout(layout, &g);
    if (st) return st;
    if (n_new < 0 || pos0 < 0) return fail(KVQ_ERR_INVALID_ARG, "pos0 %d and n_new %d must be >= 0", pos0, n_new);
    if (d_pool == nullptr || d_page_table == nullptr || d_k == nullptr || d_v == nullptr)
        return fail(KVQ_ERR_INVALID_ARG, "pool, page_table, k and v must be non-NULL");
    if (n_table < 1) return fail(KVQ_ERR_INVALID_ARG, "n_table %d < 1", n_table);
    if ((int64_t)pos0 + n_new > (int64_t)n_table * layout->page_size)
        return fail(KVQ_ERR_CAPACITY, "positions up to %lld exceed the page table (%d pages of %d)",
                    (long long)pos0 + n_new, n_table, layout->page_size);
    if ((int64_t)pos0 + n_new > INT32_MAX) return fail(KVQ_ERR_CAPACITY, "positions overflow int32");
    if (((uintptr_t)d_pool & 255) != 0) return fail(KVQ_ERR_INVALID_ARG, "pool must be 256-byte aligned");
    if (n_new == 0) return ok();
    hipError_t e = kvq::launch_append(g, static_cast<uint8_t*>(d_pool), d_page_table, pos0, n_new, d_k, d_v,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
    return ok();
}

int kvq_workspace_bytes(const kvq_layout* layout, int32_t n_heads, int32_t ctx_len, int32_t n_q,
                        int32_t prefill, size_t* bytes) {
    return workspace_impl(layout, n_heads, ctx_len, n_q, prefill != 0, nullptr, bytes);
}

int kvq_workspace_bytes_ex(const kvq_layout* layout, int32_t n_heads, int32_t ctx_len, int32_t n_q,
                           const kvq_attn_opts* opts, size_t* bytes) {
    return workspace_impl(layout, n_heads, ctx_len, n_q, n_q > KVQ_MAX_NQ_DECODE, opts, bytes);
}

int kvq_decode_attn(const kvq_layout* layout, const void* d_pool, const int32_t* d_page_table, int32_t n_table,
                    int32_t ctx_len, int32_t n_heads, int32_t n_q, const float* d_q, float scale,
                    float* d_out, float* d_lse, void* d_ws, size_t ws_bytes, void* stream) {
    return attn_impl(layout, d_pool, d_page_table, n_table, ctx_len, n_heads, n_q, d_q, scale, d_out, d_lse,
                     d_ws, ws_bytes, false, nullptr, stream);
}

int kvq_prefill_attn(const kvq_layout* layout, const void* d_pool, const int32_t* d_page_table, int32_t n_table,
                     int32_t ctx_len, int32_t n_heads, int32_t n_q, const float* d_q, float scale,
                     float* d_out, float* d_lse, void* d_ws, size_t ws_bytes, void* stream) {
    return attn_impl(layout, d_pool, d_page_table, n_table, ctx_len, n_heads, n_q, d_q, scale, d_out, d_lse,
                     d_ws, ws_bytes, true, nullptr, stream);
}

int kvq_append_attn_workspace_bytes(const kvq_layout* layout, int32_t n_heads, int32_t pos0, int32_t n_new,
                                    const kvq_attn_opts* opts, size_t* bytes) {
    kvq::Geom g;
    int st = check_layout(layout, &g);
    if (st) return st;
    if (bytes == nullptr) return fail(KVQ_ERR_INVALID_ARG, "bytes is NULL");
    st = check_append_attn(layout, INT32_MAX / layout->page_size, pos0, n_new, n_heads);
    if (st) return st;
    const bool fused = append_attn_fused(layout, n_heads, pos0, n_new, opts);
    kvq::AttnPlan pl;
    st = append_attn_plan(layout, n_heads, pos0, n_new, opts, fused, &pl);
    if (st) return st;
    *bytes = fused ? fused_ws_bytes(pl, n_new, n_heads, layout->head_dim)
                   : pl.n_splits > 0 ? kvq::ws_bytes_for(pl, n_new, n_heads, layout->head_dim) : 0;
    return ok();
}

}  // extern "C"

namespace {

int append_attn_impl(const kvq_layout* layout, void* d_pool, const int32_t* d_page_table, int32_t n_table,
                     int32_t pos0, int32_t n_new, const float* d_k, const float* d_v, int32_t n_heads,
                     const float* d_q, float scale, float* d_out, float* d_lse, void* d_ws, size_t ws_bytes,
                     const kvq_attn_opts* opts, void* stream) {
    kvq::Geom g;
    int st = check_layout(layout, &g);
    if (st) return st;
    if (d_pool == nullptr || d_page_table == nullptr || d_k == nullptr || d_v == nullptr || d_q == nullptr ||
        d_out == nullptr)
        return fail(KVQ_ERR_INVALID_ARG, "pool, page_table, k, v, q and out must be non-NULL");
    st = check_append_attn(layout, n_table, pos0, n_new, n_heads);
    if (st) return st;
    if (((uintptr_t)d_pool & 255) != 0) return fail(KVQ_ERR_INVALID_ARG, "pool must be 256-byte aligned");
    const bool fused = append_attn_fused(layout, n_heads, pos0, n_new, opts);
    if (!fused) {
        st = kvq_append(layout, d_pool, d_page_table, n_table, pos0, n_new, d_k, d_v, stream);
        if (st) return st;
        return attn_impl(layout, d_pool, d_page_table, n_table, pos0 + n_new, n_heads, n_new, d_q, scale, d_out,
                         d_lse, d_ws, ws_bytes, false, opts, stream);
    }
    kvq::AttnPlan pl;
    st = append_attn_plan(layout, n_heads, pos0, n_new, opts, true, &pl);
    if (st) return st;
    const size_t need = fused_ws_bytes(pl, n_new, n_heads, layout->head_dim);
    if (need > 0 && (d_ws == nullptr || ws_bytes < need))
        return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, ws_bytes,
                    d_ws == nullptr ? " (NULL)" : "");
    if (((uintptr_t)d_ws & 15) != 0) return fail(KVQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

    kvq::AttnArgs a;
    a.g = g;
    a.pool = static_cast<const uint8_t*>(d_pool);
    a.page_table = d_page_table;
    a.ctx = pos0;
    a.n_heads = n_heads;
    a.n_q = n_new;
    a.q = d_q;
    a.scale = scale;
    a.out = d_out;
    a.lse = d_lse;
    a.causal = 0;
    const int parts = fused_parts(pl, n_new);
    const size_t rows = (size_t)n_new * n_heads;
    const size_t ml = (rows * parts * sizeof(float) + 255) / 256 * 256;
    uint8_t* ws = static_cast<uint8_t*>(d_ws);
    a.ws_m = reinterpret_cast<float*>(ws);
    a.ws_l = reinterpret_cast<float*>(ws + ml);
    a.ws_acc = reinterpret_cast<float*>(ws + 2 * ml);
    const kvq::NewRows nr{static_cast<uint8_t*>(d_pool), d_k, d_v, pos0, n_new};

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (opts != nullptr && opts->kernel_begin_event != nullptr)
        e = hipEventRecord(static_cast<hipEvent_t>(opts->kernel_begin_event), s);
    // The split pass over the cached keys either also appends the new rows
    // and leaves their partials (the merge then only folds), or leaves them
    // to the merge kernel, which appends and scores them itself (also when
    // there are no cached keys, pos0 = 0).
    const bool in_split = new_rows_in_split(pl);
    if (e == hipSuccess && in_split)
        e = pl.kernel == 4 ? kvq::launch_attn_int2_new(a, pl, nr, s) : kvq::launch_attn_mfma_stream_new(a, pl, nr, s);
    else if (e == hipSuccess && pl.n_splits > 0) e = kvq::launch_attn_mfma_stream(a, pl, s);
    if (e == hipSuccess && opts != nullptr && opts->kernel_end_event != nullptr)
        e = hipEventRecord(static_cast<hipEvent_t>(opts->kernel_end_event), s);
    if (e == hipSuccess && in_split) {
        kvq::AttnPlan pm = pl;
        pm.n_splits = parts;
        e = kvq::launch_merge(a, pm, s);
    } else if (e == hipSuccess) {
        e = kvq::launch_merge_new(a, nr, pl.n_splits, s);
    }
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Scratch of kvq_append_attn_noalloc: the split partials live here instead
// of in a caller's workspace.  Host code never names the array itself (its
// host-side name is not a device address): it takes the device address once
// per device with hipGetSymbolAddress and passes that to the kernels.
constexpr size_t kScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table covers", dev, kMaxDevices);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return KVQ_OK;
}

}  // namespace

extern "C" {

int kvq_append_attn(const kvq_layout* layout, void* d_pool, const int32_t* d_page_table, int32_t n_table,
                    int32_t pos0, int32_t n_new, const float* d_k, const float* d_v, int32_t n_heads,
                    const float* d_q, float scale, float* d_out, float* d_lse, void* d_ws, size_t ws_bytes,
                    const kvq_attn_opts* opts, void* stream) {
    return append_attn_impl(layout, d_pool, d_page_table, n_table, pos0, n_new, d_k, d_v, n_heads, d_q, scale, d_out,
                            d_lse, d_ws, ws_bytes, opts, stream);
}

size_t kvq_noalloc_scratch_bytes(void) { return kScratchBytes; }

int kvq_append_attn_noalloc(const kvq_layout* layout, void* d_pool, const int32_t* d_page_table, int32_t n_table,
                            int32_t pos0, int32_t n_new, const float* d_k, const float* d_v, int32_t n_heads,
                            const float* d_q, float scale, float* d_out, float* d_lse, const kvq_attn_opts* opts,
                            void* stream) {
    size_t need = 0;
    int st = kvq_append_attn_workspace_bytes(layout, n_heads, pos0, n_new, opts, &need);
    if (st) return st;
    if (need > kScratchBytes)
        return fail(KVQ_ERR_WORKSPACE,
                    "this step needs %zu bytes of scratch; the static scratch holds %zu (use kvq_append_attn with a "
                    "workspace, or fewer query rows or a shorter context)",
                    need, kScratchBytes);
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st) return st;
    return append_attn_impl(layout, d_pool, d_page_table, n_table, pos0, n_new, d_k, d_v, n_heads, d_q, scale, d_out,
                            d_lse, ws, kScratchBytes, opts, stream);
}

int kvq_attn_ex(const kvq_layout* layout, const void* d_pool, const int32_t* d_page_table, int32_t n_table,
                int32_t ctx_len, int32_t n_heads, int32_t n_q, const float* d_q, float scale,
                float* d_out, float* d_lse, void* d_ws, size_t ws_bytes, const kvq_attn_opts* opts,
                void* stream) {
    return attn_impl(layout, d_pool, d_page_table, n_table, ctx_len, n_heads, n_q, d_q, scale, d_out, d_lse,
                     d_ws, ws_bytes, n_q > KVQ_MAX_NQ_DECODE, opts, stream);
}

int kvq_decode_attn_batch_workspace_bytes(const kvq_layout* layout, int32_t n_seqs, const int32_t* ctx_lens,
                                          int32_t n_heads, int32_t n_q, size_t* bytes) {
    if (bytes == nullptr) return fail(KVQ_ERR_INVALID_ARG, "bytes is NULL");
    kvq::AttnPlan pl;
    kvq::SeqBatch sb;
    size_t parts = 0;
    // the plan does not depend on the page table: pass a table that fits
    int32_t n_table = 1;
    if (layout != nullptr && ctx_lens != nullptr && n_seqs >= 1 && n_seqs <= KVQ_MAX_SEQS && layout->page_size > 0)
        for (int b = 0; b < n_seqs; ++b)
            n_table = std::max(n_table, (ctx_lens[b] + layout->page_size - 1) / layout->page_size);
    int st = batch_plan(layout, n_table, n_seqs, ctx_lens, n_heads, n_q, &pl, &sb, &parts);
    if (st) return st;
    *bytes = batch_ws_bytes(parts, layout->head_dim);
    return ok();
}

int kvq_decode_attn_batch(const kvq_layout* layout, const void* d_pool, const int32_t* d_page_tables, int32_t n_table,
                          int32_t n_seqs, const int32_t* ctx_lens, int32_t n_heads, int32_t n_q,
                          const float* d_q, float scale, float* d_out, float* d_lse,
                          void* d_ws, size_t ws_bytes, const kvq_attn_opts* opts, void* stream) {
    if (d_pool == nullptr || d_page_tables == nullptr || d_q == nullptr || d_out == nullptr)
        return fail(KVQ_ERR_INVALID_ARG, "pool, page_tables, q and out must be non-NULL");
    if (opts != nullptr && opts->kernel != 0 && opts->kernel != 2 && opts->kernel != 4)
        return fail(KVQ_ERR_INVALID_ARG, "batched decode runs a streaming kernel (kernel 0, 2 or 4, got %d)",
                    opts->kernel);
    if (layout != nullptr && opts != nullptr && opts->kernel != 0 &&
        opts->kernel != (layout->codec == KVQ_CODEC_INT2 ? 4 : 2))
        return fail(KVQ_ERR_UNSUPPORTED, "kernel %d does not read codec %d", opts->kernel, layout->codec);
    kvq::AttnPlan pl;
    kvq::SeqBatch sb;
    size_t parts = 0;
    int st = batch_plan(layout, n_table, n_seqs, ctx_lens, n_heads, n_q, &pl, &sb, &parts);
    if (st) return st;
    const size_t need = batch_ws_bytes(parts, layout->head_dim);
    if (d_ws == nullptr || ws_bytes < need)
        return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, ws_bytes,
                    d_ws == nullptr ? " (NULL)" : "");
    if (((uintptr_t)d_pool & 255) != 0) return fail(KVQ_ERR_INVALID_ARG, "pool must be 256-byte aligned");
    if (((uintptr_t)d_ws & 15) != 0) return fail(KVQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    kvq::Geom g;
    check_layout(layout, &g);
    kvq::AttnArgs a;
    a.g = g;
    a.pool = static_cast<const uint8_t*>(d_pool);
    a.page_table = d_page_tables;
    a.ctx = sb.ctx[0];
    a.n_heads = n_heads;
    a.n_q = n_q;
    a.q = d_q;
    a.scale = scale;
    a.out = d_out;
    a.lse = d_lse;
    uint8_t* ws = static_cast<uint8_t*>(d_ws);
    const size_t ml = (parts * sizeof(float) + 255) / 256 * 256;
    a.ws_m = reinterpret_cast<float*>(ws);
    a.ws_l = reinterpret_cast<float*>(ws + ml);
    a.ws_acc = reinterpret_cast<float*>(ws + 2 * ml);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (opts != nullptr && opts->kernel_begin_event != nullptr)
        e = hipEventRecord(static_cast<hipEvent_t>(opts->kernel_begin_event), s);
    if (e == hipSuccess)
        e = pl.kernel == 4 ? kvq::launch_attn_int2(a, pl, s, &sb) : kvq::launch_attn_mfma_stream(a, pl, s, &sb);
    if (e == hipSuccess && opts != nullptr && opts->kernel_end_event != nullptr)
        e = hipEventRecord(static_cast<hipEvent_t>(opts->kernel_end_event), s);
    if (e == hipSuccess) e = kvq::launch_merge(a, pl, s, &sb);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

int kvq_hadamard(float* d_x, int64_t n_rows, int32_t dim, void* stream) {
    if (dim < 2 || dim > 1024 || (dim & (dim - 1)) != 0)
        return fail(KVQ_ERR_INVALID_ARG, "dim %d must be a power of two in [2, 1024]", dim);
    if (n_rows < 0 || n_rows > INT32_MAX)
        return fail(KVQ_ERR_INVALID_ARG, "n_rows %lld outside [0, 2^31 - 1]", (long long)n_rows);
    // one workgroup of dim/2 threads per row: the grid's work-items must stay
    // below 2^32
    if ((uint64_t)n_rows * (uint64_t)(dim / 2) >= (1ull << 32))
        return fail(KVQ_ERR_INVALID_ARG, "n_rows %lld x dim/2 %d reaches 2^32 work-items; rotate in several calls",
                    (long long)n_rows, dim / 2);
    if (n_rows == 0) return ok();
    if (d_x == nullptr) return fail(KVQ_ERR_INVALID_ARG, "x is NULL");
    if (((uintptr_t)d_x & 3) != 0) return fail(KVQ_ERR_INVALID_ARG, "x must be 4-byte aligned");
    const hipError_t e = kvq::launch_hadamard(d_x, n_rows, dim, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

int kvq_stage_pages(const kvq_layout* host_layout, const void* h_pool, const int32_t* h_page_table, int32_t n_copy,
                    const kvq_layout* dev_layout, void* d_pool, int32_t dst_first, void* stream) {
    kvq::Geom gh, gd;
    int st = check_layout(host_layout, &gh);
    if (st) return st;
    st = check_layout(dev_layout, &gd);
    if (st) return st;
    if (h_pool == nullptr || d_pool == nullptr || h_page_table == nullptr)
        return fail(KVQ_ERR_INVALID_ARG, "pools and page table must be non-NULL");
    if (n_copy < 0) return fail(KVQ_ERR_INVALID_ARG, "n_copy %d < 0", n_copy);
    // the copies are sized from the host layout, so every field that sets the
    // bytes of a page must agree (a different codec changes the unit size)
    if (gh.D != gd.D || gh.P != gd.P || gh.n_kv != gd.n_kv || gh.codec != gd.codec)
        return fail(KVQ_ERR_INVALID_ARG, "host and device layouts differ (head_dim, page_size, n_kv_heads or codec)");
    if (dst_first < 0 || (int64_t)dst_first + n_copy > gd.n_pages)
        return fail(KVQ_ERR_INVALID_ARG, "device pages %d..%d outside the pool of %d", dst_first,
                    dst_first + n_copy - 1, gd.n_pages);
    for (int i = 0; i < n_copy; ++i)
        if (h_page_table[i] < 0 || h_page_table[i] >= gh.n_pages)
            return fail(KVQ_ERR_INVALID_ARG, "host page %d (entry %d) outside the pool of %d", h_page_table[i], i,
                        gh.n_pages);
    if (n_copy == 0) return ok();
    // one page of the pool = the units of all KV heads, contiguous
    const size_t page_bytes = (size_t)gh.unit_bytes() * gh.n_kv;
    const uint8_t* src = static_cast<const uint8_t*>(h_pool);
    uint8_t* dst = static_cast<uint8_t*>(d_pool) + (size_t)dst_first * page_bytes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int i = 0; i < n_copy;) {
        int j = i + 1;
        while (j < n_copy && h_page_table[j] == h_page_table[j - 1] + 1) ++j;   // a run of consecutive pages
        const hipError_t e = hipMemcpyAsync(dst + (size_t)i * page_bytes, src + (size_t)h_page_table[i] * page_bytes,
                                            (size_t)(j - i) * page_bytes, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipMemcpyAsync failed: %s", hipGetErrorString(e));
        i = j;
    }
    return ok();
}

}  // extern "C"
