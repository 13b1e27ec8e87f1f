// api.cpp -- the C ABI of libdsa: argument validation, workspace sizing,
// device checks and launch sequencing.  See include/dsa.h for the contract.
#include "dsa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "dsa_internal.h"

namespace {

thread_local char g_detail[512] = "";

dsa_status_t fail(dsa_status_t s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof g_detail, fmt, ap);
    va_end(ap);
    return s;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool good_scale(float s) { return std::isfinite(s) && s > 0.f; }

constexpr int32_t kMaxRows = 1 << 24;

dsa_status_t check_rows(const dsa_rows_t* rows)
{
    if (!rows) return fail(DSA_ERR_INVALID_ARGUMENT, "rows is NULL");
    if (rows->num_rows < 1 || rows->num_rows > kMaxRows)
        return fail(DSA_ERR_INVALID_ARGUMENT, "num_rows=%d outside [1, %d]", rows->num_rows, kMaxRows);
    if (rows->max_visible < 1 || rows->max_visible > DSA_MAX_VISIBLE)
        return fail(DSA_ERR_INVALID_ARGUMENT, "max_visible=%d outside [1, %d]", rows->max_visible, DSA_MAX_VISIBLE);
    if (!rows->visible_len) return fail(DSA_ERR_INVALID_ARGUMENT, "rows->visible_len is NULL");
    if (!rows->row_cache_base) return fail(DSA_ERR_INVALID_ARGUMENT, "rows->row_cache_base is NULL");
    if (!aligned(rows->visible_len, 4)) return fail(DSA_ERR_MISALIGNED, "visible_len not 4-byte aligned");
    if (!aligned(rows->row_cache_base, 8)) return fail(DSA_ERR_MISALIGNED, "row_cache_base not 8-byte aligned");
    if (rows->flags & ~DSA_ROWS_DISTINCT_SEQUENCES) return fail(DSA_ERR_INVALID_ARGUMENT, "unknown rows->flags bits 0x%x", rows->flags);
    return DSA_OK;
}

dsa_status_t check_ptr16(const void* p, const char* name)
{
    if (!p) return fail(DSA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(DSA_ERR_MISALIGNED, "%s not 16-byte aligned", name);
    return DSA_OK;
}

dsa_status_t check_k(int32_t k)
{
    if (k < 1 || k > DSA_TOPK_MAX) return fail(DSA_ERR_INVALID_ARGUMENT, "k=%d outside [1, %d]", k, DSA_TOPK_MAX);
    return DSA_OK;
}

dsa_status_t check_ld(const dsa_rows_t* rows, int64_t ld)
{
    if (ld < rows->max_visible) return fail(DSA_ERR_INVALID_ARGUMENT, "ld=%lld < max_visible=%d", (long long)ld, rows->max_visible);
    if (ld % 4 != 0) return fail(DSA_ERR_MISALIGNED, "ld=%lld is not a multiple of 4", (long long)ld);
    return DSA_OK;
}

dsa_status_t check_ws(const void* ws, size_t ws_bytes, size_t need)
{
    if (ws_bytes < need)
        return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", ws_bytes, need);
    if (need > 0) {
        if (!ws) return fail(DSA_ERR_INVALID_ARGUMENT, "workspace is NULL");
        if (!aligned(ws, 256)) return fail(DSA_ERR_MISALIGNED, "workspace not 256-byte aligned");
    }
    return DSA_OK;
}

// Per-device "is this a gfx950" cache.
std::mutex g_dev_mu;
int g_dev_state[64];  // 0 unknown, 1 ok, 2 unsupported

dsa_status_t check_device()
{
    int dev = -1;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return fail(DSA_ERR_NO_DEVICE, "no HIP device present");
    }
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(DSA_ERR_NO_DEVICE, "hipGetDevice failed");
    }
    if (dev < 64) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (g_dev_state[dev] == 1) return DSA_OK;
        if (g_dev_state[dev] == 2) return fail(DSA_ERR_NO_DEVICE, "device %d is not gfx950", dev);
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(DSA_ERR_NO_DEVICE, "hipGetDeviceProperties(%d) failed", dev);
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        g_dev_state[dev] = ok ? 1 : 2;
    }
    if (!ok) return fail(DSA_ERR_NO_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
    return DSA_OK;
}

dsa_status_t after_launch(hipStream_t stream, const char* what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    if (dsa::sync_debug()) {
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    }
    return DSA_OK;
}

size_t scores_ld(int32_t max_visible) { return dsa::align_up((size_t)max_visible, 4); }

// Rows the fused step scores and selects at a time (see dsa_decode_step in
// dsa.h): all of them while their fp32 score rows fit the budget, else the
// largest multiple of 256 rows that fits (a whole number of rows per CU for
// the per-row kernels), or of 32 rows below that (at least 32).  Chunks start
// on multiples of 32 rows, so the indexer's 32-row blocks are those of the
// whole call and the results do not depend on the chunking.
int32_t step_chunk_rows(int32_t num_rows, int32_t max_visible)
{
    const size_t row_bytes = scores_ld(max_visible) * 4;
    if ((size_t)num_rows * row_bytes <= (size_t)DSA_STEP_SCORES_BUDGET) return num_rows;
    const size_t fit = (size_t)DSA_STEP_SCORES_BUDGET / row_bytes;
    size_t c = fit >= 256 ? fit / 256 * 256 : fit / 32 * 32;
    if (c < 32) c = 32;
    return c < (size_t)num_rows ? (int32_t)c : num_rows;
}

// Workspace of the fused step when it scores C rows at a time: the chunk's
// score rows, the indexer's row list and the top-k state for C rows, and the
// attention's split partials for all rows.
size_t step_ws_bytes(int32_t num_rows, int32_t max_visible, int32_t k, int32_t C)
{
    size_t b = dsa::align_up((size_t)C * scores_ld(max_visible) * 4, 256);
    b += dsa::align_up(dsa::indexer_list_bytes(C), 256);
    b += dsa::align_up(dsa::topk_workspace_bytes(C, max_visible), 256);
    b += dsa::align_up(dsa::attn_workspace_bytes(num_rows, k), 256);
    return b;
}

constexpr dsa::PagedCache kPacked{nullptr, 0, 0};

// Validates a block-table description against the rows and converts it.
dsa_status_t check_paged(const dsa_rows_t* rows, const dsa_paged_t* paged, dsa::PagedCache* out)
{
    if (!paged) return fail(DSA_ERR_INVALID_ARGUMENT, "paged is NULL");
    if (!paged->block_table) return fail(DSA_ERR_INVALID_ARGUMENT, "paged->block_table is NULL");
    if (!aligned(paged->block_table, 4)) return fail(DSA_ERR_MISALIGNED, "block_table not 4-byte aligned");
    const int32_t B = paged->block_size;
    if (B < 16 || B > 65536 || (B & (B - 1)) != 0)
        return fail(DSA_ERR_INVALID_ARGUMENT, "block_size=%d is not a power of two in [16, 65536]", B);
    const int64_t need = ((int64_t)rows->max_visible + B - 1) / B;
    if (paged->max_blocks < need)
        return fail(DSA_ERR_INVALID_ARGUMENT, "max_blocks=%d < %lld blocks of max_visible", paged->max_blocks,
                    (long long)need);
    int lg = 0;
    while ((1 << lg) < B) lg++;
    *out = dsa::PagedCache{paged->block_table, paged->max_blocks, lg};
    return DSA_OK;
}

#define DSA_TRY(expr)                        \
    do {                                     \
        dsa_status_t _s = (expr);            \
        if (_s != DSA_OK) return _s;         \
    } while (0)

}  // namespace

namespace dsa {
bool sync_debug()
{
    static const bool on = [] {
        const char* e = std::getenv("DSA_SYNC_DEBUG");
        return e && e[0] == '1';
    }();
    return on;
}
}  // namespace dsa

extern "C" {

const char* dsa_version(void) { return "libdsa 0.1.0 (gfx950)"; }

const char* dsa_status_string(dsa_status_t s)
{
    switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARGUMENT: return "DSA_ERR_INVALID_ARGUMENT";
    case DSA_ERR_MISALIGNED: return "DSA_ERR_MISALIGNED";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "DSA_ERR_WORKSPACE_TOO_SMALL";
    case DSA_ERR_NO_DEVICE: return "DSA_ERR_NO_DEVICE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
    }
    return "DSA_ERR_UNKNOWN_STATUS";
}

const char* dsa_last_error_detail(void) { return g_detail; }

}  // extern "C"

namespace {

dsa_status_t indexer_impl(const dsa_rows_t* rows, const dsa::PagedCache& pc, const void* q_idx, const float* w,
                          const void* k_idx, float index_scale, float* scores, int64_t ld, void* hip_stream)
{
    DSA_TRY(check_ptr16(q_idx, "q_idx"));
    DSA_TRY(check_ptr16(w, "w"));
    DSA_TRY(check_ptr16(k_idx, "k_idx"));
    DSA_TRY(check_ptr16(scores, "scores"));
    DSA_TRY(check_ld(rows, ld));
    if (!good_scale(index_scale)) return fail(DSA_ERR_INVALID_ARGUMENT, "index_scale must be finite and > 0");
    DSA_TRY(check_device());
    hipStream_t st = (hipStream_t)hip_stream;
    dsa::launch_indexer_scores(rows->num_rows, rows->max_visible, rows->visible_len, rows->row_cache_base,
                               (const uint16_t*)q_idx, w, (const uint16_t*)k_idx, index_scale, scores, ld,
                               (rows->flags & DSA_ROWS_DISTINCT_SEQUENCES) != 0, pc, st);
    return after_launch(st, "indexer");
}

dsa_status_t attn_impl(const dsa_rows_t* rows, const dsa::PagedCache& pc, const void* q_abs, const void* kv_latent,
                       const int32_t* indices, int32_t k, float softmax_scale, float* out_latent, float* out_lse,
                       void* ws, hipStream_t st)
{
    const int64_t* base = rows->row_cache_base;
    const int32_t* idx = indices;
    void* aws = ws;
    if (pc.block_table) {
        // Selected positions -> pool rows (and zero row bases) ahead of the
        // attention's workspace.
        const int32_t R = rows->num_rows;
        char* p = (char*)ws;
        int32_t* phys = (int32_t*)p;
        p += dsa::align_up((size_t)R * k * 4, 256);
        int64_t* zero = (int64_t*)p;
        p += dsa::align_up((size_t)R * 8, 256);
        aws = p;
        dsa::launch_page_indices(R, k, rows->row_cache_base, indices, pc, phys, zero, st);
        DSA_TRY(after_launch(st, "sparse_mla/page_indices"));
        base = zero;
        idx = phys;
    }
    dsa::launch_sparse_mla(rows->num_rows, base, (const uint16_t*)q_abs, (const uint16_t*)kv_latent, idx, k,
                           softmax_scale, out_latent, out_lse, aws, st, rows->max_visible, pc.block_table != nullptr);
    return after_launch(st, "sparse_mla");
}

size_t paged_attn_extra(int32_t num_rows, int32_t k)
{
    return dsa::align_up((size_t)num_rows * k * 4, 256) + dsa::align_up((size_t)num_rows * 8, 256);
}

}  // namespace

extern "C" {

dsa_status_t dsa_indexer_scores(const dsa_rows_t* rows, const void* q_idx, const float* w, const void* k_idx,
                                float index_scale, float* scores, int64_t ld, void* hip_stream)
{
    g_detail[0] = '\0';
    DSA_TRY(check_rows(rows));
    return indexer_impl(rows, kPacked, q_idx, w, k_idx, index_scale, scores, ld, hip_stream);
}

dsa_status_t dsa_indexer_scores_paged(const dsa_rows_t* rows, const dsa_paged_t* paged, const void* q_idx,
                                      const float* w, const void* k_pool, float index_scale, float* scores,
                                      int64_t ld, void* hip_stream)
{
    g_detail[0] = '\0';
    DSA_TRY(check_rows(rows));
    dsa::PagedCache pc;
    DSA_TRY(check_paged(rows, paged, &pc));
    return indexer_impl(rows, pc, q_idx, w, k_pool, index_scale, scores, ld, hip_stream);
}

size_t dsa_topk_workspace_size(int32_t num_rows, int32_t max_visible, int32_t k)
{
    (void)k;
    if (num_rows < 1 || max_visible < 1) return 0;
    return dsa::topk_workspace_bytes(num_rows, max_visible);
}

dsa_status_t dsa_topk_select(const dsa_rows_t* rows, const float* scores, int64_t ld, int32_t k, int32_t* indices,
                             void* ws, size_t ws_bytes, void* hip_stream)
{
    g_detail[0] = '\0';
    DSA_TRY(check_rows(rows));
    DSA_TRY(check_ptr16(scores, "scores"));
    DSA_TRY(check_ld(rows, ld));
    DSA_TRY(check_k(k));
    if (!indices) return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL");
    if (!aligned(indices, 4)) return fail(DSA_ERR_MISALIGNED, "indices not 4-byte aligned");
    DSA_TRY(check_ws(ws, ws_bytes, dsa_topk_workspace_size(rows->num_rows, rows->max_visible, k)));
    DSA_TRY(check_device());
    hipStream_t st = (hipStream_t)hip_stream;
    dsa::TopkWorkspace tw = dsa::topk_workspace_carve(ws, rows->num_rows, rows->max_visible);
    dsa::launch_topk(rows->num_rows, rows->max_visible, rows->visible_len, scores, ld, k, indices, tw, st);
    return after_launch(st, "topk");
}

size_t dsa_sparse_mla_workspace_size(int32_t num_rows, int32_t k)
{
    if (num_rows < 1 || k < 1 || k > DSA_TOPK_MAX) return 0;
    return dsa::attn_workspace_bytes(num_rows, k);
}

size_t dsa_sparse_mla_paged_workspace_size(int32_t num_rows, int32_t k)
{
    if (num_rows < 1 || k < 1 || k > DSA_TOPK_MAX) return 0;
    return paged_attn_extra(num_rows, k) + dsa::attn_workspace_bytes(num_rows, k);
}

}  // extern "C"

namespace {

dsa_status_t check_attn_args(const dsa_rows_t* rows, const void* q_abs, const void* kv_latent,
                             const int32_t* indices, int32_t k, float softmax_scale, const float* out_latent,
                             const float* out_lse)
{
    (void)rows;
    DSA_TRY(check_ptr16(q_abs, "q_abs"));
    DSA_TRY(check_ptr16(kv_latent, "kv_latent"));
    DSA_TRY(check_k(k));
    if (!indices) return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL");
    if (!aligned(indices, 4)) return fail(DSA_ERR_MISALIGNED, "indices not 4-byte aligned");
    DSA_TRY(check_ptr16(out_latent, "out_latent"));
    if (out_lse && !aligned(out_lse, 4)) return fail(DSA_ERR_MISALIGNED, "out_lse not 4-byte aligned");
    if (!good_scale(softmax_scale)) return fail(DSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
    return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status_t dsa_sparse_mla_attn(const dsa_rows_t* rows, const void* q_abs, const void* kv_latent,
                                 const int32_t* indices, int32_t k, float softmax_scale, float* out_latent,
                                 float* out_lse, void* ws, size_t ws_bytes, void* hip_stream)
{
    g_detail[0] = '\0';
    DSA_TRY(check_rows(rows));
    DSA_TRY(check_attn_args(rows, q_abs, kv_latent, indices, k, softmax_scale, out_latent, out_lse));
    DSA_TRY(check_ws(ws, ws_bytes, dsa_sparse_mla_workspace_size(rows->num_rows, k)));
    DSA_TRY(check_device());
    return attn_impl(rows, kPacked, q_abs, kv_latent, indices, k, softmax_scale, out_latent, out_lse, ws,
                     (hipStream_t)hip_stream);
}

dsa_status_t dsa_sparse_mla_attn_paged(const dsa_rows_t* rows, const dsa_paged_t* paged, const void* q_abs,
                                       const void* kv_pool, const int32_t* indices, int32_t k, float softmax_scale,
                                       float* out_latent, float* out_lse, void* ws, size_t ws_bytes,
                                       void* hip_stream)
{
    g_detail[0] = '\0';
    DSA_TRY(check_rows(rows));
    dsa::PagedCache pc;
    DSA_TRY(check_paged(rows, paged, &pc));
    DSA_TRY(check_attn_args(rows, q_abs, kv_pool, indices, k, softmax_scale, out_latent, out_lse));
    DSA_TRY(check_ws(ws, ws_bytes, dsa_sparse_mla_paged_workspace_size(rows->num_rows, k)));
    DSA_TRY(check_device());
    return attn_impl(rows, pc, q_abs, kv_pool, indices, k, softmax_scale, out_latent, out_lse, ws,
                     (hipStream_t)hip_stream);
}

size_t dsa_decode_step_workspace_size(int32_t num_rows, int32_t max_visible, int32_t k)
{
    if (num_rows < 1 || max_visible < 1 || k < 1 || k > DSA_TOPK_MAX) return 0;
    return step_ws_bytes(num_rows, max_visible, k, step_chunk_rows(num_rows, max_visible));
}

size_t dsa_decode_step_paged_workspace_size(int32_t num_rows, int32_t max_visible, int32_t k)
{
    const size_t b = dsa_decode_step_workspace_size(num_rows, max_visible, k);
    return b ? b + paged_attn_extra(num_rows, k) : 0;
}

}  // extern "C"

namespace {

// The fused step with C rows scored at a time (0: the default chunking of
// dsa_decode_step_workspace_size).
dsa_status_t check_step_args(const void* q_idx, const float* w, const void* k_idx, float index_scale,
                             const void* q_abs, const void* kv_latent, float softmax_scale, int32_t k,
                             const int32_t* indices, const float* out_latent, const float* out_lse)
{
    DSA_TRY(check_ptr16(q_idx, "q_idx"));
    DSA_TRY(check_ptr16(w, "w"));
    DSA_TRY(check_ptr16(k_idx, "k_idx"));
    DSA_TRY(check_ptr16(q_abs, "q_abs"));
    DSA_TRY(check_ptr16(kv_latent, "kv_latent"));
    DSA_TRY(check_k(k));
    if (!indices) return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL");
    if (!aligned(indices, 4)) return fail(DSA_ERR_MISALIGNED, "indices not 4-byte aligned");
    DSA_TRY(check_ptr16(out_latent, "out_latent"));
    if (out_lse && !aligned(out_lse, 4)) return fail(DSA_ERR_MISALIGNED, "out_lse not 4-byte aligned");
    if (!good_scale(index_scale)) return fail(DSA_ERR_INVALID_ARGUMENT, "index_scale must be finite and > 0");
    if (!good_scale(softmax_scale)) return fail(DSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
    return DSA_OK;
}

// Enqueues the fused step with C rows scored at a time (arguments already
// validated, workspace large enough for C).
dsa_status_t decode_run(const dsa_rows_t* rows, const dsa::PagedCache& pc, const void* q_idx, const float* w,
                        const void* k_idx, float index_scale, const void* q_abs, const void* kv_latent,
                        float softmax_scale, int32_t k, int32_t* indices, float* out_latent, float* out_lse,
                        void* ws, void* hip_stream, int32_t C)
{
    hipStream_t st = (hipStream_t)hip_stream;
    const int32_t R = rows->num_rows;
    const int32_t maxv = rows->max_visible;
    const int64_t ld = (int64_t)scores_ld(maxv);
    char* p = (char*)ws;
    float* scores = (float*)p;
    p += dsa::align_up((size_t)C * ld * 4, 256);
    void* lws = p;  // the indexer's row list (used when rows may share blocks)
    p += dsa::align_up(dsa::indexer_list_bytes(C), 256);
    void* tws = p;
    p += dsa::align_up(dsa_topk_workspace_size(C, maxv, k), 256);
    void* aws = p;

    // Scores and selection chunk by chunk (the index lists land in
    // `indices`), then one attention launch over every row.
    const bool distinct = (rows->flags & DSA_ROWS_DISTINCT_SEQUENCES) != 0;
    for (int32_t c0 = 0; c0 < R; c0 += C) {
        const int32_t nc = R - c0 < C ? R - c0 : C;
        const int32_t* vis = rows->visible_len + c0;
        const int64_t* base = rows->row_cache_base + c0;
        dsa::launch_indexer_scores(nc, maxv, vis, base, (const uint16_t*)q_idx + (int64_t)c0 * DSA_INDEX_HEADS * DSA_INDEX_DIM,
                                   w + (int64_t)c0 * DSA_INDEX_HEADS, (const uint16_t*)k_idx, index_scale, scores, ld,
                                   distinct, pc, st, lws);
        DSA_TRY(after_launch(st, "decode_step/indexer"));
        dsa::TopkWorkspace tw = dsa::topk_workspace_carve(tws, nc, maxv);
        dsa::launch_topk(nc, maxv, vis, scores, ld, k, indices + (int64_t)c0 * k, tw, st);
        DSA_TRY(after_launch(st, "decode_step/topk"));
    }
    return attn_impl(rows, pc, q_abs, kv_latent, indices, k, softmax_scale, out_latent, out_lse, aws, st);
}

dsa_status_t decode_impl(const dsa_rows_t* rows, const dsa::PagedCache& pc, const void* q_idx, const float* w,
                         const void* k_idx, float index_scale, const void* q_abs, const void* kv_latent,
                         float softmax_scale, int32_t k, int32_t* indices, float* out_latent, float* out_lse,
                         void* ws, size_t ws_bytes, void* hip_stream)
{
    DSA_TRY(check_step_args(q_idx, w, k_idx, index_scale, q_abs, kv_latent, softmax_scale, k, indices, out_latent,
                            out_lse));
    const int32_t R = rows->num_rows;
    const int32_t C = step_chunk_rows(R, rows->max_visible);
    DSA_TRY(check_ws(ws, ws_bytes,
                     step_ws_bytes(R, rows->max_visible, k, C) + (pc.block_table ? paged_attn_extra(R, k) : 0)));
    DSA_TRY(check_device());
    return decode_run(rows, pc, q_idx, w, k_idx, index_scale, q_abs, kv_latent, softmax_scale, k, indices,
                      out_latent, out_lse, ws, hip_stream, C);
}

}  // namespace

namespace dsa {

dsa_status_t decode_step_in_scratch(const dsa_rows_t* rows, const void* q_idx, const float* w, const void* k_idx,
                                    float index_scale, const void* q_abs, const void* kv_latent, float softmax_scale,
                                    int32_t k, int32_t* indices, float* out_latent, float* out_lse,
                                    size_t scratch_bytes, void* (*scratch_ptr)(), void* hip_stream)
{
    g_detail[0] = '\0';
    DSA_TRY(check_rows(rows));
    DSA_TRY(check_step_args(q_idx, w, k_idx, index_scale, q_abs, kv_latent, softmax_scale, k, indices, out_latent,
                            out_lse));
    // As many rows at a time as the scratch holds: the default chunk if it
    // fits, else the largest multiple of 32 rows (all rows when fewer than 32).
    const int32_t R = rows->num_rows, maxv = rows->max_visible;
    int32_t C = step_chunk_rows(R, maxv);
    if (step_ws_bytes(R, maxv, k, C) > scratch_bytes) {
        int32_t lo = 0, hi = C / 32;  // largest m in [1, hi] with 32 m rows fitting, 0 if none
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) / 2;
            if (step_ws_bytes(R, maxv, k, 32 * mid) <= scratch_bytes) lo = mid;
            else hi = mid - 1;
        }
        if (lo == 0)
            return fail(DSA_ERR_INVALID_ARGUMENT,
                        "rows=%d, max_visible=%d, k=%d need %zu bytes of scratch even 32 rows at a time; the scratch "
                        "holds %zu",
                        R, maxv, k, step_ws_bytes(R, maxv, k, R < 32 ? R : 32), scratch_bytes);
        C = 32 * lo;
    }
    DSA_TRY(check_device());
    void* scratch = scratch_ptr();
    if (!scratch) return fail(DSA_ERR_HIP, "the scratch array's device address is unavailable");
    return decode_run(rows, kPacked, q_idx, w, k_idx, index_scale, q_abs, kv_latent, softmax_scale, k, indices,
                      out_latent, out_lse, scratch, hip_stream, C);
}

}  // namespace dsa

extern "C" {

dsa_status_t dsa_decode_step(const dsa_rows_t* rows, const void* q_idx, const float* w, const void* k_idx,
                             float index_scale, const void* q_abs, const void* kv_latent, float softmax_scale,
                             int32_t k, int32_t* indices, float* out_latent, float* out_lse, void* ws,
                             size_t ws_bytes, void* hip_stream)
{
    g_detail[0] = '\0';
    DSA_TRY(check_rows(rows));
    return decode_impl(rows, kPacked, q_idx, w, k_idx, index_scale, q_abs, kv_latent, softmax_scale, k, indices,
                       out_latent, out_lse, ws, ws_bytes, hip_stream);
}

dsa_status_t dsa_decode_step_paged(const dsa_rows_t* rows, const dsa_paged_t* paged, const void* q_idx,
                                   const float* w, const void* k_pool, float index_scale, const void* q_abs,
                                   const void* kv_pool, float softmax_scale, int32_t k, int32_t* indices,
                                   float* out_latent, float* out_lse, void* ws, size_t ws_bytes, void* hip_stream)
{
    g_detail[0] = '\0';
    DSA_TRY(check_rows(rows));
    dsa::PagedCache pc;
    DSA_TRY(check_paged(rows, paged, &pc));
    return decode_impl(rows, pc, q_idx, w, k_pool, index_scale, q_abs, kv_pool, softmax_scale, k, indices,
                       out_latent, out_lse, ws, ws_bytes, hip_stream);
}

dsa_status_t dsa_absorb_queries(int32_t num_rows, const void* q_nope, const void* q_pe, const void* kv_b_weight,
                                void* q_abs, void* hip_stream)
{
    g_detail[0] = '\0';
    if (num_rows < 1 || num_rows > kMaxRows)
        return fail(DSA_ERR_INVALID_ARGUMENT, "num_rows=%d outside [1, %d]", num_rows, kMaxRows);
    DSA_TRY(check_ptr16(q_nope, "q_nope"));
    DSA_TRY(check_ptr16(q_pe, "q_pe"));
    DSA_TRY(check_ptr16(kv_b_weight, "kv_b_weight"));
    DSA_TRY(check_ptr16(q_abs, "q_abs"));
    DSA_TRY(check_device());
    hipStream_t st = (hipStream_t)hip_stream;
    dsa::launch_absorb_queries(num_rows, (const uint16_t*)q_nope, (const uint16_t*)q_pe,
                               (const uint16_t*)kv_b_weight, (uint16_t*)q_abs, st);
    return after_launch(st, "absorb_queries");
}

dsa_status_t dsa_v_up_proj(int32_t num_rows, const float* o_latent, const void* kv_b_weight, float* out,
                           void* hip_stream)
{
    g_detail[0] = '\0';
    if (num_rows < 1 || num_rows > kMaxRows)
        return fail(DSA_ERR_INVALID_ARGUMENT, "num_rows=%d outside [1, %d]", num_rows, kMaxRows);
    DSA_TRY(check_ptr16(o_latent, "o_latent"));
    DSA_TRY(check_ptr16(kv_b_weight, "kv_b_weight"));
    DSA_TRY(check_ptr16(out, "out"));
    DSA_TRY(check_device());
    hipStream_t st = (hipStream_t)hip_stream;
    dsa::launch_v_up_proj(num_rows, o_latent, (const uint16_t*)kv_b_weight, out, st);
    return after_launch(st, "v_up_proj");
}

size_t dsa_cache_write_workspace_size(int32_t num_tokens)
{
    if (num_tokens < 1 || num_tokens > kMaxRows) return 0;
    return dsa::cache_write_workspace_bytes(num_tokens);
}

dsa_status_t dsa_cache_write(int32_t num_tokens, const void* hidden, const void* wk_weight,
                             const float* k_norm_weight, const float* k_norm_bias, float k_norm_eps,
                             const void* kv_a_weight, const float* kv_norm_weight, float kv_norm_eps,
                             const int32_t* positions, const int64_t* slots, double rope_theta, void* k_idx_cache,
                             void* kv_latent_cache, void* ws, size_t ws_bytes, void* hip_stream)
{
    g_detail[0] = '\0';
    if (num_tokens < 1 || num_tokens > kMaxRows)
        return fail(DSA_ERR_INVALID_ARGUMENT, "num_tokens=%d outside [1, %d]", num_tokens, kMaxRows);
    DSA_TRY(check_ptr16(hidden, "hidden"));
    DSA_TRY(check_ptr16(wk_weight, "wk_weight"));
    DSA_TRY(check_ptr16(kv_a_weight, "kv_a_weight"));
    DSA_TRY(check_ptr16(kv_norm_weight, "kv_norm_weight"));
    DSA_TRY(check_ptr16(k_idx_cache, "k_idx_cache"));
    DSA_TRY(check_ptr16(kv_latent_cache, "kv_latent_cache"));
    if (!k_norm_weight || !k_norm_bias || !positions || !slots)
        return fail(DSA_ERR_INVALID_ARGUMENT, "k_norm_weight, k_norm_bias, positions and slots must not be NULL");
    if (!aligned(k_norm_weight, 8) || !aligned(k_norm_bias, 8))
        return fail(DSA_ERR_MISALIGNED, "k_norm_weight and k_norm_bias need 8-byte alignment");
    if (!aligned(positions, 4)) return fail(DSA_ERR_MISALIGNED, "positions not 4-byte aligned");
    if (!aligned(slots, 8)) return fail(DSA_ERR_MISALIGNED, "slots not 8-byte aligned");
    if (!std::isfinite(k_norm_eps) || k_norm_eps < 0.f || !std::isfinite(kv_norm_eps) || kv_norm_eps < 0.f)
        return fail(DSA_ERR_INVALID_ARGUMENT, "norm eps must be finite and >= 0");
    if (!std::isfinite(rope_theta) || rope_theta <= 0.0)
        return fail(DSA_ERR_INVALID_ARGUMENT, "rope_theta must be finite and > 0");
    DSA_TRY(check_ws(ws, ws_bytes, dsa::cache_write_workspace_bytes(num_tokens)));
    DSA_TRY(check_device());
    hipStream_t st = (hipStream_t)hip_stream;
    dsa::launch_cache_write(num_tokens, (const uint16_t*)hidden, (const uint16_t*)wk_weight, k_norm_weight,
                            k_norm_bias, k_norm_eps, (const uint16_t*)kv_a_weight, kv_norm_weight, kv_norm_eps,
                            positions, slots, rope_theta, (uint16_t*)k_idx_cache, (uint16_t*)kv_latent_cache, ws, st);
    return after_launch(st, "cache_write");
}

int32_t dsa_index_share_source(int32_t layer, int32_t num_layers, int32_t leading_full, int32_t freq)
{
    if (num_layers < 1 || layer < 0 || layer >= num_layers || leading_full < 1 || freq < 1) return -1;
    if (layer < leading_full) return layer;
    const int32_t pos = (layer - leading_full) % freq;  // 0 .. freq-2 shared, freq-1 full
    return pos == freq - 1 ? layer : layer - pos - 1;
}

}  // extern "C"
