/*
 * dsa.h -- C ABI of libdsa: the DSA hot path (lightning indexer -> causal
 * top-k -> absorbed sparse MLA attention) for AMD Instinct MI355X (gfx950).
 *
 * The method is the one the GLM-5 / GLM-5.1 pages describe:
 *  - "GLM-5.1 架构深度拆解" (GLM-5.1 architecture teardown,
 *    cctoctofx.netlify.app), CH3 §3.2 "Indexer 公式" and §3.6
 *    "GlmMoeDsaIndexer.forward" (indexer score, causal mask, top-k), CH4 §4.1
 *    and §4.5 "GlmMoeDsaAttention.forward" (MLA latent rows, sparse attention).
 *  - GLM-5 explainer (ailearn.mscapital.top): the indexer paragraph (one
 *    128-d key per position, 32 x 128 queries, ReLU, 32 weights, causal
 *    Top-2,048 returning position IDs), the latent-cache paragraph (512 latent
 *    + 64 RoPE key per position; the IDs only drive the gather) and the
 *    "shorter than 2,048 keeps every position" rule.
 *  - "GLM-5.2 架构 QA" (pillumina.github.io), Q1.1 config listing
 *    (qk_nope_head_dim 192 + qk_rope_head_dim 64 = qk_head_dim 256).
 *
 * Conventions for every entry point:
 *  - Every array pointer is a DEVICE pointer unless marked "host".  The caller
 *    owns every buffer and the stream; the library allocates nothing and keeps
 *    no mutable global state besides a per-device properties cache and a
 *    thread-local error message.
 *  - bf16 arrays are passed as `const void*` holding IEEE bfloat16 bit
 *    patterns.  Row-major layouts, innermost dimension last.
 *  - All work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL
 *    means the null stream).  No call synchronizes the host.
 *  - Host-side validation runs first and in full.  On any error nothing is
 *    enqueued and every output is left untouched.  HIP launch failures map to
 *    DSA_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Device array contents (visible lengths, cache bases, index lists) are
 *    trusted: values outside the documented ranges are undefined behaviour.
 *  - Results are deterministic: identical inputs give bitwise-identical
 *    outputs (no floating-point atomics anywhere).
 *  - Calls are re-entrant; calls on different streams may overlap as long as
 *    they do not share output or workspace buffers.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point is exported with default visibility. */
#if defined(__GNUC__) || defined(__clang__)
#define DSA_API __attribute__((visibility("default")))
#else
#define DSA_API
#endif

/* Geometry (fixed at compile time).  32 index heads x 128 dims with one
 * 128-d key per position (teardown §3.6 steps 1-2); 64 attention heads over a
 * 576-wide latent row = 512 c_kv + 64 RoPE key (teardown CH4 §4.1, §4.2);
 * top-k up to index_topk = 2048 (teardown CH2 constraint 1, §3.6 step 7). */
#define DSA_INDEX_HEADS 32
#define DSA_INDEX_DIM 128
#define DSA_HEADS 64
#define DSA_LATENT_DIM 512
#define DSA_ROPE_DIM 64
#define DSA_ROW_DIM 576
#define DSA_TOPK_MAX 2048
/* Largest visible length a row may have (positions per sequence). */
#define DSA_MAX_VISIBLE (1 << 24)

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARGUMENT = 1,    /* null pointer, bad size, bad scale ... */
    DSA_ERR_MISALIGNED = 2,          /* a pointer or stride breaks its alignment rule */
    DSA_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes below the *_workspace_size value */
    DSA_ERR_NO_DEVICE = 4,           /* no HIP device, or the current device is not gfx950 */
    DSA_ERR_HIP = 5                  /* a HIP runtime call or kernel launch failed */
} dsa_status_t;

/*
 * Query rows.  Row r belongs to a sequence whose caches start at packed cache
 * row row_cache_base[r]; it sees positions [0, visible_len[r]) of that
 * sequence (causal, its own position included: keys are appended before
 * scoring, teardown §3.6 step 3 and §4.5 steps 5-6).  A decode row of a
 * sequence of length T has visible_len = T; prefill row i has i + 1.
 */
typedef struct {
    int32_t num_rows;              /* host: R >= 1 */
    int32_t max_visible;           /* host: >= every visible_len[r]; <= DSA_MAX_VISIBLE */
    const int32_t* visible_len;    /* [R], each in [1, max_visible] */
    const int64_t* row_cache_base; /* [R], each >= 0 */
    uint32_t flags;                /* host: DSA_ROWS_* hints (0 = none) */
} dsa_rows_t;

/* Hint: no two rows read the same sequence (e.g. a decode batch with one query
 * per sequence).  The indexer then skips its shared-sequence pass (blocks of
 * 32 consecutive rows on one sequence, as in a prefill chunk, are scored with
 * query tiles on MFMA).  Hints never change results: with or without the
 * flag, and whether or not it is true, every call computes the same values. */
#define DSA_ROWS_DISTINCT_SEQUENCES 1u

/* Library version string (static storage). */
DSA_API const char* dsa_version(void);
/* Human-readable name of a status code (static storage; never NULL). */
DSA_API const char* dsa_status_string(dsa_status_t status);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
DSA_API const char* dsa_last_error_detail(void);

/*
 * Lightning-indexer scores (teardown §3.6 step 5, §3.2 steps 4-6; explainer
 * indexer paragraph):
 *     scores[r, t] = sum_h w[r,h] * ReLU(index_scale * sum_d q_idx[r,h,d] * k_idx[base_r + t, d])
 * for 0 <= t < visible_len[r].  Columns >= visible_len[r] are not written.
 *  q_idx  [R, 32, 128] bf16, 16-B aligned (post-RoPE index queries)
 *  w      [R, 32] fp32, 16-B aligned (already multiplied by 32^-1/2 upstream,
 *         teardown §3.6 step 4)
 *  k_idx  [*, 128] bf16 packed index-key cache, 16-B aligned
 *  index_scale  > 0 and finite
 *  scores [R, ld] fp32, 16-B aligned; ld >= max_visible and ld % 4 == 0
 * Products are exact in fp32 (bf16 x bf16); sums are fp32.
 */
DSA_API dsa_status_t dsa_indexer_scores(const dsa_rows_t* rows, const void* q_idx, const float* w,
                                const void* k_idx, float index_scale, float* scores, int64_t ld,
                                void* hip_stream);

/* Workspace bytes dsa_topk_select needs for these sizes (host arithmetic only). */
DSA_API size_t dsa_topk_workspace_size(int32_t num_rows, int32_t max_visible, int32_t k);

/*
 * Causal top-k select (teardown §3.6 step 7 "topk = min(index_topk,
 * total_len)", §3.4 determinism requirement; explainer "shorter than 2,048
 * keeps all; the top-k is a set of positions").
 * For each row picks k_r = min(k, visible_len[r]) positions of scores[r, 0:n_r)
 * with the largest scores.  Order: larger score first; -0.0 equals +0.0; equal
 * scores go to the lower position; NaN ranks below every number.
 *  scores   [R, ld] fp32, 16-B aligned, ld >= max_visible, ld % 4 == 0
 *  k        1 .. 2048
 *  indices  [R, k] int32, 4-B aligned: the k_r positions in ascending order,
 *           then -1 padding up to k
 *  ws       device workspace of ws_bytes >= dsa_topk_workspace_size(R, max_visible, k),
 *           256-B aligned; contents need no initialisation and are clobbered
 */
DSA_API dsa_status_t dsa_topk_select(const dsa_rows_t* rows, const float* scores, int64_t ld, int32_t k,
                             int32_t* indices, void* ws, size_t ws_bytes, void* hip_stream);

/* Workspace bytes dsa_sparse_mla_attn needs for these sizes (host arithmetic only). */
DSA_API size_t dsa_sparse_mla_workspace_size(int32_t num_rows, int32_t k);

/*
 * Absorbed-MLA attention over the selected positions (teardown §4.5 steps 2,
 * 6, 7; explainer latent-cache paragraph; GLM-5.2 QA Q1.1 for the 256-wide
 * original QK head that fixes softmax_scale = 1/sqrt(256)):
 *     z[h,j]   = softmax_scale * sum_{d<576} q_abs[r,h,d] * kv[base_r + idx_j, d]
 *     p[h,j]   = softmax_j(z[h,:])
 *     out[r,h,c] = sum_j p[h,j] * kv[base_r + idx_j, c]        c < 512
 *     lse[r,h] = log sum_j exp(z[h,j])
 * over the entries idx_j >= 0 of indices[r, 0:k] (negative entries are
 * padding and are skipped).  q_abs = [W_UK^T q_nope (512) || q_pe (64)] per
 * head; the latent row is [c_kv (512) || k_pe (64)]; the output is the
 * 512-wide latent before the per-head V up-projection.
 *  q_abs      [R, 64, 576] bf16, 16-B aligned
 *  kv_latent  [*, 576] bf16 packed latent cache, 16-B aligned
 *  indices    [R, k] int32, entries in [0, visible_len[r]) or negative
 *  k          1 .. 2048;  softmax_scale > 0 and finite
 *  out_latent [R, 64, 512] fp32, 16-B aligned
 *  out_lse    [R, 64] fp32 or NULL
 *  ws         ws_bytes >= dsa_sparse_mla_workspace_size(R, k), 256-B aligned
 * A row whose entries are all negative gets out = 0 and lse = -inf.
 * P is rounded to bf16 (round-to-nearest-even) for the P.V product; all sums
 * are fp32.
 */
DSA_API dsa_status_t dsa_sparse_mla_attn(const dsa_rows_t* rows, const void* q_abs, const void* kv_latent,
                                 const int32_t* indices, int32_t k, float softmax_scale,
                                 float* out_latent, float* out_lse, void* ws, size_t ws_bytes,
                                 void* hip_stream);

/* Budget, in bytes, of the fp32 score rows dsa_decode_step holds at a time. */
#define DSA_STEP_SCORES_BUDGET (1u << 30)

/* Workspace bytes dsa_decode_step needs for these sizes (host arithmetic only):
 *   align256(C * ld * 4) + align256(4 C) + 256 + align256(dsa_topk_workspace_size(C, max_visible, k))
 *   + align256(dsa_sparse_mla_workspace_size(R, k))
 * with ld = max_visible rounded up to a multiple of 4 and C the rows scored at
 * a time: C = R when R * ld * 4 <= DSA_STEP_SCORES_BUDGET; otherwise, with
 * F = floor(DSA_STEP_SCORES_BUDGET / (ld * 4)) rows fitting the budget, C is
 * F rounded down to a multiple of 256 when F >= 256, else to a multiple of
 * 32, and at least 32 (at most R).  The score rows of a call thus take at
 * most max(1 GiB, 32 * ld * 4). */
DSA_API size_t dsa_decode_step_workspace_size(int32_t num_rows, int32_t max_visible, int32_t k);

/*
 * The whole path in one call: dsa_indexer_scores into workspace, then
 * dsa_topk_select into `indices`, then dsa_sparse_mla_attn.  Arguments mean
 * what they mean above; `indices` [R, k] int32 receives the selection.
 * ws_bytes >= dsa_decode_step_workspace_size(R, max_visible, k).  Rows are
 * scored and selected C at a time (C as above; chunks start at multiples of
 * 32 rows), then attended in one pass; results are those of the separate
 * calls over all rows at once, bit for bit.
 */
DSA_API dsa_status_t dsa_decode_step(const dsa_rows_t* rows, const void* q_idx, const float* w,
                             const void* k_idx, float index_scale, const void* q_abs,
                             const void* kv_latent, float softmax_scale, int32_t k,
                             int32_t* indices, float* out_latent, float* out_lse, void* ws,
                             size_t ws_bytes, void* hip_stream);

/* ---- The fused step without a workspace argument -----------------------
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as dsa_decode_step, with the workspace taken from a scratch array of
 * DSA_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device it
 * runs on, from the first call there until the process ends.  The call itself
 * allocates nothing.  Rows are scored and selected as many at a time as the
 * scratch holds (the dsa_decode_step_workspace_size formula with C the
 * largest multiple of 32 rows that fits, or all rows when fewer than 32);
 * results equal dsa_decode_step's bit for bit.  Every call on one device uses that
 * device's single array: calls that overlap on one device (other streams,
 * other host threads) race and must be serialized by the caller.
 * Errors: as for dsa_decode_step, plus DSA_ERR_INVALID_ARGUMENT when even 32
 * rows at a time (with the attention's split partials for every row) exceed
 * the scratch (from max_visible of about 900,000 positions up, depending on
 * the row count); DSA_ERR_HIP if
 * the scratch array's device address cannot be obtained. */
#define DSA_NOALLOC_SCRATCH_BYTES (128u << 20)

DSA_API dsa_status_t dsa_decode_step_noalloc(const dsa_rows_t* rows, const void* q_idx, const float* w,
                                             const void* k_idx, float index_scale, const void* q_abs,
                                             const void* kv_latent, float softmax_scale, int32_t k,
                                             int32_t* indices, float* out_latent, float* out_lse,
                                             void* hip_stream);

/* ---- Paged caches -------------------------------------------------------
 *
 * The same calls over caches kept in fixed-size blocks of a shared pool, with
 * a block table per sequence (the serving layout of vLLM's PagedAttention,
 * which "GLM-5.2 架构 QA" CH2 Q2.6 and CH4 Q4.2 name as the paged store of
 * the compressed cache in GLM-5.2's serving stack).  Only the
 * addressing changes: position p of the sequence whose block-table row is s
 * lives at pool row
 *     block_table[s * max_blocks + p / block_size] * block_size + p % block_size
 * in both pools (index keys [*, 128] and latent rows [*, 576]), which share
 * the block table.  dsa_cache_write fills a pool when its slots are these
 * rows.  In the *_paged calls rows->row_cache_base[r] is the block-table row
 * s of row r's sequence (not a cache row); everything else means what it
 * means above, and `indices` stay logical positions.  Results are bitwise
 * those of the packed calls on the same logical caches.
 */
typedef struct {
    const int32_t* block_table; /* device: [num_seqs, max_blocks] int32 pool block numbers, 4-B aligned */
    int32_t max_blocks;         /* host: row stride of block_table, >= ceil(max_visible / block_size) */
    int32_t block_size;         /* host: positions per block, a power of two in [16, 65536] */
} dsa_paged_t;
/* The entries a call reads (blocks below ceil(visible_len[r] / block_size))
 * must name blocks inside both pools, and pool rows must stay below 2^31;
 * neither is checked (device data).  Errors: as for the packed calls, plus a
 * NULL or misaligned block table, a block size that is not a power of two in
 * [16, 65536], or max_blocks too small for max_visible. */

DSA_API dsa_status_t dsa_indexer_scores_paged(const dsa_rows_t* rows, const dsa_paged_t* paged, const void* q_idx,
                                              const float* w, const void* k_pool, float index_scale, float* scores,
                                              int64_t ld, void* hip_stream);

/* Workspace bytes dsa_sparse_mla_attn_paged needs (the packed size plus the
 * translated index lists). */
DSA_API size_t dsa_sparse_mla_paged_workspace_size(int32_t num_rows, int32_t k);

DSA_API dsa_status_t dsa_sparse_mla_attn_paged(const dsa_rows_t* rows, const dsa_paged_t* paged,
                                               const void* q_abs, const void* kv_pool, const int32_t* indices,
                                               int32_t k, float softmax_scale, float* out_latent, float* out_lse,
                                               void* ws, size_t ws_bytes, void* hip_stream);

DSA_API size_t dsa_decode_step_paged_workspace_size(int32_t num_rows, int32_t max_visible, int32_t k);

DSA_API dsa_status_t dsa_decode_step_paged(const dsa_rows_t* rows, const dsa_paged_t* paged, const void* q_idx,
                                           const float* w, const void* k_pool, float index_scale, const void* q_abs,
                                           const void* kv_pool, float softmax_scale, int32_t k, int32_t* indices,
                                           float* out_latent, float* out_lse, void* ws, size_t ws_bytes,
                                           void* hip_stream);

/* ---- Projections on either side of the path ----------------------------
 *
 * kv_b_proj expands the 512-d latent into 64 heads x (192 non-RoPE key dims
 * + 256 value dims) ("GLM-5.1 架构深度拆解" CH4 §4.1; §4.5 step 2 splits each
 * head's 448 output rows as [k_nope || value]).  Both calls take that weight
 * as the model holds it:
 *   kv_b_weight  [64, 448, 512] bf16: head h's rows 0..191 are W_UK,h, rows
 *                192..447 are W_UV,h; each row is 512 latent columns.
 * Because kv_b_proj is linear, q_nope . (W_UK,h c) = (W_UK,h^T q_nope) . c
 * and the values W_UV,h c can be up-projected after the attention sum, which
 * is what lets the attention run on the 576-wide latent rows.
 */

/* Query absorption: for each row r < num_rows and head h < 64,
 *   q_abs[r,h,c]       = sum_{d<192} W_UK,h[d,c] * q_nope[r,h,d]   (c < 512)
 *   q_abs[r,h,512 + i] = q_pe[r,h,i]                                (i < 64)
 * computed on bf16 matrix cores with fp32 accumulation and rounded to bf16
 * (round-to-nearest-even): the q_abs layout dsa_sparse_mla_attn and
 * dsa_decode_step take.
 *   q_nope [R,64,192] bf16, q_pe [R,64,64] bf16 (RoPE already applied),
 *   kv_b_weight as above, q_abs [R,64,576] bf16 (written).
 * Errors: num_rows outside [1, 2^24]; a NULL or not 16-byte-aligned pointer;
 * no gfx950 device.  No workspace. */
DSA_API dsa_status_t dsa_absorb_queries(int32_t num_rows, const void* q_nope, const void* q_pe,
                                        const void* kv_b_weight, void* q_abs, void* hip_stream);

/* V up-projection: for each row r < num_rows and head h < 64,
 *   out[r,h,v] = sum_{c<512} W_UV,h[v,c] * bf16(o_latent[r,h,c])   (v < 256)
 * where bf16() rounds to nearest even (the precision of the bf16 matrix-core
 * operand); fp32 accumulation.  o_latent is the attention output
 * (out_latent of dsa_sparse_mla_attn / dsa_decode_step).
 *   o_latent [R,64,512] fp32, kv_b_weight as above, out [R,64,256] fp32.
 * Errors: as for dsa_absorb_queries. */
DSA_API dsa_status_t dsa_v_up_proj(int32_t num_rows, const float* o_latent, const void* kv_b_weight,
                                   float* out, void* hip_stream);

/* ---- Cache writers -----------------------------------------------------
 *
 * The rows the path reads, made from a new token's hidden state x (6144-d):
 *  - indexer key ("GLM-5.1 架构深度拆解" CH3 §3.6 step 2):
 *      v = LayerNorm(wk x) over 128 dims (population variance, weight, bias),
 *      key = [RoPE(v[0:64]) || v[64:128]];
 *  - latent row (same page, CH4 §4.1, §4.5 steps 2-3):
 *      [c || p] = kv_a_proj_with_mqa x  (512 + 64 outputs),
 *      row = [RMSNorm(c) over 512 (weight) || RoPE(p)];
 *  - RoPE ("GLM-5.2 架构 QA" CH1 Q1.4): in a 64-d block, dims i and i + 32
 *    (i < 32) turn by a = position * rope_theta^(-2i/64):
 *      y[i] = x[i] cos a - x[i+32] sin a,  y[i+32] = x[i+32] cos a + x[i] sin a.
 * Projections accumulate in fp32 on bf16 matrix cores; norms run in fp32;
 * RoPE angles are formed in fp64; results are rounded to bf16
 * (round-to-nearest-even) as they are stored.
 */

#define DSA_HIDDEN 6144

/* Workspace bytes dsa_cache_write needs (host arithmetic only; 0 when
 * num_tokens is outside [1, 2^24]). */
DSA_API size_t dsa_cache_write_workspace_size(int32_t num_tokens);

/* Computes both cache rows of num_tokens new tokens and writes them at row
 * slots[t] of each cache (a token whose slot is negative writes nothing):
 *   hidden          [N, 6144] bf16, 16-B aligned
 *   wk_weight       [128, 6144] bf16 (nn.Linear layout: one output per row)
 *   k_norm_weight, k_norm_bias  [128] fp32, 8-B aligned;  k_norm_eps >= 0
 *   kv_a_weight     [576, 6144] bf16 (rows 0..511 c_kv, 512..575 k_pe)
 *   kv_norm_weight  [512] fp32, 16-B aligned;  kv_norm_eps >= 0
 *   positions       [N] int32 RoPE positions;  slots [N] int64 cache rows
 *   rope_theta      > 0 (1e6 for GLM-5/5.1, 8e6 for GLM-5.2)
 *   k_idx_cache     [*, 128] bf16 and kv_latent_cache [*, 576] bf16, the
 *                   caches dsa_indexer_scores / dsa_sparse_mla_attn read; only
 *                   the rows named by slots are written
 *   ws              >= dsa_cache_write_workspace_size(N) bytes, 256-B aligned
 * Slots must be distinct (two tokens on one slot race) and inside the caches
 * (not checked: the library cannot see their sizes).  Errors: num_tokens
 * outside [1, 2^24]; NULL or misaligned pointers; a negative or non-finite
 * eps; rope_theta not finite and > 0; workspace too small; no gfx950 device.
 */
DSA_API dsa_status_t dsa_cache_write(int32_t num_tokens, const void* hidden, const void* wk_weight,
                                     const float* k_norm_weight, const float* k_norm_bias, float k_norm_eps,
                                     const void* kv_a_weight, const float* kv_norm_weight, float kv_norm_eps,
                                     const int32_t* positions, const int64_t* slots, double rope_theta,
                                     void* k_idx_cache, void* kv_latent_cache, void* ws, size_t ws_bytes,
                                     void* hip_stream);

/* ---- IndexShare: one selection serving several layers ------------------
 *
 * Only "full" layers run the indexer and the top-k; a "shared" layer has no
 * indexer (and no index-key cache) and attends over the index list of the
 * latest full layer below it ("GLM-5.2 架构 QA" CH2 Q2.1 and Q2.2; the layer
 * pattern is CH1 Q1.2 and CH2 Q2.4).  With this library a full layer calls
 * dsa_decode_step, which writes `indices`; each shared layer after it calls
 * dsa_sparse_mla_attn with its own q_abs and kv_latent and that same
 * `indices` buffer, which nothing in between may overwrite.  Attention reads
 * the indices only, so the buffer is the model's shared top-k cache as is.
 */

/* The layer whose selection `layer` attends over: `layer` itself when it is
 * a full layer, else the latest full layer below it.  The first
 * `leading_full` layers are full; above them the layers repeat with period
 * `freq`, each period being freq - 1 shared layers followed by one full
 * layer.  num_layers = 78, leading_full = 3, freq = 4 gives the GLM-5.2
 * pattern: layers 0, 1, 2, 6, 10, ..., 74 full (21 of 78), layers 3..5
 * reuse layer 2, layers 75..77 reuse layer 74.  freq = 1 makes every layer
 * full.  Host arithmetic only (no device needed).  Returns -1 when
 * num_layers < 1, layer is outside [0, num_layers), leading_full < 1 or
 * freq < 1. */
DSA_API int32_t dsa_index_share_source(int32_t layer, int32_t num_layers, int32_t leading_full, int32_t freq);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
