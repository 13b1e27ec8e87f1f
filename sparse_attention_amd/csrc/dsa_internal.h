// dsa_internal.h -- host-side launcher declarations shared by api.cpp and the
// kernel translation units.  Launchers only enqueue work; validation happens
// in api.cpp before any of them is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// A paged cache: position p of the sequence whose block-table row is s sits at
// pool row (block_table[s * max_blocks + (p >> log2_block)] << log2_block) |
// (p & (2^log2_block - 1)).  block_table == nullptr: a packed cache.
struct PagedCache {
    const int32_t* block_table;
    int64_t max_blocks;
    int log2_block;
};

// ---- indexer -------------------------------------------------------------
// Indexer workgroups per row.
int indexer_pick_chunk(int32_t num_rows, int32_t max_visible);
void launch_indexer_scores(int32_t num_rows, int32_t max_visible, const int32_t* vis,
                           const int64_t* base, const uint16_t* q, const float* w,
                           const uint16_t* kc, float scale, float* scores, int64_t ld,
                           bool distinct_sequences, const PagedCache& paged, hipStream_t stream,
                           void* list_ws = nullptr);
// Workspace the row list of launch_indexer_scores needs (list_ws, 256-B aligned).
size_t indexer_list_offset(int32_t num_rows);
size_t indexer_list_bytes(int32_t num_rows);

// ---- top-k ---------------------------------------------------------------
constexpr int TK_CHUNK = 4096;     // scores one top-k workgroup owns
constexpr int TK_BINS = 4096;      // 12-bit top radix digit
constexpr int TK_CAP = 8192;       // candidate slots per row
constexpr int TK_ROWST = 8;        // u32 words of per-row state
constexpr int TK_CHUNKST = 4;      // u32 words of per-chunk state
constexpr int TK_MAX_CHUNKS = 4096;  // DSA_MAX_VISIBLE / TK_CHUNK

constexpr int TR_ROW_PATH_MAXN = 65536;  // calls with max_visible up to this use it

struct TopkWorkspace {
    uint32_t* rowst;           // [R][TK_ROWST]
    uint32_t* chunkst;         // [R][CH][TK_CHUNKST]
    unsigned long long* cand;  // [R][TK_CAP]
    int32_t* longrows;         // [R]: rows the multi-workgroup kernels own, in row order
    uint32_t* nlong;           // their count
    int32_t chunks;            // CH
    uint32_t* crec;            // chunked path for few rows: [R][CH] (count, largest key, theta_lo, -)
    unsigned long long* mcand; //   [R][CH][slots] (key, position) in position order
};
size_t topk_workspace_bytes(int32_t num_rows, int32_t max_visible);
TopkWorkspace topk_workspace_carve(void* ws, int32_t num_rows, int32_t max_visible);
void launch_topk(int32_t num_rows, int32_t max_visible, const int32_t* vis, const float* scores,
                 int64_t ld, int32_t k, int32_t* indices, const TopkWorkspace& tw,
                 hipStream_t stream);

// ---- sparse MLA attention --------------------------------------------------
int attn_pick_splits(int32_t num_rows, int32_t k);
size_t attn_workspace_bytes(int32_t num_rows, int32_t k);
void launch_sparse_mla(int32_t num_rows, const int64_t* base, const uint16_t* qa,
                       const uint16_t* kv, const int32_t* idx, int32_t k, float softmax_scale,
                       float* out, float* lse, void* ws, hipStream_t stream, int32_t max_visible,
                       bool pad_rows = false);

// Logical selection -> physical pool rows of a paged latent cache; a negative
// entry becomes -1 - (pool row of the sequence's position 0), the row the
// attention's padding slots then fetch (launch_sparse_mla with pad_rows).
// Also zeroes the num_rows cache bases the attention adds.  Enqueued on
// `stream`.
void launch_page_indices(int32_t num_rows, int32_t k, const int64_t* seq, const int32_t* idx,
                         const PagedCache& paged, int32_t* phys, int64_t* zero_base, hipStream_t stream);

// ---- projections on either side of the attention -------------------------
void launch_absorb_queries(int32_t num_rows, const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* kvb,
                           uint16_t* q_abs, hipStream_t stream);
void launch_v_up_proj(int32_t num_rows, const float* o, const uint16_t* kvb, float* out, hipStream_t stream);

// ---- cache writers ---------------------------------------------------------
int cache_write_splits(int32_t num_tokens);
size_t cache_write_workspace_bytes(int32_t num_tokens);
void launch_cache_write(int32_t num_tokens, const uint16_t* hidden, const uint16_t* wk, const float* k_norm_weight,
                        const float* k_norm_bias, float k_norm_eps, const uint16_t* kv_a, const float* kv_norm_weight,
                        float kv_norm_eps, const int32_t* positions, const int64_t* slots, double rope_theta,
                        uint16_t* k_idx_cache, uint16_t* kv_latent_cache, void* ws, hipStream_t stream);

// ---- fused step over a fixed scratch region ------------------------------
// Validates the call in full, picks the rows scored at a time so that the
// step's workspace fits scratch_bytes (an error if 32 rows do not fit), checks
// the device, then asks scratch_ptr() for the region's device address and
// enqueues the step there.  scratch_ptr returns nullptr on failure.
dsa_status_t decode_step_in_scratch(const dsa_rows_t* rows, const void* q_idx, const float* w, const void* k_idx,
                                    float index_scale, const void* q_abs, const void* kv_latent, float softmax_scale,
                                    int32_t k, int32_t* indices, float* out_latent, float* out_lse,
                                    size_t scratch_bytes, void* (*scratch_ptr)(), void* hip_stream);

// Debug aid: when DSA_SYNC_DEBUG=1, synchronize after every launch.
bool sync_debug();

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace dsa
