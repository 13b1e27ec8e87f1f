// indexer.hip -- lightning-indexer scores on gfx950.
//
// Computes scores[r, t] = sum_h w[r,h] * ReLU(scale * q[r,h,:] . K[base_r + t, :])
// for t < n_r ("GLM-5.1 架构深度拆解" §3.6 step 5 and §3.2 steps 4-6; the
// GLM-5 explainer's indexer paragraph: one 128-d key per position shared by
// all 32 index heads).
//
// Design (decode rows, each row streaming its own key cache):
//  - The work is HBM-bound (256 key bytes per position against 8192 MFMA
//    flops), so the kernel's job is keeping enough 16-byte loads in flight
//    with good DRAM locality: the waves of a row sweep it together in
//    interleaved 64-position blocks, each wave prefetching its next block.
//  - The contraction runs on v_mfma_f32_16x16x32_bf16 with the 32 index heads
//    as M (two 16-row blocks) and 16 positions as N: the key rows are the B
//    operand and are loaded straight from HBM into registers.  Lane (j, g)
//    loads bytes [64 s + 16 g, +16) of position j's 256-byte row at k-step s,
//    so the four lanes of a position read 64 contiguous bytes per load; Q uses
//    the same k order and stays in registers for the whole chunk.
//  - The output layout puts 4 heads of one position in each lane, so the
//    ReLU and head weighting stay in registers; a reduce-scatter over the
//    lanes j, j+16, j+32, j+48 (three VALU lane swaps for four position
//    groups) leaves each lane group the full score of a different 16-position
//    group, so one store covers 64 consecutive scores.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int IDX_WAVES = 4;
constexpr int IDX_GROUPS = 4;               // 16-position groups per block
constexpr int IDX_BLOCK = 16 * IDX_GROUPS;  // positions per wave iteration

// ---------------------------------------------------------------------------
// Prefill tile kernel.  Rows come in blocks of IDX_TILE_ROWS consecutive rows;
// a block is "shared" when all its rows exist and read the same sequence
// (equal cache base), as the rows of one prefill chunk do.  Shared blocks are
// scored here, every other row by the row kernel; both kernels evaluate the
// same test, so each row is scored exactly once.
//
// One 512-thread workgroup scores a shared block (32 rows x 32 heads = 1024
// MFMA rows) against 128-position key tiles: each tile is loaded once into LDS
// (256 B per position, rows padded to 272 B so the 16 rows an operand read
// touches sit in distinct banks), and each wave multiplies its 4 rows' queries
// (128 heads, kept in registers) by the tile: 256 MFMAs per wave per 32 KB of
// keys and one barrier.  The causal triangle is skipped: a block only visits positions
// below its longest row, and scores past a row's own length are not stored.
// Workgroups of one block take every CX-th tile, for load balance across
// blocks of different lengths.
constexpr int IDX_TILE_ROWS = 32;
constexpr int IDX_TILE_POS = 128;
constexpr int IDX_KEY_PITCH = 272;  // bytes per staged key row

// Called by whole waves; the result is wave-uniform.
__device__ __forceinline__ bool block_is_shared(const int64_t* __restrict__ base, int num_rows, int b)
{
    const int r0 = b * IDX_TILE_ROWS;
    if (r0 + IDX_TILE_ROWS > num_rows) return false;
    const int64_t mine = base[r0 + (threadIdx.x & (IDX_TILE_ROWS - 1))];
    return __ballot(mine != base[r0]) == 0ull;
}

// Paged caches: positions live in blocks of 2^lg rows; row base[r]'s sequence
// has its physical block numbers in bt[base[r] * mb ..].  Blocks hold at least
// 16 positions, so a 16-aligned position group never straddles two blocks.
template <bool PAGED>
__global__ __launch_bounds__(512) void indexer_tile_kernel(
    const int32_t* __restrict__ vis, const int64_t* __restrict__ base, const uint16_t* __restrict__ q,
    const float* __restrict__ w, const uint16_t* __restrict__ kc, float scale, float* __restrict__ scores,
    int64_t ld, int num_rows, PagedCache pm)
{
    // Last blocks first: in a causal prefill chunk they see the most
    // positions, so starting them early shortens the tail (measured on an
    // 8,192-position prefill: 267 vs 336 us).
    const int nblk = num_rows / IDX_TILE_ROWS;
    if (grid_item() >= nblk) return;
    const int blk = nblk - 1 - grid_item();
    if (!block_is_shared(base, num_rows, blk)) return;
    const int r0 = blk * IDX_TILE_ROWS;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;  // 0..7: rows r0 + 4 wave .. + 3
    const int j = lane & 15;
    const int g = lane >> 4;

    __shared__ __attribute__((aligned(16))) uint8_t keys[2][IDX_TILE_POS * IDX_KEY_PITCH];
    __shared__ int s_nmax;
    // Each wave's 4 rows x 128 scores of the current tile, gathered here so
    // that they leave as 16-byte row pieces (two stores per lane per tile
    // instead of eight 4-byte ones).
    __shared__ __attribute__((aligned(16))) float sst[8][4][IDX_TILE_POS + 4];
    if (threadIdx.x == 0) s_nmax = 0;
    __syncthreads();
    if (threadIdx.x < IDX_TILE_ROWS) atomicMax(&s_nmax, vis[r0 + threadIdx.x]);

    // Queries and head weights of this wave's 4 rows (the positive index
    // scale is folded into the weights: ReLU(s x) = s ReLU(x) for s > 0).
    bf16x8 qa[4][2][4];
    float wv[4][8];
    int nrow[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int r = r0 + 4 * wave + i;
        nrow[i] = vis[r];
        const uint16_t* qr = q + (int64_t)r * (32 * 128);
#pragma unroll
        for (int hb = 0; hb < 2; hb++)
#pragma unroll
            for (int s = 0; s < 4; s++) qa[i][hb][s] = load_bf16x8(qr + (hb * 16 + j) * 128 + 32 * s + 8 * g);
#pragma unroll
        for (int v = 0; v < 4; v++) {
            wv[i][v] = w[r * 32 + 4 * g + v] * scale;
            wv[i][4 + v] = w[r * 32 + 16 + 4 * g + v] * scale;
        }
    }
    __syncthreads();
    const int nmax = s_nmax;
    const int ntile = (nmax + IDX_TILE_POS - 1) / IDX_TILE_POS;
    const uint16_t* kb = PAGED ? kc : kc + base[r0] * 128;
    const int32_t* btr = PAGED ? pm.block_table + base[r0] * pm.max_blocks : nullptr;

    // Staging roles: thread t moves 16 bytes (chunk t & 15) of positions
    // (t >> 4) + 32 h, h < NH, of a tile.  Positions past nmax are clamped
    // onto nmax - 1.
    const int sp_pos = threadIdx.x >> 4, sp_chunk = threadIdx.x & 15;
    constexpr int NH = IDX_TILE_POS / 32;  // staging loads per thread per tile
    auto load_tile = [&](int tt, u32x4 (&dst)[NH]) {
#pragma unroll
        for (int h = 0; h < NH; h++) {
            const int pos = min(tt * IDX_TILE_POS + sp_pos + 32 * h, nmax - 1);
            int64_t prow = pos;
            if constexpr (PAGED)
                prow = ((int64_t)btr[pos >> pm.log2_block] << pm.log2_block) | (pos & ((1 << pm.log2_block) - 1));
            dst[h] = load_u32x4(kb + prow * 128 + sp_chunk * 8);
        }
    };
    int tt = blockIdx.x;
    u32x4 pre[NH];
#pragma unroll
    for (int h = 0; h < NH; h++) pre[h] = u32x4{0u, 0u, 0u, 0u};
    if (tt < ntile) load_tile(tt, pre);
    int buf = 0;
    for (; tt < ntile; tt += gridDim.x, buf ^= 1) {
#pragma unroll
        for (int h = 0; h < NH; h++)
            *reinterpret_cast<u32x4*>(&keys[buf][(sp_pos + 32 * h) * IDX_KEY_PITCH + sp_chunk * 16]) = pre[h];
        __syncthreads();  // tile visible; the other buffer is free again
        if (tt + (int)gridDim.x < ntile) load_tile(tt + gridDim.x, pre);
        const int p0 = tt * IDX_TILE_POS;
        // B operands of position group pg (positions 16 pg + j, k-step s ->
        // bytes 64 s + 16 g), read one group ahead into a double buffer.
        bf16x8 kv[2][4];
        auto ldkv = [&](int pg) {
            const uint8_t* kp = &keys[buf][(16 * pg + j) * IDX_KEY_PITCH + 16 * g];
#pragma unroll
            for (int s = 0; s < 4; s++) kv[pg & 1][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp + 64 * s));
        };
        // Sixteen units (position group pg, row i), software-pipelined: the
        // MFMAs of unit u + 1 are issued before the ReLU / head weighting of
        // unit u, so the VALU work runs in the MFMA shadow.  Each lane sums
        // its 8 heads; once a position group is done, one reduce-scatter
        // leaves row 4 wave + g's 32-head score in lane group g, and its store
        // overlaps the next group's MFMAs.
        float part[4];
        floatx4 acc[2][2];
        auto mm = [&](int u) {
            const int pg = u >> 2, i = u & 3;
            floatx4 a0 = {0.f, 0.f, 0.f, 0.f};
            floatx4 a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s++) {
                a0 = mfma_16x16x32(qa[i][0][s], kv[pg & 1][s], a0);
                a1 = mfma_16x16x32(qa[i][1][s], kv[pg & 1][s], a1);
            }
            acc[u & 1][0] = a0;
            acc[u & 1][1] = a1;
        };
        auto epi = [&](int u) {
            const int i = u & 3;
            const floatx4 a0 = acc[u & 1][0], a1 = acc[u & 1][1];
            float sum = 0.f;
#pragma unroll
            for (int v = 0; v < 4; v++) sum += wv[i][v] * relu_bits(a0[v]);
#pragma unroll
            for (int v = 0; v < 4; v++) sum += wv[i][4 + v] * relu_bits(a1[v]);
            part[i] = sum;
        };
        constexpr int NU = 4 * (IDX_TILE_POS / 16);  // units per tile
        ldkv(0);
        ldkv(1);
        mm(0);
#pragma unroll
        for (int u = 0; u < NU; u++) {
            if (u + 1 < NU) mm(u + 1);
            epi(u);
            if ((u & 3) == 3) {
                const int pg = u >> 2;
                if (pg + 2 < NU / 4) ldkv(pg + 2);  // its buffer's last reader was unit u
                // Lane group g holds row 4 wave + g: 16 consecutive scores.
                sst[wave][g][16 * pg + j] = xrow_reduce_scatter4(part);
            }
            if (u + 1 < NU) {
#pragma unroll
                for (int q = 0; q < 8; q++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU (measured best of 1..4)
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // The tile's scores, lane l taking row 4 wave + (l >> 4), positions
        // 8 (l & 15) .. + 7 (same wave, so no barrier).  Non-temporal: read
        // once, by the top-k; dirty L2 lines would cost the kernel-end
        // write-back.
        const int g2 = lane >> 4, c = (lane & 15) * 8;
        const float4 v0 = *reinterpret_cast<const float4*>(&sst[wave][g2][c]);
        const float4 v1 = *reinterpret_cast<const float4*>(&sst[wave][g2][c + 4]);
        int lim = nrow[0];
#pragma unroll
        for (int i = 1; i < 4; i++) lim = (g2 == i) ? nrow[i] : lim;
        float* dst = scores + (int64_t)(r0 + 4 * wave + g2) * ld + p0 + c;
        if (p0 + c + 8 <= lim) {
            __builtin_nontemporal_store(floatx4{v0.x, v0.y, v0.z, v0.w}, reinterpret_cast<floatx4*>(dst));
            __builtin_nontemporal_store(floatx4{v1.x, v1.y, v1.z, v1.w}, reinterpret_cast<floatx4*>(dst + 4));
        } else {
            const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int e = 0; e < 8; e++)
                if (p0 + c + e < lim) __builtin_nontemporal_store(vv[e], dst + e);
        }
    }
}

// One wave's share of row r: 64-position blocks wr, wr + nw, wr + 2 nw, ...
// (nw = waves per row; every wave works on its own, no workgroup barrier).
// The waves of a row thus read one compact, advancing window of the key cache
// instead of thousands of scattered streams, which keeps DRAM pages open.
// Each wave loads each 16-position group of its next block as soon as the
// same group of the current block has gone through the matrix cores.
template <bool PAGED>
__device__ __forceinline__ void indexer_row(int r, int wr, int nw, const int32_t* __restrict__ vis,
                                            const int64_t* __restrict__ base, const uint16_t* __restrict__ q,
                                            const float* __restrict__ w, const uint16_t* __restrict__ kc,
                                            float scale, float* __restrict__ scores, int64_t ld,
                                            const PagedCache& pm)
{
    const int n = vis[r];
    const int lane = threadIdx.x & 63;
    const int j = lane & 15;
    const int g = lane >> 4;
    if (wr * IDX_BLOCK >= n) return;

    // A operands: Q[r][16 hb + j][32 s + 8 g .. +8] for head blocks hb = 0, 1.
    const uint16_t* qr = q + (int64_t)r * (32 * 128);
    bf16x8 qa[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; hb++)
#pragma unroll
        for (int s = 0; s < 4; s++) qa[hb][s] = load_bf16x8(qr + (hb * 16 + j) * 128 + 32 * s + 8 * g);
    // Head weights of the output rows this lane holds: heads 4g+v and 16+4g+v,
    // with the positive index scale folded in (ReLU(s x) = s ReLU(x), s > 0).
    float w0[4], w1[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        w0[v] = w[r * 32 + 4 * g + v] * scale;
        w1[v] = w[r * 32 + 16 + 4 * g + v] * scale;
    }

    const uint16_t* kb = PAGED ? kc : kc + base[r] * 128;
    const int32_t* btr = PAGED ? pm.block_table + base[r] * pm.max_blocks : nullptr;
    float* srow = scores + (int64_t)r * ld;

    bf16x8 kv[IDX_GROUPS][4];
    // Paged: pool block of each 16-position group of a 64-position block
    // (wave-uniform; a group never straddles two blocks, and clamped lanes
    // stay in their group's block).  Looked up one block-step ahead of the
    // key loads that use it, so those loads do not wait on the table.
    int pbn[IDX_GROUPS] = {}, pbnn[IDX_GROUPS] = {};
    auto lookup = [&](int p0, int (&dst)[IDX_GROUPS]) {
        if constexpr (PAGED) {
#pragma unroll
            for (int u = 0; u < IDX_GROUPS; u++) dst[u] = btr[min(p0 + 16 * u, n - 1) >> pm.log2_block];
        }
    };
    auto load = [&](int p0, int u, const int (&pb)[IDX_GROUPS]) {
        // Reads past the row's visible range are clamped onto its last
        // position; their results are never stored.
        const int pc = min(p0 + 16 * u + j, n - 1);
        int64_t prow = pc;
        if constexpr (PAGED) prow = ((int64_t)pb[u] << pm.log2_block) | (pc & ((1 << pm.log2_block) - 1));
        const uint16_t* kp = kb + prow * 128 + 8 * g;
#pragma unroll
        for (int s = 0; s < 4; s++) kv[u][s] = load_bf16x8(kp + 32 * s);
    };

    lookup(wr * IDX_BLOCK, pbn);
#pragma unroll
    for (int u = 0; u < IDX_GROUPS; u++) load(wr * IDX_BLOCK, u, pbn);
    lookup((wr + nw) * IDX_BLOCK, pbn);
    for (int b = wr; b * IDX_BLOCK < n; b += nw) {
        const int p0 = b * IDX_BLOCK;
        const bool more = (b + nw) * IDX_BLOCK < n;  // wave-uniform
        if (PAGED && (b + 2 * nw) * IDX_BLOCK < n) lookup((b + 2 * nw) * IDX_BLOCK, pbnn);
        float part[IDX_GROUPS];
#pragma unroll
        for (int u = 0; u < IDX_GROUPS; u++) {
            floatx4 a0 = {0.f, 0.f, 0.f, 0.f};
            floatx4 a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s++) {
                a0 = mfma_16x16x32(qa[0][s], kv[u][s], a0);
                a1 = mfma_16x16x32(qa[1][s], kv[u][s], a1);
            }
            // The group's registers are free once its MFMAs have issued: the
            // next block's group goes out now, not after the whole block.
            if (more) load((b + nw) * IDX_BLOCK, u, pbn);
            float acc = 0.f;
#pragma unroll
            for (int v = 0; v < 4; v++) acc += w0[v] * relu_bits(a0[v]);
#pragma unroll
            for (int v = 0; v < 4; v++) acc += w1[v] * relu_bits(a1[v]);
            part[u] = acc;  // this lane's 8 heads
        }
        // Lane group g takes group u == g, summed over all 32 heads: 64
        // consecutive scores per store.
        const float mine = xrow_reduce_scatter4(part);
        const int pos = p0 + 16 * g + j;
        // Scores go out as non-temporal stores: they are read once, by the
        // next kernel, and dirty lines left in L2 cost the kernel-end write-back.
        if (pos < n) __builtin_nontemporal_store(mine, &srow[pos]);
        if constexpr (PAGED) {
#pragma unroll
            for (int u = 0; u < IDX_GROUPS; u++) pbn[u] = pbnn[u];
        }
    }
}

// Grid: (workgroups per row, rows as items): item r scores row r.  With
// rowlist set, grid row y walks list entries y, y + gridDim.y, ... instead
// (the rows no shared block owns; see indexer_list_kernel).
template <bool PAGED>
__global__ __launch_bounds__(256) void indexer_rows_kernel(
    const int32_t* __restrict__ vis, const int64_t* __restrict__ base, const uint16_t* __restrict__ q,
    const float* __restrict__ w, const uint16_t* __restrict__ kc, float scale, float* __restrict__ scores,
    int64_t ld, int num_rows, int skip_shared, PagedCache pm, const int32_t* __restrict__ rowlist,
    const uint32_t* __restrict__ nlist)
{
    const int wr = blockIdx.x * IDX_WAVES + (threadIdx.x >> 6);
    const int nw = gridDim.x * IDX_WAVES;
    if (!rowlist) {
        const int r = grid_item();
        if (r >= num_rows) return;
        if (skip_shared && block_is_shared(base, num_rows, r / IDX_TILE_ROWS)) return;  // the tile kernel owns it
        indexer_row<PAGED>(r, wr, nw, vis, base, q, w, kc, scale, scores, ld, pm);
        return;
    }
    const uint32_t cnt = *nlist;
    for (uint32_t li = blockIdx.y; li < cnt; li += gridDim.y)
        indexer_row<PAGED>(rowlist[li], wr, nw, vis, base, q, w, kc, scale, scores, ld, pm);
}

// One workgroup: lists, in row order, the rows that no shared 32-row block
// owns (the rows the row kernel scores), so that a batch mixing a long
// prefill chunk with decode rows can give those rows many workgroups each
// instead of the one per row a grid over all rows affords.
constexpr int IL_THREADS = 1024;
constexpr int IL_GRID = 64;  // grid rows of the row kernel in list mode
__global__ __launch_bounds__(IL_THREADS) void indexer_list_kernel(const int64_t* __restrict__ base, int num_rows,
                                                                  int32_t* __restrict__ rowlist,
                                                                  uint32_t* __restrict__ nlist)
{
    __shared__ uint32_t sh[IL_THREADS / 64];
    const int nb = (num_rows + IDX_TILE_ROWS - 1) / IDX_TILE_ROWS;
    const int per = (nb + IL_THREADS - 1) / IL_THREADS;
    const int b0 = threadIdx.x * per, b1 = min(nb, b0 + per);
    auto listed = [&](int b) {  // rows of block b the row kernel owns
        const int r0 = b * IDX_TILE_ROWS;
        const int rn = min(IDX_TILE_ROWS, num_rows - r0);
        if (rn < IDX_TILE_ROWS) return rn;  // a partial block is never shared
        // Every load issued before any compare: one memory round trip.
        int64_t v[IDX_TILE_ROWS];
#pragma unroll
        for (int i = 0; i < IDX_TILE_ROWS; i++) v[i] = base[r0 + i];
        bool same = true;
#pragma unroll
        for (int i = 1; i < IDX_TILE_ROWS; i++) same &= v[i] == v[0];
        return same ? 0 : IDX_TILE_ROWS;
    };
    // The first 32 blocks' verdicts are kept for the second pass.
    uint32_t cnt = 0, owned = 0;
    for (int b = b0; b < b1; b++) {
        const int nr = listed(b);
        if (b - b0 < 32 && nr > 0) owned |= 1u << (b - b0);
        cnt += (uint32_t)nr;
    }
    // Exclusive scan of the per-thread counts.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_inclusive_scan(cnt);
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
    for (int i = 0; i < IL_THREADS / 64; i++) {
        before += i < wave ? sh[i] : 0u;
        total += sh[i];
    }
    uint32_t slot = before + incl - cnt;
    for (int b = b0; b < b1; b++) {
        const int nr = b - b0 < 32 ? ((owned >> (b - b0)) & 1u ? min(IDX_TILE_ROWS, num_rows - b * IDX_TILE_ROWS) : 0)
                                   : listed(b);
        for (int i = 0; i < nr; i++) rowlist[slot++] = b * IDX_TILE_ROWS + i;
    }
    if (threadIdx.x == 0) *nlist = total;
}

}  // namespace

int indexer_pick_chunk(int32_t num_rows, int32_t max_visible)
{
    // Workgroups per row: about 8192 in total, but at least two 64-position
    // blocks of the longest row per wave (measured on 64 x 32,768 and
    // 16 x 202,752 decode: 94 and 143 us, against 94-102 and 149 us with 4096
    // workgroups and 96 and 145 us with one block per wave).
    const int64_t blocks = (max_visible + IDX_BLOCK - 1) / IDX_BLOCK;
    int64_t cx = (8192 + num_rows - 1) / num_rows;
    const int64_t cap = (blocks + 2 * IDX_WAVES - 1) / (2 * IDX_WAVES);
    if (cx > cap) cx = cap;
    if (cx < 1) cx = 1;
    return (int)cx;
}

void launch_indexer_scores(int32_t num_rows, int32_t max_visible, const int32_t* vis, const int64_t* base,
                           const uint16_t* q, const float* w, const uint16_t* kc, float scale, float* scores,
                           int64_t ld, bool distinct_sequences, const PagedCache& paged, hipStream_t stream,
                           void* list_ws)
{
    const bool pg = paged.block_table != nullptr;
    const int nblk = distinct_sequences ? 0 : num_rows / IDX_TILE_ROWS;
    if (nblk > 0) {
        // Workgroups per shared block: enough for ~2 per CU overall (up to
        // 32 per block, for calls with few blocks), never more than the
        // block's key tiles.
        const int tiles = (max_visible + IDX_TILE_POS - 1) / IDX_TILE_POS;
        int cx = (512 + nblk - 1) / nblk;
        if (cx > 32) cx = 32;
        if (cx > tiles) cx = tiles;
        if (cx < 1) cx = 1;
        if (pg)
            hipLaunchKernelGGL(indexer_tile_kernel<true>, item_grid(cx, nblk), dim3(512), 0, stream, vis, base, q, w, kc,
                               scale, scores, ld, num_rows, paged);
        else
            hipLaunchKernelGGL(indexer_tile_kernel<false>, item_grid(cx, nblk), dim3(512), 0, stream, vis, base, q, w, kc,
                               scale, scores, ld, num_rows, paged);
    }
    int32_t* rowlist = nullptr;
    uint32_t* nlist = nullptr;
    dim3 grid = item_grid(indexer_pick_chunk(num_rows, max_visible), num_rows);
    if (nblk > 0 && list_ws) {
        // Rows that may share blocks: list the others and give each of them
        // the workgroups of a batch of at most IL_GRID rows.
        rowlist = reinterpret_cast<int32_t*>(list_ws);
        nlist = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(list_ws) + indexer_list_offset(num_rows));
        hipLaunchKernelGGL(indexer_list_kernel, dim3(1), dim3(IL_THREADS), 0, stream, base, (int)num_rows, rowlist,
                           nlist);
        const int G = num_rows < IL_GRID ? num_rows : IL_GRID;
        grid = dim3(indexer_pick_chunk(G, max_visible), G);
    }
    if (pg)
        hipLaunchKernelGGL(indexer_rows_kernel<true>, grid, dim3(256), 0, stream, vis, base, q, w, kc, scale, scores,
                           ld, num_rows, nblk > 0 ? 1 : 0, paged, rowlist, nlist);
    else
        hipLaunchKernelGGL(indexer_rows_kernel<false>, grid, dim3(256), 0, stream, vis, base, q, w, kc, scale, scores,
                           ld, num_rows, nblk > 0 ? 1 : 0, paged, rowlist, nlist);
}

size_t indexer_list_offset(int32_t num_rows) { return align_up((size_t)num_rows * 4, 256); }
size_t indexer_list_bytes(int32_t num_rows) { return indexer_list_offset(num_rows) + 256; }

}  // namespace dsa
