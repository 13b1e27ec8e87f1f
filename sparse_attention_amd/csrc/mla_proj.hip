// mla_proj.hip -- the two per-head projections on either side of the
// absorbed sparse attention, on gfx950 matrix cores.
//
// kv_b_proj expands the 512-d latent into 64 heads x (192 non-RoPE key dims +
// 256 value dims) ("GLM-5.1 架构深度拆解" CH4 §4.1; §4.5 step 2 splits each
// head's 448 output rows as [k_nope || value]).  Being linear, it can move
// off the cache side:
//  - query absorption: q_abs[r,h] = [W_UK,h^T q_nope[r,h] (512) || q_pe[r,h] (64)],
//    W_UK,h = head h's first 192 rows, so that q_abs . [c_kv || k_pe] equals
//    the expanded q_nope . k_nope + q_pe . k_pe;
//  - V up-projection: out[r,h] = W_UV,h o[r,h], W_UV,h = head h's last 256
//    rows, applied once to the attention's 512-wide latent output instead of
//    to every selected value row.
// Both are per-head GEMMs, C_h[R x N] = A_h[R x K] B_h[K x N], run on
// v_mfma_f32_16x16x32_bf16 (fp32 accumulate):
//   absorption:     A = q_nope (K = 192), B = W_UK,h (N = 512 latent columns)
//   up-projection:  A = bf16(o) (K = 512), B = W_UV,h^T (N = 256 value dims)
// A workgroup (4 waves) owns one head and one 64-column tile of N, stages that
// tile of the weight in LDS once, and walks the 64-row tiles of R (wave w:
// rows 16w..16w+15, all four 16-column blocks).  At decode batch sizes the
// weights (12.6 + 16.8 MB) are the traffic; at prefill sizes the MFMAs.
//  - W_UK rows are 512 latent values each, so its K (= row) direction is
//    strided; the staged tile is read with transposing LDS reads
//    (ds_read_b64_tr_b16), which deliver 4 consecutive rows of one column per
//    lane, so two reads give the 8 consecutive K values of a B operand.
//  - W_UV rows are already K-contiguous: plain 16-byte LDS reads.
//  - o arrives as fp32 and is rounded to bf16 (round-to-nearest-even) as it
//    is loaded, the precision of the MFMA operand.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int PJ_NOPE = 192;   // qk_nope_head_dim
constexpr int PJ_VDIM = 256;   // v_head_dim
constexpr int PJ_LAT = 512;    // kv_lora_rank
constexpr int PJ_ROPE = 64;    // qk_rope_head_dim
constexpr int PJ_ROW = PJ_LAT + PJ_ROPE;
constexpr int PJ_KVB = PJ_NOPE + PJ_VDIM;  // kv_b_proj rows per head
constexpr int PJ_TM = 64;      // rows of R per tile
constexpr int VU_PITCH = 1040; // bytes per staged W_UV row (512 bf16 + 16)
// Columns of N per workgroup (TN, a template parameter): 64 for small R (the
// weights are the traffic: more workgroups stream them); for the absorption at
// large R 256 (each A row tile is re-read from L2 by every column tile of its
// head, so fewer, wider column tiles cut that traffic: 8192 rows in 306
// instead of ~395 us).
constexpr int PJ_WIDE_ROWS = 512;  // R above this takes the wide absorption tiles

__device__ __forceinline__ uint16_t to_bf16(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);  // round-to-nearest-even
}

// Workgroup -> (column tile, head, row group).  Workgroups are handed to the
// 8 XCDs round-robin, and the NT column tiles of one (head, row group) read
// the same A rows: numbering them 8 apart puts them on one XCD, where its L2
// serves A to all of them (only locality depends on this, not correctness).
struct ProjTile {
    int nt, h, grp;
};
template <int NT>
__device__ __forceinline__ ProjTile proj_tile()
{
    const int L = blockIdx.x;
    const int c = L & 7, b = (L >> 3) % NT, a = L / (8 * NT);
    const int p = 8 * a + c;  // (head, row group) pair
    return ProjTile{b, p & 63, p >> 6};
}

template <int TN>
__global__ __launch_bounds__(256) void absorb_kernel(int R, const uint16_t* __restrict__ qn,
                                                     const uint16_t* __restrict__ qp,
                                                     const uint16_t* __restrict__ kvb, uint16_t* __restrict__ qa)
{
    constexpr int ABP = 2 * TN + 32;  // bytes per staged W_UK row (TN bf16 + 32: spreads the rows a read touches)
    constexpr int CPR = TN / 8;       // 16-byte chunks per staged row
    constexpr int NB = TN / 16;       // 16-column blocks per wave
    const ProjTile tile = proj_tile<PJ_LAT / TN>();
    const int nt = tile.nt, h = tile.h, grp = tile.grp, ngrp = gridDim.x / (64 * (PJ_LAT / TN));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 15, g = lane >> 4;
    __shared__ __attribute__((aligned(16))) uint8_t wt[PJ_NOPE * ABP];
    __shared__ __attribute__((aligned(16))) uint16_t ct[4][16][TN + 8];  // output staging, per wave
    constexpr int KS = PJ_NOPE / 32;  // k-steps

    // A operand of row tile mt: lane (j, g) holds q_nope[row][32 s + 8 g .. +8]
    // (rows clamped inside R; their results are not stored).
    auto load_a = [&](int mt, bf16x8 (&a)[KS]) {
        const int ra = min(mt * PJ_TM + 16 * wave + j, R - 1);
        const uint16_t* arow = qn + ((int64_t)ra * 64 + h) * PJ_NOPE + 8 * g;
#pragma unroll
        for (int s = 0; s < KS; s++) a[s] = load_bf16x8(arow + 32 * s);
    };

    // Every global load of the prologue goes out before the one barrier:
    // W_UK,h[0:192][TN nt .. +TN] (192 rows x CPR chunks of 16 bytes) and the
    // first row tile's A operand.
    const uint16_t* W = kvb + (int64_t)h * PJ_KVB * PJ_LAT + TN * nt;
    constexpr int WPT = PJ_NOPE * CPR / 256;  // chunks per thread
    u32x4 wreg[WPT];
#pragma unroll
    for (int i = 0; i < WPT; i++) {
        const int c = threadIdx.x + 256 * i;
        wreg[i] = load_u32x4(W + (int64_t)(c / CPR) * PJ_LAT + 8 * (c % CPR));
    }
    const int mtiles = (R + PJ_TM - 1) / PJ_TM;
    bf16x8 a[KS];
    load_a(grp, a);
#pragma unroll
    for (int i = 0; i < WPT; i++) {
        const int c = threadIdx.x + 256 * i;
        *reinterpret_cast<u32x4*>(wt + (c / CPR) * ABP + 16 * (c % CPR)) = wreg[i];
    }
    __syncthreads();

    for (int mt = grp; mt < mtiles; mt += ngrp) {
        // The next row tile's A goes out before this tile's MFMAs.
        const bool more = mt + ngrp < mtiles;  // uniform
        bf16x8 an[KS];
        if (more) load_a(mt + ngrp, an);
        floatx4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; nb++) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; s++) {
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                // Lane (j, g): rows 32 s + 8 g + (j >> 2) (+4), columns
                // 16 nb + 4 (j & 3) .. +3; it receives column 16 nb + j of
                // rows 32 s + 8 g .. +7, the same K order as its A operand.
                const uint8_t* lo = wt + (32 * s + 8 * g + (j >> 2)) * ABP + 2 * (16 * nb + 4 * (j & 3));
                const bf16x8 b = lds_read_tr_pair((const uint16_t*)lo, (const uint16_t*)(lo + 4 * ABP));
                acc[nb] = mfma_16x16x32(a[s], b, acc[nb]);
            }
        }
        // Lane (j, g) holds C[16 wave + 4 g + v][16 nb + j]; the wave's 16 rows
        // go through its own staging rows (only this wave touches them, and
        // LDS keeps one wave's accesses in order) and leave as 16-byte stores.
#pragma unroll
        for (int v = 0; v < 4; v++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++) ct[wave][4 * g + v][16 * nb + j] = to_bf16(acc[nb][v]);
#pragma unroll
        for (int i = 0; i < 16 * CPR / 64; i++) {
            const int q = 64 * i + lane, rr = q / CPR, ch = q % CPR;  // row of the wave's 16, 16-byte chunk
            const int r = mt * PJ_TM + 16 * wave + rr;
            const u32x4 val = *reinterpret_cast<const u32x4*>(&ct[wave][rr][8 * ch]);
            // Non-temporal: the output is not re-read here, and dirty L2 lines
            // cost the kernel-end write-back.
            if (r < R)
                __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(qa + ((int64_t)r * 64 + h) * PJ_ROW +
                                                                          TN * nt + 8 * ch));
        }
        if (nt == 0) {
            // q_pe passes through: 64 rows x 8 chunks of 16 bytes.
            for (int i = threadIdx.x; i < PJ_TM * 8; i += 256) {
                const int r = mt * PJ_TM + (i >> 3), ch = i & 7;
                if (r < R)
                    *reinterpret_cast<u32x4*>(qa + ((int64_t)r * 64 + h) * PJ_ROW + PJ_LAT + 8 * ch) =
                        load_u32x4(qp + ((int64_t)r * 64 + h) * PJ_ROPE + 8 * ch);
            }
        }
        if (more) {
#pragma unroll
            for (int s = 0; s < KS; s++) a[s] = an[s];
        }
    }
}

template <int TN>
__global__ __launch_bounds__(256) void vup_kernel(int R, const float* __restrict__ o,
                                                  const uint16_t* __restrict__ kvb, float* __restrict__ out)
{
    constexpr int NB = TN / 16;  // 16-column blocks per wave
    const ProjTile tile = proj_tile<PJ_VDIM / TN>();
    const int nt = tile.nt, h = tile.h, grp = tile.grp, ngrp = gridDim.x / (64 * (PJ_VDIM / TN));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 15, g = lane >> 4;
    __shared__ __attribute__((aligned(16))) uint8_t wt[TN * VU_PITCH];
    constexpr int KS = PJ_LAT / 32;  // k-steps

    // A operand of row tile mt, rounded to bf16 as it arrives: lane (j, g)
    // holds bf16(o[row][32 s + 8 g .. +8]).
    auto load_a = [&](int mt, bf16x8 (&a)[KS]) {
        const int ra = min(mt * PJ_TM + 16 * wave + j, R - 1);
        const float* arow = o + ((int64_t)ra * 64 + h) * PJ_LAT + 8 * g;
        float4 x[2 * KS];
#pragma unroll
        for (int s = 0; s < KS; s++) {
            x[2 * s] = *reinterpret_cast<const float4*>(arow + 32 * s);
            x[2 * s + 1] = *reinterpret_cast<const float4*>(arow + 32 * s + 4);
        }
#pragma unroll
        for (int s = 0; s < KS; s++) {
            const float4 x0 = x[2 * s], x1 = x[2 * s + 1];
            a[s] = bf16x8{(__bf16)x0.x, (__bf16)x0.y, (__bf16)x0.z, (__bf16)x0.w,
                          (__bf16)x1.x, (__bf16)x1.y, (__bf16)x1.z, (__bf16)x1.w};
        }
    };

    // Prologue: W_UV,h rows TN nt .. +TN (all 512 columns, 64 chunks of 16
    // bytes per row) into LDS, 64 rows per pass so that at most 64 KB are
    // held in registers, then the first row tile.
    const uint16_t* W = kvb + ((int64_t)h * PJ_KVB + PJ_NOPE + TN * nt) * PJ_LAT;
    const int mtiles = (R + PJ_TM - 1) / PJ_TM;
    bf16x8 a[KS];
#pragma unroll
    for (int half = 0; half < TN / 64; half++) {
        u32x4 wreg[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int c = 4096 * half + threadIdx.x + 256 * i;
            wreg[i] = load_u32x4(W + (int64_t)(c >> 6) * PJ_LAT + 8 * (c & 63));
        }
        if (half == TN / 64 - 1) load_a(grp, a);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int c = 4096 * half + threadIdx.x + 256 * i;
            *reinterpret_cast<u32x4*>(wt + (c >> 6) * VU_PITCH + 16 * (c & 63)) = wreg[i];
        }
    }
    __syncthreads();

    for (int mt = grp; mt < mtiles; mt += ngrp) {
        const bool more = mt + ngrp < mtiles;  // uniform
        floatx4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; nb++) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; s++) {
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                // Lane (j, g): value dim 16 nb + j, latent columns 32 s + 8 g .. +7.
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(wt + (16 * nb + j) * VU_PITCH + 2 * (32 * s + 8 * g)));
                acc[nb] = mfma_16x16x32(a[s], b, acc[nb]);
            }
        }
        // The next row tile's A goes out once this tile's MFMAs have read theirs.
        if (more) load_a(mt + ngrp, a);
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int r = mt * PJ_TM + 16 * wave + 4 * g + v;
            if (r < R) {
                float* orow = out + ((int64_t)r * 64 + h) * PJ_VDIM + TN * nt + j;
#pragma unroll
                for (int nb = 0; nb < NB; nb++) __builtin_nontemporal_store(acc[nb][v], &orow[16 * nb]);  // not re-read
            }
        }
    }
}

// Row-tile groups per (column tile, head): about 2048 workgroups in all, each
// walking the row tiles of its group (its weight tile is staged once).
int proj_row_groups(int32_t num_rows, int col_tiles)
{
    const int mtiles = (num_rows + PJ_TM - 1) / PJ_TM;
    int groups = 2048 / (col_tiles * 64);
    if (groups < 1) groups = 1;
    return mtiles < groups ? mtiles : groups;
}

}  // namespace

void launch_absorb_queries(int32_t num_rows, const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* kvb,
                           uint16_t* q_abs, hipStream_t stream)
{
    if (num_rows > PJ_WIDE_ROWS) {
        constexpr int ct = PJ_LAT / 256;
        hipLaunchKernelGGL(absorb_kernel<256>, dim3(ct * 64 * proj_row_groups(num_rows, ct)), dim3(256), 0, stream,
                           num_rows, q_nope, q_pe, kvb, q_abs);
    } else {
        constexpr int ct = PJ_LAT / 64;
        hipLaunchKernelGGL(absorb_kernel<64>, dim3(ct * 64 * proj_row_groups(num_rows, ct)), dim3(256), 0, stream,
                           num_rows, q_nope, q_pe, kvb, q_abs);
    }
}

void launch_v_up_proj(int32_t num_rows, const float* o, const uint16_t* kvb, float* out, hipStream_t stream)
{
    // 64-column tiles at every size: with 128 the fp32 A prefetch, its bf16
    // operands and the accumulators exceed the register file (measured at
    // 8192 rows: 1211 us with spills, against 530 us).
    constexpr int ct = PJ_VDIM / 64;
    hipLaunchKernelGGL(vup_kernel<64>, dim3(ct * 64 * proj_row_groups(num_rows, ct)), dim3(256), 0, stream,
                       num_rows, o, kvb, out);
}

}  // namespace dsa
