// sparse_mla.hip -- absorbed-MLA attention over selected positions on gfx950.
//
// For each query row r and head h, over the selected positions idx_j >= 0:
//   z[h,j]   = softmax_scale * q_abs[r,h,:] . L[base_r + idx_j, 0:576]
//   out[r,h] = sum_j softmax(z[h,:])_j * L[base_r + idx_j, 0:512]
//   lse[r,h] = log sum_j exp(z[h,j])
// ("GLM-5.1 架构深度拆解" §4.5 steps 2, 6 and 7; GLM-5 explainer: the
// selected IDs only drive the gather of 512 latent + 64 RoPE values per
// position, and the 64 MLA heads attend inside the selected set; the query is
// in absorbed form so one 576-wide latent row serves every head).
//
// Design:
//  - One workgroup = one row x one contiguous split of its index list; 4 waves,
//    wave w owns heads 16w..16w+15 (the MFMA M dimension) for the whole split.
//  - Per tile of 32 selected positions the workgroup gathers the 32 latent
//    rows (1152 B each) into LDS with 16-byte loads, one wave-instruction
//    covering 1 KB of one row.  The row pitch is padded to 1168 B so the MFMA
//    operand reads do not collide in LDS banks.
//  - QK: v_mfma_f32_16x16x32_bf16 with the wave's absorbed queries as the A
//    operand (kept in registers, 72 VGPRs) and latent rows as B (one 16-byte
//    LDS read per lane and k-step).
//  - Online softmax in fp32 (base-2 exponent), head statistics reduced across
//    the 16 lanes of a head with xor-shuffles.
//  - PV: O[16 heads x 512] += P[16 x 32] . V[32 x 512].  P goes through a small
//    per-wave LDS buffer (bf16, round-to-nearest-even) and both operands are
//    read with ds_read_tr16_b64, which delivers the k = position direction
//    from row-major tiles.  O lives in 128 accumulation registers.
//  - Splits write unnormalized partials (O, running max, running sum); a
//    combine kernel merges them in split order, so results do not depend on
//    scheduling.  A single split normalizes in place.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int AT_TILE = 32;        // selected positions per tile
constexpr int AT_CHUNKS = 72;      // 16-byte chunks per latent row
constexpr int AT_TILE_BYTES = AT_TILE * AT_CHUNKS * 16;  // 36,864
constexpr int AT_STAGES = 4;       // tiles in flight per workgroup
constexpr int AT_MAX_SPLIT = 2048; // largest split (slots)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_LOG2 = 8.f;  // lazy-rescale threshold (log2 units)
constexpr float LN2 = 0.6931471805599453f;

// Tile layout: 32 rows x 72 16-byte chunks, dense (1152 B per row, the
// direct global->LDS loads write 64 consecutive chunks per instruction).
// Logical chunk c of row r sits at chunk c ^ swz(r), swz(r) = (r bit 2, r bit
// 1, r bit 3) in bits (0, 1, 2).  With the row parity that the 1152-byte pitch
// already spreads over the two 128-byte halves of a 256-byte bank window:
//  - QK operand reads (rows 0..15, one logical chunk) hit 16 distinct 16-byte
//    slots;
//  - transposing PV reads (rows 8g+4h+{0..3}, two adjacent chunks, 8-byte
//    halves) hit 16 distinct 8-byte slots;
// and both read sets stay affine in the unrolled loop index, so the compiler
// folds them into a few base registers plus immediate offsets.
__device__ __forceinline__ int swz(int row)
{
    return ((row >> 2) & 1) | (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
}
__device__ __forceinline__ int tile_chunk_offset(int row, int chunk)
{
    return row * (AT_CHUNKS * 16) + 16 * (chunk ^ swz(row));
}

// s_waitcnt immediates (gfx9 encoding): vmcnt in bits [3:0] and [15:14],
// expcnt [6:4] and lgkmcnt [11:8] left at their "no wait" maxima.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__global__ __launch_bounds__(256, 1) void sparse_mla_kernel(const int64_t* __restrict__ base,
                                                           const uint16_t* __restrict__ qa,
                                                           const uint16_t* __restrict__ kv,
                                                           const int32_t* __restrict__ idx, int k,
                                                           float scale_log2, int split_len,
                                                           float* __restrict__ out, float* __restrict__ lse,
                                                           float* __restrict__ part_o,
                                                           float2* __restrict__ part_ml)
{
    const int r = blockIdx.y;
    const int sp = blockIdx.x;
    const int nsplit = gridDim.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int tc = lane & 3;         // transposed-read roles inside a 16-lane group
    const int tk = (lane >> 2) & 3;
    const int h0 = wave * 16;

    const int slot_begin = sp * split_len;
    const int slot_end = min(k, slot_begin + split_len);
    const int nslots = slot_end - slot_begin;
    const int ntiles = (nslots + AT_TILE - 1) / AT_TILE;

    // AT_STAGES tiles of 32 latent rows, filled by direct global->LDS loads.
    __shared__ __attribute__((aligned(1024))) uint8_t ring[AT_STAGES][AT_TILE_BYTES];
    __shared__ __attribute__((aligned(16))) uint16_t plds[4][AT_TILE * 16];
    __shared__ int32_t sidx[AT_MAX_SPLIT + AT_TILE];

    // The split's index list, padded with -1 to a whole number of tiles.
    const int32_t* irow = idx + (int64_t)r * k + slot_begin;
    for (int i = threadIdx.x; i < split_len + AT_TILE; i += 256) sidx[i] = i < nslots ? irow[i] : -1;

    bf16x8 qreg[18];
    {
        const uint16_t* qrow = qa + ((int64_t)r * 64 + h0 + j) * 576 + 8 * g;
#pragma unroll
        for (int s = 0; s < 18; s++) qreg[s] = load_bf16x8(qrow + 32 * s);
    }
    const uint16_t* kvrow = kv + base[r] * 576;
    __syncthreads();  // sidx visible; nothing asynchronous is in flight yet

    // Gather roles.  Wave w fills tile chunks [576 w, 576 w + 576): its i-th
    // load instruction writes 64 consecutive 16-byte LDS chunks (lane order),
    // and lane L fetches whichever logical chunk belongs at LDS chunk
    // 576 w + 64 i + L under the swizzle.  Padding slots fetch the sequence's
    // first latent row (always present); their softmax weight is zero.
    auto issue = [&](int t) {
        uint8_t* dst = ring[t % AT_STAGES] + wave * 9 * 1024;
        const int t0 = t * AT_TILE;
#pragma unroll
        for (int i = 0; i < 9; i++) {
            const int p = (wave * 9 + i) * 64 + lane;
            const int row = p / AT_CHUNKS;
            const int part = (p - row * AT_CHUNKS) ^ swz(row);
            const int id = sidx[t0 + row];
            const uint16_t* src = kvrow + (int64_t)(id < 0 ? 0 : id) * 576 + part * 8;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                             (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
        }
    };

    float m_run[4], l_run[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        m_run[v] = -INFINITY;
        l_run[v] = 0.f;
    }
    floatx4 o[32];
#pragma unroll
    for (int cb = 0; cb < 32; cb++) o[cb] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int t = 0; t < AT_STAGES - 1; t++)
        if (t < ntiles) issue(t);

    for (int t = 0; t < ntiles; t++) {
        // Keep AT_STAGES - 1 tiles in flight; wait only for tile t's loads.
        // Raw s_barrier (no fence) so outstanding loads of later tiles are not
        // drained; the data dependence is carried by the explicit vmcnt wait.
        if (t + AT_STAGES - 1 < ntiles) {
            issue(t + AT_STAGES - 1);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(9 * (AT_STAGES - 1)));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        __builtin_amdgcn_s_barrier();
        const uint8_t* tl = ring[t % AT_STAGES];
        const int t0 = t * AT_TILE;
        const bool ok0 = sidx[t0 + j] >= 0;
        const bool ok1 = sidx[t0 + 16 + j] >= 0;

        // QK: s0 -> positions 0..15 of the tile, s1 -> 16..31.  Logical chunk
        // 4s + g = 8 (s >> 1) + (4 (s & 1) + g): two per-lane bases per row,
        // the rest is an immediate 128 (s >> 1).
        floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        {
            const uint8_t* q0e0 = tl + tile_chunk_offset(j, g);
            const uint8_t* q0e1 = tl + tile_chunk_offset(j, 4 + g);
            const uint8_t* q1e0 = tl + tile_chunk_offset(16 + j, g);
            const uint8_t* q1e1 = tl + tile_chunk_offset(16 + j, 4 + g);
            // Operand reads run QK_AHEAD steps ahead of the MFMAs that use
            // them; scheduling barriers keep the compiler from collapsing the
            // pipeline (LDS reads return in order, so the waits stay partial).
            constexpr int QK_AHEAD = 3;
            bf16x8 b0[18], b1[18];
            auto rd = [&](int st) {
                const int off = 128 * (st >> 1);
                b0[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(((st & 1) ? q0e1 : q0e0) + off));
                b1[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(((st & 1) ? q1e1 : q1e0) + off));
            };
#pragma unroll
            for (int st = 0; st < QK_AHEAD; st++) rd(st);
#pragma unroll
            for (int st = 0; st < 18; st++) {
                if (st + QK_AHEAD < 18) rd(st + QK_AHEAD);
                s0 = mfma_16x16x32(qreg[st], b0[st], s0);
                s1 = mfma_16x16x32(qreg[st], b1[st], s1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // Online softmax.  Lane (j, g) holds heads h0 + 4g + v at positions j, 16 + j.
        // The reference maximum m_run of a head moves only when the tile's
        // maximum exceeds it by more than 2^RESCALE_LOG2; weights are then at
        // most 2^RESCALE_LOG2, far from fp32 or bf16 overflow, and the result
        // o / l and lse = m_run + log2 l do not depend on which reference is
        // used.  In steady state no tile rescales the 128 O accumulators.
        float p0[4], p1[4], z0[4], z1[4], mt[4];
        bool need = false;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            z0[v] = ok0 ? s0[v] * scale_log2 : -INFINITY;
            z1[v] = ok1 ? s1[v] * scale_log2 : -INFINITY;
            mt[v] = wave_max_16(fmaxf(z0[v], z1[v]));
            need |= mt[v] > m_run[v] + RESCALE_LOG2;
        }
        if (__builtin_amdgcn_read_exec() & __ballot(need)) {  // wave-uniform
            float alpha[4];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float m_new = fmaxf(m_run[v], mt[v]);
                alpha[v] = (m_run[v] == -INFINITY) ? 0.f : exp2f(m_run[v] - m_new);
                l_run[v] *= alpha[v];
                m_run[v] = m_new;
            }
#pragma unroll
            for (int cb = 0; cb < 32; cb++)
#pragma unroll
                for (int v = 0; v < 4; v++) o[cb][v] *= alpha[v];
        }
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const bool live = m_run[v] != -INFINITY;
            p0[v] = (ok0 && live) ? exp2f(z0[v] - m_run[v]) : 0.f;
            p1[v] = (ok1 && live) ? exp2f(z1[v] - m_run[v]) : 0.f;
            l_run[v] += wave_sum_16(p0[v] + p1[v]);
        }

        // P (bf16) into the wave's buffer, row = tile position, column = head.
        {
            uint16_t* pw = plds[wave];
            typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
            u16x4 a = {f32_to_bf16_rne(p0[0]), f32_to_bf16_rne(p0[1]), f32_to_bf16_rne(p0[2]),
                       f32_to_bf16_rne(p0[3])};
            u16x4 b = {f32_to_bf16_rne(p1[0]), f32_to_bf16_rne(p1[1]), f32_to_bf16_rne(p1[2]),
                       f32_to_bf16_rne(p1[3])};
            *reinterpret_cast<u16x4*>(&pw[j * 16 + 4 * g]) = a;
            *reinterpret_cast<u16x4*>(&pw[(16 + j) * 16 + 4 * g]) = b;
        }
        // The P buffer is private to the wave and one wave's LDS operations
        // complete in order, so only the compiler needs fencing here.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // A operand: lane (head j, group g) gets P at tile positions 8g .. 8g+7.
        const bf16x8 pa = lds_read_tr_pair(&plds[wave][(8 * g + tk) * 16 + 4 * tc],
                                           &plds[wave][(8 * g + 4 + tk) * 16 + 4 * tc]);
        // PV over 32 column blocks of 16; B lane (column j, group g) gets V at
        // the same positions 8g .. 8g+7: source lane (tc, tk) points at row
        // 8g + tk (+4), columns 16 cb + 4 tc .. +3, i.e. logical chunk
        // 2 cb + (tc >> 1), byte 8 (tc & 1) inside it.
        // Column block cb = 4m + e covers logical chunks 8m + 2e + (tc >> 1):
        // four per-lane bases per row, the rest is an immediate 128 m.
        const int rlo = 8 * g + tk, rhi = 8 * g + 4 + tk;
        const uint8_t* vlo[4];
        const uint8_t* vhi[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            vlo[e] = tl + tile_chunk_offset(rlo, 2 * e + (tc >> 1)) + 8 * (tc & 1);
            vhi[e] = tl + tile_chunk_offset(rhi, 2 * e + (tc >> 1)) + 8 * (tc & 1);
        }
        constexpr int PV_AHEAD = 4;
        bf16x8 vb[32];
        auto rdv = [&](int cb) {
            const int off = 128 * (cb >> 2);
            vb[cb] = lds_read_tr_pair((const uint16_t*)(vlo[cb & 3] + off), (const uint16_t*)(vhi[cb & 3] + off));
        };
#pragma unroll
        for (int cb = 0; cb < PV_AHEAD; cb++) rdv(cb);
#pragma unroll
        for (int cb = 0; cb < 32; cb++) {
            if (cb + PV_AHEAD < 32) rdv(cb + PV_AHEAD);
            o[cb] = mfma_16x16x32(pa, vb[cb], o[cb]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Every wave is done with this ring slot before it is refilled.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(63) & ~(15 << 8));  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
    }

    // Epilogue.  Lane (j, g) holds O[h0 + 4g + v][16 cb + j].
    if (nsplit == 1) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int h = h0 + 4 * g + v;
            const float inv = l_run[v] > 0.f ? 1.f / l_run[v] : 0.f;
            float* orow = out + ((int64_t)r * 64 + h) * 512;
#pragma unroll
            for (int cb = 0; cb < 32; cb++) orow[16 * cb + j] = o[cb][v] * inv;
            if (lse && j == 0)
                lse[(int64_t)r * 64 + h] = l_run[v] > 0.f ? (m_run[v] + log2f(l_run[v])) * LN2 : -INFINITY;
        }
    } else {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int h = h0 + 4 * g + v;
            float* prow = part_o + (((int64_t)r * nsplit + sp) * 64 + h) * 512;
#pragma unroll
            for (int cb = 0; cb < 32; cb++) prow[16 * cb + j] = o[cb][v];
            if (j == 0) part_ml[((int64_t)r * nsplit + sp) * 64 + h] = make_float2(m_run[v], l_run[v]);
        }
    }
}

// Merges split partials in split order: one workgroup per (head, row), each
// thread four latent columns.
__global__ __launch_bounds__(128) void sparse_mla_combine_kernel(const float* __restrict__ part_o,
                                                                const float2* __restrict__ part_ml, int nsplit,
                                                                float* __restrict__ out, float* __restrict__ lse)
{
    const int h = blockIdx.x;
    const int r = blockIdx.y;
    const float2* ml = part_ml + (int64_t)r * nsplit * 64 + h;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; s++) M = fmaxf(M, ml[(int64_t)s * 64].x);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < nsplit; s++) {
            const float2 e = ml[(int64_t)s * 64];
            const float f = exp2f(e.x - M);
            L += e.y * f;
            const float4 p = *reinterpret_cast<const float4*>(
                part_o + (((int64_t)r * nsplit + s) * 64 + h) * 512 + 4 * threadIdx.x);
            acc.x += p.x * f;
            acc.y += p.y * f;
            acc.z += p.z * f;
            acc.w += p.w * f;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float4 res = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    *reinterpret_cast<float4*>(out + ((int64_t)r * 64 + h) * 512 + 4 * threadIdx.x) = res;
    if (lse && threadIdx.x == 0) lse[(int64_t)r * 64 + h] = L > 0.f ? (M + log2f(L)) * LN2 : -INFINITY;
}

}  // namespace

int attn_pick_splits(int32_t num_rows, int32_t k)
{
    const int tiles = (k + AT_TILE - 1) / AT_TILE;
    // One 256-thread workgroup per CU (the kernel uses the whole register
    // file of its SIMDs): aim for 256 workgroups.
    int s = (int)((256 + num_rows - 1) / num_rows);
    if (s > 16) s = 16;
    if (s > tiles) s = tiles;
    if (s < 1) s = 1;
    // Equal whole-tile splits.
    const int per = (tiles + s - 1) / s;
    return (tiles + per - 1) / per;
}

size_t attn_workspace_bytes(int32_t num_rows, int32_t k)
{
    const int s = attn_pick_splits(num_rows, k);
    if (s == 1) return 0;
    const size_t R = (size_t)num_rows;
    return align_up(R * s * 64 * 512 * 4, 256) + align_up(R * s * 64 * 8, 256);
}

void launch_sparse_mla(int32_t num_rows, const int64_t* base, const uint16_t* qa, const uint16_t* kv,
                       const int32_t* idx, int32_t k, float softmax_scale, float* out, float* lse, void* ws,
                       hipStream_t stream)
{
    const int s = attn_pick_splits(num_rows, k);
    const int tiles = (k + AT_TILE - 1) / AT_TILE;
    const int split_len = ((tiles + s - 1) / s) * AT_TILE;
    float* part_o = nullptr;
    float2* part_ml = nullptr;
    if (s > 1) {
        part_o = (float*)ws;
        part_ml = (float2*)((char*)ws + align_up((size_t)num_rows * s * 64 * 512 * 4, 256));
    }
    hipLaunchKernelGGL(sparse_mla_kernel, dim3(s, num_rows), dim3(256), 0, stream, base, qa, kv, idx, k,
                       softmax_scale * LOG2E, split_len, out, lse, part_o, part_ml);
    if (s > 1)
        hipLaunchKernelGGL(sparse_mla_combine_kernel, dim3(64, num_rows), dim3(128), 0, stream, part_o, part_ml, s,
                           out, lse);
}

}  // namespace dsa
