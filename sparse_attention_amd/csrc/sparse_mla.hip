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
constexpr int AT_PITCH = 584;      // LDS row pitch in bf16 (576 + 8 pad)
constexpr int AT_CHUNKS = 72;      // 16-byte chunks per latent row
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__global__ __launch_bounds__(256, 2) void sparse_mla_kernel(const int64_t* __restrict__ base,
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

    __shared__ __attribute__((aligned(16))) uint16_t tile[AT_TILE * AT_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t plds[4][AT_TILE * 16];

    bf16x8 qreg[18];
    {
        const uint16_t* qrow = qa + ((int64_t)r * 64 + h0 + j) * 576 + 8 * g;
#pragma unroll
        for (int s = 0; s < 18; s++) qreg[s] = load_bf16x8(qrow + 32 * s);
    }
    const int64_t rbase = base[r];
    const int32_t* irow = idx + (int64_t)r * k;

    float m_run[4], l_run[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        m_run[v] = -INFINITY;
        l_run[v] = 0.f;
    }
    floatx4 o[32];
#pragma unroll
    for (int cb = 0; cb < 32; cb++) o[cb] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int t0 = slot_begin; t0 < slot_end; t0 += AT_TILE) {
        __syncthreads();  // the previous tile is fully consumed
        // Gather: 32 rows x 72 chunks of 16 B, 9 per thread.
#pragma unroll
        for (int i = 0; i < 9; i++) {
            const int c = threadIdx.x + 256 * i;
            const int slot = c / AT_CHUNKS;
            const int part = c - slot * AT_CHUNKS;
            const int gs = t0 + slot;
            const int id = gs < slot_end ? irow[gs] : -1;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (id >= 0) val = load_u32x4(kv + (rbase + id) * 576 + part * 8);
            *reinterpret_cast<u32x4*>(&tile[slot * AT_PITCH + part * 8]) = val;
        }
        __syncthreads();

        const int gs0 = t0 + j, gs1 = t0 + 16 + j;
        const bool ok0 = gs0 < slot_end && irow[gs0] >= 0;
        const bool ok1 = gs1 < slot_end && irow[gs1] >= 0;

        // QK: s0 -> positions 0..15 of the tile, s1 -> 16..31.
        floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 18; s++) {
            const bf16x8 b0 = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(&tile[j * AT_PITCH + 32 * s + 8 * g]));
            const bf16x8 b1 = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(&tile[(16 + j) * AT_PITCH + 32 * s + 8 * g]));
            s0 = mfma_16x16x32(qreg[s], b0, s0);
            s1 = mfma_16x16x32(qreg[s], b1, s1);
        }

        // Online softmax.  Lane (j, g) holds heads h0 + 4g + v at positions j, 16 + j.
        float p0[4], p1[4], alpha[4];
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const float z0 = ok0 ? s0[v] * scale_log2 : -INFINITY;
            const float z1 = ok1 ? s1[v] * scale_log2 : -INFINITY;
            const float mt = wave_max_16(fmaxf(z0, z1));
            const float m_new = fmaxf(m_run[v], mt);
            if (m_new == -INFINITY) {
                alpha[v] = 1.f;
                p0[v] = 0.f;
                p1[v] = 0.f;
            } else {
                alpha[v] = exp2f(m_run[v] - m_new);
                p0[v] = ok0 ? exp2f(z0 - m_new) : 0.f;
                p1[v] = ok1 ? exp2f(z1 - m_new) : 0.f;
            }
            l_run[v] = l_run[v] * alpha[v] + wave_sum_16(p0[v] + p1[v]);
            m_run[v] = m_new;
        }
#pragma unroll
        for (int cb = 0; cb < 32; cb++)
#pragma unroll
            for (int v = 0; v < 4; v++) o[cb][v] *= alpha[v];

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
        __syncthreads();
        // A operand: lane (head j, group g) gets P at tile positions 8g .. 8g+7.
        const bf16x8 pa = lds_read_tr_pair(&plds[wave][(8 * g + tk) * 16 + 4 * tc],
                                           &plds[wave][(8 * g + 4 + tk) * 16 + 4 * tc]);
        // PV over 32 column blocks of 16; B lane (column j, group g) gets V at
        // the same positions 8g .. 8g+7.
        const uint16_t* vlo = &tile[(8 * g + tk) * AT_PITCH + 4 * tc];
        const uint16_t* vhi = &tile[(8 * g + 4 + tk) * AT_PITCH + 4 * tc];
#pragma unroll
        for (int cb = 0; cb < 32; cb++) {
            const bf16x8 vb = lds_read_tr_pair(vlo + 16 * cb, vhi + 16 * cb);
            o[cb] = mfma_16x16x32(pa, vb, o[cb]);
        }
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
    int s = (int)((512 + num_rows - 1) / num_rows);
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
