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
// Design.  Each phase of a tile saturates a different unit (the address
// unit for the gathers, the matrix cores for QK and PV, the VALU and LDS
// round trips for the softmax), so the workgroup is split into two kinds of
// waves that work on consecutive tiles at the same time:
//  - One workgroup = one row x one contiguous split of its index list;
//    8 waves, one "score" wave and one "output" wave per SIMD.
//  - Tiles of 32 selected positions: the 32 latent rows (1152 B each) are
//    gathered into a 4-slot LDS ring with direct global->LDS loads.
//  - Score waves (w = 0..3) own heads 16w..16w+15.  QK computes
//    S^T[32 positions x 16 heads] on v_mfma_f32_16x16x32_bf16 with the latent
//    rows as the A operand (16-byte LDS reads) and the absorbed queries as B
//    (registers); each lane then holds one head and eight positions, so the
//    online softmax (fp32, base-2 exponent, lazily moved reference maximum)
//    needs in-lane work plus two cross-row swaps.  P is rounded to bf16
//    (round-to-nearest-even) and stored in the exact layout of the PV A
//    operand (16 bytes per lane).
//  - Output waves (w = 4..7) own latent columns 128(w-4)..+127 for all 64
//    heads: O[64 x 128] += P[64 x 32] . V[32 x 128] one tile behind the score
//    waves, reading each V element once (transposing ds_read_b64_tr_b16) and P
//    as four plain 16-byte reads.  They also issue the gathers.
//  - One barrier per tile: score waves hand over P(t) while output waves
//    finish PV(t-1); P, the rescale factors and the selected indices live in
//    small double / quadruple buffers.
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
constexpr int AT_STAGES = 4;       // ring slots
constexpr int AT_MAX_SPLIT = 2048; // largest split (slots)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_LOG2 = 8.f;  // lazy-rescale threshold (log2 units)
constexpr float LN2 = 0.6931471805599453f;

// Tile layout: 32 rows x 72 16-byte chunks, dense (1152 B per row, the
// direct global->LDS loads write 64 consecutive chunks per instruction).
// Logical chunk c of row r sits at chunk c ^ (r & 7).  With 1152 = 4.5 x 256
// the row parity already alternates the 128-byte half of the bank window, and
// the XOR spreads the rest, so that both operand read patterns are free of
// bank conflicts: QK reads (rows m0..m0+15, one logical chunk, 16 bytes per
// lane) and transposing PV reads (rows 4g+k and 16+4g+k of the four lane
// groups g, two adjacent chunks, 8 bytes per lane).
__device__ __forceinline__ int tile_chunk_offset(int row, int chunk)
{
    return row * (AT_CHUNKS * 16) + 16 * (chunk ^ (row & 7));
}

// Ring synchronisation.  The gathers are direct global->LDS loads issued
// through inline asm, so the compiler neither sees them as LDS writes (it
// would otherwise drain every outstanding gather before each LDS read of the
// ring) nor waits on them: the kernel does.  Each wave issues 9 loads per
// tile, loads complete in order, and a tile is read only after
// "vmcnt <= 9 x (tiles issued after it)" on every wave plus a barrier.  The
// waits and barriers carry memory clobbers so no LDS access moves across them.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 16-byte-per-lane direct load into LDS: lane L's bytes land at
// lds_base + 16 L.  M0 carries the LDS base; nothing else in this file uses
// M0, so clobbering it here is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void gather16_to_lds(const void* src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

__global__ __launch_bounds__(512, 1) void sparse_mla_kernel(const int64_t* __restrict__ base,
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
    const bool scorer = wave < 4;  // wave-uniform role
    const int wr = wave & 3;        // head block (score waves) / column block (output waves)
    const int j = lane & 15;
    const int g = lane >> 4;

    const int slot_begin = sp * split_len;
    const int slot_end = min(k, slot_begin + split_len);
    const int nslots = slot_end - slot_begin;
    const int32_t* irow = idx + (int64_t)r * k + slot_begin;

    __shared__ __attribute__((aligned(1024))) uint8_t ring[AT_STAGES][AT_TILE_BYTES];
    __shared__ __attribute__((aligned(16))) u32x4 plds[2][4][64];  // P of tile t: [t & 1][head block][lane]
    __shared__ __attribute__((aligned(16))) float alpha_l[2][64];  // per-head rescale factor of tile t
    __shared__ __attribute__((aligned(16))) int flag_l[2][4];      // head block rescaled in tile t
    __shared__ __attribute__((aligned(16))) int32_t sid[AT_STAGES][AT_TILE];  // indices of tile t: [t % 4]
    __shared__ __attribute__((aligned(16))) float lfin[64];
    __shared__ int s_last;

    // Last valid slot of the split: tiles past it hold no position and are skipped.
    if (threadIdx.x == 0) s_last = -1;
    __syncthreads();
    {
        int last = -1;
        for (int i = threadIdx.x; i < nslots; i += 512)
            if (irow[i] >= 0) last = i;
        if (last >= 0) atomicMax(&s_last, last);
    }
    __syncthreads();
    const int ntiles = (s_last + AT_TILE) / AT_TILE;
    // Indices of a tile (padding slots past the split read as -1).
    auto tile_index = [&](int t, int p) -> int32_t {
        const int i = t * AT_TILE + p;
        return (t < ntiles && i < nslots) ? irow[i] : -1;
    };
    if (threadIdx.x < (AT_STAGES - 1) * AT_TILE)
        sid[threadIdx.x / AT_TILE][threadIdx.x % AT_TILE] = tile_index(threadIdx.x / AT_TILE, threadIdx.x % AT_TILE);

    if (scorer) {
        // ------------------------------------------------------------ score waves
        const int h0 = wr * 16;
        // B operands of QK: Q[r][h0 + j][32 s + 8 g .. +8].
        bf16x8 qreg[18];
        {
            const uint16_t* qrow = qa + ((int64_t)r * 64 + h0 + j) * 576 + 8 * g;
#pragma unroll
            for (int s = 0; s < 18; s++) qreg[s] = load_bf16x8(qrow + 32 * s);
        }
        __syncthreads();  // indices of tiles 0..2 visible
        lds_barrier();    // tile 0 landed (the output waves waited for it)

        // QK A-operand bases: rows j and 16 + j, logical chunk 4 s + g =
        // 8 (s >> 1) + (4 (s & 1) + g) -> two bases per row plus immediate 128 (s >> 1).
        const int qa00 = tile_chunk_offset(j, g), qa01 = tile_chunk_offset(j, 4 + g);
        const int qa10 = tile_chunk_offset(16 + j, g), qa11 = tile_chunk_offset(16 + j, 4 + g);
        float m_run = -INFINITY, l_run = 0.f;  // head h0 + j; l_run: this lane's positions

        for (int t = 0; t < ntiles; t++) {
            // Indices of tile t + 3 (one score wave loads them; they are
            // stored at the end of this step, into the slot of tile t - 1).
            int32_t next_id = -1;
            if (wr == 0) next_id = tile_index(t + AT_STAGES - 1, lane & 31);

            const uint8_t* tl = ring[t % AT_STAGES];
            // QK: s0 -> tile positions 0..15, s1 -> 16..31 (rows of S^T);
            // lane (j, g) ends with S[head h0 + j][position 16 mb + 4 g + v] in s_mb[v].
            floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            {
                constexpr int QK_AHEAD = 3;
                bf16x8 a0[18], a1[18];
                auto rd = [&](int st) {
                    const int off = 128 * (st >> 1);
                    a0[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tl + ((st & 1) ? qa01 : qa00) + off));
                    a1[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tl + ((st & 1) ? qa11 : qa10) + off));
                };
#pragma unroll
                for (int st = 0; st < QK_AHEAD; st++) rd(st);
#pragma unroll
                for (int st = 0; st < 18; st++) {
                    if (st + QK_AHEAD < 18) rd(st + QK_AHEAD);
                    s0 = mfma_16x16x32(a0[st], qreg[st], s0);
                    s1 = mfma_16x16x32(a1[st], qreg[st], s1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // Validity of the tile's 32 slots (bit p: slot p holds a position).
            const uint32_t vbits = (uint32_t)__ballot(sid[t % AT_STAGES][lane & 31] >= 0);
            float z[8];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                z[v] = s0[v] * scale_log2;
                z[4 + v] = s1[v] * scale_log2;
            }
#pragma unroll
            for (int e = 0; e < 8; e++)
                z[e] = ((vbits >> (16 * (e >> 2) + 4 * g + (e & 3))) & 1u) ? z[e] : -INFINITY;
            float mt = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
            mt = xrow_max(mt);

            // Lazy reference maximum: m_run moves only when the tile's maximum
            // exceeds it by more than 2^RESCALE_LOG2, so weights stay below
            // 2^RESCALE_LOG2 (far from fp32 or bf16 overflow) and the result
            // o / l and lse = m_run + log2 l do not depend on the reference
            // used.  In steady state no tile rescales the output accumulators.
            const bool need = mt > m_run + RESCALE_LOG2;
            const float m_new = need ? mt : m_run;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 when m_run = -inf
            l_run *= alpha;
            m_run = m_new;
            const float m_safe = (m_run == -INFINITY) ? 0.f : m_run;  // then every z is -inf

            // P = 2^(z - m_run) (zero for empty slots), rounded to bf16, stored
            // as this lane's PV A operand: row = head h0 + j, k = positions
            // {4g..4g+3, 16+4g..16+4g+3}.
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float p0 = __builtin_amdgcn_exp2f(z[2 * e] - m_safe);
                const float p1 = __builtin_amdgcn_exp2f(z[2 * e + 1] - m_safe);
                l_run += p0 + p1;
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const bf16x2 h = {(__bf16)p0, (__bf16)p1};
                pk[e] = __builtin_bit_cast(uint32_t, h);
            }
            plds[t & 1][wr][lane] = pk;
            if (g == 0) alpha_l[t & 1][h0 + j] = alpha;
            const bool any_need = __ballot(need) != 0ull;
            if (lane == 0) flag_l[t & 1][wr] = any_need ? 1 : 0;
            if (wr == 0 && lane < AT_TILE) sid[(t + AT_STAGES - 1) % AT_STAGES][lane] = next_id;
            lds_barrier();  // step t: P(t) handed over; tile t + 1 landed
        }

        // Row sums (the four lanes of a head), log-sum-exp, split statistics.
        const float l_tot = xrow_sum(l_run);
        if (g == 0) {
            lfin[h0 + j] = l_tot;
            if (nsplit == 1) {
                if (lse) lse[(int64_t)r * 64 + h0 + j] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : -INFINITY;
            } else {
                part_ml[((int64_t)r * nsplit + sp) * 64 + h0 + j] = make_float2(m_run, l_tot);
            }
        }
        __syncthreads();  // lfin visible to the output waves
    } else {
        // ----------------------------------------------------------- output waves
        const int c0 = wr * 128;
        const int tc = lane & 3;  // transposed-read roles inside a 16-lane group
        const int tk = (lane >> 2) & 3;
        const uint16_t* kvrow = kv + base[r] * 576;

        // Gather roles.  Output wave b fills tile rows 8b..8b+7 (LDS chunks
        // [576 b, 576 b + 576)): its i-th load instruction writes 64
        // consecutive 16-byte LDS chunks (lane order), and lane L fetches
        // whichever logical chunk belongs at LDS chunk 576 b + 64 i + L under
        // the swizzle.  Padding slots fetch the sequence's first latent row
        // (always present); their softmax weight is zero.
        // The address unit takes ~30 clocks per such instruction, so the nine
        // loads of a refill are spread over the PV MFMAs (gather_one) rather
        // than issued back to back, which would stall this wave meanwhile.
        int gid[9];
        auto gather_ids = [&](int t) {
#pragma unroll
            for (int i = 0; i < 9; i++) gid[i] = sid[t % AT_STAGES][((wr * 9 + i) * 64 + lane) / AT_CHUNKS];
        };
        auto gather_one = [&](int t, int i) {
            const uint32_t dst = __builtin_amdgcn_readfirstlane(
                (uint32_t)(uintptr_t)(ring[t % AT_STAGES] + wr * 9 * 1024 + i * 1024));
            const int p = (wr * 9 + i) * 64 + lane;
            const int row = p / AT_CHUNKS;
            const int part = (p - row * AT_CHUNKS) ^ (row & 7);
            gather16_to_lds(kvrow + (int64_t)max(gid[i], 0) * 576 + part * 8, dst);
        };
        auto issue = [&](int t) {
            gather_ids(t);
#pragma unroll
            for (int i = 0; i < 9; i++) gather_one(t, i);
        };

        // Transposed-read bases (tile rows 4g + tk and 16 + 4g + tk, columns
        // c0 + 16 cb + 4 tc .. +3 = logical chunk 16 b + 2 cb + (tc >> 1),
        // byte 8 (tc & 1)); cb = 4 m + e -> immediate 128 m on top of base e.
        const int vrlo = 4 * g + tk, vrhi = 16 + 4 * g + tk;
        int vlo[4], vhi[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            vlo[e] = tile_chunk_offset(vrlo, 16 * wr + 2 * e + (tc >> 1)) + 8 * (tc & 1);
            vhi[e] = tile_chunk_offset(vrhi, 16 * wr + 2 * e + (tc >> 1)) + 8 * (tc & 1);
        }
        // O[16 mb + 4 g + v][c0 + 16 cb + j] = o[mb][cb][v].
        floatx4 o[4][8];
#pragma unroll
        for (int mb = 0; mb < 4; mb++)
#pragma unroll
            for (int cb = 0; cb < 8; cb++) o[mb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};

        // PV of tile t: rescale the O rows of head blocks whose reference
        // moved, then O[64 x 128] += P[64 x 32] . V[32 x 128].  With refill
        // >= 0 the loads of tile `refill` go out between the MFMAs.
        auto pv = [&](int t, int refill) {
            const uint8_t* tl = ring[t % AT_STAGES];
            bf16x8 pa[4];
#pragma unroll
            for (int mb = 0; mb < 4; mb++) pa[mb] = __builtin_bit_cast(bf16x8, plds[t & 1][mb][lane]);
            const u32x4 fl = *reinterpret_cast<const u32x4*>(flag_l[t & 1]);
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
                if (__builtin_amdgcn_readfirstlane(fl[mb])) {
                    const floatx4 al = *reinterpret_cast<const floatx4*>(&alpha_l[t & 1][16 * mb + 4 * g]);
#pragma unroll
                    for (int cb = 0; cb < 8; cb++)
#pragma unroll
                        for (int v = 0; v < 4; v++) o[mb][cb][v] *= al[v];
                }
            }
            constexpr int PV_AHEAD = 2;
            bf16x8 vb[8];
            auto rdv = [&](int cb) {
                const int off = 128 * (cb >> 2);
                vb[cb] = lds_read_tr_pair((const uint16_t*)(tl + vlo[cb & 3] + off), (const uint16_t*)(tl + vhi[cb & 3] + off));
            };
#pragma unroll
            for (int cb = 0; cb < PV_AHEAD; cb++) rdv(cb);
#pragma unroll
            for (int cb = 0; cb < 8; cb++) {
                if (cb + PV_AHEAD < 8) rdv(cb + PV_AHEAD);
#pragma unroll
                for (int mb = 0; mb < 4; mb++) o[mb][cb] = mfma_16x16x32(pa[mb], vb[cb], o[mb][cb]);
                if (refill >= 0) gather_one(refill, cb);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (refill >= 0) gather_one(refill, 8);
        };

        __syncthreads();  // indices of tiles 0..2 visible
        // Pipeline: at step t the score waves work on tile t and the output
        // waves on tile t - 1; tiles t + 1 (landed) and t + 2 (in flight) fill
        // the other two slots.  Loads in flight per output wave after the
        // issue of step t: tiles t + 1, t + 2.
        if (ntiles > 0) issue(0);
        if (ntiles > 1) issue(1);
        if (ntiles > 1) wait_vm<9>();
        else wait_vm<0>();
        lds_barrier();  // tile 0 landed
        for (int t = 0; t < ntiles; t++) {
            // Refill: tile t + 2 into the slot of tile t - 2 (finished at step t - 1).
            const int refill = t + 2 < ntiles ? t + 2 : -1;  // wave-uniform
            if (refill >= 0) gather_ids(refill);
            if (t > 0) pv(t - 1, refill);
            else if (refill >= 0)
#pragma unroll
                for (int i = 0; i < 9; i++) gather_one(refill, i);
            if (t + 1 < ntiles) {
                if (t + 2 < ntiles) wait_vm<9>();
                else wait_vm<0>();
            }
            lds_barrier();  // step t: P(t) handed over; tile t + 1 landed
        }
        if (ntiles > 0) pv(ntiles - 1, -1);
        __syncthreads();  // lfin visible

        // Epilogue.  Lane (j, g) holds O[16 mb + 4 g + v][c0 + 16 cb + j].
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            const floatx4 lv = *reinterpret_cast<const floatx4*>(&lfin[16 * mb + 4 * g]);
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int h = 16 * mb + 4 * g + v;
                float* orow;
                float scl;
                if (nsplit == 1) {
                    orow = out + ((int64_t)r * 64 + h) * 512 + c0;
                    scl = lv[v] > 0.f ? 1.f / lv[v] : 0.f;
                } else {
                    orow = part_o + (((int64_t)r * nsplit + sp) * 64 + h) * 512 + c0;
                    scl = 1.f;
                }
#pragma unroll
                for (int cb = 0; cb < 8; cb++) orow[16 * cb + j] = o[mb][cb][v] * scl;
            }
        }
    }
}

// Merges split partials in split order: one workgroup per (head, row), each
// thread four latent columns.  Every split's loads are issued before any is
// used (one memory round trip per thread); the arithmetic still runs in
// split order, so results do not depend on scheduling.
__global__ __launch_bounds__(128) void sparse_mla_combine_kernel(const float* __restrict__ part_o,
                                                                const float2* __restrict__ part_ml, int nsplit,
                                                                float* __restrict__ out, float* __restrict__ lse)
{
    constexpr int MAXS = 16;  // attn_pick_splits never returns more
    const int h = blockIdx.x;
    const int r = blockIdx.y;
    const float2* ml = part_ml + (int64_t)r * nsplit * 64 + h;
    const float* po = part_o + ((int64_t)r * nsplit * 64 + h) * 512 + 4 * threadIdx.x;
    float2 e[MAXS];
    float4 p[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; s++) {
        if (s < nsplit) {
            e[s] = ml[(int64_t)s * 64];
            p[s] = *reinterpret_cast<const float4*>(po + (int64_t)s * 64 * 512);
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < MAXS; s++)
        if (s < nsplit) M = fmaxf(M, e[s].x);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int s = 0; s < MAXS; s++) {
            if (s < nsplit) {
                const float f = exp2f(e[s].x - M);
                L += e[s].y * f;
                acc.x += p[s].x * f;
                acc.y += p[s].y * f;
                acc.z += p[s].z * f;
                acc.w += p[s].w * f;
            }
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
    hipLaunchKernelGGL(sparse_mla_kernel, dim3(s, num_rows), dim3(512), 0, stream, base, qa, kv, idx, k,
                       softmax_scale * LOG2E, split_len, out, lse, part_o, part_ml);
    if (s > 1)
        hipLaunchKernelGGL(sparse_mla_combine_kernel, dim3(64, num_rows), dim3(128), 0, stream, part_o, part_ml, s,
                           out, lse);
}

}  // namespace dsa
