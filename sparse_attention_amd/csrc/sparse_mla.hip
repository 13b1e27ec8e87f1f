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
//    12 waves: per SIMD one "score" wave and two "output" waves.
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
//  - Output waves (w = 4..11) own latent columns 64(w-4)..+63 for all 64
//    heads: O[64 x 64] += P[64 x 32] . V[32 x 64] one tile behind the score
//    waves, reading each V element once (transposing ds_read_b64_tr_b16, into
//    registers during the tile's QK step, so its ring slot is free one step
//    later and three tiles stay in flight) and P as four plain 16-byte reads.
//    They also issue the gathers; with two of them per SIMD, one waiting for
//    the address unit leaves the matrix core to the other.
//  - One barrier per tile: score waves hand over P(t) while output waves
//    finish PV(t-1); P, the rescale factors and the selected indices live in
//    small double / octuple buffers.
//  - A split writes its own normalized output, rounded to bf16, with its
//    running maximum and sum; a combine kernel merges the splits in split
//    order (in fp32), so results do not depend on scheduling.  A single split
//    writes the fp32 output itself.
#include <algorithm>
#include <cmath>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int AT_TILE = 32;        // selected positions per tile
constexpr int AT_CHUNKS = 72;      // 16-byte chunks per latent row
constexpr int AT_TILE_BYTES = AT_TILE * AT_CHUNKS * 16;  // 36,864
constexpr int AT_STAGES = 4;       // ring slots
constexpr int AT_SID = 8;          // index ring slots
constexpr int AT_MAX_SPLIT = 2048; // largest split (slots)
constexpr int AT_OWAVES = 8;       // output waves
constexpr int AT_OCOLS = 512 / AT_OWAVES;  // latent columns per output wave (64)
constexpr int AT_OCB = AT_OCOLS / 16;      // 16-column blocks per output wave
constexpr int AT_GQ = AT_TILE_BYTES / 1024;  // gather instructions per tile (36)
constexpr int AT_THREADS = 64 * (4 + AT_OWAVES);  // 4 score waves + output waves
constexpr int AT_OPAD = AT_OCOLS + 4;  // padded row of an output block staged in LDS (floats)
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

// The same from a uniform 64-bit base plus a 32-bit per-lane byte offset
// (the scalar-base form: no 64-bit address arithmetic per lane).
__device__ __forceinline__ void gather16_to_lds_off(const void* base, uint32_t off, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(off), "s"(base)
                 : "memory", "m0");
}

// The same for 4 bytes per lane (lane L's word lands at lds_base + 4 L).
__device__ __forceinline__ void load4_to_lds(const void* src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

// Byte offset of a shared-memory object inside the workgroup's LDS, as the
// direct loads take it in M0.
template <typename T>
__device__ __forceinline__ uint32_t lds_offset(T* p)
{
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) T*)p);
}

// OFF32: every gathered row lies within 2^32 bytes of the row's cache base
// (no paged pool), so a gather address is the base plus a 32-bit offset.
template <bool OFF32>
__global__ __launch_bounds__(AT_THREADS, 1) void sparse_mla_kernel(const int64_t* __restrict__ base,
                                                           const uint16_t* __restrict__ qa,
                                                           const uint16_t* __restrict__ kv,
                                                           const int32_t* __restrict__ idx, int k,
                                                           int num_rows, float scale_log2, int split_len,
                                                           int nsplit, int pad_rows,
                                                           float* __restrict__ out, float* __restrict__ lse,
                                                           uint16_t* __restrict__ part_o,
                                                           float2* __restrict__ part_ml)
{
    // One split per row: rows in reverse (in a causal prefill chunk the last
    // rows select the most positions, and starting them first shortens the
    // tail).  Several splits: a one-dimensional grid numbered so that the
    // splits of a row share an XCD (workgroups go to the eight XCDs in turn),
    // and the later splits find the row's queries in that XCD's L2.  Results
    // do not depend on the order.
    int r, sp;
    if (nsplit == 1) {
        if (grid_item() >= num_rows) return;
        r = num_rows - 1 - grid_item();
        sp = 0;
    } else {
        const int id = blockIdx.x, blk = id / (8 * nsplit), j = id - blk * 8 * nsplit;
        r = blk * 8 + (j & 7);
        sp = j >> 3;
        if (r >= num_rows) return;
    }
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
    __shared__ __attribute__((aligned(16))) int32_t sid[AT_SID][AT_TILE];  // indices of tile t: [t % 8]
    __shared__ __attribute__((aligned(16))) float lfin[64];
    __shared__ int s_wlast[AT_THREADS / 64];

    // Prologue, one memory round trip before the first gathers: every thread
    // reads its slots of the split (at most three), posting the first tiles'
    // indices to the index ring and the last valid slot (tiles past it hold no
    // position and are skipped) as a per-wave maximum.
    static_assert(AT_MAX_SPLIT <= 3 * AT_THREADS, "three slots per thread");
    int32_t v[3];
#pragma unroll
    for (int u = 0; u < 3; u++) v[u] = irow[min((int)threadIdx.x + AT_THREADS * u, nslots - 1)];  // nslots >= 1
    {
        int last = -1;
#pragma unroll
        for (int u = 0; u < 3; u++) {
            const int i = threadIdx.x + AT_THREADS * u;
            last = (i < nslots && v[u] >= 0) ? i : last;  // slots past the split hold its last slot: masked by nslots
        }
        if (threadIdx.x < AT_STAGES * AT_TILE) sid[threadIdx.x / AT_TILE][threadIdx.x % AT_TILE] = v[0];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) last = max(last, __shfl_xor(last, d));
        if (lane == 0) s_wlast[wave] = last;
    }
    // The queries go out after the indices have been used (so that waiting
    // for the indices does not mean waiting for them): they still land before
    // the first tile, which needs a second round trip.
    bf16x8 qreg[18];  // score waves: B operands of QK, Q[r][16 wr + j][32 s + 8 g .. +8]
    if (scorer) {
        const uint16_t* qrow = qa + ((int64_t)r * 64 + wr * 16 + j) * 576 + 8 * g;
#pragma unroll
        for (int s = 0; s < 18; s++) qreg[s] = load_bf16x8(qrow + 32 * s);
    }
    __syncthreads();
    int s_last = -1;
#pragma unroll
    for (int w = 0; w < AT_THREADS / 64; w++) s_last = max(s_last, s_wlast[w]);
    const int ntiles = (s_last + AT_TILE) / AT_TILE;

    if (scorer) {
        // ------------------------------------------------------------ score waves
        const int h0 = wr * 16;
        // Complete the query loads here: otherwise the compiler's wait counts
        // at the loop head assume they may still be in flight and make every
        // step wait for the index prefetches below as well.
#pragma unroll
        for (int s = 0; s < 18; s++) asm volatile("" ::"v"(qreg[s]));
        lds_barrier();  // tile 0 landed (the output waves waited for it)

        // QK A-operand bases: rows j and 16 + j, logical chunk 4 s + g =
        // 8 (s >> 1) + (4 (s & 1) + g) -> two bases per row plus immediate 128 (s >> 1).
        const int qa00 = tile_chunk_offset(j, g), qa01 = tile_chunk_offset(j, 4 + g);
        const int qa10 = tile_chunk_offset(16 + j, g), qa11 = tile_chunk_offset(16 + j, 4 + g);
        float m_run = -INFINITY, l_run = 0.f;  // head h0 + j; l_run: this lane's positions

        // The index ring is refilled by direct loads into LDS (wave 0, lanes
        // 0..31), two steps ahead: the indices of tile t + 5 go out at the
        // start of step t and are waited for at the end of step t + 1, before
        // the barrier after which the output waves issue that tile's gathers.
        // Slots past the split read its last slot and are masked as invalid.
        auto fetch_ids = [&](int tt) {
            if (lane < AT_TILE) {
                const int i = min(tt * AT_TILE + lane, nslots - 1);
                load4_to_lds(irow + i, lds_offset(&sid[tt % AT_SID][0]));
            }
        };
        if (wr == 0 && AT_STAGES < ntiles) fetch_ids(AT_STAGES);
        auto score_step = [&](int t) {
            const bool fetch = wr == 0 && t + AT_STAGES + 1 < ntiles;  // wave-uniform
            if (fetch) fetch_ids(t + AT_STAGES + 1);
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
            const uint32_t vbits =
                (uint32_t)__ballot(sid[t % AT_SID][lane & 31] >= 0 && t * AT_TILE + (lane & 31) < nslots);
            // Raw scores; the scale (> 0, so the maximum commutes with it) is
            // applied to the tile maximum and inside the exponent's fma.
            float z[8];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                z[v] = s0[v];
                z[4 + v] = s1[v];
            }
            if (vbits != 0xffffffffu) {  // wave-uniform: only tiles with empty slots
#pragma unroll
                for (int e = 0; e < 8; e++)
                    z[e] = ((vbits >> (16 * (e >> 2) + 4 * g + (e & 3))) & 1u) ? z[e] : -INFINITY;
            }
            float mt = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
            mt = xrow_max(mt) * scale_log2;

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

            // P = 2^(scale z - m_run) (zero for empty slots), rounded to bf16,
            // stored as this lane's PV A operand: row = head h0 + j, k =
            // positions {4g..4g+3, 16+4g..16+4g+3}.
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(z[2 * e], scale_log2, -m_safe));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(z[2 * e + 1], scale_log2, -m_safe));
                l_run += p0 + p1;
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const bf16x2 h = {(__bf16)p0, (__bf16)p1};
                pk[e] = __builtin_bit_cast(uint32_t, h);
            }
            plds[t & 1][wr][lane] = pk;
            if (g == 0) alpha_l[t & 1][h0 + j] = alpha;
            const bool any_need = __ballot(need) != 0ull;
            if (lane == 0) flag_l[t & 1][wr] = any_need ? 1 : 0;
            // Indices of tile t + 4 landed (those of t + 5 may be in flight).
            if (wr == 0) {
                if (fetch) wait_vm<1>();
                else wait_vm<0>();
            }
            lds_barrier();  // step t: P(t) handed over; tile t + 1 landed
        };
        for (int t = 0; t < ntiles; t++) score_step(t);

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
        const int ob = wave - 4;    // output wave 0..7
        const int c0 = ob * AT_OCOLS;
        const int tc = lane & 3;    // transposed-read roles inside a 16-lane group
        const int tk = (lane >> 2) & 3;
        const uint16_t* kvrow = kv + base[r] * 576;

        // Gather roles.  A tile is 36 load instructions, each writing 64
        // consecutive 16-byte LDS chunks (lane order); output wave ob issues
        // instructions q = ob + 8 i (five for ob < 4, four otherwise), and lane
        // L fetches whichever logical chunk belongs at LDS chunk 64 q + L
        // under the swizzle.  Padding slots fetch a row that is always present
        // (their softmax weight is zero, but a non-finite row would still
        // poison P.V): the sequence's first latent row, or, when pad_rows is
        // set (index lists translated to pool rows), row -1 - entry, which
        // the translation points at the sequence's first row.  The loads are
        // spread over the PV MFMAs: a wave waiting for the address unit leaves
        // the matrix core to the other output wave of its SIMD.
        const bool five = ob < AT_GQ - 4 * AT_OWAVES;  // wave-uniform
        // Per gather i: the tile row lane L fetches for (clamped for the
        // fifth gather of waves that issue only four) and the byte offset of
        // its swizzled chunk in that latent row.  Both are fixed for the
        // whole loop.
        int grow[5], gbyte[5];
#pragma unroll
        for (int i = 0; i < 5; i++) {
            const int p = min((ob + AT_OWAVES * i) * 64 + lane, AT_TILE * AT_CHUNKS - 1);
            grow[i] = p / AT_CHUNKS;
            gbyte[i] = 16 * ((p - grow[i] * AT_CHUNKS) ^ (grow[i] & 7));
        }
        int gid[5];
        auto gather_ids = [&](int t) {
#pragma unroll
            for (int i = 0; i < 5; i++) gid[i] = sid[t % AT_SID][grow[i]];
        };
        const uint8_t* kvbytes = reinterpret_cast<const uint8_t*>(kvrow);
        const uint32_t ring_lds = lds_offset(&ring[0][0]);
        auto gather_one = [&](int t, int i) {
            const int q = ob + AT_OWAVES * i;
            const uint32_t dst =
                __builtin_amdgcn_readfirstlane(ring_lds + (uint32_t)((t % AT_STAGES) * AT_TILE_BYTES + q * 1024));
            if constexpr (OFF32) {
                // No pool: padding fetches row 0.  Rows stay below 2^24 here
                // (2^32 / 1152), so the offset is one 24-bit multiply-add.
                const uint32_t gr = (uint32_t)min(max(gid[i], 0), 0xffffff);
                gather16_to_lds_off(kvbytes, gr * 1152u + (uint32_t)gbyte[i], dst);
            } else {
                const int64_t gr = gid[i] >= 0 ? (int64_t)gid[i] : (pad_rows ? -1 - (int64_t)gid[i] : 0);
                gather16_to_lds(kvbytes + gr * 1152 + gbyte[i], dst);
            }
        };
        auto issue = [&](int t) {
            gather_ids(t);
#pragma unroll
            for (int i = 0; i < 4; i++) gather_one(t, i);
            if (five) gather_one(t, 4);
        };
        // Tile t + 1 landed, `after` tiles issued later possibly not.
        auto wait_tiles = [&](int after) {
            if (five) {
                if (after >= 2) wait_vm<10>();
                else if (after == 1) wait_vm<5>();
                else wait_vm<0>();
            } else {
                if (after >= 2) wait_vm<8>();
                else if (after == 1) wait_vm<4>();
                else wait_vm<0>();
            }
        };

        // Transposed-read bases: tile rows 4g + tk and 16 + 4g + tk, columns
        // c0 + 16 cb + 4 tc .. +3 = logical chunk 8 ob + 2 cb + (tc >> 1),
        // byte 8 (tc & 1).
        const int vrlo = 4 * g + tk, vrhi = 16 + 4 * g + tk;
        int vlo[AT_OCB], vhi[AT_OCB];
#pragma unroll
        for (int cb = 0; cb < AT_OCB; cb++) {
            vlo[cb] = tile_chunk_offset(vrlo, 8 * ob + 2 * cb + (tc >> 1)) + 8 * (tc & 1);
            vhi[cb] = tile_chunk_offset(vrhi, 8 * ob + 2 * cb + (tc >> 1)) + 8 * (tc & 1);
        }
        // O[16 mb + 4 g + v][c0 + 16 cb + j] = o[mb][cb][v].
        floatx4 o[4][AT_OCB];
#pragma unroll
        for (int mb = 0; mb < 4; mb++)
#pragma unroll
            for (int cb = 0; cb < AT_OCB; cb++) o[mb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};

        // V operands of the current tile, read from the ring one step before
        // their PV, so that a slot is free as soon as both roles have read it
        // (the step after its QK) and three tiles stay in flight.
        bf16x8 vb[AT_OCB];
        auto rescale = [&](int tp) {
            const u32x4 fl = *reinterpret_cast<const u32x4*>(flag_l[tp]);
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
                if (__builtin_amdgcn_readfirstlane(fl[mb])) {
                    const floatx4 al = *reinterpret_cast<const floatx4*>(&alpha_l[tp][16 * mb + 4 * g]);
#pragma unroll
                    for (int cb = 0; cb < AT_OCB; cb++)
#pragma unroll
                        for (int v = 0; v < 4; v++) o[mb][cb][v] *= al[v];
                }
            }
        };
        // Step body of the output waves at step t: rescale the O rows of head
        // blocks whose reference moved in tile t - 1 and accumulate
        // O[64 x 64] += P(t-1)[64 x 32] . V(t-1)[32 x 64] (if t > 0), then
        // read V(t) into vb.  With refill >= 0 the loads of tile `refill` go
        // out between the MFMAs.
        auto step = [&](int t, int refill) {
            const uint8_t* tl = ring[t % AT_STAGES];
            if (t > 0) {
                const int tp = (t - 1) & 1;
                bf16x8 pa[4];
#pragma unroll
                for (int mb = 0; mb < 4; mb++) pa[mb] = __builtin_bit_cast(bf16x8, plds[tp][mb][lane]);
                rescale(tp);
#pragma unroll
                for (int cb = 0; cb < AT_OCB; cb++) {
#pragma unroll
                    for (int mb = 0; mb < 4; mb++) o[mb][cb] = mfma_16x16x32(pa[mb], vb[cb], o[mb][cb]);
                    vb[cb] = lds_read_tr_pair((const uint16_t*)(tl + vlo[cb]), (const uint16_t*)(tl + vhi[cb]));
                    if (refill >= 0) gather_one(refill, cb);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int cb = 0; cb < AT_OCB; cb++) {
                    vb[cb] = lds_read_tr_pair((const uint16_t*)(tl + vlo[cb]), (const uint16_t*)(tl + vhi[cb]));
                    if (refill >= 0) gather_one(refill, cb);
                }
            }
            if (refill >= 0 && five) gather_one(refill, 4);
        };
        // PV of the last tile, after the final hand-over.
        auto pv_last = [&](int t) {
            const int tp = t & 1;
            bf16x8 pa[4];
#pragma unroll
            for (int mb = 0; mb < 4; mb++) pa[mb] = __builtin_bit_cast(bf16x8, plds[tp][mb][lane]);
            rescale(tp);
#pragma unroll
            for (int cb = 0; cb < AT_OCB; cb++)
#pragma unroll
                for (int mb = 0; mb < 4; mb++) o[mb][cb] = mfma_16x16x32(pa[mb], vb[cb], o[mb][cb]);
        };

        // Pipeline: at step t the score waves work on tile t and the output
        // waves on tiles t - 1 (PV) and t (V reads); tiles t + 1 (landed),
        // t + 2 and t + 3 (in flight) fill the other slots.  The refill of
        // step t goes into the slot of tile t - 1, which both roles finished
        // reading in step t - 1.
        if (ntiles > 0) issue(0);
        if (ntiles > 1) issue(1);
        if (ntiles > 2) issue(2);
        wait_tiles(min(ntiles, 3) - 1);
        lds_barrier();  // tile 0 landed
        for (int t = 0; t < ntiles; t++) {
            const int refill = t + 3 < ntiles ? t + 3 : -1;  // wave-uniform
            if (refill >= 0) gather_ids(refill);
            step(t, refill);
            if (t + 1 < ntiles) wait_tiles(min(ntiles - 1, t + 3) - (t + 1));
            lds_barrier();  // step t: P(t) handed over; tile t + 1 landed
        }
        if (ntiles > 0) pv_last(ntiles - 1);
        __syncthreads();  // lfin visible

        // Epilogue.  Lane (j, g) holds O[16 mb + 4 g + v][c0 + 16 cb + j],
        // normalized by the head's sum (a split normalizes by its own).  The
        // block goes through this wave's own region of the (now idle) ring,
        // rows padded to AT_OPAD floats, so that the stores leave as 16-byte
        // pieces of row segments.
        float* ot = reinterpret_cast<float*>(&ring[0][0]) + ob * (64 * AT_OPAD);
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            const floatx4 lv = *reinterpret_cast<const floatx4*>(&lfin[16 * mb + 4 * g]);
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float scl = lv[v] > 0.f ? 1.f / lv[v] : 0.f;
                float* orow = ot + (16 * mb + 4 * g + v) * AT_OPAD + j;
#pragma unroll
                for (int cb = 0; cb < AT_OCB; cb++) orow[16 * cb] = o[mb][cb][v] * scl;
            }
        }
        // Only this wave touches its region: LDS keeps its accesses in order.
        // Non-temporal stores: the output (or the split partials, read once
        // by the combine kernel) would otherwise be written back from L2 at
        // the kernel's end.
        if (nsplit == 1) {
            float* dst = out + (int64_t)r * 64 * 512 + c0;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int h = 4 * i + (lane >> 4), c = 4 * (lane & 15);
                const floatx4 val = *reinterpret_cast<const floatx4*>(ot + h * AT_OPAD + c);
                __builtin_nontemporal_store(val, reinterpret_cast<floatx4*>(dst + (int64_t)h * 512 + c));
            }
        } else {
            // A split's partial, rounded to bf16 (to nearest even): a convex
            // combination of V rows, so each element is off by at most
            // 2^-9 max|V|, the precision of a bf16 output.
            uint16_t* dst = part_o + ((int64_t)r * nsplit + sp) * 64 * 512 + c0;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int h = 8 * i + (lane >> 3), c = 8 * (lane & 7);
                const floatx4 a = *reinterpret_cast<const floatx4*>(ot + h * AT_OPAD + c);
                const floatx4 b = *reinterpret_cast<const floatx4*>(ot + h * AT_OPAD + c + 4);
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                u32x4 pk;
                pk[0] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a[0], (__bf16)a[1]});
                pk[1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a[2], (__bf16)a[3]});
                pk[2] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)b[0], (__bf16)b[1]});
                pk[3] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)b[2], (__bf16)b[3]});
                __builtin_nontemporal_store(pk, reinterpret_cast<u32x4*>(dst + (int64_t)h * 512 + c));
            }
        }
    }
}

// Merges split partials in split order: one workgroup per (head, row), each
// thread four latent columns.  A split's partial is its own normalized output
// (bf16) with its running maximum m_s and sum l_s, so the merge weighs split s
// by l_s 2^(m_s - M).  Every split's loads are issued before any is used (one
// memory round trip per thread); the arithmetic still runs in split order, so
// results do not depend on scheduling.
__global__ __launch_bounds__(128) void sparse_mla_combine_kernel(const uint16_t* __restrict__ part_o,
                                                                const float2* __restrict__ part_ml, int nsplit,
                                                                int num_rows, float* __restrict__ out,
                                                                float* __restrict__ lse)
{
    constexpr int MAXS = 16;  // attn_pick_splits never returns more
    const int h = blockIdx.x;
    const int r = grid_item();
    if (r >= num_rows) return;
    const float2* ml = part_ml + (int64_t)r * nsplit * 64 + h;
    const uint16_t* po = part_o + ((int64_t)r * nsplit * 64 + h) * 512 + 4 * threadIdx.x;
    float2 e[MAXS];
    uint2 p[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; s++) {
        if (s < nsplit) {
            e[s] = ml[(int64_t)s * 64];
            p[s] = *reinterpret_cast<const uint2*>(po + (int64_t)s * 64 * 512);
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
                const float wgt = e[s].y * exp2f(e[s].x - M);
                L += wgt;
                acc.x += __uint_as_float(p[s].x << 16) * wgt;
                acc.y += __uint_as_float(p[s].x & 0xffff0000u) * wgt;
                acc.z += __uint_as_float(p[s].y << 16) * wgt;
                acc.w += __uint_as_float(p[s].y & 0xffff0000u) * wgt;
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float4 res = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    __builtin_nontemporal_store(floatx4{res.x, res.y, res.z, res.w},
                                reinterpret_cast<floatx4*>(out + ((int64_t)r * 64 + h) * 512 + 4 * threadIdx.x));
    if (lse && threadIdx.x == 0) lse[(int64_t)r * 64 + h] = L > 0.f ? (M + log2f(L)) * LN2 : -INFINITY;
}

}  // namespace

int attn_pick_splits(int32_t num_rows, int32_t k)
{
    // The split count with the least modelled time.  One 768-thread
    // workgroup fills a CU (LDS ring and registers), so at most 256 run at
    // once and the rest start in later rounds.  A workgroup costs ~7 us
    // besides its tiles (index list and queries in, output or partial out);
    // a tile takes the longer of ~1.03 us (one CU's gather rate, three tiles
    // in flight) and the time the busy CUs' tiles take together at ~6.5 TB/s.
    // Every split adds a 64 KB bf16 partial per row, written and read back
    // by the merge, which is one more launch.  Fitted to decode batches of
    // 2,048 selected rows (attention + merge, then re-measured with the bf16
    // partials): 64 rows 36.6-37.0 us with 3 splits against 36.8-37.0 with 4
    // (whose step is 2 us slower) and 44.1 with 2; 16 rows 20.0-20.5 us with
    // 8 to 13 splits against 21.8 with 6 and 21.2 with 16; and, with fp32
    // partials, 48 rows 34.4 us with 4 against 49.2 with 6 (two rounds), 100
    // rows 55.6 with 2 against 78.5 with 3.
    constexpr double kTileFloor = 1.03e-6, kGatherBw = 6.5e12, kFixed = 7e-6, kMergeLaunch = 2e-6;
    constexpr double kPartialBytes = 64.0 * 512 * 2 * 2;  // per row and split: written, then read
    const int tiles = (k + AT_TILE - 1) / AT_TILE;
    int best = 1;
    double best_t = 0.0;
    for (int s = 1; s <= 16 && s <= tiles; s++) {
        const int per = (tiles + s - 1) / s;  // equal whole-tile splits
        if ((tiles + per - 1) / per != s) continue;  // the same splits as a smaller count
        const double wgs = (double)num_rows * s;
        auto round_time = [&](double busy) {
            return kFixed + per * std::max(kTileFloor, busy * AT_TILE_BYTES / kGatherBw);
        };
        const double full = std::floor(wgs / 256.0), rest = wgs - 256.0 * full;
        double t = full * round_time(256.0) + (rest > 0.0 ? round_time(rest) : 0.0);
        if (s > 1) t += kMergeLaunch + wgs * kPartialBytes / kGatherBw;
        // A further split has to save at least 2%: the merge's partials are
        // the model's least certain part.
        if (s == 1 || t < 0.98 * best_t) {
            best = s;
            best_t = t;
        }
    }
    return best;
}

size_t attn_workspace_bytes(int32_t num_rows, int32_t k)
{
    const int s = attn_pick_splits(num_rows, k);
    if (s == 1) return 0;
    const size_t R = (size_t)num_rows;
    return align_up(R * s * 64 * 512 * 2, 256) + align_up(R * s * 64 * 8, 256);
}

void launch_sparse_mla(int32_t num_rows, const int64_t* base, const uint16_t* qa, const uint16_t* kv,
                       const int32_t* idx, int32_t k, float softmax_scale, float* out, float* lse, void* ws,
                       hipStream_t stream, int32_t max_visible, bool pad_rows)
{
    const int s = attn_pick_splits(num_rows, k);
    const int tiles = (k + AT_TILE - 1) / AT_TILE;
    const int split_len = ((tiles + s - 1) / s) * AT_TILE;
    uint16_t* part_o = nullptr;
    float2* part_ml = nullptr;
    if (s > 1) {
        part_o = (uint16_t*)ws;
        part_ml = (float2*)((char*)ws + align_up((size_t)num_rows * s * 64 * 512 * 2, 256));
    }
    // Several splits only occur below 256 rows (attn_pick_splits), so their
    // one-dimensional grid stays small.
    const dim3 grid = s == 1 ? item_grid(1, num_rows) : dim3((unsigned)(((num_rows + 7) / 8) * 8 * s));
    // Selected positions lie below max_visible; pool rows (pad_rows) are not bounded.
    const bool off32 = !pad_rows && (uint64_t)max_visible * 1152 <= 0xffffffffull;
    if (off32)
        hipLaunchKernelGGL(sparse_mla_kernel<true>, grid, dim3(AT_THREADS), 0, stream, base, qa, kv, idx, k,
                           (int)num_rows, softmax_scale * LOG2E, split_len, s, 0, out, lse, part_o, part_ml);
    else
        hipLaunchKernelGGL(sparse_mla_kernel<false>, grid, dim3(AT_THREADS), 0, stream, base, qa, kv, idx, k,
                           (int)num_rows, softmax_scale * LOG2E, split_len, s, pad_rows ? 1 : 0, out, lse, part_o,
                           part_ml);
    if (s > 1)
        hipLaunchKernelGGL(sparse_mla_combine_kernel, item_grid(64, num_rows), dim3(128), 0, stream, part_o, part_ml,
                           s, (int)num_rows, out, lse);
}

}  // namespace dsa
