// cache_write.hip -- the cache rows of new tokens: the indexer key and the
// MLA latent row, computed from the hidden state and scattered into the two
// caches the path reads.
//
// Per token x (the 6144-d hidden state):
//  - indexer key ("GLM-5.1 架构深度拆解" CH3 §3.6 step 2):
//      k = LayerNorm_128(wk x), RoPE on dims 0..63, dims 64..127 unchanged;
//  - latent row (same page, CH4 §4.1 and §4.5 steps 2-3):
//      [c_kv || k_pe] = kv_a_proj_with_mqa x  (512 + 64),
//      row = [RMSNorm_512(c_kv) || RoPE(k_pe)];
//  - RoPE ("GLM-5.2 架构 QA" Q1.4): dims i and i + 32 of a 64-d block turn by
//    m * theta^(-2i/64), m the token's position (half-split pairing).
//
// Two kernels:
//  1. cw_gemm_kernel / cw_gemm_resident_kernel: Y = x [N x 6144] times
//     [wk; kv_a]^T [6144 x 704] on v_mfma_f32_16x16x32_bf16.  Both operands
//     are K-contiguous (hidden rows, weight rows), which is the MFMA operand
//     layout as is: 64 x 64 output tiles, 64-deep K stages in LDS (144-byte
//     pitch: the 16 rows a 16-byte operand read touches land on disjoint
//     banks).  K is split so that the grid fills the chip; each split writes
//     its own fp32 partial tile (no atomics).  With few tokens (decode: the
//     8.65 MB of weights are the traffic) each workgroup requests its whole
//     4-stage K chunk at once.
//  2. cw_epilogue_kernel: sums the splits in a fixed order,
//     applies LayerNorm / RMSNorm in fp32 and RoPE with angles formed and
//     reduced modulo 2 pi in fp64 (an fp32 angle loses ~0.06 rad at position
//     10^6), rounds to bf16
//     (round-to-nearest-even) and writes the two cache rows at the token's
//     slot.
#include <cmath>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int CW_HID = 6144;                 // hidden_size
constexpr int CW_KEY = 128;                  // index_head_dim
constexpr int CW_LAT = 512;                  // kv_lora_rank
constexpr int CW_ROW = 576;                  // latent row: 512 + 64 (qk_rope_head_dim)
constexpr int CW_COLS = CW_KEY + CW_ROW;     // 704 projected values per token
constexpr int CW_CT = CW_COLS / 64;          // 11 column tiles: 2 of wk, 9 of kv_a
constexpr int CW_TM = 64;                    // tokens per tile
constexpr int CW_TK = 64;                    // K per stage
constexpr int CW_PITCH = CW_TK + 8;          // staged row, bf16 elements (144 bytes)
constexpr int CW_STAGES = CW_HID / CW_TK;    // 96

__device__ __forceinline__ float wave_sum64(float v)
{
    // Butterfly: every lane ends with the bitwise same sum (each step adds the
    // same two values, in either order).
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    return (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
}

// Workgroup -> (column tile, token tile, K split).  Workgroups go to the 8
// XCDs round-robin; numbering the 11 column tiles of one (token tile, split)
// 8 apart puts them on one XCD, whose L2 then serves their shared hidden-state
// tile (only locality depends on this).  Numbers past the last pair exit.
struct CwTile {
    int ct, mt, s;
    bool live;
};
__device__ __forceinline__ CwTile cw_tile(int mtiles, int S)
{
    const int L = blockIdx.x, x = L & 7, i = L >> 3;
    const int pp = (i / CW_CT) * 8 + x;
    return CwTile{i % CW_CT, pp % mtiles, pp / mtiles, pp < mtiles * S};
}

// Loader: thread -> rows lr and lr + 32 of both 64-row tiles, 8 K values at lk.
struct CwLoader {
    const uint16_t *xa0, *xa1, *wb0, *wb1;
    int so0, so1;
    __device__ CwLoader(int N, int mt, int ct, int k0, const uint16_t* x, const uint16_t* wk, const uint16_t* kva)
    {
        const int tid = threadIdx.x, lr = tid >> 3, lk = (tid & 7) * 8;
        const int ra = min(mt * CW_TM + lr, N - 1), rb = min(mt * CW_TM + lr + 32, N - 1);  // ragged tail: clamp
        const uint16_t* W = ct < 2 ? wk + (size_t)ct * 64 * CW_HID : kva + (size_t)(ct - 2) * 64 * CW_HID;
        xa0 = x + (size_t)ra * CW_HID + k0 + lk;
        xa1 = x + (size_t)rb * CW_HID + k0 + lk;
        wb0 = W + (size_t)lr * CW_HID + k0 + lk;
        wb1 = W + (size_t)(lr + 32) * CW_HID + k0 + lk;
        so0 = lr * CW_PITCH + lk;
        so1 = (lr + 32) * CW_PITCH + lk;
    }
};

// One 64-deep stage of the wave's 32 x 32 tile (2 x 2 MFMA blocks).
__device__ __forceinline__ void cw_stage(const uint16_t* A, const uint16_t* B, int wr, int wc, int j, int g,
                                         floatx4 (&acc)[2][2])
{
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
        const int ko = kk * 32 + g * 8;
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(A + (wr + j) * CW_PITCH + ko));
        const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(A + (wr + 16 + j) * CW_PITCH + ko));
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(B + (wc + j) * CW_PITCH + ko));
        const bf16x8 b1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(B + (wc + 16 + j) * CW_PITCH + ko));
        acc[0][0] = mfma_16x16x32(a0, b0, acc[0][0]);
        acc[0][1] = mfma_16x16x32(a0, b1, acc[0][1]);
        acc[1][0] = mfma_16x16x32(a1, b0, acc[1][0]);
        acc[1][1] = mfma_16x16x32(a1, b1, acc[1][1]);
    }
}

// D lane layout: element v of block (a, b) is D[4g + v][j].
__device__ __forceinline__ void cw_store(float* part, int N, int mt, int ct, int s, int wr, int wc, int j, int g,
                                         const floatx4 (&acc)[2][2])
{
    float* P = part + (size_t)s * N * CW_COLS;
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int row = mt * CW_TM + wr + 16 * a + 4 * g + v;
            if (row < N) {
#pragma unroll
                for (int b = 0; b < 2; b++) P[(size_t)row * CW_COLS + ct * 64 + wc + 16 * b + j] = acc[a][b][v];
            }
        }
}

// Many K stages per workgroup: double-buffered LDS, next stage's loads in
// flight during the current stage's MFMAs.
__global__ __launch_bounds__(256) void cw_gemm_kernel(int N, int S, int mtiles, const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ wk,
                                                      const uint16_t* __restrict__ kva, float* __restrict__ part)
{
    const CwTile tl = cw_tile(mtiles, S);
    if (!tl.live) return;
    const int nstage = CW_STAGES / S;
    const CwLoader ld(N, tl.mt, tl.ct, tl.s * nstage * CW_TK, x, wk, kva);

    __shared__ __attribute__((aligned(16))) uint16_t sa[2][CW_TM * CW_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sb[2][64 * CW_PITCH];

    u32x4 ga0 = load_u32x4(ld.xa0), ga1 = load_u32x4(ld.xa1), gb0 = load_u32x4(ld.wb0), gb1 = load_u32x4(ld.wb1);
    *reinterpret_cast<u32x4*>(&sa[0][ld.so0]) = ga0;
    *reinterpret_cast<u32x4*>(&sa[0][ld.so1]) = ga1;
    *reinterpret_cast<u32x4*>(&sb[0][ld.so0]) = gb0;
    *reinterpret_cast<u32x4*>(&sb[0][ld.so1]) = gb1;
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32, j = lane & 15, g = lane >> 4;
    floatx4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int st = 0; st < nstage; st++) {
        const bool more = st + 1 < nstage;
        if (more) {
            const int off = (st + 1) * CW_TK;
            ga0 = load_u32x4(ld.xa0 + off);
            ga1 = load_u32x4(ld.xa1 + off);
            gb0 = load_u32x4(ld.wb0 + off);
            gb1 = load_u32x4(ld.wb1 + off);
        }
        cw_stage(sa[st & 1], sb[st & 1], wr, wc, j, g, acc);
        if (more) {
            const int nb = (st + 1) & 1;
            *reinterpret_cast<u32x4*>(&sa[nb][ld.so0]) = ga0;
            *reinterpret_cast<u32x4*>(&sa[nb][ld.so1]) = ga1;
            *reinterpret_cast<u32x4*>(&sb[nb][ld.so0]) = gb0;
            *reinterpret_cast<u32x4*>(&sb[nb][ld.so1]) = gb1;
        }
        __syncthreads();
    }
    cw_store(part, N, tl.mt, tl.ct, tl.s, wr, wc, j, g, acc);
}

// Few tokens (decode): every workgroup's whole K chunk (CW_RES stages) is
// requested at once and held in LDS, so a workgroup waits for memory once.
constexpr int CW_RES = 4;
__global__ __launch_bounds__(256) void cw_gemm_resident_kernel(int N, int mtiles, const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wk,
                                                               const uint16_t* __restrict__ kva,
                                                               float* __restrict__ part)
{
    constexpr int S = CW_STAGES / CW_RES;
    const CwTile tl = cw_tile(mtiles, S);
    if (!tl.live) return;
    const CwLoader ld(N, tl.mt, tl.ct, tl.s * CW_RES * CW_TK, x, wk, kva);

    __shared__ __attribute__((aligned(16))) uint16_t sa[CW_RES][CW_TM * CW_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sb[CW_RES][64 * CW_PITCH];

    u32x4 ga0[CW_RES], ga1[CW_RES], gb0[CW_RES], gb1[CW_RES];
#pragma unroll
    for (int st = 0; st < CW_RES; st++) {
        ga0[st] = load_u32x4(ld.xa0 + st * CW_TK);
        ga1[st] = load_u32x4(ld.xa1 + st * CW_TK);
        gb0[st] = load_u32x4(ld.wb0 + st * CW_TK);
        gb1[st] = load_u32x4(ld.wb1 + st * CW_TK);
    }
#pragma unroll
    for (int st = 0; st < CW_RES; st++) {
        *reinterpret_cast<u32x4*>(&sa[st][ld.so0]) = ga0[st];
        *reinterpret_cast<u32x4*>(&sa[st][ld.so1]) = ga1[st];
        *reinterpret_cast<u32x4*>(&sb[st][ld.so0]) = gb0[st];
        *reinterpret_cast<u32x4*>(&sb[st][ld.so1]) = gb1[st];
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32, j = lane & 15, g = lane >> 4;
    floatx4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < CW_RES; st++) cw_stage(sa[st], sb[st], wr, wc, j, g, acc);
    cw_store(part, N, tl.mt, tl.ct, tl.s, wr, wc, j, g, acc);
}

// Large batches: 128 x 128 output tiles, four waves of 64 x 64 (4 x 4 MFMA
// blocks each), no K split.  Each staged byte of A now feeds 128 columns and
// each of B 128 tokens (a 64 x 64 tile re-reads both from L2 twice as
// often), and a wave issues 8 LDS reads per 16 MFMAs instead of 8 per 8.
// Loads run three stages ahead through a register ring (the loop is unrolled
// by three so the ring slots are static and the compiler's wait counts exact),
// then move to a double-buffered LDS stage.  Column tile 0 is wk, tiles 1..5
// are kv_a rows 128 (t - 1) .. +127 (the last one half past row 575: those
// rows are clamped on load and their columns never stored).
constexpr int CB_T = 128;                      // tile rows and columns
constexpr int CB_CT = (CW_COLS + CB_T - 1) / CB_T;  // 6 column tiles
constexpr int CB_PITCH = CW_TK + 8;            // staged row, bf16 (144 bytes)
constexpr int CB_MIN_TOKENS = 2048;            // batches from this size take this kernel

struct CbLoader {
    const uint16_t* xa[4];
    const uint16_t* wb[4];
    int so[4];
    __device__ CbLoader(int N, int mt, int ct, const uint16_t* x, const uint16_t* wk, const uint16_t* kva)
    {
        const int tid = threadIdx.x, lr = tid >> 3, lk = (tid & 7) * 8;
        const uint16_t* W = ct == 0 ? wk : kva + (size_t)(ct - 1) * CB_T * CW_HID;
        const int wrows = ct == 0 ? CW_KEY : min(CB_T, CW_ROW - (ct - 1) * CB_T);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = lr + 32 * i;
            xa[i] = x + (size_t)min(mt * CB_T + r, N - 1) * CW_HID + lk;  // ragged tail: clamp
            wb[i] = W + (size_t)min(r, wrows - 1) * CW_HID + lk;
            so[i] = r * CB_PITCH + lk;
        }
    }
};

__global__ __launch_bounds__(256, 2) void cw_gemm_big_kernel(int N, int mtiles, const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wk,
                                                            const uint16_t* __restrict__ kva,
                                                            float* __restrict__ part)
{
    // Workgroup -> (column tile, token tile): the 6 column tiles of a token
    // tile are numbered 8 apart, so they share an XCD and its L2.
    const int L = blockIdx.x, xc = L & 7, i8 = L >> 3;
    const int ct = i8 % CB_CT, mt = (i8 / CB_CT) * 8 + xc;
    if (mt >= mtiles) return;
    const CbLoader ld(N, mt, ct, x, wk, kva);

    __shared__ __attribute__((aligned(16))) uint16_t sa[2][CB_T * CB_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sb[2][CB_T * CB_PITCH];

    u32x4 ra[3][4], rb[3][4];  // register ring: stage st lives in slot st % 3
    auto issue = [&](u32x4 (&a)[4], u32x4 (&b)[4], int st) {
        const int off = st * CW_TK;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            a[i] = load_u32x4(ld.xa[i] + off);
            b[i] = load_u32x4(ld.wb[i] + off);
        }
    };
    auto stage_to_lds = [&](const u32x4 (&a)[4], const u32x4 (&b)[4], int buf) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            *reinterpret_cast<u32x4*>(&sa[buf][ld.so[i]]) = a[i];
            *reinterpret_cast<u32x4*>(&sb[buf][ld.so[i]]) = b[i];
        }
    };

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64, j = lane & 15, g = lane >> 4;
    floatx4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto mfma_stage = [&](int buf) {
        const uint16_t* A = sa[buf];
        const uint16_t* B = sb[buf];
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
            const int ko = kk * 32 + g * 8;
            bf16x8 av[4], bv[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                av[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(A + (wr + 16 * q + j) * CB_PITCH + ko));
                bv[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(B + (wc + 16 * q + j) * CB_PITCH + ko));
            }
#pragma unroll
            for (int a = 0; a < 4; a++)
#pragma unroll
                for (int b = 0; b < 4; b++) acc[a][b] = mfma_16x16x32(av[a], bv[b], acc[a][b]);
        }
    };

    // Prologue: stages 0..2 requested, stage 0 staged.
    issue(ra[0], rb[0], 0);
    issue(ra[1], rb[1], 1);
    issue(ra[2], rb[2], 2);
    stage_to_lds(ra[0], rb[0], 0);
    __syncthreads();
    // Step st: request stage st + 3 into slot st % 3 (stage st is in LDS),
    // multiply stage st, stage st + 1 into the other LDS buffer.
    auto step = [&](int st, u32x4 (&a0)[4], u32x4 (&b0)[4], u32x4 (&a1)[4], u32x4 (&b1)[4]) {
        if (st + 3 < CW_STAGES) issue(a0, b0, st + 3);
        mfma_stage(st & 1);
        if (st + 1 < CW_STAGES) stage_to_lds(a1, b1, (st + 1) & 1);
        __syncthreads();
    };
    static_assert(CW_STAGES % 3 == 0, "the ring walks whole rounds");
    for (int st = 0; st < CW_STAGES; st += 3) {
        step(st, ra[0], rb[0], ra[1], rb[1]);
        step(st + 1, ra[1], rb[1], ra[2], rb[2]);
        step(st + 2, ra[2], rb[2], ra[0], rb[0]);
    }

    // D lane layout: element v of block (a, b) is D[4g + v][j].
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int row = mt * CB_T + wr + 16 * a + 4 * g + v;
            if (row < N) {
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    const int col = ct * CB_T + wc + 16 * b + j;
                    if (col < CW_COLS) part[(size_t)row * CW_COLS + col] = acc[a][b][v];
                }
            }
        }
}

// WPT waves per token (1, or 4 when K is split at least 4 ways).  Wave sub of
// a token sums splits [sub * per, (sub + 1) * per) in split order with every
// load issued first; with WPT = 4 the four partial sums meet in LDS and wave
// 0 adds them in wave order (a fixed order: results do not depend on timing).
// Wave 0 of a token then finishes it: lane l owns key dims 2l, 2l+1; c_kv
// dims 8l..8l+7; (lanes < 32) k_pe dims 2l, 2l+1.  In a 64-d RoPE block,
// dims 2l, 2l+1 of lane l < 16 pair with dims 2l+32, 2l+33 of lane l + 16.
struct CwSums {
    float k0, k1, p0, p1, c[8];
};

__device__ __forceinline__ void cw_add(CwSums& a, const float* row, int l)
{
    const float2 kk = *reinterpret_cast<const float2*>(row + 2 * l);
    const float4 u = *reinterpret_cast<const float4*>(row + CW_KEY + 8 * l);
    const float4 w = *reinterpret_cast<const float4*>(row + CW_KEY + 8 * l + 4);
    const float2 pp = l < 32 ? *reinterpret_cast<const float2*>(row + CW_KEY + CW_LAT + 2 * l) : float2{0.f, 0.f};
    a.k0 += kk.x; a.k1 += kk.y;
    a.c[0] += u.x; a.c[1] += u.y; a.c[2] += u.z; a.c[3] += u.w;
    a.c[4] += w.x; a.c[5] += w.y; a.c[6] += w.z; a.c[7] += w.w;
    a.p0 += pp.x; a.p1 += pp.y;
}

constexpr int CW_SUM_BATCH = 8;  // splits whose loads are in flight together

// theta^(-i/32) for the 32 RoPE pairs, formed on the host in fp64.
struct CwInvFreq {
    double f[32];
};

// cos and sin of m * f: the product and its reduction modulo 2 pi in fp64 (2 pi
// split in two doubles, so the remainder keeps ~1e-16 relative accuracy for
// any int32 m), then fp32 sincos of a value within [-pi, pi].
__device__ __forceinline__ void cw_angle(int32_t m, double f, float& c, float& s)
{
    constexpr double kTwoPiHi = 6.283185307179586;       // 2 pi rounded to double
    constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2 pi - kTwoPiHi
    const double a = (double)m * f;
    const double k = rint(a * (1.0 / kTwoPiHi));
    const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, a));
    sincosf((float)r, &s, &c);
}

__global__ __launch_bounds__(256) void cw_epilogue_kernel(int N, int S, int WPT, const float* __restrict__ part,
                                                          const float* __restrict__ kg, const float* __restrict__ kb,
                                                          float keps, const float* __restrict__ kvg, float kveps,
                                                          const int32_t* __restrict__ pos,
                                                          const int64_t* __restrict__ slots, CwInvFreq inv_freq,
                                                          uint16_t* __restrict__ kcache, uint16_t* __restrict__ lcache)
{
    __shared__ float xs[3][64][12];
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, sub = wave % WPT;
    const int t = blockIdx.x * (4 / WPT) + wave / WPT;
    if (t >= N) return;  // uniform over the token's waves (with WPT = 4, the whole workgroup)
    // Every load that does not depend on another is issued here, so the wave
    // waits for memory about once.
    const int64_t slot = slots[t];
    const int32_t m = pos[t];
    const float2 kg2 = *reinterpret_cast<const float2*>(kg + 2 * l);
    const float2 kb2 = *reinterpret_cast<const float2*>(kb + 2 * l);
    const float4 g0 = *reinterpret_cast<const float4*>(kvg + 8 * l);
    const float4 g1 = *reinterpret_cast<const float4*>(kvg + 8 * l + 4);

    CwSums a = {};
    const int per = (S + WPT - 1) / WPT, s_lo = sub * per, s_hi = min(S, s_lo + per);
    for (int s0 = s_lo; s0 < s_hi; s0 += CW_SUM_BATCH) {
        CwSums b[CW_SUM_BATCH];
#pragma unroll
        for (int e = 0; e < CW_SUM_BATCH; e++) {
            b[e] = CwSums{};
            if (s0 + e < s_hi) cw_add(b[e], part + ((size_t)(s0 + e) * N + t) * CW_COLS, l);
        }
#pragma unroll
        for (int e = 0; e < CW_SUM_BATCH; e++) {
            if (s0 + e < s_hi) {
                a.k0 += b[e].k0; a.k1 += b[e].k1; a.p0 += b[e].p0; a.p1 += b[e].p1;
#pragma unroll
                for (int q = 0; q < 8; q++) a.c[q] += b[e].c[q];
            }
        }
    }
    if (WPT > 1) {
        if (sub > 0) {
            float* d = xs[sub - 1][l];
            d[0] = a.k0; d[1] = a.k1; d[2] = a.p0; d[3] = a.p1;
#pragma unroll
            for (int q = 0; q < 8; q++) d[4 + q] = a.c[q];
        }
        __syncthreads();
        if (sub > 0) return;
#pragma unroll
        for (int w = 0; w < 3; w++) {
            const float* d = xs[w][l];
            a.k0 += d[0]; a.k1 += d[1]; a.p0 += d[2]; a.p1 += d[3];
#pragma unroll
            for (int q = 0; q < 8; q++) a.c[q] += d[4 + q];
        }
    }

    if (slot < 0) return;  // wave-uniform: a padding token writes nothing

    // RoPE angles of this lane's two dims (lanes < 32; pair index = dim mod 32).
    float cs0 = 1.f, sn0 = 0.f, cs1 = 1.f, sn1 = 0.f;
    if (l < 32) {
        cw_angle(m, inv_freq.f[(2 * l) & 31], cs0, sn0);
        cw_angle(m, inv_freq.f[(2 * l + 1) & 31], cs1, sn1);
    }
    const float sgn = l < 16 ? -1.f : 1.f;  // first half: x cos - x' sin; second half: x cos + x' sin

    // Indexer key: LayerNorm over 128, then RoPE on dims 0..63.
    const float mean = wave_sum64(a.k0 + a.k1) * (1.f / CW_KEY);
    const float d0 = a.k0 - mean, d1 = a.k1 - mean;
    const float var = wave_sum64(d0 * d0 + d1 * d1) * (1.f / CW_KEY);
    const float inv = 1.f / sqrtf(var + keps);
    float y0 = d0 * inv * kg2.x + kb2.x;
    float y1 = d1 * inv * kg2.y + kb2.y;
    const float q0 = __shfl_xor(y0, 16, 64), q1 = __shfl_xor(y1, 16, 64);
    if (l < 32) {
        y0 = y0 * cs0 + sgn * q0 * sn0;
        y1 = y1 * cs1 + sgn * q1 * sn1;
    }
    *reinterpret_cast<uint32_t*>(kcache + (size_t)slot * CW_KEY + 2 * l) = pack_bf16x2(y0, y1);

    // Latent row: RMSNorm over c_kv, RoPE on k_pe.
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) ss += a.c[e] * a.c[e];
    const float rinv = 1.f / sqrtf(wave_sum64(ss) * (1.f / CW_LAT) + kveps);
    u32x4 o;
    o[0] = pack_bf16x2(a.c[0] * rinv * g0.x, a.c[1] * rinv * g0.y);
    o[1] = pack_bf16x2(a.c[2] * rinv * g0.z, a.c[3] * rinv * g0.w);
    o[2] = pack_bf16x2(a.c[4] * rinv * g1.x, a.c[5] * rinv * g1.y);
    o[3] = pack_bf16x2(a.c[6] * rinv * g1.z, a.c[7] * rinv * g1.w);
    uint16_t* lrow = lcache + (size_t)slot * CW_ROW;
    *reinterpret_cast<u32x4*>(lrow + 8 * l) = o;
    const float r0 = __shfl_xor(a.p0, 16, 64), r1 = __shfl_xor(a.p1, 16, 64);
    if (l < 32) {
        const float z0 = a.p0 * cs0 + sgn * r0 * sn0;
        const float z1 = a.p1 * cs1 + sgn * r1 * sn1;
        *reinterpret_cast<uint32_t*>(lrow + CW_LAT + 2 * l) = pack_bf16x2(z0, z1);
    }
}

int cw_row_tiles(int32_t n) { return (n + CW_TM - 1) / CW_TM; }

}  // namespace

// K splits.  Few token tiles (<= 3): the resident kernel, K in 24 chunks of
// 4 stages.  Otherwise the smallest split (a divisor of 96) that gives at
// least 512 workgroups, each split at least 8 stages deep.
int cache_write_splits(int32_t num_tokens)
{
    if (num_tokens >= CB_MIN_TOKENS) return 1;  // the 128 x 128 kernel
    const int mtiles = cw_row_tiles(num_tokens);
    if (mtiles <= 3) return CW_STAGES / CW_RES;
    static const int kDiv[] = {1, 2, 3, 4, 6, 8, 12};
    for (int d : kDiv)
        if (mtiles * CW_CT * d >= 512) return d;
    return 12;
}

size_t cache_write_workspace_bytes(int32_t num_tokens)
{
    return align_up((size_t)cache_write_splits(num_tokens) * num_tokens * CW_COLS * sizeof(float), 256);
}

void launch_cache_write(int32_t num_tokens, const uint16_t* hidden, const uint16_t* wk, const float* k_norm_weight,
                        const float* k_norm_bias, float k_norm_eps, const uint16_t* kv_a, const float* kv_norm_weight,
                        float kv_norm_eps, const int32_t* positions, const int64_t* slots, double rope_theta,
                        uint16_t* k_idx_cache, uint16_t* kv_latent_cache, void* ws, hipStream_t stream)
{
    const int S = cache_write_splits(num_tokens);
    const int mtiles = cw_row_tiles(num_tokens);
    const int pairs8 = (mtiles * S + 7) / 8 * 8;  // (token tile, split) pairs, padded to whole XCD rounds
    float* part = reinterpret_cast<float*>(ws);
    if (num_tokens >= CB_MIN_TOKENS) {
        const int mt128 = (num_tokens + CB_T - 1) / CB_T;
        const int rounds = (mt128 + 7) / 8;  // token tiles per XCD slot, padded to whole rounds
        hipLaunchKernelGGL(cw_gemm_big_kernel, dim3(CB_CT * 8 * rounds), dim3(256), 0, stream, (int)num_tokens,
                           mt128, hidden, wk, kv_a, part);
    } else if (S == CW_STAGES / CW_RES)
        hipLaunchKernelGGL(cw_gemm_resident_kernel, dim3(CW_CT * pairs8), dim3(256), 0, stream, (int)num_tokens,
                           mtiles, hidden, wk, kv_a, part);
    else
        hipLaunchKernelGGL(cw_gemm_kernel, dim3(CW_CT * pairs8), dim3(256), 0, stream, (int)num_tokens, S, mtiles,
                           hidden, wk, kv_a, part);
    CwInvFreq inv_freq;
    for (int i = 0; i < 32; i++) inv_freq.f[i] = std::pow(rope_theta, -(double)i / 32.0);
    const int wpt = S >= 4 ? 4 : 1;
    const int tok_per_wg = 4 / wpt;
    hipLaunchKernelGGL(cw_epilogue_kernel, dim3((num_tokens + tok_per_wg - 1) / tok_per_wg), dim3(256), 0, stream,
                       (int)num_tokens, S, wpt, (const float*)part, k_norm_weight, k_norm_bias, k_norm_eps,
                       kv_norm_weight, kv_norm_eps, positions, slots, inv_freq, k_idx_cache, kv_latent_cache);
}

}  // namespace dsa
