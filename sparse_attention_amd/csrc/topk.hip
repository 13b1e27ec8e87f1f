// topk.hip -- deterministic causal top-k over fp32 score rows on gfx950.
//
// Selects, for each row, k_r = min(k, n_r) positions of scores[r, 0:n_r) with
// the largest scores, returned in ascending position order and padded with
// -1 ("GLM-5.1 架构深度拆解" §3.6 step 7 and §3.4, which require a
// deterministic top-k; GLM-5 explainer: the top-k is a set of positions and
// rows shorter than 2,048 keep every position).  Order: larger score first,
// -0.0 == +0.0, equal scores go to the lower position, NaN lowest.
//
// Design: a radix select on the order-preserving 32-bit key of each score.
// Rows of at most 65,536 positions take one 1024-thread workgroup each (one
// streaming pass over the row, the rest in LDS; see topk_rows_kernel).
// Longer rows are split over workgroups, because a single CU streams too
// slowly for them; only integer counts are combined across workgroups, so the
// result does not depend on scheduling:
//   1. zero     per-row histogram and counters
//   2. hist     rows x chunks: LDS histogram of the top 12 key bits, merged
//               into the row histogram with integer atomics
//   3. filter   rows x chunks: every workgroup finds the same threshold bin b0
//               from the row histogram; counts the chunk's elements above b0
//               and appends the elements inside b0 (candidates) to a per-row
//               candidate list
//   4. resolve  one workgroup per row: radix-selects the remaining 20 key bits
//               among the candidates (or, if they overflowed the list, among
//               the row itself) to get the exact threshold key theta and the
//               number need_eq of theta-valued elements to keep; then turns
//               per-chunk counts into per-chunk output offsets
//   5. write    rows x chunks: ordered compaction; an element is kept if its
//               key exceeds theta, or equals theta and fewer than need_eq
//               theta-valued elements precede it in position order
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int TK_THREADS = 256;
constexpr int TK_PER_THREAD = TK_CHUNK / TK_THREADS;  // 16
constexpr int RS_THREADS = 512;

// Row state words.
constexpr int RS_CAND = 0, RS_B0 = 1, RS_GT0 = 2, RS_THETA = 3, RS_NEEDEQ = 4;
// Chunk state words.
constexpr int CS_GTBIN = 0, CS_OFFSET = 1, CS_EQBEFORE = 2;

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64).
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total, uint32_t* sh /*[NT/64]*/)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; i++) {
        uint32_t t = sh[i];
        before += (i < wave) ? t : 0u;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

// Finds, in a histogram h[0..B) (larger bin = larger key), the bin b holding
// the need-th largest element (need >= 1, need <= sum of h): the number of
// elements in bins above b is < need and including b is >= need.  Returns b
// and the count strictly above it via shared outputs.  NT threads, B a
// multiple of NT.
template <int NT, int B>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* h, uint32_t need, uint32_t* out_bin,
                                                   uint32_t* out_above, uint32_t* sh)
{
    constexpr int PER = B / NT;
    const int t = threadIdx.x;
    // Thread t owns bins [B - PER (t+1), B - PER t), scanned from the top.
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) mine += h[B - 1 - (PER * t + i)];
    uint32_t total;
    uint32_t pre = block_exclusive_scan<NT>(mine, &total, sh);
    if (pre < need && pre + mine >= need) {
        uint32_t acc = pre;
        for (int i = 0; i < PER; i++) {
            const int b = B - 1 - (PER * t + i);
            if (acc + h[b] >= need) {
                *out_bin = (uint32_t)b;
                *out_above = acc;
                break;
            }
            acc += h[b];
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t* __restrict__ hist, uint32_t* __restrict__ rowst)
{
    const int r = blockIdx.x;
    uint32_t* h = hist + (int64_t)r * TK_BINS;
    for (int i = threadIdx.x; i < TK_BINS; i += 256) h[i] = 0u;
    if (threadIdx.x < TK_ROWST) rowst[(int64_t)r * TK_ROWST + threadIdx.x] = 0u;
}

// Loads the TK_PER_THREAD keys of thread `tid` in chunk [start, end): thread
// tid owns positions start + 16 tid .. +15 (position order = thread order).
// Keys of positions >= end are returned as "absent".
__device__ __forceinline__ void load_chunk_keys(const float* __restrict__ row, int start, int end,
                                                uint32_t (&key)[TK_PER_THREAD], uint32_t& present)
{
    const int t0 = start + TK_PER_THREAD * threadIdx.x;
    present = 0u;
#pragma unroll
    for (int q4 = 0; q4 < TK_PER_THREAD / 4; q4++) {
        const int t = t0 + 4 * q4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        // A 4-aligned group starting below `end` lies inside the row
        // allocation because ld is a multiple of 4 and end <= ld.
        if (t < end) v = *reinterpret_cast<const float4*>(row + t);
        key[4 * q4 + 0] = score_key(v.x);
        key[4 * q4 + 1] = score_key(v.y);
        key[4 * q4 + 2] = score_key(v.z);
        key[4 * q4 + 3] = score_key(v.w);
#pragma unroll
        for (int e = 0; e < 4; e++)
            if (t + e < end) present |= 1u << (4 * q4 + e);
    }
}

__global__ __launch_bounds__(TK_THREADS) void topk_hist_kernel(const int32_t* __restrict__ vis,
                                                               const float* __restrict__ scores, int64_t ld, int k,
                                                               uint32_t* __restrict__ hist, int min_n)
{
    const int r = blockIdx.y;
    const int n = vis[r];
    const int start = blockIdx.x * TK_CHUNK;
    if (n <= k || n <= min_n || start >= n) return;
    const int end = min(n, start + TK_CHUNK);
    __shared__ uint32_t h[TK_BINS];
    for (int i = threadIdx.x; i < TK_BINS; i += TK_THREADS) h[i] = 0u;
    __syncthreads();
    uint32_t key[TK_PER_THREAD], present;
    load_chunk_keys(scores + (int64_t)r * ld, start, end, key, present);
#pragma unroll
    for (int i = 0; i < TK_PER_THREAD; i++)
        if (present & (1u << i)) atomicAdd(&h[key[i] >> 20], 1u);
    __syncthreads();
    uint32_t* gh = hist + (int64_t)r * TK_BINS;
    for (int i = threadIdx.x; i < TK_BINS; i += TK_THREADS)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

__global__ __launch_bounds__(TK_THREADS) void topk_filter_kernel(const int32_t* __restrict__ vis,
                                                                 const float* __restrict__ scores, int64_t ld, int k,
                                                                 const uint32_t* __restrict__ hist,
                                                                 uint32_t* __restrict__ rowst,
                                                                 uint32_t* __restrict__ chunkst, int chunks,
                                                                 unsigned long long* __restrict__ cand, int min_n)
{
    const int r = blockIdx.y;
    const int c = blockIdx.x;
    const int n = vis[r];
    const int start = c * TK_CHUNK;
    if (n <= k || n <= min_n || start >= n) return;
    const int end = min(n, start + TK_CHUNK);
    __shared__ uint32_t h[TK_BINS];
    __shared__ uint32_t sh[TK_THREADS / 64];
    __shared__ uint32_t s_b0, s_gt0, s_base;
    const uint32_t* gh = hist + (int64_t)r * TK_BINS;
    for (int i = threadIdx.x; i < TK_BINS; i += TK_THREADS) h[i] = gh[i];
    __syncthreads();
    find_threshold_bin<TK_THREADS, TK_BINS>(h, (uint32_t)k, &s_b0, &s_gt0, sh);
    const uint32_t b0 = s_b0;

    uint32_t key[TK_PER_THREAD], present;
    load_chunk_keys(scores + (int64_t)r * ld, start, end, key, present);
    uint32_t gt = 0, nc = 0;
#pragma unroll
    for (int i = 0; i < TK_PER_THREAD; i++) {
        if (!(present & (1u << i))) continue;
        const uint32_t b = key[i] >> 20;
        gt += (b > b0) ? 1u : 0u;
        nc += (b == b0) ? 1u : 0u;
    }
    uint32_t gt_total, nc_total;
    (void)block_exclusive_scan<TK_THREADS>(gt, &gt_total, sh);
    const uint32_t nc_pre = block_exclusive_scan<TK_THREADS>(nc, &nc_total, sh);
    if (threadIdx.x == 0) {
        s_base = nc_total ? atomicAdd(&rowst[(int64_t)r * TK_ROWST + RS_CAND], nc_total) : 0u;
        chunkst[((int64_t)r * chunks + c) * TK_CHUNKST + CS_GTBIN] = gt_total;
        if (c == 0) {
            rowst[(int64_t)r * TK_ROWST + RS_B0] = b0;
            rowst[(int64_t)r * TK_ROWST + RS_GT0] = s_gt0;
        }
    }
    __syncthreads();
    uint32_t slot = s_base + nc_pre;
    unsigned long long* cr = cand + (int64_t)r * TK_CAP;
    const int t0 = start + TK_PER_THREAD * threadIdx.x;
#pragma unroll
    for (int i = 0; i < TK_PER_THREAD; i++) {
        if (!(present & (1u << i))) continue;
        if ((key[i] >> 20) != b0) continue;
        if (slot < (uint32_t)TK_CAP) cr[slot] = ((unsigned long long)key[i] << 32) | (uint32_t)(t0 + i);
        slot++;
    }
}

// One workgroup per row (rows with n > k only).
__global__ __launch_bounds__(RS_THREADS) void topk_resolve_kernel(const int32_t* __restrict__ vis,
                                                                  const float* __restrict__ scores, int64_t ld,
                                                                  int k, uint32_t* __restrict__ rowst,
                                                                  uint32_t* __restrict__ chunkst, int chunks,
                                                                  const unsigned long long* __restrict__ cand, int min_n)
{
    const int r = blockIdx.x;
    const int n = vis[r];
    if (n <= k || n <= min_n) return;
    __shared__ unsigned long long cl[TK_CAP];
    __shared__ uint32_t h[TK_BINS];
    __shared__ uint32_t cgt[TK_MAX_CHUNKS / 2];  // per-chunk counts, see note below
    __shared__ uint32_t ceq[TK_MAX_CHUNKS / 2];
    __shared__ uint32_t sh[RS_THREADS / 64];
    __shared__ uint32_t s_bin, s_above;

    uint32_t* rs = rowst + (int64_t)r * TK_ROWST;
    const uint32_t m = rs[RS_CAND];
    const uint32_t b0 = rs[RS_B0];
    const uint32_t need = (uint32_t)k - rs[RS_GT0];
    const bool overflow = m > (uint32_t)TK_CAP;
    const float* row = scores + (int64_t)r * ld;
    const int nch = (n + TK_CHUNK - 1) / TK_CHUNK;

    if (!overflow)
        for (uint32_t i = threadIdx.x; i < m; i += RS_THREADS) cl[i] = cand[(int64_t)r * TK_CAP + i];

    // Digit 2: key bits 19..8 among elements whose top 12 bits equal b0.
    for (int i = threadIdx.x; i < TK_BINS; i += RS_THREADS) h[i] = 0u;
    __syncthreads();
    if (!overflow) {
        for (uint32_t i = threadIdx.x; i < m; i += RS_THREADS) {
            const uint32_t key = (uint32_t)(cl[i] >> 32);
            atomicAdd(&h[(key >> 8) & 0xfffu], 1u);
        }
    } else {
        for (int t = threadIdx.x; t < n; t += RS_THREADS) {
            const uint32_t key = score_key(row[t]);
            if ((key >> 20) == b0) atomicAdd(&h[(key >> 8) & 0xfffu], 1u);
        }
    }
    __syncthreads();
    find_threshold_bin<RS_THREADS, TK_BINS>(h, need, &s_bin, &s_above, sh);
    const uint32_t b1 = s_bin;
    const uint32_t need2 = need - s_above;
    const uint32_t pre20 = (b0 << 12) | b1;  // top 24 bits of theta

    // Digit 3: key bits 7..0 among elements whose top 24 bits equal pre20.
    for (int i = threadIdx.x; i < 512; i += RS_THREADS) h[i] = 0u;
    __syncthreads();
    if (!overflow) {
        for (uint32_t i = threadIdx.x; i < m; i += RS_THREADS) {
            const uint32_t key = (uint32_t)(cl[i] >> 32);
            if ((key >> 8) == pre20) atomicAdd(&h[key & 0xffu], 1u);
        }
    } else {
        for (int t = threadIdx.x; t < n; t += RS_THREADS) {
            const uint32_t key = score_key(row[t]);
            if ((key >> 8) == pre20) atomicAdd(&h[key & 0xffu], 1u);
        }
    }
    __syncthreads();
    find_threshold_bin<RS_THREADS, 512>(h, need2, &s_bin, &s_above, sh);
    const uint32_t theta = (pre20 << 8) | s_bin;
    const uint32_t need_eq = need2 - s_above;

    // Per-chunk counts, inside bin b0, of keys > theta and keys == theta.
    // Chunks are processed in windows of TK_MAX_CHUNKS / 2 to bound LDS.
    uint32_t offs = 0, eqb = 0;  // running totals (thread 0)
    for (int w0 = 0; w0 < nch; w0 += TK_MAX_CHUNKS / 2) {
        const int w1 = min(nch, w0 + TK_MAX_CHUNKS / 2);
        for (int i = threadIdx.x; i < w1 - w0; i += RS_THREADS) {
            cgt[i] = 0u;
            ceq[i] = 0u;
        }
        __syncthreads();
        if (!overflow) {
            for (uint32_t i = threadIdx.x; i < m; i += RS_THREADS) {
                const uint32_t key = (uint32_t)(cl[i] >> 32);
                const int pos = (int)(uint32_t)cl[i];
                const int cc = pos / TK_CHUNK;
                if (cc < w0 || cc >= w1) continue;
                if (key > theta) atomicAdd(&cgt[cc - w0], 1u);
                else if (key == theta) atomicAdd(&ceq[cc - w0], 1u);
            }
        } else {
            const int t_end = min(n, w1 * TK_CHUNK);
            for (int t = w0 * TK_CHUNK + threadIdx.x; t < t_end; t += RS_THREADS) {
                const uint32_t key = score_key(row[t]);
                if ((key >> 20) != b0) continue;
                const int cc = t / TK_CHUNK - w0;
                if (key > theta) atomicAdd(&cgt[cc], 1u);
                else if (key == theta) atomicAdd(&ceq[cc], 1u);
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int cc = w0; cc < w1; cc++) {
                uint32_t* cs = chunkst + ((int64_t)r * chunks + cc) * TK_CHUNKST;
                const uint32_t gtc = cs[CS_GTBIN] + cgt[cc - w0];
                const uint32_t eqc = ceq[cc - w0];
                const uint32_t left = need_eq > eqb ? need_eq - eqb : 0u;
                const uint32_t take = left < eqc ? left : eqc;
                cs[CS_OFFSET] = offs;
                cs[CS_EQBEFORE] = eqb;
                offs += gtc + take;
                eqb += eqc;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        rs[RS_THETA] = theta;
        rs[RS_NEEDEQ] = need_eq;
    }
}

__global__ __launch_bounds__(TK_THREADS) void topk_write_kernel(const int32_t* __restrict__ vis,
                                                                const float* __restrict__ scores, int64_t ld, int k,
                                                                const uint32_t* __restrict__ rowst,
                                                                const uint32_t* __restrict__ chunkst, int chunks,
                                                                int32_t* __restrict__ indices, int min_n)
{
    const int r = blockIdx.y;
    const int c = blockIdx.x;
    const int n = vis[r];
    if (n <= min_n) return;  // the one-workgroup-per-row kernel owns this row
    const int start = c * TK_CHUNK;
    int32_t* out = indices + (int64_t)r * k;
    if (n <= k) {
        // Every visible position is kept; chunk 0 also writes the padding.
        for (int t = start + threadIdx.x; t < min(n, start + TK_CHUNK); t += TK_THREADS) out[t] = t;
        if (c == 0)
            for (int t = n + threadIdx.x; t < k; t += TK_THREADS) out[t] = -1;
        return;
    }
    if (start >= n) return;
    const int end = min(n, start + TK_CHUNK);
    __shared__ uint32_t sh[TK_THREADS / 64];
    const uint32_t theta = rowst[(int64_t)r * TK_ROWST + RS_THETA];
    const uint32_t need_eq = rowst[(int64_t)r * TK_ROWST + RS_NEEDEQ];
    const uint32_t* cs = chunkst + ((int64_t)r * chunks + c) * TK_CHUNKST;
    const uint32_t offs = cs[CS_OFFSET];
    const uint32_t eqb = cs[CS_EQBEFORE];

    uint32_t key[TK_PER_THREAD], present;
    load_chunk_keys(scores + (int64_t)r * ld, start, end, key, present);
    uint32_t neq = 0;
#pragma unroll
    for (int i = 0; i < TK_PER_THREAD; i++) neq += ((present >> i) & 1u) && key[i] == theta;
    uint32_t tot;
    uint32_t eq_rank = eqb + block_exclusive_scan<TK_THREADS>(neq, &tot, sh);
    uint32_t keep = 0u;
#pragma unroll
    for (int i = 0; i < TK_PER_THREAD; i++) {
        if (!((present >> i) & 1u)) continue;
        if (key[i] > theta) keep |= 1u << i;
        else if (key[i] == theta) {
            if (eq_rank < need_eq) keep |= 1u << i;
            eq_rank++;
        }
    }
    const uint32_t nk = __popc(keep);
    uint32_t pos = offs + block_exclusive_scan<TK_THREADS>(nk, &tot, sh);
    const int t0 = start + TK_PER_THREAD * threadIdx.x;
#pragma unroll
    for (int i = 0; i < TK_PER_THREAD; i++)
        if ((keep >> i) & 1u) {
            // The counts guarantee pos < k; the bound keeps a logic slip from
            // writing outside the row.
            if (pos < (uint32_t)k) out[pos] = t0 + i;
            pos++;
        }
}

// ---------------------------------------------------------------------------
// One workgroup per row, for rows of at most TR_MAXN positions.
//
// Fast path (sampled bound):
//   1. A strided sample of about 4096 scores gives a conservative lower bound
//      theta_lo on the k-th largest key: the lower edge of the 12-bit key bin
//      holding the sample's rho-th largest, rho about 1.5x the rank the k-th
//      largest has in the sample plus a margin.
//   2. One streaming pass appends every element with key >= theta_lo
//      (key, position) to its wave's private segment of an LDS candidate list
//      (a wave-uniform counter: no atomics).
//   3. If at least k candidates were found and no segment overflowed, the k-th
//      largest key lies among them, and a radix select over the candidates
//      alone is exact.  Its bins are taken relative to the candidates' own key
//      range (12 bits per round, at most three rounds), which spreads them
//      over the histogram instead of piling onto a few hot bins.
// Fallback (exact for any input, e.g. huge tie groups or a misleading
// sample): an LDS histogram of the top 12 key bits of the whole row gives the
// threshold bin b0; elements above b0 go straight to the result bitmap and
// those inside b0 become the candidates (if they overflow, the radix rounds
// rescan the row instead of the list).
// Finally candidates above theta join a position bitmap, theta-valued ones go
// to a tie bitmap, and an ordered pass over the bitmaps (one block scan for
// ties, one for output offsets) keeps the first need_eq ties in position
// order and writes the selected positions in ascending order.
constexpr int TR_THREADS = 1024;
constexpr int TR_WAVES = TR_THREADS / 64;
constexpr int TR_SEG = 512;                    // candidate slots per wave
constexpr int TR_CAP = TR_SEG * TR_WAVES;      // 8192
constexpr int TR_BATCH = 8;  // 16-byte loads in flight per thread in row passes

// Appends (key, t) to the calling wave's segment; `count` is the wave's
// (uniform) fill level.  Must be called by every lane of the wave.
__device__ __forceinline__ void append_candidate(bool want, uint32_t key, int t, uint32_t& count,
                                                 unsigned long long* seg)
{
    const unsigned long long m = __ballot(want);
    if (m == 0) return;
    const int lane = threadIdx.x & 63;
    if (want) {
        const uint32_t slot = count + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
        if (slot < (uint32_t)TR_SEG) seg[slot] = ((unsigned long long)key << 32) | (uint32_t)t;
    }
    count += (uint32_t)__popcll(m);
}

// Visits every candidate: wave segments are dense prefixes of length segn[w].
template <class F>
__device__ __forceinline__ void for_each_candidate(const unsigned long long* cand, const uint32_t* segn, F f)
{
    for (int i = threadIdx.x; i < TR_CAP; i += TR_THREADS) {
        const int w = i / TR_SEG;
        if ((uint32_t)(i - w * TR_SEG) < segn[w]) f(cand[i]);
    }
}

__device__ __forceinline__ int bitlen(uint32_t x) { return x ? 32 - __clz(x) : 0; }

__global__ __launch_bounds__(TR_THREADS) void topk_rows_kernel(const int32_t* __restrict__ vis,
                                                               const float* __restrict__ scores, int64_t ld,
                                                               int k, int32_t* __restrict__ indices, int max_n)
{
    const int r = blockIdx.x;
    const int n = vis[r];
    if (n > max_n) return;  // the multi-workgroup kernels own this row
    int32_t* out = indices + (int64_t)r * k;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    if (n <= k) {
        for (int t = tid; t < k; t += TR_THREADS) out[t] = t < n ? t : -1;
        return;
    }
    __shared__ uint32_t hist[TK_BINS];
    __shared__ uint32_t gtbits[TR_MAXN / 32];
    __shared__ uint32_t eqbits[TR_MAXN / 32];
    __shared__ unsigned long long cand[TR_CAP];
    __shared__ uint32_t segn[TR_WAVES];
    __shared__ uint32_t sh[TR_THREADS / 64];
    __shared__ uint32_t s_bin, s_above, s_max;

    const int nwords = (n + 31) >> 5;
    const float* row = scores + (int64_t)r * ld;
    unsigned long long* seg = cand + wave * TR_SEG;
    for (int i = tid; i < TK_BINS; i += TR_THREADS) hist[i] = 0u;
    for (int i = tid; i < nwords; i += TR_THREADS) {
        gtbits[i] = 0u;
        eqbits[i] = 0u;
    }
    if (tid == 0) s_max = 0u;
    __syncthreads();

    // ---- 1. sampled lower bound -------------------------------------------
    const int stride = max(1, n >> 12);
    const int msamp = (n + stride - 1) / stride;
    const uint32_t rho = (uint32_t)min((int64_t)msamp, ((int64_t)3 * k * msamp) / (2 * (int64_t)n) + 32);
#pragma unroll 4
    for (int i = tid; i < msamp; i += TR_THREADS) atomicAdd(&hist[score_key(row[(int64_t)i * stride]) >> 20], 1u);
    __syncthreads();
    find_threshold_bin<TR_THREADS, TK_BINS>(hist, rho, &s_bin, &s_above, sh);
    const uint32_t theta_lo = (rho >= (uint32_t)msamp) ? 0u : (s_bin << 20);

    // ---- 2. filter pass ------------------------------------------------------
    // TR_BATCH independent 16-byte loads per thread are issued before any is
    // used, so each wave keeps several KB in flight.
    uint32_t count = 0;  // wave-uniform
    for (int bb = 0; bb < n; bb += 4 * TR_THREADS * TR_BATCH) {
        float4 v[TR_BATCH];
#pragma unroll
        for (int u = 0; u < TR_BATCH; u++) {
            const int b = bb + 4 * (tid + TR_THREADS * u);
            // A 4-aligned group starting below n lies inside the row
            // allocation because ld is a multiple of 4 and n <= ld.
            v[u] = b < n ? *reinterpret_cast<const float4*>(row + b) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < TR_BATCH; u++) {
            const int b = bb + 4 * (tid + TR_THREADS * u);
            const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint32_t key = score_key(e[q]);
                append_candidate(b + q < n && key >= theta_lo, key, b + q, count, seg);
            }
        }
    }
    if (lane == 0) segn[wave] = count;
    __syncthreads();
    uint32_t total = 0;
    bool seg_over = false;
#pragma unroll
    for (int w = 0; w < TR_WAVES; w++) {
        total += segn[w];
        seg_over |= segn[w] > (uint32_t)TR_SEG;
    }
    const bool fast = total >= (uint32_t)k && !seg_over;

    uint32_t need = (uint32_t)k;
    uint32_t lo, hi;            // every key still in play lies in [lo, hi]
    bool from_row = false;      // candidates overflowed: rescan the row
    if (fast) {
        lo = theta_lo;
        uint32_t mx = 0;
        for_each_candidate(cand, segn, [&](unsigned long long c) { mx = max(mx, (uint32_t)(c >> 32)); });
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d));
        if (lane == 0) atomicMax(&s_max, mx);
        __syncthreads();
        hi = s_max;
    } else {
        // ---- fallback: whole-row histogram --------------------------------
        for (int i = tid; i < TK_BINS; i += TR_THREADS) hist[i] = 0u;
        __syncthreads();
        for (int bb = 0; bb < n; bb += 4 * TR_THREADS * TR_BATCH) {
            float4 v[TR_BATCH];
#pragma unroll
            for (int u = 0; u < TR_BATCH; u++) {
                const int b = bb + 4 * (tid + TR_THREADS * u);
                v[u] = b < n ? *reinterpret_cast<const float4*>(row + b) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < TR_BATCH; u++) {
                const int b = bb + 4 * (tid + TR_THREADS * u);
                const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int q = 0; q < 4; q++)
                    if (b + q < n) atomicAdd(&hist[score_key(e[q]) >> 20], 1u);
            }
        }
        __syncthreads();
        find_threshold_bin<TR_THREADS, TK_BINS>(hist, need, &s_bin, &s_above, sh);
        const uint32_t b0 = s_bin;
        need -= s_above;
        lo = b0 << 20;
        hi = lo | 0xfffffu;
        count = 0;
        for (int bb = 0; bb < n; bb += 4 * TR_THREADS * TR_BATCH) {
            float4 v[TR_BATCH];
#pragma unroll
            for (int u = 0; u < TR_BATCH; u++) {
                const int b = bb + 4 * (tid + TR_THREADS * u);
                v[u] = b < n ? *reinterpret_cast<const float4*>(row + b) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < TR_BATCH; u++) {
                const int b = bb + 4 * (tid + TR_THREADS * u);
                const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int t = b + q;
                    const uint32_t key = score_key(e[q]);
                    const uint32_t bin = key >> 20;
                    if (t < n && bin > b0) atomicOr(&gtbits[t >> 5], 1u << (t & 31));
                    append_candidate(t < n && bin == b0, key, t, count, seg);
                }
            }
        }
        __syncthreads();  // every wave has read segn (above) before it changes
        if (lane == 0) segn[wave] = count;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < TR_WAVES; w++) from_row |= segn[w] > (uint32_t)TR_SEG;
    }

    // ---- 3. radix rounds on [lo, hi], 12 bits at a time --------------------
    // Each round histograms (key - lo) >> shift over the keys in [lo, hi]
    // and narrows [lo, hi] to the bin holding the need-th largest.
    while (true) {
        const uint32_t span = hi - lo;
        const int shift = max(0, bitlen(span) - 12);
        for (int i = tid; i < TK_BINS; i += TR_THREADS) hist[i] = 0u;
        __syncthreads();
        if (!from_row) {
            for_each_candidate(cand, segn, [&](unsigned long long c) {
                const uint32_t key = (uint32_t)(c >> 32);
                if (key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1u);
            });
        } else {
            for (int t = tid; t < n; t += TR_THREADS) {
                const uint32_t key = score_key(row[t]);
                if (key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1u);
            }
        }
        __syncthreads();
        find_threshold_bin<TR_THREADS, TK_BINS>(hist, need, &s_bin, &s_above, sh);
        need -= s_above;
        const uint32_t nlo = lo + (s_bin << shift);
        const uint32_t nhi = shift == 0 ? nlo : min(hi, nlo + ((1u << shift) - 1u));
        lo = nlo;
        hi = nhi;
        if (shift == 0) break;
    }
    const uint32_t theta = lo;
    const uint32_t need_eq = need;

    // Candidates above theta join the result; theta ties are marked.  (In the
    // fallback, elements above the top-12-bit bin are already in gtbits and
    // only elements of that bin are candidates.)
    if (!from_row) {
        for_each_candidate(cand, segn, [&](unsigned long long c) {
            const uint32_t key = (uint32_t)(c >> 32);
            const int t = (int)(uint32_t)c;
            if (key > theta) atomicOr(&gtbits[t >> 5], 1u << (t & 31));
            else if (key == theta) atomicOr(&eqbits[t >> 5], 1u << (t & 31));
        });
    } else {
        const uint32_t b0 = theta >> 20;
        for (int t = tid; t < n; t += TR_THREADS) {
            const uint32_t key = score_key(row[t]);
            if ((key >> 20) != b0) continue;
            if (key > theta) atomicOr(&gtbits[t >> 5], 1u << (t & 31));
            else if (key == theta) atomicOr(&eqbits[t >> 5], 1u << (t & 31));
        }
    }
    __syncthreads();

    // ---- ordered output.  Thread tid owns the contiguous words [w0, w1). ----
    const int per = (nwords + TR_THREADS - 1) / TR_THREADS;
    const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
    uint32_t my_eq = 0;
    for (int w = w0; w < w1; w++) my_eq += __popc(eqbits[w]);
    uint32_t tot;
    uint32_t eq_before = block_exclusive_scan<TR_THREADS>(my_eq, &tot, sh);
    uint32_t my_sel = 0;
    for (int w = w0; w < w1; w++) {
        uint32_t e = eqbits[w];
        uint32_t keep = 0;
        while (e && eq_before < need_eq) {
            const uint32_t low = e & (0u - e);
            keep |= low;
            e ^= low;
            eq_before++;
        }
        const uint32_t selw = gtbits[w] | keep;
        gtbits[w] = selw;  // only this thread touches word w from here on
        my_sel += __popc(selw);
    }
    uint32_t pos = block_exclusive_scan<TR_THREADS>(my_sel, &tot, sh);
    for (int w = w0; w < w1; w++) {
        uint32_t selw = gtbits[w];
        while (selw) {
            const int bit = __ffs(selw) - 1;
            selw &= selw - 1u;
            if (pos < (uint32_t)k) out[pos] = (w << 5) + bit;
            pos++;
        }
    }
}

}  // namespace

size_t topk_workspace_bytes(int32_t num_rows, int32_t max_visible)
{
    if (max_visible <= TR_ROW_PATH_MAXN) return 0;  // the one-workgroup-per-row path needs none
    const size_t R = (size_t)num_rows;
    const size_t CH = (size_t)((max_visible + TK_CHUNK - 1) / TK_CHUNK);
    size_t b = 0;
    b += align_up(R * TK_BINS * 4, 256);
    b += align_up(R * TK_ROWST * 4, 256);
    b += align_up(R * CH * TK_CHUNKST * 4, 256);
    b += align_up(R * TK_CAP * 8, 256);
    return b;
}

TopkWorkspace topk_workspace_carve(void* ws, int32_t num_rows, int32_t max_visible)
{
    const size_t R = (size_t)num_rows;
    const int32_t CH = (max_visible + TK_CHUNK - 1) / TK_CHUNK;
    char* p = (char*)ws;
    TopkWorkspace tw;
    tw.hist = (uint32_t*)p;
    p += align_up(R * TK_BINS * 4, 256);
    tw.rowst = (uint32_t*)p;
    p += align_up(R * TK_ROWST * 4, 256);
    tw.chunkst = (uint32_t*)p;
    p += align_up(R * (size_t)CH * TK_CHUNKST * 4, 256);
    tw.cand = (unsigned long long*)p;
    tw.chunks = CH;
    return tw;
}

void launch_topk(int32_t num_rows, int32_t max_visible, const int32_t* vis, const float* scores, int64_t ld,
                 int32_t k, int32_t* indices, const TopkWorkspace& tw, hipStream_t stream)
{
    // Rows of up to TR_ROW_PATH_MAXN positions take one workgroup each; longer
    // rows (present only when max_visible exceeds it) are split over
    // workgroups.  Each kernel skips the rows the other path owns.
    hipLaunchKernelGGL(topk_rows_kernel, dim3(num_rows), dim3(TR_THREADS), 0, stream, vis, scores, ld, k,
                       indices, (int)TR_ROW_PATH_MAXN);
    if (max_visible <= TR_ROW_PATH_MAXN) return;
    const int CH = tw.chunks;
    const int min_n = TR_ROW_PATH_MAXN;
    dim3 g2(CH, num_rows);
    hipLaunchKernelGGL(topk_zero_kernel, dim3(num_rows), dim3(256), 0, stream, tw.hist, tw.rowst);
    hipLaunchKernelGGL(topk_hist_kernel, g2, dim3(TK_THREADS), 0, stream, vis, scores, ld, k, tw.hist, min_n);
    hipLaunchKernelGGL(topk_filter_kernel, g2, dim3(TK_THREADS), 0, stream, vis, scores, ld, k, tw.hist,
                       tw.rowst, tw.chunkst, CH, tw.cand, min_n);
    hipLaunchKernelGGL(topk_resolve_kernel, dim3(num_rows), dim3(RS_THREADS), 0, stream, vis, scores, ld, k,
                       tw.rowst, tw.chunkst, CH, tw.cand, min_n);
    hipLaunchKernelGGL(topk_write_kernel, g2, dim3(TK_THREADS), 0, stream, vis, scores, ld, k, tw.rowst,
                       tw.chunkst, CH, indices, min_n);
}

}  // namespace dsa
