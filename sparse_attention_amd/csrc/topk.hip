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
// Calls whose rows all have at most 8,192 positions take one 256-thread
// workgroup per row, several rows to a CU (topk_short_kernel).  Calls with
// few rows (at most 256) whose longest row has 65,537 to 262,144 positions
// split each row over 4,096-position chunks (topk_sfilter_kernel: a sampled
// bound, then the chunk's candidates in position order) and finish each row
// in one workgroup (topk_sresolve_kernel).  Calls of at least 1,024 rows give
// their rows of at most 65,536 positions one 256-thread workgroup each, four
// to a CU (topk_stream_kernel).  Otherwise rows of at most 65,536 positions
// take one 1024-thread workgroup each (one streaming pass over the row, the
// rest in LDS; see topk_rows_kernel).
// Longer rows are split over workgroups, because a single CU streams too
// slowly for them; only integer counts are combined across workgroups, so the
// result does not depend on scheduling:
//   1. sample   per long row, in the one-workgroup-per-row kernel (which owns
//               the short rows): a lower bound theta_lo on the k-th largest
//               key, the exact order statistic of 8,192 sampled keys at about
//               1.5x the k-th largest's expected sample rank.  With more than
//               64 rows, one workgroup then lists the long rows (in row
//               order) and the kernels below walk that list with fixed grids;
//               else they run one workgroup row per query row
//   2. filter   rows x chunks: elements with key >= theta_lo are appended to a
//               per-row candidate list (one atomic slot reservation per
//               workgroup; only the set matters)
//   3. resolve  one workgroup per row: a three-round radix select (12, 12, 8
//               key bits) for the exact threshold key theta and the number
//               need_eq of theta-valued elements to keep, over the candidates
//               when they number at least k and fit the list (then they hold
//               theta and everything above it), else over the row itself;
//               then per-chunk output offsets by block scans
//   4. write    rows x chunks: ordered compaction; an element is kept if its
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
constexpr int RS_CAND = 0, RS_THLO = 1, RS_THETA = 3, RS_NEEDEQ = 4;
// Chunk state words.
constexpr int CS_OFFSET = 1, CS_EQBEFORE = 2;

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
// elements in bins above b is < need and including b is >= need.  Returns b,
// the count strictly above it and (if out_count is set) the count in b via
// shared outputs.  NT threads, B a multiple of NT; two barriers: thread t
// holds bins [B - PER (t+1), B - PER t) in registers, a wave prefix sum plus
// the per-wave totals in sh[] give its offset from the top, and the one
// thread whose range holds the answer scans its own registers.
template <int NT, int B>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* h, uint32_t need, uint32_t* out_bin,
                                                   uint32_t* out_above, uint32_t* sh,
                                                   uint32_t* out_count = nullptr)
{
    constexpr int PER = B / NT;
    static_assert(PER >= 1 && PER * NT == B, "bins split evenly over the threads");
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int lo = B - PER * (t + 1);
    uint32_t c[PER];
    if constexpr (PER % 4 == 0) {  // 16-byte reads (the histograms are 16-byte aligned)
#pragma unroll
        for (int i = 0; i < PER; i += 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(h + lo + i);
            c[i] = v.x;
            c[i + 1] = v.y;
            c[i + 2] = v.z;
            c[i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < PER; i++) c[i] = h[lo + i];
    }
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) mine += c[i];
    const uint32_t incl = wave_inclusive_scan(mine);
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) before += (w < wave) ? sh[w] : 0u;
    const uint32_t pre = before + incl - mine;  // elements in bins above this thread's range
    if (pre < need && pre + mine >= need) {
        uint32_t acc = pre;
#pragma unroll
        for (int i = PER - 1; i >= 0; i--) {
            if (acc < need && acc + c[i] >= need) {
                *out_bin = (uint32_t)(lo + i);
                *out_above = acc;
                if (out_count) *out_count = c[i];
            }
            acc += c[i];
        }
    }
    __syncthreads();
}

constexpr int TR_FEW = 64;  // keys one wave ranks directly to end the radix rounds

// Ends a radix select once at most 64 keys remain in play: called by one
// whole wave with the m <= 64 remaining keys in few[] (16-byte aligned), it
// finds theta, the key with fewer than `need` larger keys among them and at
// least `need` larger-or-equal ones (a single value, and lanes holding it
// agree on every count), the number need_eq of theta-valued keys to keep and
// their total.
__device__ __forceinline__ void rank_few(const uint32_t* few, uint32_t m, uint32_t need, uint32_t* s_theta,
                                         uint32_t* s_needeq, uint32_t* s_eqtot)
{
    const int lane = threadIdx.x & 63;
    const uint32_t mine = lane < (int)m ? few[lane] : 0u;
    uint32_t gt = 0, eq = 0;
    for (uint32_t i = 0; i < m; i += 4) {
        const uint4 o4 = *reinterpret_cast<const uint4*>(&few[i]);
        const uint32_t o[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const bool live = i + e < m;
            gt += (live && o[e] > mine) ? 1u : 0u;
            eq += (live && o[e] == mine) ? 1u : 0u;
        }
    }
    if (lane < (int)m && gt < need && need <= gt + eq) {
        *s_theta = mine;
        *s_needeq = need - gt;
        *s_eqtot = eq;
    }
}

// Sampled lower bound of one long row (n > TR_ROW_PATH_MAXN, so n is well
// above TS_SAMPLES): TS_BLOCKS blocks of TS_BLOCK consecutive positions spread
// evenly over the row; theta_lo = the key of the rho-th largest sample, with
// rho = 1.5 x the rank the k-th largest element has in the sample (k m / n)
// plus 16, found exactly by a three-round radix select over the sample keys.
// Stores theta_lo and clears the row's candidate counter.  Called by a whole
// TP_THREADS workgroup; keys[] and h[] are its LDS.
constexpr int TP_THREADS = 1024;
constexpr int TS_BLOCKS = 32;
constexpr int TS_BLOCK = 256;
constexpr int TS_SAMPLES = TS_BLOCKS * TS_BLOCK;  // 8 per thread
static_assert(TS_SAMPLES == 8 * TP_THREADS, "eight samples per thread");

__device__ void topk_sample_row(const float* __restrict__ row, int n, int k, uint32_t* __restrict__ rs,
                                uint32_t* keys, uint32_t* h, uint32_t* sh, uint32_t* s_bin, uint32_t* s_above)
{
    const int t = threadIdx.x;
    const int blk = t >> 5, o = 8 * (t & 31);
    // 4-aligned block start, the block inside the row: start + 255 < n.
    const int start = (int)(((int64_t)(n - TS_BLOCK) * blk / (TS_BLOCKS - 1)) & ~3LL);
    const float4 v0 = *reinterpret_cast<const float4*>(row + start + o);
    const float4 v1 = *reinterpret_cast<const float4*>(row + start + o + 4);
    uint32_t kk[8] = {score_key(v0.x), score_key(v0.y), score_key(v0.z), score_key(v0.w),
                      score_key(v1.x), score_key(v1.y), score_key(v1.z), score_key(v1.w)};
    for (int i = t; i < TK_BINS; i += TP_THREADS) h[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; e++) atomicAdd(&h[kk[e] >> 20], 1u);
    __syncthreads();
    const uint32_t rho = min((uint32_t)TS_SAMPLES,
                             (uint32_t)((3LL * k * TS_SAMPLES + 2LL * n - 1) / (2LL * n)) + 16u);
    find_threshold_bin<TP_THREADS, TK_BINS>(h, rho, s_bin, s_above, sh);
    const uint32_t b0 = *s_bin, need1 = rho - *s_above;
    for (int i = t; i < TK_BINS; i += TP_THREADS) h[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; e++)
        if ((kk[e] >> 20) == b0) atomicAdd(&h[(kk[e] >> 8) & 0xfffu], 1u);
    __syncthreads();
    find_threshold_bin<TP_THREADS, TK_BINS>(h, need1, s_bin, s_above, sh);
    const uint32_t pre = (b0 << 12) | *s_bin, need2 = need1 - *s_above;
    for (int i = t; i < 256; i += TP_THREADS) h[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; e++)
        if ((kk[e] >> 8) == pre) atomicAdd(&h[kk[e] & 0xffu], 1u);
    __syncthreads();
    if (t < 256) {
        // 256 bins over 1024 threads: the bin search runs in the first 256.
        uint32_t c = h[255 - t];
        const uint32_t incl = wave_inclusive_scan(c);
        if ((t & 63) == 63) sh[t >> 6] = incl;
        keys[t] = incl;  // scratch: inclusive count from the top, per bin
    }
    __syncthreads();
    if (t < 256) {
        uint32_t before = 0;
        for (int w = 0; w < (t >> 6); w++) before += sh[w];
        const uint32_t incl = before + keys[t], c = h[255 - t];
        if (incl >= need2 && incl - c < need2) {
            rs[RS_THLO] = (pre << 8) | (uint32_t)(255 - t);
            rs[RS_CAND] = 0u;
        }
    }
    __syncthreads();  // LDS free for the caller's next row
}

// Many rows: one workgroup lists, in row order, the rows the multi-workgroup
// kernels own (n > min_n, hence n > k); the kernels below walk that list with
// grids of a fixed size, so a call with many short rows and a few long ones
// does not launch rows x chunks workgroups that would mostly exit at once.
// (Few rows: no list; the kernels below run one workgroup row per query row.)
__global__ __launch_bounds__(TP_THREADS) void topk_prep_kernel(const int32_t* __restrict__ vis, int num_rows,
                                                               int min_n, int32_t* __restrict__ longrows,
                                                               uint32_t* __restrict__ nlong)
{
    __shared__ uint32_t sh[TP_THREADS / 64];
    // Thread t owns rows [t * per, (t + 1) * per): count, scan, then write.
    const int per = (num_rows + TP_THREADS - 1) / TP_THREADS;
    const int r0 = threadIdx.x * per, r1 = min(num_rows, r0 + per);
    uint32_t cnt = 0;
    for (int r = r0; r < r1; r++) cnt += vis[r] > min_n ? 1u : 0u;
    uint32_t total;
    uint32_t slot = block_exclusive_scan<TP_THREADS>(cnt, &total, sh);
    for (int r = r0; r < r1; r++)
        if (vis[r] > min_n) longrows[slot++] = r;
    if (threadIdx.x == 0) *nlong = total;
}

// Item li of the list-walking kernels: query row li itself (direct mode,
// longrows == nullptr; short rows are skipped), or list entry li.
__device__ __forceinline__ uint32_t topk_items(const int32_t* longrows, const uint32_t* nlong, int num_rows)
{
    return longrows ? *nlong : (uint32_t)num_rows;
}
__device__ __forceinline__ int topk_item_row(const int32_t* longrows, uint32_t li)
{
    return longrows ? longrows[li] : (int)li;
}

// Grid rows of the list-walking kernels.
constexpr int TK_LIST_GRID = 64;

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

// Rows x chunks: every element whose key is >= the row's sampled bound
// theta_lo becomes a candidate (key, position); one integer atomic per
// workgroup reserves its slots in the row's list (the list order is
// irrelevant: the selection below depends only on the set).
__global__ __launch_bounds__(TK_THREADS) void topk_filter_kernel(const int32_t* __restrict__ vis,
                                                                 const float* __restrict__ scores, int64_t ld,
                                                                 uint32_t* __restrict__ rowst,
                                                                 unsigned long long* __restrict__ cand,
                                                                 const int32_t* __restrict__ longrows,
                                                                 const uint32_t* __restrict__ nlong, int num_rows,
                                                                 int min_n)
{
    __shared__ uint32_t sh[TK_THREADS / 64];
    __shared__ uint32_t s_base;
    const uint32_t nl = topk_items(longrows, nlong, num_rows);
    for (uint32_t li = blockIdx.y; li < nl; li += gridDim.y) {
        const int r = topk_item_row(longrows, li);
        const int n = vis[r];
        const int start = blockIdx.x * TK_CHUNK;
        if (n <= min_n || start >= n) continue;
        const int end = min(n, start + TK_CHUNK);
        uint32_t* rs = rowst + (int64_t)r * TK_ROWST;
        const uint32_t thlo = rs[RS_THLO];
        uint32_t key[TK_PER_THREAD], present;
        load_chunk_keys(scores + (int64_t)r * ld, start, end, key, present);
        uint32_t sel = 0u;
#pragma unroll
        for (int i = 0; i < TK_PER_THREAD; i++)
            if (((present >> i) & 1u) && key[i] >= thlo) sel |= 1u << i;
        uint32_t total;
        const uint32_t pre = block_exclusive_scan<TK_THREADS>(__popc(sel), &total, sh);
        if (threadIdx.x == 0) s_base = total ? atomicAdd(&rs[RS_CAND], total) : 0u;
        __syncthreads();
        uint32_t slot = s_base + pre;
        unsigned long long* cr = cand + (int64_t)r * TK_CAP;
        const int t0 = start + TK_PER_THREAD * threadIdx.x;
#pragma unroll
        for (int i = 0; i < TK_PER_THREAD; i++)
            if ((sel >> i) & 1u) {
                if (slot < (uint32_t)TK_CAP) cr[slot] = ((unsigned long long)key[i] << 32) | (uint32_t)(t0 + i);
                slot++;
            }
        __syncthreads();  // s_base is read before the next item overwrites it
    }
}

// One workgroup per long row: the exact threshold key theta (the k-th
// largest key) and need_eq (theta-valued elements to keep) by a three-round
// radix select, then per-chunk output offsets.  Fast path: the candidates
// (every element >= theta_lo) number at least k and fit the list, so theta
// is among them and every element above theta is a candidate.  Otherwise (a
// misleading sample, or ties filling the list) the same rounds run over the
// whole row, read from memory: slower, equally exact.
__global__ __launch_bounds__(RS_THREADS) void topk_resolve_kernel(const int32_t* __restrict__ vis,
                                                                  const float* __restrict__ scores, int64_t ld,
                                                                  int k, uint32_t* __restrict__ rowst,
                                                                  uint32_t* __restrict__ chunkst, int chunks,
                                                                  const unsigned long long* __restrict__ cand,
                                                                  const int32_t* __restrict__ longrows,
                                                                  const uint32_t* __restrict__ nlong, int num_rows,
                                                                  int min_n)
{
    __shared__ unsigned long long cl[TK_CAP];
    __shared__ __attribute__((aligned(16))) uint32_t h[TK_BINS];
    __shared__ uint32_t cgt[TK_MAX_CHUNKS / 2];  // per-chunk counts, in windows of chunks
    __shared__ uint32_t ceq[TK_MAX_CHUNKS / 2];
    __shared__ uint32_t sh[RS_THREADS / 64];
    __shared__ uint32_t s_bin, s_above, s_cnt;
    __shared__ __attribute__((aligned(16))) uint32_t few[TR_FEW];  // the last keys in play (early finish)
    __shared__ uint32_t s_nfew, s_theta, s_needeq, s_eqtot;
    const uint32_t nl = topk_items(longrows, nlong, num_rows);
    for (uint32_t li = blockIdx.x; li < nl; li += gridDim.x) {
    const int r = topk_item_row(longrows, li);
    const int n = vis[r];
    if (n <= min_n) continue;
    __syncthreads();  // the previous item is done with the shared state
    if (threadIdx.x == 0) s_nfew = 0u;

    uint32_t* rs = rowst + (int64_t)r * TK_ROWST;
    const uint32_t m = rs[RS_CAND];
    const bool fast = m >= (uint32_t)k && m <= (uint32_t)TK_CAP;
    const float* row = scores + (int64_t)r * ld;
    const int nch = (n + TK_CHUNK - 1) / TK_CHUNK;
    if (fast)
        for (uint32_t i = threadIdx.x; i < m; i += RS_THREADS) cl[i] = cand[(int64_t)r * TK_CAP + i];

    uint32_t theta, need_eq;
    if (fast) {
        // Radix rounds relative to the candidates' own key range [theta_lo,
        // max]: 12 bits of (key - lo) per round, so the candidates (which
        // share few top-bit bins) spread over the histogram instead of piling
        // onto a handful of LDS counters.
        uint32_t mx = 0u;
        for (uint32_t i = threadIdx.x; i < m; i += RS_THREADS) mx = max(mx, (uint32_t)(cl[i] >> 32));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
        if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = mx;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < RS_THREADS / 64; w++) mx = max(mx, sh[w]);
        __syncthreads();
        uint32_t lo = rs[RS_THLO], hi = mx, nd = (uint32_t)k;
        for (;;) {
            const uint32_t span = hi - lo;
            const int shift = span < (uint32_t)TK_BINS ? 0 : (32 - __clz(span)) - 12;
            for (int i = threadIdx.x; i < TK_BINS; i += RS_THREADS) h[i] = 0u;
            __syncthreads();
            for (uint32_t i = threadIdx.x; i < m; i += RS_THREADS) {
                const uint32_t key = (uint32_t)(cl[i] >> 32);
                if (key >= lo && key <= hi) atomicAdd(&h[(key - lo) >> shift], 1u);
            }
            __syncthreads();
            find_threshold_bin<RS_THREADS, TK_BINS>(h, nd, &s_bin, &s_above, sh, &s_cnt);
            nd -= s_above;
            lo += s_bin << shift;
            hi = (uint32_t)min((uint64_t)hi, (uint64_t)lo + ((1ull << shift) - 1));
            if (shift == 0) break;  // wave-uniform: every thread holds the same lo, hi
            // Few candidates left in [lo, hi]: one wave ranks them (see rank_few).
            if (s_cnt <= (uint32_t)TR_FEW) {
                for (uint32_t i = threadIdx.x; i < m; i += RS_THREADS) {
                    const uint32_t key = (uint32_t)(cl[i] >> 32);
                    if (key >= lo && key <= hi) few[atomicAdd(&s_nfew, 1u)] = key;
                }
                __syncthreads();
                if (threadIdx.x < 64) rank_few(few, s_cnt, nd, &s_theta, &s_needeq, &s_eqtot);
                __syncthreads();
                lo = s_theta;
                nd = s_needeq;
                break;
            }
        }
        theta = lo;
        need_eq = nd;
    } else {
    // Whole row, absolute key bits.  Round 1: bits 31..20.
    for (int i = threadIdx.x; i < TK_BINS; i += RS_THREADS) h[i] = 0u;
    __syncthreads();
    for (int t = threadIdx.x; t < n; t += RS_THREADS) atomicAdd(&h[score_key(row[t]) >> 20], 1u);
    __syncthreads();
    find_threshold_bin<RS_THREADS, TK_BINS>(h, (uint32_t)k, &s_bin, &s_above, sh);
    const uint32_t b0 = s_bin;
    const uint32_t need = (uint32_t)k - s_above;

    // Round 2: key bits 19..8 among keys whose top 12 bits equal b0.
    for (int i = threadIdx.x; i < TK_BINS; i += RS_THREADS) h[i] = 0u;
    __syncthreads();
    for (int t = threadIdx.x; t < n; t += RS_THREADS) {
        const uint32_t key = score_key(row[t]);
        if ((key >> 20) == b0) atomicAdd(&h[(key >> 8) & 0xfffu], 1u);
    }
    __syncthreads();
    find_threshold_bin<RS_THREADS, TK_BINS>(h, need, &s_bin, &s_above, sh);
    const uint32_t b1 = s_bin;
    const uint32_t need2 = need - s_above;
    const uint32_t pre20 = (b0 << 12) | b1;  // top 24 bits of theta

    // Round 3: key bits 7..0 among keys whose top 24 bits equal pre20.
    for (int i = threadIdx.x; i < 512; i += RS_THREADS) h[i] = 0u;
    __syncthreads();
    for (int t = threadIdx.x; t < n; t += RS_THREADS) {
        const uint32_t key = score_key(row[t]);
        if ((key >> 8) == pre20) atomicAdd(&h[key & 0xffu], 1u);
    }
    __syncthreads();
    find_threshold_bin<RS_THREADS, 512>(h, need2, &s_bin, &s_above, sh);
    theta = (pre20 << 8) | s_bin;
    need_eq = need2 - s_above;
    }

    // Per-chunk counts of keys > theta and keys == theta (all such elements
    // are candidates on the fast path).  Chunks are processed in windows of
    // TK_MAX_CHUNKS / 2 to bound LDS.
    uint32_t offs = 0, eqb = 0;  // running totals (the same in every thread)
    for (int w0 = 0; w0 < nch; w0 += TK_MAX_CHUNKS / 2) {
        const int w1 = min(nch, w0 + TK_MAX_CHUNKS / 2);
        for (int i = threadIdx.x; i < w1 - w0; i += RS_THREADS) {
            cgt[i] = 0u;
            ceq[i] = 0u;
        }
        __syncthreads();
        if (fast) {
            for (uint32_t i = threadIdx.x; i < m; i += RS_THREADS) {
                const uint32_t key = (uint32_t)(cl[i] >> 32);
                const int cc = (int)(uint32_t)cl[i] / TK_CHUNK;
                if (cc < w0 || cc >= w1) continue;
                if (key > theta) atomicAdd(&cgt[cc - w0], 1u);
                else if (key == theta) atomicAdd(&ceq[cc - w0], 1u);
            }
        } else {
            const int t_end = min(n, w1 * TK_CHUNK);
            for (int t = w0 * TK_CHUNK + threadIdx.x; t < t_end; t += RS_THREADS) {
                const uint32_t key = score_key(row[t]);
                const int cc = t / TK_CHUNK - w0;
                if (key > theta) atomicAdd(&cgt[cc], 1u);
                else if (key == theta) atomicAdd(&ceq[cc], 1u);
            }
        }
        __syncthreads();
        // Output offsets in chunk order: chunk i keeps its elements above
        // theta plus as many theta-valued ones as remain of need_eq after the
        // chunks before it (two block scans per RS_THREADS chunks).
        for (int c0 = 0; c0 < w1 - w0; c0 += RS_THREADS) {
            const int i = c0 + threadIdx.x;
            const bool in = i < w1 - w0;
            const uint32_t gtc = in ? cgt[i] : 0u;
            const uint32_t eqc = in ? ceq[i] : 0u;
            uint32_t eq_tot, o_tot;
            const uint32_t eq_before = eqb + block_exclusive_scan<RS_THREADS>(eqc, &eq_tot, sh);
            const uint32_t left = need_eq > eq_before ? need_eq - eq_before : 0u;
            const uint32_t take = left < eqc ? left : eqc;
            const uint32_t o_before = offs + block_exclusive_scan<RS_THREADS>(gtc + take, &o_tot, sh);
            if (in) {
                uint32_t* cs = chunkst + ((int64_t)r * chunks + w0 + i) * TK_CHUNKST;
                cs[CS_OFFSET] = o_before;
                cs[CS_EQBEFORE] = eq_before;
            }
            offs += o_tot;
            eqb += eq_tot;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        rs[RS_THETA] = theta;
        rs[RS_NEEDEQ] = need_eq;
    }
    }
}

__global__ __launch_bounds__(TK_THREADS) void topk_write_kernel(const int32_t* __restrict__ vis,
                                                                const float* __restrict__ scores, int64_t ld, int k,
                                                                const uint32_t* __restrict__ rowst,
                                                                const uint32_t* __restrict__ chunkst, int chunks,
                                                                int32_t* __restrict__ indices,
                                                                const int32_t* __restrict__ longrows,
                                                                const uint32_t* __restrict__ nlong, int num_rows,
                                                                int min_n)
{
    __shared__ uint32_t sh[TK_THREADS / 64];
    const uint32_t nl = topk_items(longrows, nlong, num_rows);
    for (uint32_t li = blockIdx.y; li < nl; li += gridDim.y) {
    const int r = topk_item_row(longrows, li);
    const int c = blockIdx.x;
    const int n = vis[r];  // > min_n > k for the rows this path owns
    const int start = c * TK_CHUNK;
    int32_t* out = indices + (int64_t)r * k;
    if (n <= min_n || start >= n) continue;
    const int end = min(n, start + TK_CHUNK);
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
}

// ---------------------------------------------------------------------------
// One workgroup per row, for rows of at most TR_ROW_PATH_MAXN positions (for
// longer rows the workgroup runs the sampling step of the multi-workgroup
// path and leaves the rest to it).  The row is read from memory once, into
// registers: thread t holds the scores of
// positions 4 (t + TR_THREADS u) + q, q < 4, for every group u the row
// reaches.  A workgroup of 16 waves shares one CU, so the per-element work is
// kept to a few VALU operations: the full pass compares raw floats (exact:
// fp32 denormals are kept, -0.0 == +0.0 and NaN compares false, the same
// order as the keys), and only sampled elements and candidates are turned
// into keys.
//
// Fast path (sampled bound):
//   1. The keys at positions 4 (t + TR_THREADS u) of every su-th group (about
//      4096 samples) give a conservative lower bound theta_lo on the k-th
//      largest key: the lower edge of the 12-bit key bin holding the sample's
//      rho-th largest, rho about 1.5x the rank the k-th largest has in the
//      sample plus a margin.
//   2. Every element whose key is >= theta_lo (a float compare against the
//      bound's float) is a candidate; lanes count their own, the wave and
//      block prefix sums place them densely in an LDS list.  NaN (and any
//      position past the row, loaded as NaN) is never a candidate; when that
//      matters, fewer than k candidates remain and the fallback runs.
//   3. If there are at least k candidates and they fit the list, the k-th
//      largest key lies among them, and a radix select over the candidates
//      alone (held in registers, 12 bits per round relative to their own key
//      range, at most three rounds) is exact.
// Fallback (exact for any input, e.g. huge tie groups or a misleading
// sample): an LDS histogram of the top 12 key bits of the whole row gives the
// threshold bin b0; elements above b0 are marked selected at once, and the
// elements inside b0 become the candidates (if they overflow the list, the
// radix rounds histogram the row again, from memory).
// Finally candidates above theta are marked in a position bitmap and
// theta-valued ones in a tie bitmap, and an ordered pass over the bitmaps
// writes the selected positions in ascending order.  When every theta-valued
// element is kept (the usual case) one block scan gives the output offsets;
// otherwise a first scan ranks the ties so that the first need_eq of them in
// position order are kept.
constexpr int TR_THREADS = 1024;
constexpr int TR_WAVES = TR_THREADS / 64;
constexpr int TR_CAP = 8192;                                       // candidate list slots
constexpr int TR_CPT = TR_CAP / TR_THREADS;                        // candidate slots per thread
constexpr int TR_GROUPS = TR_ROW_PATH_MAXN / (4 * TR_THREADS);     // 16 float4 groups per thread
constexpr int TR_WORDS = TR_ROW_PATH_MAXN / 32;

// The order-preserving key of a score, branch-free (see score_key).
__device__ __forceinline__ uint32_t key_of(float f)
{
    const uint32_t b = __float_as_uint(f), a = b & 0x7fffffffu;
    return a > 0x7f800000u ? 0u : (a == 0u ? 0x80000000u : ((b >> 31) ? ~b : (b | 0x80000000u)));
}

// The float whose key is k, for keys of non-NaN scores (k in
// [key(-inf), key(+inf)]); key(-0.0) maps back to -0.0, which compares like
// +0.0.
__device__ __forceinline__ float float_of_key(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Maximum over the wave, valid in lane 63 (DPP row shifts and broadcasts);
// NaN is ignored.
__device__ __forceinline__ float wave_max_lane63(float x)
{
    const int ninf = __float_as_int(-__builtin_inff());
#define TR_MAX_STEP(ctrl, rm)                                                                   \
    {                                                                                           \
        const float y = __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), ctrl, rm, 0xF, false)); \
        x = y > x ? y : x;                                                                      \
    }
    TR_MAX_STEP(0x111, 0xF)  // row_shr:1
    TR_MAX_STEP(0x112, 0xF)  // row_shr:2
    TR_MAX_STEP(0x114, 0xF)  // row_shr:4
    TR_MAX_STEP(0x118, 0xF)  // row_shr:8
    TR_MAX_STEP(0x142, 0xA)  // row_bcast:15
    TR_MAX_STEP(0x143, 0xC)  // row_bcast:31
#undef TR_MAX_STEP
    return x;
}

__device__ __forceinline__ int bitlen(uint32_t x) { return x ? 32 - __clz(x) : 0; }

__global__ __launch_bounds__(TR_THREADS) void topk_rows_kernel(const int32_t* __restrict__ vis,
                                                               const float* __restrict__ scores, int64_t ld,
                                                               int k, int32_t* __restrict__ indices, int max_n,
                                                               uint32_t* __restrict__ long_rowst, int num_rows,
                                                               int sample_only)
{
    static_assert(TR_THREADS == TP_THREADS, "the sampling step runs on this workgroup");
    const int r = grid_item();
    if (r >= num_rows) return;
    const int n = vis[r];
    if (sample_only && n <= max_n) return;  // topk_stream_kernel owns this row
    int32_t* out = indices + (int64_t)r * k;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    if (n <= k) {
        for (int t = tid; t < k; t += TR_THREADS) out[t] = t < n ? t : -1;
        return;
    }
    __shared__ __attribute__((aligned(16))) uint32_t hs[TK_BINS];     // sample, then fallback histogram
    __shared__ __attribute__((aligned(16))) uint32_t hr[2][TK_BINS];  // radix rounds, alternating
    __shared__ uint32_t gtbits[TR_WORDS];
    __shared__ uint32_t eqbits[TR_WORDS];
    __shared__ unsigned long long cand[TR_CAP];  // (score bits, position)
    __shared__ uint32_t wcnt[TR_WAVES];
    __shared__ float wmax[TR_WAVES];
    __shared__ uint32_t sh[TR_THREADS / 64];
    __shared__ uint32_t s_bin, s_above, s_cnt;
    __shared__ __attribute__((aligned(16))) uint32_t few[TR_FEW];  // the last keys in play (early finish)
    __shared__ uint32_t s_nfew, s_theta, s_needeq, s_eqtot;
    if (n > max_n) {
        // The multi-workgroup kernels own this row; its first step, the
        // sampled lower bound, runs here (the candidate list is free LDS).
        topk_sample_row(scores + (int64_t)r * ld, n, k, long_rowst + (int64_t)r * TK_ROWST,
                        reinterpret_cast<uint32_t*>(cand), hs, sh, &s_bin, &s_above);
        return;
    }

    // ---- the row, into registers ---------------------------------------------
    const float* row = scores + (int64_t)r * ld;
    const int nu = (n + 4 * TR_THREADS - 1) / (4 * TR_THREADS);  // groups the row reaches
    float x[TR_GROUPS][4];
#pragma unroll
    for (int u = 0; u < TR_GROUPS; u++) {
        if (u < nu) {
            // A 4-aligned group starting below n lies inside the row allocation
            // (ld is a multiple of 4 and n <= ld); lanes past the row re-read
            // its last group and turn it into NaN below.
            const int p = min(4 * (tid + TR_THREADS * u), (n - 1) & ~3);
            const float4 v = *reinterpret_cast<const float4*>(row + p);
            x[u][0] = v.x;
            x[u][1] = v.y;
            x[u][2] = v.z;
            x[u][3] = v.w;
        }
    }
    const int nwords = (n + 31) >> 5;
    for (int i = tid; i < TK_BINS; i += TR_THREADS) {
        hs[i] = 0u;
        hr[0][i] = 0u;
        hr[1][i] = 0u;
    }
    for (int i = tid; i < nwords; i += TR_THREADS) {
        gtbits[i] = 0u;
        eqbits[i] = 0u;
    }
    if (tid == 0) s_nfew = 0u;
    // Only the last group can run past the row.
#pragma unroll
    for (int u = 0; u < TR_GROUPS; u++) {
        if (u == nu - 1 && 4 * TR_THREADS * nu > n) {
            const int p = 4 * (tid + TR_THREADS * u);
#pragma unroll
            for (int q = 0; q < 4; q++)
                if (p + q >= n) x[u][q] = __uint_as_float(0xffffffffu);
        }
    }
    __syncthreads();  // histograms and bitmaps cleared

    // ---- 1. sampled lower bound ------------------------------------------------
    // Samples past the row are NaN, key 0, bin 0: below the rho-th largest of
    // the real samples, so they change nothing.
    const int su = nu <= 4 ? 1 : (nu <= 8 ? 2 : 4);  // sample every su-th group
    int msamp = 0;
    for (int u = 0; u < nu; u += su) msamp += min(TR_THREADS, (n - 4 * TR_THREADS * u + 3) >> 2);
#pragma unroll
    for (int u = 0; u < TR_GROUPS; u++)
        if (u < nu && (u & (su - 1)) == 0) atomicAdd(&hs[key_of(x[u][0]) >> 20], 1u);
    __syncthreads();
    const uint32_t rho = (uint32_t)min((int64_t)msamp, ((int64_t)3 * k * msamp) / (2 * (int64_t)n) + 32);
    find_threshold_bin<TR_THREADS, TK_BINS>(hs, rho, &s_bin, &s_above, sh);
    // Candidates: keys >= lo0, i.e. scores >= flo (key(-inf) is the lowest
    // key of a non-NaN score).
    const uint32_t lo0 = max((rho >= (uint32_t)msamp) ? 0u : (s_bin << 20), 0x007fffffu);
    const float flo = float_of_key(lo0);

    // ---- 2. candidates ----------------------------------------------------------
    uint32_t c = 0;
    float mx = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < TR_GROUPS; u++) {
        if (u < nu) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                c += x[u][q] >= flo ? 1u : 0u;
                mx = x[u][q] > mx ? x[u][q] : mx;
            }
        }
    }
    const uint32_t incl = wave_inclusive_scan(c);
    mx = wave_max_lane63(mx);
    if (lane == 63) {
        wcnt[wave] = incl;
        wmax[wave] = mx;
    }
    __syncthreads();
    uint32_t total = 0, base = 0;
    float row_max = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < TR_WAVES; w++) {
        const uint32_t t = wcnt[w];
        base += w < wave ? t : 0u;
        total += t;
        row_max = wmax[w] > row_max ? wmax[w] : row_max;
    }
    const bool fast = total >= (uint32_t)k && total <= (uint32_t)TR_CAP;
    if (fast) {
        uint32_t slot = base + incl - c;
#pragma unroll
        for (int u = 0; u < TR_GROUPS; u++) {
            if (u < nu) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    if (x[u][q] >= flo) {
                        cand[slot] = ((unsigned long long)__float_as_uint(x[u][q]) << 32) |
                                     (uint32_t)(4 * (tid + TR_THREADS * u) + q);
                        slot++;
                    }
                }
            }
        }
    }

    uint32_t need = (uint32_t)k;
    uint32_t lo, hi;          // every key still in play lies in [lo, hi]
    bool from_regs = false;   // fallback candidates overflowed: rescan the row
    uint32_t ncand = total;
    if (fast) {
        lo = lo0;
        hi = key_of(row_max);  // >= lo0, since some candidate exists
    } else {
        // ---- fallback: whole-row histogram -----------------------------------
        // (every thread read wcnt above; the barriers below order its reuse)
        for (int i = tid; i < TK_BINS; i += TR_THREADS) hs[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < TR_GROUPS; u++) {
            if (u < nu) {
                const int p = 4 * (tid + TR_THREADS * u);
#pragma unroll
                for (int q = 0; q < 4; q++)
                    if (p + q < n) atomicAdd(&hs[key_of(x[u][q]) >> 20], 1u);
            }
        }
        __syncthreads();
        find_threshold_bin<TR_THREADS, TK_BINS>(hs, need, &s_bin, &s_above, sh);
        const uint32_t b0 = s_bin;
        need -= s_above;
        lo = b0 << 20;
        hi = lo | 0xfffffu;
        // Elements above b0 are selected; those inside b0 are the candidates.
        uint32_t cb = 0;
#pragma unroll
        for (int u = 0; u < TR_GROUPS; u++) {
            if (u < nu) {
                const int p = 4 * (tid + TR_THREADS * u);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const uint32_t kk = key_of(x[u][q]);
                    if (p + q < n && (kk >> 20) > b0) atomicOr(&gtbits[(p + q) >> 5], 1u << ((p + q) & 31));
                    cb += (p + q < n && (kk >> 20) == b0) ? 1u : 0u;
                }
            }
        }
        const uint32_t incl_b = wave_inclusive_scan(cb);
        if (lane == 63) wcnt[wave] = incl_b;
        __syncthreads();
        uint32_t base_b = 0;
        ncand = 0;
#pragma unroll
        for (int w = 0; w < TR_WAVES; w++) {
            const uint32_t t = wcnt[w];
            base_b += w < wave ? t : 0u;
            ncand += t;
        }
        from_regs = ncand > (uint32_t)TR_CAP;
        if (!from_regs) {
            uint32_t slot = base_b + incl_b - cb;
#pragma unroll
            for (int u = 0; u < TR_GROUPS; u++) {
                if (u < nu) {
                    const int p = 4 * (tid + TR_THREADS * u);
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        if (p + q < n && (key_of(x[u][q]) >> 20) == b0) {
                            cand[slot] = ((unsigned long long)__float_as_uint(x[u][q]) << 32) | (uint32_t)(p + q);
                            slot++;
                        }
                    }
                }
            }
        }
    }
    __syncthreads();  // candidate list written

    // Candidate i lives in thread i % TR_THREADS, slot i / TR_THREADS.
    uint32_t ck[TR_CPT], cp[TR_CPT];
#pragma unroll
    for (int j = 0; j < TR_CPT; j++) {
        const uint32_t i = (uint32_t)(tid + TR_THREADS * j);
        ck[j] = 0u;
        cp[j] = 0u;
        if (!from_regs && i < ncand) {
            const unsigned long long cv = cand[i];
            ck[j] = key_of(__uint_as_float((uint32_t)(cv >> 32)));
            cp[j] = (uint32_t)cv;
        }
    }

    // ---- 3. radix rounds on [lo, hi], 12 bits at a time --------------------
    // Each round histograms (key - lo) >> shift over the keys in [lo, hi]
    // and narrows [lo, hi] to the bin holding the need-th largest.  Rounds
    // alternate between two histograms, each cleared for the round after next.
    uint32_t eq_total = 0;  // theta-valued elements in play, from the last round
    for (int round = 0;; round++) {
        uint32_t* h = hr[round & 1];
        const uint32_t span = hi - lo;
        const int shift = max(0, bitlen(span) - 12);
        if (!from_regs) {
#pragma unroll
            for (int j = 0; j < TR_CPT; j++) {
                const uint32_t kk = ck[j];
                if ((uint32_t)(tid + TR_THREADS * j) < ncand && kk >= lo && kk <= hi)
                    atomicAdd(&h[(kk - lo) >> shift], 1u);
            }
        } else {
            // (rare) the row again, from memory, so the registers above can go
            for (int t = tid; t < n; t += TR_THREADS) {
                const uint32_t kk = key_of(row[t]);
                if (kk >= lo && kk <= hi) atomicAdd(&h[(kk - lo) >> shift], 1u);
            }
        }
        __syncthreads();
        find_threshold_bin<TR_THREADS, TK_BINS>(h, need, &s_bin, &s_above, sh, &s_cnt);
        const uint32_t bin = s_bin;
        need -= s_above;
        for (int i = tid; i < TK_BINS; i += TR_THREADS) h[i] = 0u;  // for round + 2
        const uint32_t nlo = lo + (bin << shift);
        const uint32_t nhi = shift == 0 ? nlo : min(hi, nlo + ((1u << shift) - 1u));
        lo = nlo;
        hi = nhi;
        if (shift == 0) {
            eq_total = s_cnt;
            break;
        }
        // Few keys left in [lo, hi] (the usual case after the first round):
        // instead of more histogram rounds, one wave ranks them directly.
        if (!from_regs && s_cnt <= (uint32_t)TR_FEW) {
#pragma unroll
            for (int j = 0; j < TR_CPT; j++) {
                const uint32_t kk = ck[j];
                if ((uint32_t)(tid + TR_THREADS * j) < ncand && kk >= lo && kk <= hi) few[atomicAdd(&s_nfew, 1u)] = kk;
            }
            __syncthreads();
            if (wave == 0) rank_few(few, s_cnt, need, &s_theta, &s_needeq, &s_eqtot);
            __syncthreads();
            lo = s_theta;
            need = s_needeq;
            eq_total = s_eqtot;
            break;
        }
    }
    const uint32_t theta = lo;
    const uint32_t need_eq = need;
    // When every theta-valued element is kept, ties go straight to the result.
    const bool keep_all_ties = need_eq == eq_total;

    // ---- bitmaps ----------------------------------------------------------------
    // Candidates hold every element at or above theta except, in the
    // fallback, those above b0, which are marked already.
    if (!from_regs) {
#pragma unroll
        for (int j = 0; j < TR_CPT; j++) {
            const uint32_t kk = ck[j], t = cp[j];
            if ((uint32_t)(tid + TR_THREADS * j) < ncand && kk >= theta) {
                if (kk > theta || keep_all_ties) atomicOr(&gtbits[t >> 5], 1u << (t & 31));
                else atomicOr(&eqbits[t >> 5], 1u << (t & 31));
            }
        }
    } else {
        for (int t = tid; t < n; t += TR_THREADS) {
            const uint32_t kk = key_of(row[t]);
            if (kk >= theta) {
                if (kk > theta || keep_all_ties) atomicOr(&gtbits[t >> 5], 1u << (t & 31));
                else atomicOr(&eqbits[t >> 5], 1u << (t & 31));
            }
        }
    }
    __syncthreads();

    // ---- ordered output.  Thread tid owns the contiguous words [w0, w1). ----
    const int per = (nwords + TR_THREADS - 1) / TR_THREADS;
    const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
    uint32_t tot;
    if (!keep_all_ties) {
        uint32_t my_eq = 0;
        for (int w = w0; w < w1; w++) my_eq += __popc(eqbits[w]);
        uint32_t eq_before = block_exclusive_scan<TR_THREADS>(my_eq, &tot, sh);
        for (int w = w0; w < w1; w++) {
            uint32_t e = eqbits[w];
            uint32_t keep = 0;
            while (e && eq_before < need_eq) {
                const uint32_t low = e & (0u - e);
                keep |= low;
                e ^= low;
                eq_before++;
            }
            gtbits[w] |= keep;  // only this thread touches word w from here on
        }
    }
    uint32_t my_sel = 0;
    for (int w = w0; w < w1; w++) my_sel += __popc(gtbits[w]);
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

// ---------------------------------------------------------------------------
// Few rows (a decode batch) longer than one workgroup streams quickly (the
// longest above 65,536 positions, up to TM_MAXN).  Each row is split over
// 4,096-position chunks:
//   topk_sfilter_kernel   rows x chunks, 256 threads.  Every workgroup of a
//       row draws the same sample of 2,048 scores (32 blocks of 64 consecutive
//       positions spread evenly over the row) and finds the same bound
//       theta_lo: the lower edge of the 12-bit key bin that holds the sample's
//       rho-th largest key, rho = 1.3 x the rank the k-th largest element has
//       in the sample, plus 8.  Rows of at most TM_MINSAMPLE_N positions use
//       theta_lo = 0, i.e. every element.  The chunk's elements with key >=
//       theta_lo go to the chunk's own slots, in position order (thread t
//       holds positions 16 t .. 16 t + 15), with their count, their largest
//       key and theta_lo; nothing crosses workgroups, so nothing needs
//       clearing first.
//   topk_sresolve_kernel  one 1024-thread workgroup per row.  If the
//       candidates number at least k and fit in LDS, they hold the k-th largest key theta and every key above it, and
//       the radix rounds of topk_resolve_kernel (over [theta_lo, largest
//       candidate], early finish) give theta and need_eq.  The concatenated lists
//       are in position order, so two block scans over them give the
//       ascending output (theta-valued elements kept up to need_eq in
//       position order).  Otherwise (a misleading sample, huge tie groups, NaN)
//       three radix rounds and the ordered output run over the row itself,
//       read from memory: slower, equally exact.
// The sample only decides how fast a row goes, never what it selects.
constexpr int TM_MAXN = 262144;
constexpr int TM_MAXROWS = 256;
constexpr int TM_THREADS = 256;
constexpr int TM_SBLOCKS = 32;
constexpr int TM_SBLOCK = 64;
constexpr int TM_SAMPLES = TM_SBLOCKS * TM_SBLOCK;  // 8 per thread
constexpr int TM_CCAP = TK_CHUNK;                   // candidate slots per chunk (never overflow)
constexpr int TM_LCAP = 8192;                       // candidates the resolve holds in LDS
constexpr int TM_MINSAMPLE_N = 8192;
constexpr int TM_MAXCH = TM_MAXN / TK_CHUNK;        // 64 chunks
static_assert(TM_SAMPLES == 8 * TM_THREADS, "two sample float4 per thread");
static_assert(TK_CHUNK == TK_PER_THREAD * TM_THREADS, "one chunk per workgroup");
static_assert(TM_MAXCH == 64, "the resolve scans chunk counts with one wave");
constexpr int TM_RTHREADS = 1024;  // topk_sresolve_kernel

// Per-chunk record written by topk_sfilter_kernel: candidate count, largest
// candidate key, theta_lo.
constexpr int TM_CREC = 4;

__global__ __launch_bounds__(TM_THREADS) void topk_sfilter_kernel(const int32_t* __restrict__ vis,
                                                                  const float* __restrict__ scores, int64_t ld, int k,
                                                                  uint32_t* __restrict__ crec,
                                                                  unsigned long long* __restrict__ mcand, int chunks,
                                                                  int num_rows)
{
    const int r = grid_item();
    if (r >= num_rows) return;
    const int c = blockIdx.x;
    const int n = vis[r];
    const int start = c * TK_CHUNK;
    if (n <= k || start >= n) return;  // the resolve reads counts of chunks below n only, and only when n > k
    const int end = min(n, start + TK_CHUNK);
    const float* row = scores + (int64_t)r * ld;
    const int t = threadIdx.x;
    __shared__ __attribute__((aligned(16))) uint32_t h[TK_BINS];
    __shared__ uint32_t sh[TM_THREADS / 64];
    __shared__ uint32_t s_bin, s_above;

    // The chunk's keys and the sample go out together.
    uint32_t key[TK_PER_THREAD], present;
    load_chunk_keys(row, start, end, key, present);
    uint32_t thlo = 0u;
    if (n > TM_MINSAMPLE_N) {
        uint32_t sk[8];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            // 4-aligned block start with the block inside the row: s0 + 63 < n.
            const int blk = (t >> 4) + 16 * j;
            const int s0 = (int)(((int64_t)(n - TM_SBLOCK) * blk / (TM_SBLOCKS - 1)) & ~3LL);
            const float4 v = *reinterpret_cast<const float4*>(row + s0 + 4 * (t & 15));
            sk[4 * j + 0] = score_key(v.x);
            sk[4 * j + 1] = score_key(v.y);
            sk[4 * j + 2] = score_key(v.z);
            sk[4 * j + 3] = score_key(v.w);
        }
        const uint32_t rho = (uint32_t)min((int64_t)TM_SAMPLES,
                                           (13LL * k * TM_SAMPLES + 10LL * n - 1) / (10LL * n) + 8);
        for (int i = t; i < TK_BINS; i += TM_THREADS) h[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; e++) atomicAdd(&h[sk[e] >> 20], 1u);
        __syncthreads();
        find_threshold_bin<TM_THREADS, TK_BINS>(h, rho, &s_bin, &s_above, sh);
        thlo = s_bin << 20;
    }
    uint32_t sel = 0u, kmax = 0u;
#pragma unroll
    for (int i = 0; i < TK_PER_THREAD; i++)
        if (((present >> i) & 1u) && key[i] >= thlo) {
            sel |= 1u << i;
            kmax = max(kmax, key[i]);
        }
    // Exclusive scan of the counts and maximum of the keys, one barrier pair.
    const int lane = t & 63, wave = t >> 6;
    const uint32_t cnt = __popc(sel);
    const uint32_t incl = wave_inclusive_scan(cnt);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    __shared__ uint32_t smax[TM_THREADS / 64];
    if (lane == 63) sh[wave] = incl;
    if (lane == 0) smax[wave] = kmax;
    __syncthreads();
    uint32_t before = 0, total = 0, cmax = 0;
#pragma unroll
    for (int w = 0; w < TM_THREADS / 64; w++) {
        before += w < wave ? sh[w] : 0u;
        total += sh[w];
        cmax = max(cmax, smax[w]);
    }
    uint32_t slot = before + incl - cnt;
    unsigned long long* cc = mcand + ((int64_t)r * chunks + c) * TM_CCAP;
    const int t0 = start + TK_PER_THREAD * t;
#pragma unroll
    for (int i = 0; i < TK_PER_THREAD; i++)
        if ((sel >> i) & 1u) {
            if (slot < (uint32_t)TM_CCAP) cc[slot] = ((unsigned long long)key[i] << 32) | (uint32_t)(t0 + i);
            slot++;
        }
    if (t == 0) {
        uint32_t* rec = crec + ((int64_t)r * chunks + c) * TM_CREC;
        rec[0] = total;
        rec[1] = cmax;
        rec[2] = thlo;
    }
}

__global__ __launch_bounds__(TM_RTHREADS) void topk_sresolve_kernel(const int32_t* __restrict__ vis,
                                                                   const float* __restrict__ scores, int64_t ld,
                                                                   int k, int32_t* __restrict__ indices,
                                                                   const uint32_t* __restrict__ crec,
                                                                   const unsigned long long* __restrict__ mcand,
                                                                   int chunks, int num_rows)
{
    const int r = grid_item();
    if (r >= num_rows) return;
    const int n = vis[r];
    int32_t* out = indices + (int64_t)r * k;
    const int t = threadIdx.x;
    if (n <= k) {
        for (int i = t; i < k; i += TM_RTHREADS) out[i] = i < n ? i : -1;
        return;
    }
    __shared__ unsigned long long cl[TM_LCAP];
    __shared__ __attribute__((aligned(16))) uint32_t h[TK_BINS];
    __shared__ uint32_t coff[TM_MAXCH + 1];
    __shared__ uint32_t sh[TM_RTHREADS / 64];
    __shared__ uint32_t s_bin, s_above, s_cnt, s_total, s_over, s_max, s_thlo;
    __shared__ __attribute__((aligned(16))) uint32_t few[TR_FEW];
    __shared__ uint32_t s_nfew, s_theta, s_needeq, s_eqtot;
    const int nch = (n + TK_CHUNK - 1) / TK_CHUNK;  // <= TM_MAXCH

    // Chunk records -> offsets of each chunk's list in the concatenation,
    // the largest candidate key, theta_lo.
    if (t < 64) {
        uint4 rec = make_uint4(0u, 0u, 0u, 0u);
        if (t < nch) rec = *reinterpret_cast<const uint4*>(crec + ((int64_t)r * chunks + t) * TM_CREC);
        const uint32_t cnt = rec.x;
        const uint32_t incl = wave_inclusive_scan(cnt);
        coff[t] = incl - cnt;
        const bool over = __ballot(cnt > (uint32_t)TM_CCAP) != 0ull;
        uint32_t mx = rec.y;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
        if (t == 0) s_thlo = rec.z;
        if (t == 63) {
            coff[64] = incl;
            s_total = incl;
            s_over = over ? 1u : 0u;
            s_max = mx;
        }
    }
    if (t == 0) s_nfew = 0u;
    __syncthreads();
    const uint32_t m = s_total;
    const bool fast = !s_over && m >= (uint32_t)k && m <= (uint32_t)TM_LCAP;

    uint32_t theta, need_eq, eq_total = 0;
    bool keep_all_ties = false;
    if (fast) {
        // Each wave copies whole chunk lists (64 lanes per pass).
        for (int ch = t >> 6; ch < nch; ch += TM_RTHREADS / 64) {
            const uint32_t o = coff[ch], cnt = coff[ch + 1] - o;
            const unsigned long long* src = mcand + ((int64_t)r * chunks + ch) * TM_CCAP;
            for (uint32_t j = t & 63; j < cnt; j += 64) cl[o + j] = src[j];
        }
        __syncthreads();
        // Radix rounds over [theta_lo, largest candidate]: every candidate's
        // key lies there (and m >= k >= 1 makes the maximum a real key).
        uint32_t lo = s_thlo, hi = s_max, nd = (uint32_t)k;
        for (;;) {
            const uint32_t span = hi - lo;
            const int shift = span < (uint32_t)TK_BINS ? 0 : (32 - __clz(span)) - 12;
            for (int i = t; i < TK_BINS; i += TM_RTHREADS) h[i] = 0u;
            __syncthreads();
            for (uint32_t i = t; i < m; i += TM_RTHREADS) {
                const uint32_t key = (uint32_t)(cl[i] >> 32);
                if (key >= lo && key <= hi) atomicAdd(&h[(key - lo) >> shift], 1u);
            }
            __syncthreads();
            find_threshold_bin<TM_RTHREADS, TK_BINS>(h, nd, &s_bin, &s_above, sh, &s_cnt);
            nd -= s_above;
            lo += s_bin << shift;
            hi = (uint32_t)min((uint64_t)hi, (uint64_t)lo + ((1ull << shift) - 1));
            if (shift == 0) {  // wave-uniform: every thread holds the same lo, hi
                eq_total = s_cnt;
                break;
            }
            if (s_cnt <= (uint32_t)TR_FEW) {
                for (uint32_t i = t; i < m; i += TM_RTHREADS) {
                    const uint32_t key = (uint32_t)(cl[i] >> 32);
                    if (key >= lo && key <= hi) few[atomicAdd(&s_nfew, 1u)] = key;
                }
                __syncthreads();
                if (t < 64) rank_few(few, s_cnt, nd, &s_theta, &s_needeq, &s_eqtot);
                __syncthreads();
                lo = s_theta;
                nd = s_needeq;
                eq_total = s_eqtot;
                break;
            }
        }
        theta = lo;
        need_eq = nd;
        keep_all_ties = need_eq == eq_total;

        // Ordered output: thread t owns candidates [t per, (t + 1) per) of the
        // position-ordered list.
        const uint32_t per = (m + TM_RTHREADS - 1) / TM_RTHREADS;
        const uint32_t i0 = min(m, t * per), i1 = min(m, i0 + per);
        uint32_t tot, eq_rank = 0;
        if (!keep_all_ties) {
            uint32_t neq = 0;
            for (uint32_t i = i0; i < i1; i++) neq += (uint32_t)(cl[i] >> 32) == theta;
            eq_rank = block_exclusive_scan<TM_RTHREADS>(neq, &tot, sh);
        }
        uint32_t nk = 0, er = eq_rank;
        for (uint32_t i = i0; i < i1; i++) {
            const uint32_t key = (uint32_t)(cl[i] >> 32);
            if (key > theta) nk++;
            else if (key == theta) nk += (keep_all_ties || er++ < need_eq) ? 1u : 0u;
        }
        uint32_t pos = block_exclusive_scan<TM_RTHREADS>(nk, &tot, sh);
        er = eq_rank;
        for (uint32_t i = i0; i < i1; i++) {
            const uint32_t key = (uint32_t)(cl[i] >> 32);
            bool keep = key > theta;
            if (key == theta) keep = keep_all_ties || er++ < need_eq;
            if (keep) {
                if (pos < (uint32_t)k) out[pos] = (int32_t)(uint32_t)cl[i];
                pos++;
            }
        }
        return;
    }

    // Exact path over the row itself (a misleading sample, ties or NaN
    // filling the chunk slots).  Three radix rounds on absolute key bits.
    const float* row = scores + (int64_t)r * ld;
    for (int i = t; i < TK_BINS; i += TM_RTHREADS) h[i] = 0u;
    __syncthreads();
    for (int p = t; p < n; p += TM_RTHREADS) atomicAdd(&h[score_key(row[p]) >> 20], 1u);
    __syncthreads();
    find_threshold_bin<TM_RTHREADS, TK_BINS>(h, (uint32_t)k, &s_bin, &s_above, sh);
    const uint32_t b0 = s_bin;
    const uint32_t need = (uint32_t)k - s_above;
    for (int i = t; i < TK_BINS; i += TM_RTHREADS) h[i] = 0u;
    __syncthreads();
    for (int p = t; p < n; p += TM_RTHREADS) {
        const uint32_t key = score_key(row[p]);
        if ((key >> 20) == b0) atomicAdd(&h[(key >> 8) & 0xfffu], 1u);
    }
    __syncthreads();
    find_threshold_bin<TM_RTHREADS, TK_BINS>(h, need, &s_bin, &s_above, sh);
    const uint32_t pre20 = (b0 << 12) | s_bin;
    const uint32_t need2 = need - s_above;
    for (int i = t; i < 1024; i += TM_RTHREADS) h[i] = 0u;
    __syncthreads();
    for (int p = t; p < n; p += TM_RTHREADS) {
        const uint32_t key = score_key(row[p]);
        if ((key >> 8) == pre20) atomicAdd(&h[key & 0xffu], 1u);
    }
    __syncthreads();
    find_threshold_bin<TM_RTHREADS, 1024>(h, need2, &s_bin, &s_above, sh);
    theta = (pre20 << 8) | s_bin;
    need_eq = need2 - s_above;
    // Thread t owns positions [t per, (t + 1) per): ties ranked in position
    // order, then the kept positions written in order.
    const int per = (n + TM_RTHREADS - 1) / TM_RTHREADS;
    const int p0 = min(n, t * per), p1 = min(n, p0 + per);
    uint32_t tot, neq = 0;
    for (int p = p0; p < p1; p++) neq += score_key(row[p]) == theta;
    const uint32_t eq_rank = block_exclusive_scan<TM_RTHREADS>(neq, &tot, sh);
    uint32_t nk = 0, er = eq_rank;
    for (int p = p0; p < p1; p++) {
        const uint32_t key = score_key(row[p]);
        if (key > theta) nk++;
        else if (key == theta) nk += er++ < need_eq ? 1u : 0u;
    }
    uint32_t pos = block_exclusive_scan<TM_RTHREADS>(nk, &tot, sh);
    er = eq_rank;
    for (int p = p0; p < p1; p++) {
        const uint32_t key = score_key(row[p]);
        bool keep = key > theta;
        if (key == theta) keep = er++ < need_eq;
        if (keep) {
            if (pos < (uint32_t)k) out[pos] = p;
            pos++;
        }
    }
}

// Calls whose rows all have at most TS_MAXN positions (a prefill chunk of up
// to 8,192 tokens, short decode rows): 256 threads per row and the row's keys
// held in registers, 32 per thread.  The radix rounds histogram those
// registers directly (11-bit digits relative to the row's key range, so at
// most three rounds), without a candidate list, so a workgroup needs ~19 KB
// of LDS and several rows share a CU, where the 1024-thread kernel holds a CU
// for each row in turn.  Same order and output as topk_rows_kernel: theta is
// the k-th largest key, every larger key is kept, and of the theta-valued
// elements the first need_eq in position order.
constexpr int TS_THREADS = 256;
constexpr int TS_GROUPS = 8;                         // float4 groups per thread
constexpr int TS_MAXN = 4 * TS_THREADS * TS_GROUPS;  // 8,192
constexpr int TS_BINS = 2048;                        // 11-bit digit
constexpr int TS_WORDS = TS_MAXN / 32;               // bitmap words: one per thread
static_assert(TS_WORDS == TS_THREADS, "thread t owns bitmap word t");

__global__ __launch_bounds__(TS_THREADS) void topk_short_kernel(const int32_t* __restrict__ vis,
                                                                const float* __restrict__ scores, int64_t ld,
                                                                int k, int32_t* __restrict__ indices, int num_rows)
{
    const int r = grid_item();
    if (r >= num_rows) return;
    const int n = vis[r];
    int32_t* out = indices + (int64_t)r * k;
    const int tid = threadIdx.x;
    if (n <= k) {
        for (int t = tid; t < k; t += TS_THREADS) out[t] = t < n ? t : -1;
        return;
    }
    __shared__ __attribute__((aligned(16))) uint32_t hist[2][TS_BINS];  // radix rounds, alternating
    __shared__ uint32_t gtbits[TS_WORDS];
    __shared__ uint32_t eqbits[TS_WORDS];
    __shared__ uint32_t sh[TS_THREADS / 64];
    __shared__ uint32_t wlo[TS_THREADS / 64], whi[TS_THREADS / 64];
    __shared__ uint32_t s_bin, s_above, s_cnt;
    __shared__ __attribute__((aligned(16))) uint32_t few[TR_FEW];  // the last keys in play (early finish)
    __shared__ uint32_t s_nfew, s_theta, s_needeq, s_eqtot;

    // ---- the row's keys, into registers ------------------------------------
    // Element (u, q) of thread t is position 4 (t + TS_THREADS u) + q.  A
    // 4-aligned group starting below n lies inside the row allocation (ld is
    // a multiple of 4 and n <= ld); lanes past the row re-read its last group
    // and are masked out by the position test.
    const float* row = scores + (int64_t)r * ld;
    const int nu = (n + 4 * TS_THREADS - 1) / (4 * TS_THREADS);
    const int lim = n - 4 * tid;  // element (u, q) is in the row iff 4 TS_THREADS u + q < lim
    uint32_t key[TS_GROUPS][4];
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int u = 0; u < TS_GROUPS; u++) {
        if (u < nu) {
            const int p = min(4 * (tid + TS_THREADS * u), (n - 1) & ~3);
            const float4 v = *reinterpret_cast<const float4*>(row + p);
            key[u][0] = key_of(v.x);
            key[u][1] = key_of(v.y);
            key[u][2] = key_of(v.z);
            key[u][3] = key_of(v.w);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                if (4 * TS_THREADS * u + q < lim) {
                    kmin = min(kmin, key[u][q]);
                    kmax = max(kmax, key[u][q]);
                }
            }
        }
    }
    for (int i = tid; i < 2 * TS_BINS / 4; i += TS_THREADS)
        reinterpret_cast<uint4*>(&hist[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
    gtbits[tid] = 0u;
    eqbits[tid] = 0u;
    if (tid == 0) s_nfew = 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    const int lane = tid & 63, wave = tid >> 6;
    if (lane == 0) {
        wlo[wave] = kmin;
        whi[wave] = kmax;
    }
    __syncthreads();  // histograms and bitmaps cleared, range published
    uint32_t lo = wlo[0], hi = whi[0];
#pragma unroll
    for (int w = 1; w < TS_THREADS / 64; w++) {
        lo = min(lo, wlo[w]);
        hi = max(hi, whi[w]);
    }

    // ---- radix rounds on [lo, hi] ----------------------------------------
    // Each round histograms (key - lo) >> shift over the keys in [lo, hi]
    // and narrows [lo, hi] to the bin holding the need-th largest (k < n, so
    // it exists).  A histogram is cleared for the round after next.
    uint32_t need = (uint32_t)k;
    for (int round = 0;; round++) {
        uint32_t* h = hist[round & 1];
        const int shift = max(0, bitlen(hi - lo) - 11);
#pragma unroll
        for (int u = 0; u < TS_GROUPS; u++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint32_t kk = key[u][q];
                if (u < nu && 4 * TS_THREADS * u + q < lim && kk >= lo && kk <= hi)
                    atomicAdd(&h[(kk - lo) >> shift], 1u);
            }
        }
        __syncthreads();
        find_threshold_bin<TS_THREADS, TS_BINS>(h, need, &s_bin, &s_above, sh, &s_cnt);
        const uint32_t bin = s_bin;
        need -= s_above;
        for (int i = tid; i < TS_BINS / 4; i += TS_THREADS)
            reinterpret_cast<uint4*>(h)[i] = make_uint4(0u, 0u, 0u, 0u);
        const uint32_t nlo = lo + (bin << shift);
        hi = shift == 0 ? nlo : min(hi, nlo + ((1u << shift) - 1u));
        lo = nlo;
        if (shift == 0) break;
        // Few keys left in [lo, hi]: one wave ranks them (see rank_few).
        if (s_cnt <= (uint32_t)TR_FEW) {
#pragma unroll
            for (int u = 0; u < TS_GROUPS; u++) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const uint32_t kk = key[u][q];
                    if (u < nu && 4 * TS_THREADS * u + q < lim && kk >= lo && kk <= hi)
                        few[atomicAdd(&s_nfew, 1u)] = kk;
                }
            }
            __syncthreads();
            if (tid < 64) rank_few(few, s_cnt, need, &s_theta, &s_needeq, &s_eqtot);
            __syncthreads();
            lo = s_theta;
            need = s_needeq;
            break;
        }
    }
    const uint32_t theta = lo, need_eq = need;

    // ---- bitmaps, then the ordered output (thread t owns word t) --------
#pragma unroll
    for (int u = 0; u < TS_GROUPS; u++) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const uint32_t kk = key[u][q];
            const int p = 4 * (tid + TS_THREADS * u) + q;
            if (u < nu && 4 * TS_THREADS * u + q < lim && kk >= theta) {
                if (kk > theta) atomicOr(&gtbits[p >> 5], 1u << (p & 31));
                else atomicOr(&eqbits[p >> 5], 1u << (p & 31));
            }
        }
    }
    __syncthreads();
    const uint32_t g = gtbits[tid], e = eqbits[tid];
    // Both counts in one scan (each total is at most TS_MAXN < 2^16).
    uint32_t tot;
    const uint32_t before = block_exclusive_scan<TS_THREADS>((uint32_t)__popc(g) | ((uint32_t)__popc(e) << 16),
                                                             &tot, sh);
    const uint32_t gt_before = before & 0xffffu, eq_before = before >> 16;
    // The theta-valued elements kept are the first need_eq in position order.
    uint32_t keep = 0, ee = e;
    for (uint32_t left = need_eq > eq_before ? need_eq - eq_before : 0u; ee && left; left--) {
        const uint32_t low = ee & (0u - ee);
        keep |= low;
        ee ^= low;
    }
    uint32_t sel = g | keep;
    uint32_t pos = gt_before + min(eq_before, need_eq);
    while (sel) {
        const int bit = __ffs(sel) - 1;
        sel &= sel - 1u;
        if (pos < (uint32_t)k) out[pos] = (tid << 5) + bit;  // exactly k are selected
        pos++;
    }
}


// ---------------------------------------------------------------------------
// Many rows of up to 65,536 positions (the rows of a prefill chunk): one
// 256-thread workgroup per row with ~40 KB of LDS, so four rows share a CU
// and the barrier-bound selection of one row overlaps the others' streaming
// (the 1024-thread kernel holds a CU for each row in turn).  The row is read
// from memory once, as it streams past a bound:
//   1. Bound: 4,096 sampled scores (64 blocks of 64 consecutive positions
//      spread evenly over the row).  Two 11-bit radix rounds over their keys
//      give the 22-bit prefix of the rho-th largest sample key, rho = E +
//      4 sqrt(E) + 16 with E = k 4096 / n the rank the k-th largest element
//      has in the sample on average; its lower edge is the bound theta_lo.
//      Rows of at most TQ_ALL positions take every element instead.
//   2. Stream: wave w owns the w-th quarter of the row (a multiple of 256
//      positions) and appends the elements whose key is >= theta_lo (a float
//      compare against the bound's float, as in topk_rows_kernel) to its own
//      ordered list: one wave prefix sum per 256 positions, slots in 64-slot
//      chunks of a pool the four waves share (a wave takes chunks as it
//      needs them, so rows whose large scores cluster in one quarter fit as
//      well as any other).  Key and 16-bit position per slot.
//   3. Select: if the lists hold at least k elements and the pool did not run
//      out, they hold the k-th largest key theta and every larger key, and
//      radix rounds over [theta_lo, largest candidate] (10 bits a round,
//      early finish with rank_few) give theta and need_eq.
//   4. Output: the four lists in wave order are in position order.  Each
//      thread takes a contiguous run of entries; one packed block scan gives
//      its output offset and the count of theta-valued entries before it, and
//      the first need_eq of those are kept.
// When the sampled bound fails (fewer than k candidates, or more than the
// pool holds), a histogram of the whole row's top 10 key bits gives the bin
// of the k-th largest; if that bin and everything above it fit the pool, the
// row streams once more past that exact bound and steps 3-4 run as above.
// Otherwise (huge tie groups, all-equal rows) four radix rounds and an
// ordered pass run over the row itself.  Exact for any input.
constexpr int TQ_THREADS = 256;
constexpr int TQ_WAVES = TQ_THREADS / 64;
constexpr int TQ_CHUNKS = 83;               // pool: 83 chunks of 64 slots
constexpr int TQ_CAP = TQ_CHUNKS * 64;      // 5,312 slots: 4 B key + 2 B position each
constexpr int TQ_FIT = TQ_CAP - TQ_WAVES * 63;  // candidates that always fit (each wave's last chunk partly empty)
constexpr int TQ_BINS = 1024;               // 10-bit digit
constexpr int TQ_SBLOCKS = 64;
constexpr int TQ_SBLOCK = 64;
constexpr int TQ_SAMPLES = TQ_SBLOCKS * TQ_SBLOCK;  // 16 per thread
constexpr int TQ_MAXN = 65536;              // positions fit the 16-bit slots
constexpr int TQ_ALL = 4096;                // rows of at most this take every element
constexpr int TQ_MIN_ROWS = 1024;           // calls with at least this many rows take the kernel
constexpr int TQ_PF = 4;                    // stream steps in flight per wave
static_assert(TQ_SAMPLES == 16 * TQ_THREADS, "four sample float4 per thread");
static_assert(TQ_ALL <= TQ_FIT, "a short row fits the pool whole");

__global__ __launch_bounds__(TQ_THREADS) void topk_stream_kernel(const int32_t* __restrict__ vis,
                                                                 const float* __restrict__ scores, int64_t ld,
                                                                 int k, int32_t* __restrict__ indices,
                                                                 int num_rows)
{
    const int r = grid_item();
    if (r >= num_rows) return;
    const int n = vis[r];
    if (n > TQ_MAXN) return;  // the multi-workgroup path owns this row
    int32_t* out = indices + (int64_t)r * k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (n <= k) {
        for (int t = tid; t < k; t += TQ_THREADS) out[t] = t < n ? t : -1;
        return;
    }
    __shared__ __attribute__((aligned(16))) uint32_t hist[2][TQ_BINS];  // radix rounds, alternating
    __shared__ uint32_t pkey[TQ_CAP];
    __shared__ uint16_t ppos[TQ_CAP];
    __shared__ uint8_t wch[TQ_WAVES][TQ_CHUNKS];  // each wave's chunks, in order
    __shared__ uint32_t sh[TQ_WAVES];
    __shared__ uint32_t wcnt[TQ_WAVES], wmax[TQ_WAVES];
    __shared__ uint32_t s_bin, s_above, s_cnt, s_next;
    __shared__ __attribute__((aligned(16))) uint32_t few[TR_FEW];
    __shared__ uint32_t s_nfew, s_theta, s_needeq, s_eqtot;
    const float* row = scores + (int64_t)r * ld;

    auto clear_hist = [&]() {
        for (int i = tid; i < 2 * TQ_BINS / 4; i += TQ_THREADS)
            reinterpret_cast<uint4*>(&hist[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
    };
    clear_hist();
    if (tid == 0) s_nfew = 0u;

    // ---- 1. sampled bound -------------------------------------------------
    uint32_t lo0 = 0x007fffffu;  // key(-inf): every element but NaN
    if (n > TQ_ALL) {
        uint32_t sk[16];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            // 4-aligned block start with the block inside the row: s0 + 63 < n.
            const int blk = (tid >> 4) + 16 * j;
            const int s0 = (int)(((int64_t)(n - TQ_SBLOCK) * blk / (TQ_SBLOCKS - 1)) & ~3LL);
            const float4 v = *reinterpret_cast<const float4*>(row + s0 + 4 * (tid & 15));
            sk[4 * j + 0] = key_of(v.x);
            sk[4 * j + 1] = key_of(v.y);
            sk[4 * j + 2] = key_of(v.z);
            sk[4 * j + 3] = key_of(v.w);
        }
        const float E = (float)k * (float)TQ_SAMPLES / (float)n;
        const uint32_t rho = (uint32_t)min((float)TQ_SAMPLES, E + 4.f * sqrtf(E) + 16.f);
        __syncthreads();  // histograms cleared
        // Top 11 key bits (the two 10-bit histograms side by side hold 2,048 bins).
        uint32_t* h11 = &hist[0][0];
#pragma unroll
        for (int e = 0; e < 16; e++) atomicAdd(&h11[sk[e] >> 21], 1u);
        __syncthreads();
        find_threshold_bin<TQ_THREADS, 2 * TQ_BINS>(h11, rho, &s_bin, &s_above, sh);
        const uint32_t b1 = s_bin, rho2 = rho - s_above;
        clear_hist();
        __syncthreads();
        // Next 11 bits of the samples inside that bin.
#pragma unroll
        for (int e = 0; e < 16; e++)
            if ((sk[e] >> 21) == b1) atomicAdd(&h11[(sk[e] >> 10) & 0x7ffu], 1u);
        __syncthreads();
        find_threshold_bin<TQ_THREADS, 2 * TQ_BINS>(h11, rho2, &s_bin, &s_above, sh);
        lo0 = max((b1 << 21) | (s_bin << 10), 0x007fffffu);
        clear_hist();
    }

    // ---- 2. stream the row past a bound -------------------------------------
    // Wave w: positions [w Q, min(n, (w + 1) Q)), 256 per step, lane l taking
    // the 4-aligned group at 4 l (inside the row allocation: ld is a multiple
    // of 4 and n <= ld), TQ_PF steps of loads in flight.  Returns false if the
    // pool ran out.  Counts and largest keys go to wcnt / wmax.
    const int Q = ((n + 4 * TQ_WAVES - 1) / (4 * TQ_WAVES) + 63) / 64 * 256;
    // Loads are never conditional (a branch around them would make the
    // compiler wait for every load at once): addresses past the row are
    // clamped onto its last 4-aligned group, and their elements masked.
    const int pmax = (n - 1) & ~3;
    const int wbeg = wave * Q, wend = min(n, wbeg + Q);
    const int nsteps = wend > wbeg ? (wend - wbeg + 255) / 256 : 0;
    auto stream_pass = [&](uint32_t lo) {
        const float flo = float_of_key(lo);
        if (tid == 0) s_next = 0u;
        __syncthreads();  // pool counter reset; previous readers of the lists done
        // cnt, nch and full are wave-uniform; readfirstlane keeps them scalar.
        uint32_t cnt = 0, kmax = 0, nch = 0, full = 0;
        auto load = [&](int st) {
            return *reinterpret_cast<const float4*>(row + min(wbeg + 256 * st + 4 * lane, pmax));
        };
        auto step = [&](int st, const float4& v) {
            const int p = wbeg + 256 * st + 4 * lane;
            const float x[4] = {v.x, v.y, v.z, v.w};
            uint32_t f = 0;
#pragma unroll
            for (int q = 0; q < 4; q++) f |= (p + q < wend && x[q] >= flo) ? (1u << q) : 0u;
            const uint32_t c = (uint32_t)__popc(f);
            const uint32_t incl = wave_inclusive_scan(c);
            const uint32_t step_total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            // Chunks for slots [cnt, cnt + step_total) of this wave's list.
            const uint32_t need = (uint32_t)__builtin_amdgcn_readfirstlane((int)((cnt + step_total + 63u) >> 6));
            if (!full && need > nch) {
                uint32_t first = 0;
                if (lane == 0) first = atomicAdd(&s_next, need - nch);
                first = (uint32_t)__builtin_amdgcn_readfirstlane((int)first);
                if (first + (need - nch) > (uint32_t)TQ_CHUNKS) full = 1u;
                else if ((uint32_t)lane < need - nch) wch[wave][nch + lane] = (uint8_t)(first + lane);
                nch = need;
            }
            uint32_t slot = cnt + incl - c;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                if ((f >> q) & 1u) {
                    const uint32_t kk = key_of(x[q]);
                    kmax = max(kmax, kk);
                    if (!full) {
                        const uint32_t i = (uint32_t)wch[wave][slot >> 6] * 64u + (slot & 63u);
                        pkey[i] = kk;
                        ppos[i] = (uint16_t)(p + q);
                    }
                    slot++;
                }
            }
            cnt = (uint32_t)__builtin_amdgcn_readfirstlane((int)(cnt + step_total));
        };
        // Groups of TQ_PF steps: the loads of group g + 1 go out before group g
        // is processed (two register sets, loop unrolled by two groups).
        float4 va[TQ_PF], vb[TQ_PF];
#pragma unroll
        for (int i = 0; i < TQ_PF; i++) va[i] = load(i);
        for (int g0 = 0; g0 < nsteps; g0 += 2 * TQ_PF) {
#pragma unroll
            for (int i = 0; i < TQ_PF; i++) vb[i] = load(g0 + TQ_PF + i);
#pragma unroll
            for (int i = 0; i < TQ_PF; i++)
                if (g0 + i < nsteps) step(g0 + i, va[i]);
#pragma unroll
            for (int i = 0; i < TQ_PF; i++) va[i] = load(g0 + 2 * TQ_PF + i);
#pragma unroll
            for (int i = 0; i < TQ_PF; i++)
                if (g0 + TQ_PF + i < nsteps) step(g0 + TQ_PF + i, vb[i]);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
        if (lane == 0) {
            wcnt[wave] = full ? 0xffffffffu : cnt;
            wmax[wave] = kmax;
        }
        __syncthreads();  // lists, counts and cleared histograms visible
    };
    uint32_t cw[TQ_WAVES], total = 0, hi = 0;
    auto gather_counts = [&]() {
        bool full = false;
        total = 0;
        hi = 0;
#pragma unroll
        for (int w = 0; w < TQ_WAVES; w++) {
            cw[w] = wcnt[w];
            full |= cw[w] == 0xffffffffu;
            total += full ? 0u : cw[w];
            hi = max(hi, wmax[w]);
        }
        return !full && total >= (uint32_t)k;
    };
    stream_pass(lo0);
    bool fast = gather_counts();

    uint32_t need = (uint32_t)k;
    uint32_t lo = lo0;
    auto row_keys = [&](auto&& fn) {  // every element of the row, 4 float4 per thread in flight
        for (int p0 = 4 * tid; p0 < n; p0 += 16 * TQ_THREADS) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; u++) v[u] = *reinterpret_cast<const float4*>(row + min(p0 + 4 * TQ_THREADS * u, pmax));
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int p = p0 + 4 * TQ_THREADS * u;
                const float x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int q = 0; q < 4; q++)
                    if (p + q < n) fn(key_of(x[q]));
            }
        }
    };
    bool rows_path = false;  // selection over the row itself (no lists)
    if (!fast) {
        // Exact bin of the k-th largest: top 10 key bits of the whole row
        // (NaN, key 0, included).  hist[0] is clear (stream_pass ran after the
        // last clear and uses no histogram).
        uint32_t* h = hist[0];
        row_keys([&](uint32_t kk) { atomicAdd(&h[kk >> 22], 1u); });
        __syncthreads();
        find_threshold_bin<TQ_THREADS, TQ_BINS>(h, (uint32_t)k, &s_bin, &s_above, sh, &s_cnt);
        const uint32_t b0 = s_bin;
        const uint32_t upto = s_above + s_cnt;  // elements with key >= b0 << 22
        for (int i = tid; i < TQ_BINS / 4; i += TQ_THREADS) reinterpret_cast<uint4*>(h)[i] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();  // cleared before the radix rounds or the next pass use it
        if (upto <= (uint32_t)TQ_FIT && b0 != 0u) {
            // The lists can hold them: stream again past the exact bound (keys
            // below key(-inf) belong to NaN only, and NaN keys are 0).
            lo = max(b0 << 22, 0x007fffffu);
            stream_pass(lo);
            fast = gather_counts();  // total == upto >= k, and it fits
        }
        if (!fast) {
            rows_path = true;
            lo = 0u;
            hi = 0xffffffffu;
        }
    }

    // ---- 3. radix rounds --------------------------------------------------------
    // Each round histograms (key - lo) >> shift over the keys in [lo, hi],
    // from the lists or (rows_path) the row, and narrows [lo, hi] to the bin
    // holding the need-th largest.
    auto list_slot = [&](int w, uint32_t g) { return (uint32_t)wch[w][g >> 6] * 64u + (g & 63u); };
    auto each_key = [&](auto&& fn) {
        if (!rows_path) {
#pragma unroll
            for (int w = 0; w < TQ_WAVES; w++)
                for (uint32_t g = tid; g < cw[w]; g += TQ_THREADS) fn(pkey[list_slot(w, g)]);
        } else {
            row_keys(fn);
        }
    };
    for (int round = 0;; round++) {
        uint32_t* h = hist[round & 1];
        const int shift = max(0, bitlen(hi - lo) - 10);
        const uint32_t lo_r = lo, hi_r = hi;
        each_key([&](uint32_t kk) {
            if (kk >= lo_r && kk <= hi_r) atomicAdd(&h[(kk - lo_r) >> shift], 1u);
        });
        __syncthreads();
        find_threshold_bin<TQ_THREADS, TQ_BINS>(h, need, &s_bin, &s_above, sh, &s_cnt);
        const uint32_t bin = s_bin;
        need -= s_above;
        for (int i = tid; i < TQ_BINS / 4; i += TQ_THREADS)
            reinterpret_cast<uint4*>(h)[i] = make_uint4(0u, 0u, 0u, 0u);  // for round + 2
        const uint32_t nlo = lo + (bin << shift);
        hi = shift == 0 ? nlo : min(hi, nlo + ((1u << shift) - 1u));
        lo = nlo;
        if (shift == 0) break;
        // Few keys left in [lo, hi]: one wave ranks them.
        if (!rows_path && s_cnt <= (uint32_t)TR_FEW) {
            const uint32_t lo_f = lo, hi_f = hi;
            each_key([&](uint32_t kk) {
                if (kk >= lo_f && kk <= hi_f) few[atomicAdd(&s_nfew, 1u)] = kk;
            });
            __syncthreads();
            if (tid < 64) rank_few(few, s_cnt, need, &s_theta, &s_needeq, &s_eqtot);
            __syncthreads();
            lo = s_theta;
            need = s_needeq;
            break;
        }
    }
    const uint32_t theta = lo, need_eq = need;

    // ---- 4. ordered output ------------------------------------------------------
    uint32_t tot;
    if (!rows_path) {
        // Entry e of the lists in wave order: wave w = the number of lists that
        // end at or below e, index e - (entries of the waves before w).
        const uint32_t per = (total + TQ_THREADS - 1) / TQ_THREADS;
        const uint32_t e0 = min(total, tid * per), e1 = min(total, e0 + per);
        auto entry = [&](uint32_t e) {
            int w = 0;
            uint32_t base = 0;
#pragma unroll
            for (int i = 0; i < TQ_WAVES - 1; i++) {
                if (w == i && e >= base + cw[i]) {
                    base += cw[i];
                    w++;
                }
            }
            return list_slot(w, e - base);
        };
        uint32_t gt = 0, eq = 0;
        for (uint32_t e = e0; e < e1; e++) {
            const uint32_t kk = pkey[entry(e)];
            gt += kk > theta ? 1u : 0u;
            eq += kk == theta ? 1u : 0u;
        }
        // Both counts in one scan (each total is below TQ_CAP < 2^16).
        const uint32_t before = block_exclusive_scan<TQ_THREADS>(gt | (eq << 16), &tot, sh);
        uint32_t eqb = before >> 16;
        uint32_t pos = (before & 0xffffu) + min(eqb, need_eq);
        for (uint32_t e = e0; e < e1; e++) {
            const uint32_t i = entry(e);
            const uint32_t kk = pkey[i];
            bool keep = kk > theta;
            if (kk == theta) {
                keep = eqb < need_eq;
                eqb++;
            }
            if (keep) {
                if (pos < (uint32_t)k) out[pos] = (int32_t)ppos[i];  // exactly k are kept
                pos++;
            }
        }
    } else {
        // Thread t owns positions [t S, (t + 1) S): count, two block scans
        // (counts above theta, theta-valued counts), then write in order.
        const int S = ((n + TQ_THREADS - 1) / TQ_THREADS + 3) & ~3;
        const int pb = min(n, tid * S), pe = min(n, pb + S);
        uint32_t gt = 0, eq = 0;
        for (int p = pb; p < pe; p += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + p);
            const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint32_t kk = key_of(x[q]);
                gt += (p + q < pe && kk > theta) ? 1u : 0u;
                eq += (p + q < pe && kk == theta) ? 1u : 0u;
            }
        }
        const uint32_t gt_before = block_exclusive_scan<TQ_THREADS>(gt, &tot, sh);
        uint32_t eqb = block_exclusive_scan<TQ_THREADS>(eq, &tot, sh);
        uint32_t pos = gt_before + min(eqb, need_eq);
        for (int p = pb; p < pe; p += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + p);
            const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                if (p + q >= pe) continue;
                const uint32_t kk = key_of(x[q]);
                bool keep = kk > theta;
                if (kk == theta) {
                    keep = eqb < need_eq;
                    eqb++;
                }
                if (keep) {
                    if (pos < (uint32_t)k) out[pos] = p + q;
                    pos++;
                }
            }
        }
    }
}

}  // namespace

// Calls that take the chunked path for few rows (topk_sfilter_kernel).
static bool topk_chunked_path(int32_t num_rows, int32_t max_visible)
{
    return num_rows <= TM_MAXROWS && max_visible > TR_ROW_PATH_MAXN && max_visible <= TM_MAXN;
}

size_t topk_workspace_bytes(int32_t num_rows, int32_t max_visible)
{
    if (topk_chunked_path(num_rows, max_visible)) {
        // per-chunk candidate counts and slots
        const size_t R = (size_t)num_rows;
        const size_t CH = (size_t)((max_visible + TK_CHUNK - 1) / TK_CHUNK);
        return align_up(R * CH * TM_CREC * 4, 256) + align_up(R * CH * TM_CCAP * 8, 256);
    }
    if (max_visible <= TR_ROW_PATH_MAXN) return 0;  // the one-workgroup-per-row path needs none
    const size_t R = (size_t)num_rows;
    const size_t CH = (size_t)((max_visible + TK_CHUNK - 1) / TK_CHUNK);
    size_t b = 0;
    b += align_up(R * TK_ROWST * 4, 256);
    b += align_up(R * CH * TK_CHUNKST * 4, 256);
    b += align_up(R * TK_CAP * 8, 256);
    b += align_up(R * 4, 256);  // list of long rows
    b += 256;                   // its length
    return b;
}

TopkWorkspace topk_workspace_carve(void* ws, int32_t num_rows, int32_t max_visible)
{
    const size_t R = (size_t)num_rows;
    const int32_t CH = (max_visible + TK_CHUNK - 1) / TK_CHUNK;
    char* p = (char*)ws;
    TopkWorkspace tw{};
    if (topk_chunked_path(num_rows, max_visible)) {
        tw.crec = (uint32_t*)p;
        p += align_up(R * CH * TM_CREC * 4, 256);
        tw.mcand = (unsigned long long*)p;
        tw.chunks = CH;
        return tw;
    }
    tw.rowst = (uint32_t*)p;
    p += align_up(R * TK_ROWST * 4, 256);
    tw.chunkst = (uint32_t*)p;
    p += align_up(R * (size_t)CH * TK_CHUNKST * 4, 256);
    tw.cand = (unsigned long long*)p;
    p += align_up(R * TK_CAP * 8, 256);
    tw.longrows = (int32_t*)p;
    p += align_up(R * 4, 256);
    tw.nlong = (uint32_t*)p;
    tw.chunks = CH;
    return tw;
}

void launch_topk(int32_t num_rows, int32_t max_visible, const int32_t* vis, const float* scores, int64_t ld,
                 int32_t k, int32_t* indices, const TopkWorkspace& tw, hipStream_t stream)
{
    // Rows of up to TR_ROW_PATH_MAXN positions take one workgroup each; longer
    // rows (present only when max_visible exceeds it) are split over
    // workgroups.  Each kernel skips the rows the other path owns.
    // The row kernel also samples the long rows (the first step of their
    // path), so it goes first.
    if (max_visible <= TS_MAXN) {
        hipLaunchKernelGGL(topk_short_kernel, item_grid(1, num_rows), dim3(TS_THREADS), 0, stream, vis, scores, ld, k,
                           indices, (int)num_rows);
        return;
    }
    if (topk_chunked_path(num_rows, max_visible)) {
        hipLaunchKernelGGL(topk_sfilter_kernel, item_grid(tw.chunks, num_rows), dim3(TM_THREADS), 0, stream, vis,
                           scores, ld, k, tw.crec, tw.mcand, tw.chunks, (int)num_rows);
        hipLaunchKernelGGL(topk_sresolve_kernel, item_grid(1, num_rows), dim3(TM_RTHREADS), 0, stream, vis, scores, ld,
                           k, indices, tw.crec, tw.mcand, tw.chunks, (int)num_rows);
        return;
    }
    const bool has_long = max_visible > TR_ROW_PATH_MAXN;
    // Many rows: the rows of up to TQ_MAXN positions take four small
    // workgroups per CU (topk_stream_kernel); the one-workgroup kernel then
    // only samples the long rows.
    const bool streamed = num_rows >= TQ_MIN_ROWS;
    if (streamed)
        hipLaunchKernelGGL(topk_stream_kernel, item_grid(1, num_rows), dim3(TQ_THREADS), 0, stream, vis, scores, ld,
                           k, indices, (int)num_rows);
    if (!streamed || has_long)
        hipLaunchKernelGGL(topk_rows_kernel, item_grid(1, num_rows), dim3(TR_THREADS), 0, stream, vis, scores, ld,
                           k, indices, (int)TR_ROW_PATH_MAXN, has_long ? tw.rowst : nullptr, (int)num_rows,
                           streamed ? 1 : 0);
    if (!has_long) return;
    const int CH = tw.chunks;
    const int min_n = TR_ROW_PATH_MAXN;
    // Few rows: one workgroup row per query row (short rows exit at once).
    // Many rows: a list of the long ones and fixed grids that walk it.
    const bool listed = num_rows > TK_LIST_GRID;
    int32_t* lr = listed ? tw.longrows : nullptr;
    const int G = listed ? TK_LIST_GRID : num_rows;
    dim3 g2(CH, G);
    if (listed)
        hipLaunchKernelGGL(topk_prep_kernel, dim3(1), dim3(TP_THREADS), 0, stream, vis, num_rows, min_n, lr,
                           tw.nlong);
    hipLaunchKernelGGL(topk_filter_kernel, g2, dim3(TK_THREADS), 0, stream, vis, scores, ld, tw.rowst, tw.cand, lr,
                       tw.nlong, num_rows, min_n);
    hipLaunchKernelGGL(topk_resolve_kernel, dim3(listed ? 256 : num_rows), dim3(RS_THREADS), 0, stream, vis,
                       scores, ld, k, tw.rowst, tw.chunkst, CH, tw.cand, lr, tw.nlong, num_rows, min_n);
    hipLaunchKernelGGL(topk_write_kernel, g2, dim3(TK_THREADS), 0, stream, vis, scores, ld, k, tw.rowst,
                       tw.chunkst, CH, indices, lr, tw.nlong, num_rows, min_n);
}

}  // namespace dsa
