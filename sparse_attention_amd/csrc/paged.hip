// paged.hip -- selected positions of a paged latent cache turned into pool
// rows, so that the attention gathers from the pool exactly as it gathers from
// a packed cache (a row base of 0 plus a physical row index).
//
// A paged cache keeps each sequence's positions in fixed-size blocks of a
// shared pool; a per-sequence block table names the pool block of every
// logical block (the vLLM PagedAttention layout).  Only the addressing
// differs from a packed cache: position p of the sequence with block-table
// row s is pool row  bt[s][p / B] * B + p % B,  B a power of two.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

// One thread per (row, selected slot), grid-strided past PI_MAX_GRID
// workgroups; the row's block-table row is read through the cache (a
// 2048-entry selection touches at most 2048 entries).
constexpr int64_t PI_MAX_GRID = 1 << 16;

__global__ __launch_bounds__(256) void page_indices_kernel(int64_t total, int k, const int64_t* __restrict__ seq,
                                                           const int32_t* __restrict__ idx, PagedCache pm,
                                                           int32_t* __restrict__ phys, int64_t* __restrict__ zero_base)
{
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
        const int64_t r = o / k;
        if (o - r * k == 0) zero_base[r] = 0;
        const int32_t p = idx[o];
        const int32_t* btr = pm.block_table + seq[r] * pm.max_blocks;
        // Padding: -1 - (row of position 0), a row every sequence has, for
        // the attention's masked gathers to read.
        phys[o] = p >= 0 ? (btr[p >> pm.log2_block] << pm.log2_block) | (p & ((1 << pm.log2_block) - 1))
                         : -1 - (btr[0] << pm.log2_block);
    }
}

}  // namespace

void launch_page_indices(int32_t num_rows, int32_t k, const int64_t* seq, const int32_t* idx,
                         const PagedCache& paged, int32_t* phys, int64_t* zero_base, hipStream_t stream)
{
    const int64_t total = (int64_t)num_rows * k;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(page_indices_kernel, dim3((unsigned)(blocks < PI_MAX_GRID ? blocks : PI_MAX_GRID)), dim3(256),
                       0, stream, total, (int)k, seq, idx, paged, phys, zero_base);
}

}  // namespace dsa
