// dsa_device.h -- device-side helpers shared by the libdsa kernels (gfx950).
//
// MFMA lane layouts used throughout (wave64, checked on gfx950):
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l supplies row (l & 15) and 8 consecutive k values of k-group (l >> 4)
//     B: lane l supplies column (l & 15) and the same 8 k values of k-group (l >> 4)
//     D: lane l, element v holds D[4 * (l >> 4) + v][l & 15]
//   Which k an (A, B) slot pair stands for is free as long as A and B agree,
//   so callers pick k orders that make their loads contiguous.
//
//   ds_read_tr16_b64 (per 16-lane group): source lane s = c + 4 * k (c, k in
//   0..3) names an 8-byte chunk; result lane 4 * c + e receives element e of
//   the chunks named by lanes c, c + 4, c + 8, c + 12, in that order.  With
//   source lane (c, k) pointing at row k, columns 4c..4c+3 of a row-major
//   16-bit matrix, result lane j gets column j of rows 0..3: a 4x16 -> 16x4
//   transpose, which turns row-major LDS tiles into MFMA operands whose k
//   runs over rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// Grids with one row of workgroups per item (a query row, a block of rows):
// items past what grid y takes spill into z, so that y stays within its
// launch limit and each dimension within 2^32 work-items at any item count.
// Dispatch order is unchanged: x fastest, then the items in order.
constexpr unsigned GRID_Y_MAX = 65535;

inline dim3 item_grid(unsigned x, int64_t items)
{
    const unsigned y = items < (int64_t)GRID_Y_MAX ? (unsigned)items : GRID_Y_MAX;
    return dim3(x, y, (unsigned)((items + y - 1) / y));
}

// This workgroup's item; the last z slice may run past the item count.
__device__ __forceinline__ int grid_item() { return (int)(blockIdx.z * gridDim.y + blockIdx.y); }

__device__ __forceinline__ floatx4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const floatx4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte global load of 8 bf16 values.
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 load_u32x4(const void* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}

// Two transposing LDS reads glued into one 8-element MFMA operand.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const uint16_t* lo, const uint16_t* hi)
{
    shortx4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(lo));
    shortx4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(hi));
    typedef short shortx8 __attribute__((ext_vector_type(8)));
    shortx8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// fp32 -> bf16 with round-to-nearest-even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Order-preserving 32-bit key of an fp32 score: a larger key means a larger
// score; -0.0 and +0.0 share a key; every NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Cross-lane steps on the VALU (DPP), all inside a 16-lane row: swap
// neighbours, swap pairs, mirror each half-row, mirror the row.  After the
// four steps every lane of the row holds the reduction of all 16 lanes, and
// both partners of every step combine the same two values, so all 16 lanes
// end bitwise equal.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_1032 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// Maximum / sum over the four lanes j, j+16, j+32, j+48 of a wave (gfx950
// VALU lane swaps: lanes l and l ^ 32, then l and l ^ 16; every lane ends
// with the same value).
__device__ __forceinline__ float xrow_max(float v)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xrow_sum(float v)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Reduce-scatter over the four 16-lane groups of a wave: lane group g
// returns x[g] summed over the four lanes j, j+16, j+32, j+48 (its own and
// the three other groups' values of entry g).  Three lane swaps: entries
// {0,1} / {2,3} meet across the wave halves, then across the rows.
__device__ __forceinline__ float xrow_reduce_scatter4(const float (&x)[4])
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[0]), __float_as_uint(x[2]), false, false);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[1]), __float_as_uint(x[3]), false, false);
    const float r02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // groups 0,1: entry 0; 2,3: entry 2
    const float r13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // groups 0,1: entry 1; 2,3: entry 3
    auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(r02), __float_as_uint(r13), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// max(x, 0) on the bit pattern: one integer op, and no NaN quieting of the
// input is needed (a negative float is a negative integer).
__device__ __forceinline__ float relu_bits(float x)
{
    return __int_as_float(max(__float_as_int(x), 0));
}

// Inclusive prefix sum over the 64 lanes of a wave on the VALU (DPP): a
// Hillis-Steele scan inside each 16-lane row (shifts 1, 2, 4, 8; lanes
// without a source add 0), then each row adds the totals of the rows before
// it (broadcast of lane 15 into rows 1 and 3, of lane 31 into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

__device__ __forceinline__ float wave_max_16(float v)
{
    v = fmaxf(v, dpp_f32<DPP_QUAD_1032>(v));
    v = fmaxf(v, dpp_f32<DPP_QUAD_2301>(v));
    v = fmaxf(v, dpp_f32<DPP_ROW_HALF_MIRROR>(v));
    v = fmaxf(v, dpp_f32<DPP_ROW_MIRROR>(v));
    return v;
}

__device__ __forceinline__ float wave_sum_16(float v)
{
    v += dpp_f32<DPP_QUAD_1032>(v);
    v += dpp_f32<DPP_QUAD_2301>(v);
    v += dpp_f32<DPP_ROW_HALF_MIRROR>(v);
    v += dpp_f32<DPP_ROW_MIRROR>(v);
    return v;
}

}  // namespace dsa
