// Device helpers shared by the MMQ kernels (int8 / f16 / f32 MFMA wrappers,
// workgroup-to-tile order, branch-free task indices, buffer loads).  gfx950 only.
#pragma once

#include "qmm_internal.h"

namespace qmm {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

__device__ __forceinline__ v16i mfma_i8_k32(v4i a, v4i b)
{
    const v16i z = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
}

__device__ __forceinline__ v16i mfma_i8_k16(long a, long b)
{
    const v16i z = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_i32_32x32x16_i8(a, b, z, 0, 0, 0);
}

// Two 32 x 32 outer products: lane l gives a[row l%32] and b[col l%32] of block
// l/32; result registers 16*k .. 16*k+15 hold block k in the 32 x 32 layout.
__device__ __forceinline__ v32f mfma_outer2(float a, float b)
{
    const v32f z = {};
    return __builtin_amdgcn_mfma_f32_32x32x1f32(a, b, z, 0, 0, 0);
}

// acc += A (32 x 16) . B (16 x 32) in bf16: lane l gives A[row l%32][k = 8 (l/32) ..
// + 7] and B[k = 8 (l/32) .. + 7][col l%32].
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v16f mfma_bf16_k16(v8bf a, v8bf b, v16f acc)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// acc += A (32 x 2) . B (2 x 32): lane l gives A[row l%32][k = l/32] and
// B[k = l/32][col l%32].
__device__ __forceinline__ v16f mfma_k2(float a, float b, v16f acc)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
}

// Tile index of this workgroup: consecutive tiles (same row block, successive
// token blocks) go to the same XCD.  Returns -1 for a padding workgroup.
__device__ __forceinline__ int xcd_tile(int ntiles)
{
    const int per = (ntiles + 7) >> 3;
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    return t < ntiles ? t : -1;
}

// Task index e of a thread clamped into [0, n): threads past the end repeat the
// last task -- the same loads and the same LDS stores of the same values -- so
// the prefetch and staging code has no branches (a load under a branch makes the
// compiler wait for it at once; a branch in the loop body lets it move compute
// work past the staging and keep every MFMA result live).
template <int N, int NTH, int CNT>
__device__ __forceinline__ int task(int e)
{
    if constexpr (N % NTH == 0 && CNT * NTH == N)
        return e;
    else
        return min(e, N - 1);
}

// Prefetch loads are buffer loads: a wave-uniform resource (base address in
// scalar registers) per operand, a per-thread byte offset fixed for the whole
// kernel, and the super-block step as the scalar offset -- so the loop spends no
// vector instructions on addresses.  The resource's range is the rest of the
// operand from the tile's first row / token; rows past od and tokens past nt read
// the last valid row / token (their results are never stored).
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, size_t bytes)
{
    // third descriptor word 0x00020000: raw 32-bit data, the gfx9-family setting
    const int n = (int)(bytes < 0xFFFFFFF0u ? bytes : 0xFFFFFFF0u);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ v4i bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

}  // namespace qmm
