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

// Split over K: groups 1 .. KS-1 write their partial 32 x 32 tile (v, the
// lane's 16 values) to LDS; group 0 adds them in group order.  Returns false for
// the waves that are done (groups past 0).  Called by every wave after the last
// barrier of the K loop; red is the workgroup's tile memory, free by then.
template <int NW, int KS>
__device__ __forceinline__ bool combine_k_groups(v16f& v, float* red, int kg, int gw, int lane)
{
    if constexpr (KS == 1) {
        return true;
    } else {
        if (kg > 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                red[((kg - 1) * NW + gw) * 1024 + i * 64 + lane] = v[i];
        }
        __syncthreads();
        if (kg > 0)
            return false;
#pragma unroll
        for (int g = 1; g < KS; ++g)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] += red[((g - 1) * NW + gw) * 1024 + i * 64 + lane];
        return true;
    }
}

// Q6_K staging task e = (row r = e / 8, piece c = e % 8) of super-block sb: the
// 16-byte chunks of low fields and high 2-bit fields piece c covers (h = c / 4,
// jq = c / 2 % 2, half = c % 2: low bytes 64h + 32jq + 16half, high bytes
// 128 + 32h + 16half of the block), its two group scales 2c, 2c+1 and d.  The
// unpadded 210-byte block is only 2-byte aligned: each chunk is read as the five
// dwords around it plus a byte shift; the padded 224-byte block (PAD) has both
// chunks 16-byte aligned.  psd: low half the two int8 scales, high half the f16 d.
template <bool PAD>
__device__ __forceinline__ void q6_prefetch_task(uint32_t (&pl)[5], uint32_t (&phh)[5], uint32_t& pshift,
                                                 uint32_t& psd, const uint8_t* __restrict__ W, int e, int sb,
                                                 int row0, int od, size_t row_bytes)
{
    const int r = e >> 3, c = e & 7;
    const int h = c >> 2, jq = (c >> 1) & 1, half = c & 1;
    const uint8_t* blk = W + (size_t)min(row0 + r, od - 1) * row_bytes + (size_t)sb * (PAD ? kQ6KP224Bytes : kQ6KBytes);
    const uintptr_t al = reinterpret_cast<uintptr_t>(blk + 64 * h + 32 * jq + 16 * half);
    const uintptr_t ah = reinterpret_cast<uintptr_t>(blk + 128 + 32 * h + 16 * half);
    if constexpr (PAD) {
        const uint4 l4 = *reinterpret_cast<const uint4*>(al), h4 = *reinterpret_cast<const uint4*>(ah);
        pl[0] = l4.x, pl[1] = l4.y, pl[2] = l4.z, pl[3] = l4.w, pl[4] = 0;
        phh[0] = h4.x, phh[1] = h4.y, phh[2] = h4.z, phh[3] = h4.w, phh[4] = 0;
        pshift = 0;
    } else {
        const uint32_t* wl = reinterpret_cast<const uint32_t*>(al & ~(uintptr_t)3);
        const uint32_t* wh = reinterpret_cast<const uint32_t*>(ah & ~(uintptr_t)3);
        pshift = (uint32_t)(al & 3);  // same for both chunks
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            pl[i] = wl[i];
            phh[i] = wh[i];
        }
    }
    const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(blk + 192 + 2 * c);
    const uint32_t d16 = *reinterpret_cast<const uint16_t*>(blk + 208);
    psd = sc2 | (d16 << 16);
}

// The 32 centred codes (q6 - 32, int8) of piece c, from its prefetched chunks, into
// the staged row wrow: elements 128h + 32jq + 16half .. + 15 (low nibbles with high
// bits 2jq) and the same + 64 (high nibbles with high bits 2jq + 4).
__device__ __forceinline__ void q6_stage_codes(int8_t* wrow, const uint32_t (&pl)[5], const uint32_t (&phh)[5],
                                               uint32_t sh, int c)
{
    const int h = c >> 2, jq = (c >> 1) & 1, half = c & 1;
    uint32_t L[4], H[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        L[i] = __builtin_amdgcn_alignbyte(pl[i + 1], pl[i], sh);
        H[i] = __builtin_amdgcn_alignbyte(phh[i + 1], phh[i], sh);
    }
    const int hs1 = 2 * jq, hs2 = 2 * jq + 4;
    int4 ca, cb;
    ca.x = q6_center4(L[0] & 0x0F0F0F0Fu, (H[0] >> hs1) & 0x03030303u);
    ca.y = q6_center4(L[1] & 0x0F0F0F0Fu, (H[1] >> hs1) & 0x03030303u);
    ca.z = q6_center4(L[2] & 0x0F0F0F0Fu, (H[2] >> hs1) & 0x03030303u);
    ca.w = q6_center4(L[3] & 0x0F0F0F0Fu, (H[3] >> hs1) & 0x03030303u);
    cb.x = q6_center4((L[0] >> 4) & 0x0F0F0F0Fu, (H[0] >> hs2) & 0x03030303u);
    cb.y = q6_center4((L[1] >> 4) & 0x0F0F0F0Fu, (H[1] >> hs2) & 0x03030303u);
    cb.z = q6_center4((L[2] >> 4) & 0x0F0F0F0Fu, (H[2] >> hs2) & 0x03030303u);
    cb.w = q6_center4((L[3] >> 4) & 0x0F0F0F0Fu, (H[3] >> hs2) & 0x03030303u);
    const int e1 = 128 * h + 32 * jq + 16 * half;
    *reinterpret_cast<int4*>(wrow + e1) = ca;
    *reinterpret_cast<int4*>(wrow + e1 + 64) = cb;
}

// Store one wave's 32 x 32 result tile (lane: token tg, rows r0 + 8k + 4 lh + 0..3
// from v[4k .. 4k+3]) into out [nt][od], masked at the edges.
__device__ __forceinline__ void store_tile(const v16f& v, float* __restrict__ out, int nt, int od, int tg, int r0,
                                           int lh)
{
    if (tg >= nt)
        return;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int rg = r0 + 8 * k + 4 * lh;
        float* o = out + (size_t)tg * od + rg;
        if (rg + 3 < od && (od & 3) == 0) {
            *reinterpret_cast<float4*>(o) = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
        } else {
            if (rg < od) o[0] = v[4 * k];
            if (rg + 1 < od) o[1] = v[4 * k + 1];
            if (rg + 2 < od) o[2] = v[4 * k + 2];
            if (rg + 3 < od) o[3] = v[4 * k + 3];
        }
    }
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
