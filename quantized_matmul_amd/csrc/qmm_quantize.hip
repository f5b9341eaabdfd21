// Activation quantizer: f32 [nt][id] -> int8 codes, f32 scale d and f32 d*sum(q)
// per block of 32 values.
//
// [GEMM, "The GPU path", "Activations get one scale per 32"]: int8 codes with one
// f32 scale per 32 values and the scale times the code sum stored beside it; a
// 32-value block is handled by one group of lanes with cross-lane max and sum
// reductions so loads and stores stay coalesced.  [CH04, section 2.1]: largest
// magnitude, scale, round.  Readings (the pages leave them open): d = amax / 127
// by IEEE division, q = round(x / d) half away from zero by IEEE division, a zero
// block gives d = q = s = 0, s = d * (float)sum(q) with one rounding.
//
// wave64 mapping: each lane loads 16 bytes (four values), eight lanes hold one
// block, a wave covers eight blocks = 1 KiB of input.  The eight-lane max and sum
// (quantize_lane4) use DPP (two quad permutes and a half-row mirror) -- no LDS.
// Each lane stores its four codes as one dword; the first lane of each block
// stores d and s.
#include "qmm_internal.h"

namespace qmm {

__global__ __launch_bounds__(256) void quantize_q8_kernel(const float4* __restrict__ x, int nblk,
                                                          uint32_t* __restrict__ q,
                                                          float* __restrict__ d,
                                                          float* __restrict__ s)
{
    const int g = blockIdx.x * 256 + threadIdx.x;  // index of this lane's four values
    const int blk = g >> 3;
    const bool valid = blk < nblk;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid)
        v = x[g];

    float dk, sk;
    const uint32_t codes = quantize_lane4(v, dk, sk);
    if (valid) {
        q[g] = codes;
        if ((threadIdx.x & 7) == 0) {
            d[blk] = dk;
            s[blk] = sk;
        }
    }
}

// Q8_K activations ([GEMM, "Activations: int8 with a scale per 256"]): one f32
// scale per 256 values and the sum of each 16-value group of codes, stored as
// f32.  Same rules as above over 256 values.  One wave per 256-value block: lane l
// holds values 4l .. 4l+3, the max runs over the whole wave (DPP inside rows of 16,
// then two cross-row swaps), a 16-value group is one quad of lanes.
__global__ __launch_bounds__(256) void quantize_q8k_kernel(const float4* __restrict__ x, int nblk,
                                                           uint32_t* __restrict__ q, float* __restrict__ d,
                                                           float* __restrict__ bsum)
{
    const int blk = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const bool valid = blk < nblk;
    const long g = (long)min(blk, nblk - 1) * 64 + lane;  // in bounds for every lane
    float4 v = x[g];
    if (!valid)
        v = make_float4(0.f, 0.f, 0.f, 0.f);

    float dk;
    int sum;
    const uint32_t codes = quantize_lane4_q8k(v, dk, sum);
    if (valid) {
        q[g] = codes;
        if (lane == 0)
            d[blk] = dk;
        if ((lane & 3) == 0)
            bsum[(long)blk * 16 + (lane >> 2)] = (float)sum;
    }
}

hipError_t launch_quantize_q8k(const float* x, int nt, int id, int8_t* q, float* d, float* bsum, hipStream_t st)
{
    const long nblk = (long)nt * id / kQK;
    const int grid = (int)((nblk + 3) / 4);
    if (grid == 0)
        return hipSuccess;
    hipLaunchKernelGGL(quantize_q8k_kernel, dim3(grid), dim3(256), 0, st, reinterpret_cast<const float4*>(x),
                       (int)nblk, reinterpret_cast<uint32_t*>(q), d, bsum);
    return hipGetLastError();
}

hipError_t launch_quantize(const float* x, int nt, int id, int8_t* q, float* d, float* s,
                           hipStream_t st)
{
    const long nvals = (long)nt * id;
    const int nblk = (int)(nvals / kActBlock);
    const long lanes = nvals / 4;
    const int grid = (int)((lanes + 255) / 256);
    if (grid == 0)
        return hipSuccess;
    hipLaunchKernelGGL(quantize_q8_kernel, dim3(grid), dim3(256), 0, st,
                       reinterpret_cast<const float4*>(x), nblk, reinterpret_cast<uint32_t*>(q), d, s);
    return hipGetLastError();
}

}  // namespace qmm
