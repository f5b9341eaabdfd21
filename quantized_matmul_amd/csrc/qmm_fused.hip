// Producer-side steps that feed the activation quantizer, fused with it.
//
// [GEMM, "The GPU path", "Fused elementwise kernels"]: the int8 GEMMs read
// quantized activations, so each RMS norm and the FFN activation end in the
// quantizer.  Run as separate kernels, a layer writes the normalized rows (or the
// product silu(g) * u) to HBM and reads them back; the fused kernels quantize
// from registers instead:
//   rmsnorm_kernel<CH, true,  1>   residual add + RMS norm + quantize
//   rmsnorm_kernel<CH, false, 1>   RMS norm + quantize (first layer: no add)
//   silu_mul_kernel<1>             silu(g) * u + quantize
// and with 2 in place of 1 the same steps ending in the Q8_K quantizer ([GEMM,
// "Activations: int8 with a scale per 256"]; rows of whole 256-value blocks).
// The same templates with 0 (plus residual_add_kernel) are the unfused chain's
// steps: they store the f32 values, which the plain quantizer then reads.  Fused
// and unfused evaluate the same float expressions in the same order and quantize
// through the same quantize_lane4 / quantize_lane4_q8k, so they agree bit for bit.
//
// Arithmetic (the pages fix only the fused = unfused property):
// * RMS norm, f32: 256 lane partials; lane t accumulates fma(x_i, x_i, p_t) in
//   increasing i over the values i with (i / 4) mod 256 == t (its float4 groups
//   t, t + 256, ...); the partials are combined by halving, p_t += p_{t+s} for
//   s = 128, 64, ..., 1; r = 1 / sqrtf(ss / n + eps); y = (x * r) * w.  The order
//   is part of the operation: the last bit of y decides codes.
// * silu(g) * u in f64, (g / (1 + exp(-g))) * u, rounded once to f32.
//
// wave64 mapping.  RMS norm: one 256-lane workgroup per row; lane t holds the
// float4 groups t, t + 256, ... (a row of up to 16384 values stays in registers,
// longer rows are read twice, the second time from cache).  A wave's 64 lanes
// hold 256 consecutive values = eight quantization blocks at each step, so the
// quantizer's eight-lane groups line up with the blocks (for Q8_K the wave is one
// block: rows start on a 256-value boundary).  The cross-lane sum goes
// through LDS once (strides 128 and 64, every wave reading all 256 partials) and
// then a butterfly inside the wave, which leaves the same total in every lane.
// silu: one float4 per lane, the plain quantizer's layout.
#include "qmm_internal.h"

#pragma clang fp contract(off)

namespace qmm {
namespace {

__device__ __forceinline__ float4 f4_add(float4 a, float4 b)
{
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__device__ __forceinline__ float sum_squares4(float4 v, float p)
{
    p = fmaf(v.x, v.x, p);
    p = fmaf(v.y, v.y, p);
    p = fmaf(v.z, v.z, p);
    return fmaf(v.w, v.w, p);
}

// (x * r) * w per element.
__device__ __forceinline__ float4 scale4(float4 v, float r, float4 w)
{
    return make_float4((v.x * r) * w.x, (v.y * r) * w.y, (v.z * r) * w.z, (v.w * r) * w.w);
}

// Total of the 256 lane partials in the halving order; every lane gets it.
__device__ __forceinline__ float row_total(float p, float* red)
{
    const int t = threadIdx.x;
    red[t] = p;
    __syncthreads();
    const int l = t & 63;
    const float a = red[l] + red[l + 128];       // stride 128
    const float b = red[l + 64] + red[l + 192];  // stride 128
    float v = a + b;                             // stride 64
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)            // strides 32 .. 1
        v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ float rms_scale(float ss, int n, float eps)
{
    return 1.0f / sqrtf(ss / (float)n + eps);
}

// Store one lane's four normalized values (float4 group gi): QM = 1 quantized per
// 32 (codes + the block's d and s from the first lane of each eight), QM = 2 Q8_K
// (the wave's 64 lanes are one 256-value block: codes, d from lane 0 and each
// 16-value group's code sum into s from its quad's first lane), QM = 0 as f32.
template <int QM>
__device__ __forceinline__ void emit4(float4 yv, long gi, bool valid, uint32_t* __restrict__ q,
                                      float* __restrict__ d, float* __restrict__ s, float4* y)
{
    if constexpr (QM == 1) {
        float dk, sk;
        const uint32_t codes = quantize_lane4(yv, dk, sk);
        if (valid) {
            q[gi] = codes;
            if ((threadIdx.x & 7) == 0) {
                d[gi >> 3] = dk;
                s[gi >> 3] = sk;
            }
        }
    } else if constexpr (QM == 2) {
        float dk;
        int gsum;
        const uint32_t codes = quantize_lane4_q8k(yv, dk, gsum);
        if (valid) {
            q[gi] = codes;
            if ((threadIdx.x & 63) == 0)
                d[gi >> 6] = dk;
            if ((threadIdx.x & 3) == 0)
                s[gi >> 2] = (float)gsum;
        }
    } else {
        if (valid)
            y[gi] = yv;
    }
}

// xh: the row input (x, or the residual h when ADD, updated in place to h + o).
// y may equal x (each lane reads its values before it writes them).
// CH > 0: the row is held in registers, CH float4 per lane (id <= 1024 CH);
// CH == 0: any length, the row is read a second time for the output pass.
template <int CH, bool ADD, int QM>
__global__ __launch_bounds__(256) void rmsnorm_kernel(float4* xh, const float4* __restrict__ o,
                                                      const float4* __restrict__ w, float eps, int id,
                                                      uint32_t* __restrict__ q, float* __restrict__ d,
                                                      float* __restrict__ s, float4* y)
{
    __shared__ float red[256];
    const int t = threadIdx.x;
    const int n4 = id >> 2;
    const long rb = (long)blockIdx.x * n4;
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    float p = 0.0f;

    if constexpr (CH > 0) {
        float4 v[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int g = c * 256 + t;
            const long gc = rb + min(g, n4 - 1);  // in-row clamp: every load is in bounds
            float4 a = xh[gc];
            if constexpr (ADD)
                a = f4_add(a, o[gc]);
            v[c] = g < n4 ? a : zero;
        }
        if constexpr (ADD) {
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if (c * 256 + t < n4)
                    xh[rb + c * 256 + t] = v[c];
        }
#pragma unroll
        for (int c = 0; c < CH; ++c)
            p = sum_squares4(v[c], p);  // zeros past the row end leave p unchanged

        const float r = rms_scale(row_total(p, red), id, eps);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int g = c * 256 + t;
            const float4 wv = w[min(g, n4 - 1)];
            emit4<QM>(scale4(v[c], r, wv), rb + g, g < n4, q, d, s, y);
        }
    } else {
        const int nch = (n4 + 255) >> 8;
        for (int c = 0; c < nch; ++c) {
            const int g = c * 256 + t;
            if (g < n4) {
                float4 a = xh[rb + g];
                if constexpr (ADD) {
                    a = f4_add(a, o[rb + g]);
                    xh[rb + g] = a;
                }
                p = sum_squares4(a, p);
            }
        }
        // row_total's barrier also orders the stores above before the re-reads
        const float r = rms_scale(row_total(p, red), id, eps);
        for (int c = 0; c < nch; ++c) {
            const int g = c * 256 + t;
            const int gc = min(g, n4 - 1);
            const float4 a = xh[rb + gc];
            const float4 wv = w[gc];
            emit4<QM>(scale4(g < n4 ? a : zero, r, wv), rb + g, g < n4, q, d, s, y);
        }
    }
}

__global__ __launch_bounds__(256) void residual_add_kernel(float4* __restrict__ h, const float4* __restrict__ o,
                                                           long n4)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n4)
        h[i] = f4_add(h[i], o[i]);
}

__device__ __forceinline__ float silu_mul1(float g, float u)
{
    const double gd = (double)g;
    const double sg = gd / (1.0 + exp(-gd));
    return (float)(sg * (double)u);
}

// n4 = nt * id / 4 float4 groups; a multiple of eight (id % 32 == 0).
template <int QM>
__global__ __launch_bounds__(256) void silu_mul_kernel(const float4* __restrict__ g, const float4* __restrict__ u,
                                                       long n4, uint32_t* __restrict__ q, float* __restrict__ d,
                                                       float* __restrict__ s, float4* __restrict__ y)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    const bool valid = i < n4;
    const long ic = valid ? i : n4 - 1;
    const float4 a = g[ic];
    const float4 b = u[ic];
    const float4 v = make_float4(silu_mul1(a.x, b.x), silu_mul1(a.y, b.y), silu_mul1(a.z, b.z),
                                 silu_mul1(a.w, b.w));
    emit4<QM>(v, i, valid, q, d, s, y);
}

template <bool ADD, int QM>
hipError_t launch_rms(int ch, float* xh, const float* o, const float* w, float eps, int nt, int id, int8_t* q,
                      float* d, float* s, float* y, hipStream_t st)
{
    auto X = reinterpret_cast<float4*>(xh);
    auto O = reinterpret_cast<const float4*>(o);
    auto Wv = reinterpret_cast<const float4*>(w);
    auto Q = reinterpret_cast<uint32_t*>(q);
    auto Y = reinterpret_cast<float4*>(y);
    const dim3 grid(nt), block(256);
    switch (ch) {
    case 1: hipLaunchKernelGGL((rmsnorm_kernel<1, ADD, QM>), grid, block, 0, st, X, O, Wv, eps, id, Q, d, s, Y); break;
    case 2: hipLaunchKernelGGL((rmsnorm_kernel<2, ADD, QM>), grid, block, 0, st, X, O, Wv, eps, id, Q, d, s, Y); break;
    case 4: hipLaunchKernelGGL((rmsnorm_kernel<4, ADD, QM>), grid, block, 0, st, X, O, Wv, eps, id, Q, d, s, Y); break;
    case 8: hipLaunchKernelGGL((rmsnorm_kernel<8, ADD, QM>), grid, block, 0, st, X, O, Wv, eps, id, Q, d, s, Y); break;
    case 16: hipLaunchKernelGGL((rmsnorm_kernel<16, ADD, QM>), grid, block, 0, st, X, O, Wv, eps, id, Q, d, s, Y); break;
    default: hipLaunchKernelGGL((rmsnorm_kernel<0, ADD, QM>), grid, block, 0, st, X, O, Wv, eps, id, Q, d, s, Y); break;
    }
    return hipGetLastError();
}

}  // namespace

// o != null: residual add (h = x updated in place).  q != null: quantize, else
// store y.  The unfused chain never combines the add with an f32 output.
hipError_t launch_rmsnorm(const float* x, const float* o, float* h, const float* w, float eps, int nt, int id,
                          int8_t* q, float* d, float* s, float* y, hipStream_t st, bool q8k)
{
    if (nt == 0)
        return hipSuccess;
    const int nch = (id / 4 + 255) / 256;
    const int ch = nch <= 1 ? 1 : nch <= 2 ? 2 : nch <= 4 ? 4 : nch <= 8 ? 8 : nch <= 16 ? 16 : 0;
    if (o)
        return q8k ? launch_rms<true, 2>(ch, h, o, w, eps, nt, id, q, d, s, nullptr, st)
                   : launch_rms<true, 1>(ch, h, o, w, eps, nt, id, q, d, s, nullptr, st);
    float* xh = const_cast<float*>(x);  // read only when there is no add
    if (q)
        return q8k ? launch_rms<false, 2>(ch, xh, nullptr, w, eps, nt, id, q, d, s, nullptr, st)
                   : launch_rms<false, 1>(ch, xh, nullptr, w, eps, nt, id, q, d, s, nullptr, st);
    return launch_rms<false, 0>(ch, xh, nullptr, w, eps, nt, id, nullptr, nullptr, nullptr, y, st);
}

hipError_t launch_residual_add(float* h, const float* o, long n, hipStream_t st)
{
    const long n4 = n / 4;
    const long grid = (n4 + 255) / 256;
    if (grid == 0)
        return hipSuccess;
    hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned)grid), dim3(256), 0, st, reinterpret_cast<float4*>(h),
                       reinterpret_cast<const float4*>(o), n4);
    return hipGetLastError();
}

hipError_t launch_silu_mul(const float* g, const float* u, int nt, int id, int8_t* q, float* d, float* s, float* y,
                           hipStream_t st, bool q8k)
{
    const long n4 = (long)nt * id / 4;
    const long grid = (n4 + 255) / 256;
    if (grid == 0)
        return hipSuccess;
    auto G = reinterpret_cast<const float4*>(g);
    auto U = reinterpret_cast<const float4*>(u);
    if (q && q8k)
        hipLaunchKernelGGL(silu_mul_kernel<2>, dim3((unsigned)grid), dim3(256), 0, st, G, U, n4,
                           reinterpret_cast<uint32_t*>(q), d, s, nullptr);
    else if (q)
        hipLaunchKernelGGL(silu_mul_kernel<1>, dim3((unsigned)grid), dim3(256), 0, st, G, U, n4,
                           reinterpret_cast<uint32_t*>(q), d, s, nullptr);
    else
        hipLaunchKernelGGL(silu_mul_kernel<0>, dim3((unsigned)grid), dim3(256), 0, st, G, U, n4, nullptr,
                           nullptr, nullptr, reinterpret_cast<float4*>(y));
    return hipGetLastError();
}

}  // namespace qmm
