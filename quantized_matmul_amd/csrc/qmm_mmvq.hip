// MMVQ: the decode-side quantized matmul for nt <= 8 tokens.
//
// [MMQ, section 12.2]: the token count lives in registers, not in the grid: each
// weight block is streamed once and dotted with every token, so weight traffic is
// that of nt = 1 [MMQ, section 12.4].  [CH04, section 3.4]: integer 4-way dots
// over packed 4-bit codes with the scales applied once per block in f32, min term
// folded through the activation sum.  [GEMM, "The GPU path"]: the Q4_K min and
// the Q6_K offset stay out of the integer loop.
//
// MI355X mapping (wave64):
//  * A wave owns R output rows (a row group) and all of K.  Its 64 lanes split a
//    K window of eight super-blocks: lane L takes super-block slot g = L/8 and
//    16-byte code chunk c = L%8, i.e. 32 weights.  One window load instruction
//    touches 8 consecutive super-blocks of a row (1152 contiguous bytes).
//  * Weights are read once with 16-byte loads; the lane's activation codes (two
//    16-byte pieces per token) and scales are loaded once per window and reused
//    for all R rows (tokens x rows accumulators in registers).
//  * Integer dots use v_dot4_i32_i8 (codes 0..15 are valid int8; Q6_K codes are
//    centred to -32..31 in registers), scales fold once per group in f32.
//  * At the end the R*NT partial sums are reduced across the 64 lanes with a
//    halving exchange (each step halves the values per lane), so lane l ends with
//    output number l.
#include "qmm_internal.h"

namespace qmm {

template <int N>
struct pow2_ceil {
    static constexpr int value = N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : N <= 16 ? 16 : N <= 32 ? 32 : 64;
};

// Reduce V values per lane across the wave.  After the call lane l (l < V) holds in
// a[0] the wave total of value index l.  V must be a power of two <= 64.
template <int V>
__device__ __forceinline__ float wave_reduce_spread(float (&a)[V], int lane)
{
    int cnt = V;
#pragma unroll
    for (int m = 1; m < V; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < cnt / 2; ++i) {
            const float keep = upper ? a[2 * i + 1] : a[2 * i];
            const float send = upper ? a[2 * i] : a[2 * i + 1];
            a[i] = keep + __shfl_xor(send, m, 64);
        }
        cnt >>= 1;
    }
#pragma unroll
    for (int m = V; m < 64; m <<= 1)
        a[0] += __shfl_xor(a[0], m, 64);
    return a[0];
}

// Four dwords starting at byte address p, which is 2-byte aligned: read five
// aligned dwords (all inside the same 210-byte block) and funnel-shift.
__device__ __forceinline__ uint4 load16_a2(const uint8_t* p)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(a & ~(uintptr_t)3);
    const uint32_t sh = (uint32_t)(a & 3);
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3], w4 = w[4];
    uint4 r;
    r.x = __builtin_amdgcn_alignbyte(w1, w0, sh);
    r.y = __builtin_amdgcn_alignbyte(w2, w1, sh);
    r.z = __builtin_amdgcn_alignbyte(w3, w2, sh);
    r.w = __builtin_amdgcn_alignbyte(w4, w3, sh);
    return r;
}

// ------------------------------------------------------------------ Q4_K
// Lane chunk c: code chunk p = c/2 (32 bytes: sub-block 2p in low nibbles, 2p+1
// in high nibbles, same positions), half = c%2 -> positions 16*half .. +15.
template <int NT, int R, bool DUMP>
__global__ __launch_bounds__(256) void mmvq_q4k_kernel(const uint8_t* __restrict__ W,
                                                       const int8_t* __restrict__ q,
                                                       const float* __restrict__ dx,
                                                       const float* __restrict__ sx,
                                                       float* __restrict__ out, int od, int id,
                                                       int32_t* __restrict__ S)
{
    constexpr int NTP = pow2_ceil<NT>::value;
    constexpr int V = R * NTP;
    const int lane = threadIdx.x & 63;
    const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (row0 >= od)
        return;  // whole wave leaves together
    const int g = lane >> 3, c = lane & 7;
    const int p = c >> 1, half = c & 1;
    const int nsb = id >> 8;
    const int nblk = id >> 5;
    const int nwin = (nsb + 7) >> 3;

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc[i] = 0.f;

    for (int w = 0; w < nwin; ++w) {
        const int b = 8 * w + g;
        const bool bv = b < nsb;
        // activations of this lane for every token
        int4 xa[NT], xb[NT];
        float da[NT], db[NT], sa[NT], sb[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (bv) {
                const int8_t* qt = q + (size_t)t * id + 256 * b + 64 * p + 16 * half;
                xa[t] = *reinterpret_cast<const int4*>(qt);
                xb[t] = *reinterpret_cast<const int4*>(qt + 32);
                const int ai = t * nblk + 8 * b + 2 * p;
                da[t] = dx[ai];
                db[t] = dx[ai + 1];
                // the min term of a sub-block is added once: by the half-0 lane
                sa[t] = half ? 0.f : sx[ai];
                sb[t] = half ? 0.f : sx[ai + 1];
            } else {
                xa[t] = make_int4(0, 0, 0, 0);
                xb[t] = make_int4(0, 0, 0, 0);
                da[t] = db[t] = sa[t] = sb[t] = 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r;
            uint4 hdr = make_uint4(0, 0, 0, 0), qs = make_uint4(0, 0, 0, 0);
            if (bv && row < od) {
                const uint8_t* blk = W + ((size_t)row * nsb + b) * kQ4KBytes;
                hdr = *reinterpret_cast<const uint4*>(blk);
                qs = *reinterpret_cast<const uint4*>(blk + 16 + 16 * c);
            }
            const int lo0 = (int)(qs.x & 0x0F0F0F0Fu), lo1 = (int)(qs.y & 0x0F0F0F0Fu);
            const int lo2 = (int)(qs.z & 0x0F0F0F0Fu), lo3 = (int)(qs.w & 0x0F0F0F0Fu);
            const int hi0 = (int)((qs.x >> 4) & 0x0F0F0F0Fu), hi1 = (int)((qs.y >> 4) & 0x0F0F0F0Fu);
            const int hi2 = (int)((qs.z >> 4) & 0x0F0F0F0Fu), hi3 = (int)((qs.w >> 4) & 0x0F0F0F0Fu);
            int sc0, m0, sc1, m1;
            q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * p, sc0, m0);
            q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * p + 1, sc1, m1);
            const float dw = f16_bits_to_f32(hdr.x & 0xFFFF);
            const float dm = f16_bits_to_f32(hdr.x >> 16);
            const float W0 = dw * (float)sc0, W1 = dw * (float)sc1;
            const float M0 = dm * (float)m0, M1 = dm * (float)m1;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                int s0 = sdot4(lo0, xa[t].x, 0);
                s0 = sdot4(lo1, xa[t].y, s0);
                s0 = sdot4(lo2, xa[t].z, s0);
                s0 = sdot4(lo3, xa[t].w, s0);
                int s1 = sdot4(hi0, xb[t].x, 0);
                s1 = sdot4(hi1, xb[t].y, s1);
                s1 = sdot4(hi2, xb[t].z, s1);
                s1 = sdot4(hi3, xb[t].w, s1);
                if constexpr (DUMP) {
                    const int f0 = s0 + __shfl_xor(s0, 1, 64);
                    const int f1 = s1 + __shfl_xor(s1, 1, 64);
                    if (bv && row < od && half == 0) {
                        int32_t* dst = S + (((size_t)t * od + row) * nsb + b) * 8 + 2 * p;
                        dst[0] = f0;
                        dst[1] = f1;
                    }
                } else {
                    acc[r * NTP + t] += W0 * (da[t] * (float)s0) + W1 * (db[t] * (float)s1) -
                                        (M0 * sa[t] + M1 * sb[t]);
                }
            }
        }
    }
    if constexpr (!DUMP) {
        const float v = wave_reduce_spread<V>(acc, lane);
        if (lane < V) {
            const int r = lane / NTP, t = lane % NTP;
            if (t < NT && row0 + r < od)
                out[(size_t)t * od + row0 + r] = v;
        }
    }
}

// ------------------------------------------------------------------ Q6_K
// Reading of the element map (the pages leave it open; public GGUF arrangement):
// half h of 128 elements uses low bytes 64h.., high bytes 32h..; quarter k of the
// half takes low nibbles (k < 2) or high nibbles (k >= 2) of low bytes 64h+32(k%2)+l
// and bits 2k..2k+1 of high byte 32h+l.  Lane chunk c: h = c/4, jq = (c/2)%2,
// half = c%2 -> 16 positions of quarter jq (low nibbles) and of quarter jq+2 (high
// nibbles) read from one 16-byte low chunk and one 16-byte high chunk.
template <int NT, int R, bool DUMP>
__global__ __launch_bounds__(256) void mmvq_q6k_kernel(const uint8_t* __restrict__ W,
                                                       const int8_t* __restrict__ q,
                                                       const float* __restrict__ dx,
                                                       float* __restrict__ out, int od, int id,
                                                       int32_t* __restrict__ S)
{
    constexpr int NTP = pow2_ceil<NT>::value;
    constexpr int V = R * NTP;
    const int lane = threadIdx.x & 63;
    const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (row0 >= od)
        return;
    const int g = lane >> 3, c = lane & 7;
    const int h = c >> 2, jq = (c >> 1) & 1, half = c & 1;
    const int g1 = 8 * h + 2 * jq + half;  // scale group of the low-nibble quarter
    const int g2 = g1 + 4;                 // scale group of the high-nibble quarter
    const int nsb = id >> 8;
    const int nblk = id >> 5;
    const int nwin = (nsb + 7) >> 3;

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc[i] = 0.f;

    for (int w = 0; w < nwin; ++w) {
        const int b = 8 * w + g;
        const bool bv = b < nsb;
        int4 xa[NT], xb[NT];
        float da[NT], db[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (bv) {
                const int8_t* qt = q + (size_t)t * id + 256 * b + 128 * h + 32 * jq + 16 * half;
                xa[t] = *reinterpret_cast<const int4*>(qt);
                xb[t] = *reinterpret_cast<const int4*>(qt + 64);
                const int ai = t * nblk + 8 * b + 4 * h + jq;
                da[t] = dx[ai];
                db[t] = dx[ai + 2];
            } else {
                xa[t] = make_int4(0, 0, 0, 0);
                xb[t] = make_int4(0, 0, 0, 0);
                da[t] = db[t] = 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r;
            uint4 ql = make_uint4(0, 0, 0, 0), qh = make_uint4(0, 0, 0, 0);
            int scl1 = 0, scl2 = 0;
            uint32_t dbits = 0;
            if (bv && row < od) {
                const uint8_t* blk = W + ((size_t)row * nsb + b) * kQ6KBytes;
                ql = load16_a2(blk + 64 * h + 32 * jq + 16 * half);
                qh = load16_a2(blk + 128 + 32 * h + 16 * half);
                scl1 = (int)reinterpret_cast<const int8_t*>(blk)[192 + g1];
                scl2 = (int)reinterpret_cast<const int8_t*>(blk)[192 + g2];
                dbits = *reinterpret_cast<const uint16_t*>(blk + 208);
            }
            const int hs1 = 2 * jq, hs2 = 2 * jq + 4;
            const int a0 = q6_center4(ql.x & 0x0F0F0F0Fu, (qh.x >> hs1) & 0x03030303u);
            const int a1 = q6_center4(ql.y & 0x0F0F0F0Fu, (qh.y >> hs1) & 0x03030303u);
            const int a2 = q6_center4(ql.z & 0x0F0F0F0Fu, (qh.z >> hs1) & 0x03030303u);
            const int a3 = q6_center4(ql.w & 0x0F0F0F0Fu, (qh.w >> hs1) & 0x03030303u);
            const int b0 = q6_center4((ql.x >> 4) & 0x0F0F0F0Fu, (qh.x >> hs2) & 0x03030303u);
            const int b1 = q6_center4((ql.y >> 4) & 0x0F0F0F0Fu, (qh.y >> hs2) & 0x03030303u);
            const int b2 = q6_center4((ql.z >> 4) & 0x0F0F0F0Fu, (qh.z >> hs2) & 0x03030303u);
            const int b3 = q6_center4((ql.w >> 4) & 0x0F0F0F0Fu, (qh.w >> hs2) & 0x03030303u);
            const float dw = f16_bits_to_f32(dbits);
            const float W1 = dw * (float)scl1, W2 = dw * (float)scl2;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                int s1 = sdot4(a0, xa[t].x, 0);
                s1 = sdot4(a1, xa[t].y, s1);
                s1 = sdot4(a2, xa[t].z, s1);
                s1 = sdot4(a3, xa[t].w, s1);
                int s2 = sdot4(b0, xb[t].x, 0);
                s2 = sdot4(b1, xb[t].y, s2);
                s2 = sdot4(b2, xb[t].z, s2);
                s2 = sdot4(b3, xb[t].w, s2);
                if constexpr (DUMP) {
                    if (bv && row < od) {
                        int32_t* dst = S + (((size_t)t * od + row) * nsb + b) * 16;
                        dst[g1] = s1;
                        dst[g2] = s2;
                    }
                } else {
                    acc[r * NTP + t] += W1 * (da[t] * (float)s1) + W2 * (db[t] * (float)s2);
                }
            }
        }
    }
    if constexpr (!DUMP) {
        const float v = wave_reduce_spread<V>(acc, lane);
        if (lane < V) {
            const int r = lane / NTP, t = lane % NTP;
            if (t < NT && row0 + r < od)
                out[(size_t)t * od + row0 + r] = v;
        }
    }
}

// ------------------------------------------------------------------ launch

template <int NT, int R, bool DUMP>
static hipError_t launch_one(int type, const uint8_t* W, const int8_t* q, const float* d,
                             const float* s, int od, int id, float* out, int32_t* S, hipStream_t st)
{
    const int waves = (od + R - 1) / R;
    const int grid = (waves + 3) / 4;
    if (type == 1)
        hipLaunchKernelGGL((mmvq_q4k_kernel<NT, R, DUMP>), dim3(grid), dim3(256), 0, st, W, q, d, s,
                           out, od, id, S);
    else
        hipLaunchKernelGGL((mmvq_q6k_kernel<NT, R, DUMP>), dim3(grid), dim3(256), 0, st, W, q, d, out,
                           od, id, S);
    return hipGetLastError();
}

// Rows per wave: enough waves to give every CU several (256 CUs), then fewer,
// larger row groups to reuse the activation registers.
template <int NT>
static hipError_t launch_nt(int type, const uint8_t* W, const int8_t* q, const float* d,
                            const float* s, int od, int id, float* out, int32_t* S, hipStream_t st)
{
    if (S)
        return launch_one<NT, 1, true>(type, W, q, d, s, od, id, out, S, st);
    if (od >= 4 * 2048)
        return launch_one<NT, 4, false>(type, W, q, d, s, od, id, out, S, st);
    if (od >= 2 * 2048)
        return launch_one<NT, 2, false>(type, W, q, d, s, od, id, out, S, st);
    return launch_one<NT, 1, false>(type, W, q, d, s, od, id, out, S, st);
}

hipError_t launch_mmvq(int type, const uint8_t* W, const int8_t* q, const float* d, const float* s,
                       int nt, int od, int id, float* out, int32_t* S, hipStream_t st)
{
    switch (nt) {
    case 1: return launch_nt<1>(type, W, q, d, s, od, id, out, S, st);
    case 2: return launch_nt<2>(type, W, q, d, s, od, id, out, S, st);
    case 3: return launch_nt<3>(type, W, q, d, s, od, id, out, S, st);
    case 4: return launch_nt<4>(type, W, q, d, s, od, id, out, S, st);
    case 5: return launch_nt<5>(type, W, q, d, s, od, id, out, S, st);
    case 6: return launch_nt<6>(type, W, q, d, s, od, id, out, S, st);
    case 7: return launch_nt<7>(type, W, q, d, s, od, id, out, S, st);
    case 8: return launch_nt<8>(type, W, q, d, s, od, id, out, S, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
