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
//  * K is cut into windows of eight super-blocks (2048 values).  A wave owns one
//    row group of R rows and one window (or a few, strided) of it; the waves of a
//    row group sit in one workgroup and add their partial sums through LDS.  So a
//    wave issues all of its loads at once -- R rows x two 16-byte weight loads plus
//    the activation loads of its window -- and there is no serial chain of loads.
//    One token on a K of two windows with at most 2 rows per group: one wave takes
//    both windows (all loads first), with no LDS step and no barrier.
//  * Inside a window, lane L takes super-block slot g = L/8 and 16-byte code chunk
//    c = L%8 (32 weights).  A weight load instruction covers eight consecutive
//    super-blocks of a row (1152 contiguous bytes for Q4_K).
//  * The lane's activation codes (two 16-byte pieces per token) and scales are
//    loaded once and reused for all R rows (tokens x rows accumulators in VGPRs).
//  * Integer dots use v_dot4_i32_i8 (codes 0..15 are valid int8; Q6_K codes are
//    centred to -32..31 in registers), scales fold once per group in f32.
//  * The R*NT partial sums are reduced across the 64 lanes with a halving
//    exchange (each step halves the values per lane), then across the waves of
//    the row group in LDS.
#include <stdlib.h>

#include "qmm_internal.h"

namespace qmm {

template <int N>
struct pow2_ceil {
    static constexpr int value = N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : N <= 16 ? 16 : N <= 32 ? 32 : 64;
};

constexpr int kMaxWaves = 8;   // waves per workgroup

// The value of lane (lane ^ m).  Inside a 16-lane row the exchange is a DPP move
// on the VALU (quad permutes for m = 1, 2; the row shifts by 4 selected by lane
// bit 2 for m = 4; the row rotation by 8 for m = 8); across rows it goes through
// the LDS crossbar (ds_bpermute), whose round trip is the long part of a reduction.
__device__ __forceinline__ float lane_xor(float v, int m, int lane)
{
    const int x = __float_as_int(v);
    if (m == 1)
        return __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    if (m == 2)
        return __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    if (m == 4) {
        const int up = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0xF, false);   // row_shl:4: lane + 4
        const int dn = __builtin_amdgcn_update_dpp(x, x, 0x114, 0xF, 0xF, false);   // row_shr:4: lane - 4
        return __int_as_float((lane & 4) ? dn : up);
    }
    if (m == 8)
        return __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));  // row_ror:8
    return __shfl_xor(v, m, 64);
}

// Reduce V values per lane across the wave.  Afterwards lane l (l < V) holds the
// wave total of value index l.  V must be a power of two <= 64.  Every step adds
// the same pair of partial sums whatever the exchange path, so the result does not
// depend on it.
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
            a[i] = keep + lane_xor(send, m, lane);
        }
        cnt >>= 1;
    }
#pragma unroll
    for (int m = V; m < 64; m <<= 1)
        a[0] += lane_xor(a[0], m, lane);
    return a[0];
}

// Sum the per-wave results of a row group in LDS and store them.  Every wave of
// the workgroup calls this (it holds a barrier).  v: this lane's value after the
// wave reduction (lane l < V holds value l = r * NTP + t).
template <int NT, int R, int NTP>
__device__ __forceinline__ void group_store(float v, int lane, int wave, int grp, int wk, int wpr,
                                            int row0, int od, float* __restrict__ out)
{
    constexpr int V = R * NTP;
    __shared__ float red[kMaxWaves][V];
    if (wpr > 1) {
        if (lane < V)
            red[wave][lane] = v;
        __syncthreads();
        if (wk != 0)
            return;
        if (lane < V)
            for (int k = 1; k < wpr; ++k)
                v += red[grp * wpr + k][lane];
    }
    if (lane < V) {
        const int r = lane / NTP, t = lane % NTP;
        if (t < NT && row0 + r < od)
            out[(size_t)t * od + row0 + r] = v;
    }
}

// ------------------------------------------------------------------ Q4_K
// Lane chunk c: code chunk p = c/2 (32 bytes: sub-block 2p in low nibbles, 2p+1
// in high nibbles, same positions), half = c%2 -> positions 16*half .. +15.
//
// Scales of sub-blocks 2p and 2p+1 in one pass, as bytes [sc0, sc1, m0, m1] of
// one dword.  [MMQ, section 6, get_scale_min_k4 semantics]: for p < 2 the six
// low bits of bytes 2p, 2p+1 of scale dword 1 (scales) and dword 2 (mins); for
// p >= 2 the nibbles of bytes 2p-4, 2p-3 of dword 3 (low nibble: scale, high
// nibble: min) below the top two bits of the same bytes of dword 1 (scale) or
// dword 2 (min).  Both cases use bytes k, k+1 with k = 2*(p%2), gathered with
// v_perm_b32 (selectors built once per lane).
__device__ __forceinline__ uint32_t q4k_scale_bytes(uint32_t h1, uint32_t h2, uint32_t h3, uint32_t selx,
                                                    uint32_t selz, bool plt2)
{
    const uint32_t x = __builtin_amdgcn_perm(h2, h1, selx);  // [h1.k, h1.k+1, h2.k, h2.k+1]
    const uint32_t z = __builtin_amdgcn_perm(h3, h3, selz);  // [h3.k, h3.k+1, h3.k, h3.k+1]
    const uint32_t lo = x & 0x3F3F3F3Fu;
    const uint32_t nib = (z & 0x00000F0Fu) | ((z >> 4) & 0x0F0F0000u);
    const uint32_t hi = ((x >> 2) & 0x30303030u) | nib;
    return plt2 ? lo : hi;
}

// Q5 (Q5_K, 176-byte blocks): the same sub-block structure with a fifth code bit --
// 32 bytes of high bits after the header (bit j of byte l: element l of sub-block
// j), then the 128 code bytes; the lane's 16 high-bit bytes (positions 16 half ..)
// supply bits 2p and 2p + 1.
// The activation loads of tokens T0 .. T0 + TN - 1 of one window: this lane's two
// 16-byte code pieces and its two blocks' d and s.
template <int TN>
struct K4Act {
    int4 xa[TN], xb[TN];
    float2 dd[TN], ss[TN];
};

template <int TN, int T0>
__device__ __forceinline__ void k4_act_load(K4Act<TN>& A, const int8_t* __restrict__ q, const float* __restrict__ dx,
                                            const float* __restrict__ sx, int id, int nblk, uint32_t ox, uint32_t od2)
{
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int8_t* qt = q + (size_t)(T0 + t) * id;
        A.xa[t] = *reinterpret_cast<const int4*>(qt + ox);
        A.xb[t] = *reinterpret_cast<const int4*>(qt + ox + 32);
        A.dd[t] = *reinterpret_cast<const float2*>(dx + (size_t)(T0 + t) * nblk + od2);
        A.ss[t] = *reinterpret_cast<const float2*>(sx + (size_t)(T0 + t) * nblk + od2);
    }
}

// Tokens T0 .. T0 + TN - 1 of one window (activations in A): the products with
// each of the R rows' blocks (hdr, qs, qh), added into acc, row by row in the
// order the rows' loads were issued.
template <int TN, int T0, int NTP, int R, bool DUMP, bool Q5>
__device__ __forceinline__ void k4_tokens(
    const K4Act<TN>& A, bool bv, int half, int p, uint32_t selx, uint32_t selz, bool plt2,
    const uint4 (&hdr)[R], const uint4 (&qs)[R], const uint4 (&qh)[Q5 ? R : 1], float (&acc)[R * NTP],
    int32_t* __restrict__ S, int row0, int od, int nsb, int b)
{
    const int4 (&xa)[TN] = A.xa;
    const int4 (&xb)[TN] = A.xb;
    const float2 (&dd)[TN] = A.dd;
    const float2 (&ss)[TN] = A.ss;
    // a lane past the row end adds nothing; the min term of a sub-block is
    // added by its half-0 lane only
    float da[TN], db[TN], sa[TN], sb[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        da[t] = bv ? dd[t].x : 0.f;
        db[t] = bv ? dd[t].y : 0.f;
        sa[t] = (bv && half == 0) ? ss[t].x : 0.f;
        sb[t] = (bv && half == 0) ? ss[t].y : 0.f;
    }
    // ---- compute
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint4 h = hdr[r], w4 = qs[r];
        int lo0 = (int)(w4.x & 0x0F0F0F0Fu), lo1 = (int)(w4.y & 0x0F0F0F0Fu);
        int lo2 = (int)(w4.z & 0x0F0F0F0Fu), lo3 = (int)(w4.w & 0x0F0F0F0Fu);
        int hi0 = (int)((w4.x >> 4) & 0x0F0F0F0Fu), hi1 = (int)((w4.y >> 4) & 0x0F0F0F0Fu);
        int hi2 = (int)((w4.z >> 4) & 0x0F0F0F0Fu), hi3 = (int)((w4.w >> 4) & 0x0F0F0F0Fu);
        if constexpr (Q5) {
            // fifth bits: bit 2p of each high-bit byte for sub-block 2p, 2p + 1 for 2p + 1
            const uint4 b5 = qh[r];
            const uint32_t s0 = 2u * (uint32_t)p;
            lo0 |= (int)(((b5.x >> s0) & 0x01010101u) << 4), lo1 |= (int)(((b5.y >> s0) & 0x01010101u) << 4);
            lo2 |= (int)(((b5.z >> s0) & 0x01010101u) << 4), lo3 |= (int)(((b5.w >> s0) & 0x01010101u) << 4);
            hi0 |= (int)(((b5.x >> (s0 + 1)) & 0x01010101u) << 4);
            hi1 |= (int)(((b5.y >> (s0 + 1)) & 0x01010101u) << 4);
            hi2 |= (int)(((b5.z >> (s0 + 1)) & 0x01010101u) << 4);
            hi3 |= (int)(((b5.w >> (s0 + 1)) & 0x01010101u) << 4);
        }
        const uint32_t sm = q4k_scale_bytes(h.y, h.z, h.w, selx, selz, plt2);
        const int sc0 = (int)(sm & 0xFF), sc1 = (int)((sm >> 8) & 0xFF);
        const float m0 = (float)((sm >> 16) & 0xFF), m1 = (float)(sm >> 24);
        const float dw = f16_bits_to_f32(h.x & 0xFFFF);
        const float dm = f16_bits_to_f32(h.x >> 16);
#pragma unroll
        for (int t = 0; t < TN; ++t) {
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
                if (bv && row0 + r < od && half == 0) {
                    int32_t* dst = S + (((size_t)(T0 + t) * od + row0 + r) * nsb + b) * 8 + 2 * p;
                    dst[0] = f0;
                    dst[1] = f1;
                }
            } else {
                // sc * S in integers (|sc * S| < 2^23, exact in f32), then
                // acc += d * (dx0 * sc0 S0 + dx1 * sc1 S1) - dmin * (m0 s0 + m1 s1)
                const float x0 = (float)__mul24(sc0, s0), x1 = (float)__mul24(sc1, s1);
                float a = acc[r * NTP + T0 + t];
                a = fmaf(dw, fmaf(da[t], x0, db[t] * x1), a);
                a = fmaf(-dm, fmaf(m0, sa[t], m1 * sb[t]), a);
                acc[r * NTP + T0 + t] = a;
            }
        }
    }
}

// TB < NT: the activations of tokens 0 .. TB - 1 are loaded and used before those
// of the rest -- fewer registers (more resident waves) for a second round of load
// latency per window.
template <int NT, int R, bool DUMP, bool Q5, int TB = NT>
__device__ __forceinline__ void mmvq_k4_body(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    const float* __restrict__ sx, float* __restrict__ out, int od, int id, int32_t* __restrict__ S,
    int wpr, int gpw)
{
    constexpr int NTP = pow2_ceil<NT>::value;
    constexpr int V = R * NTP;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / wpr, wk = wave - grp * wpr;
    const int row0 = (blockIdx.x * gpw + grp) * R;
    const int g = lane >> 3, c = lane & 7;
    const int p = c >> 1, half = c & 1;
    const uint32_t k = 2u * (uint32_t)(p & 1);
    const uint32_t selx = k | ((k + 1) << 8) | ((k + 4) << 16) | ((k + 5) << 24);
    const uint32_t selz = k | ((k + 1) << 8) | (k << 16) | ((k + 1) << 24);
    const bool plt2 = p < 2;
    const int nsb = id >> 8;
    const int nblk = id >> 5;
    const int nwin = (nsb + 7) >> 3;
    constexpr uint32_t BB = Q5 ? kQ5KBytes : kQ4KBytes;
    const size_t row_bytes = (size_t)nsb * BB;
    const bool live = row0 < od;  // a dead row group still reaches the barrier

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc[i] = 0.f;

    for (int w = wk; live && w < nwin; w += wpr) {
        const int b = 8 * w + g;
        const bool bv = b < nsb;
        const uint32_t bc = (uint32_t)(bv ? b : nsb - 1);
        // ---- loads: uniform row / token bases plus a 32-bit lane offset
        const uint32_t oh = bc * BB, oq = oh + (Q5 ? 48 : 16) + 32 * p + 16 * half, o5 = oh + 16 + 16 * half;
        const uint32_t ox = 256 * bc + 64 * p + 16 * half, od2 = 8 * bc + 2 * p;
        // all tokens at once: the activations (cache hits) first, then the rows'
        // blocks in row order, so the compute of row r waits only for rows <= r
        K4Act<TB> A;
        if constexpr (TB == NT)
            k4_act_load<TB, 0>(A, q, dx, sx, id, nblk, ox, od2);
        __builtin_amdgcn_sched_barrier(0);
        uint4 hdr[R], qs[R], qh[Q5 ? R : 1];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint8_t* rp = W + (size_t)min(row0 + r, od - 1) * row_bytes;
            hdr[r] = *reinterpret_cast<const uint4*>(rp + oh);
            qs[r] = *reinterpret_cast<const uint4*>(rp + oq);
            if constexpr (Q5)
                qh[r] = *reinterpret_cast<const uint4*>(rp + o5);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (TB < NT)
            k4_act_load<TB, 0>(A, q, dx, sx, id, nblk, ox, od2);
        // keep every load above this point
        __builtin_amdgcn_sched_barrier(0);
        k4_tokens<TB, 0, NTP, R, DUMP, Q5>(A, bv, half, p, selx, selz, plt2, hdr, qs, qh, acc, S, row0, od, nsb, b);
        if constexpr (TB < NT) {
            K4Act<NT - TB> B;
            k4_act_load<NT - TB, TB>(B, q, dx, sx, id, nblk, ox, od2);
            __builtin_amdgcn_sched_barrier(0);
            k4_tokens<NT - TB, TB, NTP, R, DUMP, Q5>(B, bv, half, p, selx, selz, plt2, hdr, qs, qh, acc, S, row0, od,
                                                     nsb, b);
        }
    }
    if constexpr (!DUMP) {
        const float v = wave_reduce_spread<V>(acc, lane);
        group_store<NT, R, NTP>(v, lane, wave, grp, wk, wpr, row0, od, out);
    }
}

// One token over a K of two windows (9..16 super-blocks): one wave takes both windows
// of its row group, with every load issued first (the activations, then window 0's
// rows, then window 1's), so the row group needs no second wave, no LDS round trip
// and no barrier.  The two windows' sums are reduced across the lanes apart and
// added in window order: the operations and their order are those of the
// two-wave form, so the outputs are the same bits.
template <int R>
__global__ __launch_bounds__(256) void mmvq_q4k_w2_kernel(const uint8_t* __restrict__ W,
                                                          const int8_t* __restrict__ q,
                                                          const float* __restrict__ dx,
                                                          const float* __restrict__ sx, float* __restrict__ out,
                                                          int od, int id)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (blockIdx.x * 4 + wave) * R;
    if (row0 >= od)
        return;  // whole wave; the kernel has no barrier
    const int g = lane >> 3, c = lane & 7;
    const int p = c >> 1, half = c & 1;
    const uint32_t k = 2u * (uint32_t)(p & 1);
    const uint32_t selx = k | ((k + 1) << 8) | ((k + 4) << 16) | ((k + 5) << 24);
    const uint32_t selz = k | ((k + 1) << 8) | (k << 16) | ((k + 1) << 24);
    const bool plt2 = p < 2;
    const int nsb = id >> 8, nblk = id >> 5;
    const size_t row_bytes = (size_t)nsb * kQ4KBytes;
    const int b0 = g, b1 = 8 + g;
    const bool bv0 = b0 < nsb, bv1 = b1 < nsb;
    const uint32_t c0 = (uint32_t)(bv0 ? b0 : nsb - 1), c1 = (uint32_t)(bv1 ? b1 : nsb - 1);
    const uint32_t oh0 = c0 * kQ4KBytes, oq0 = oh0 + 16 + 32 * p + 16 * half;
    const uint32_t oh1 = c1 * kQ4KBytes, oq1 = oh1 + 16 + 32 * p + 16 * half;
    K4Act<1> A0, A1;
    k4_act_load<1, 0>(A0, q, dx, sx, id, nblk, 256 * c0 + 64 * p + 16 * half, 8 * c0 + 2 * p);
    k4_act_load<1, 0>(A1, q, dx, sx, id, nblk, 256 * c1 + 64 * p + 16 * half, 8 * c1 + 2 * p);
    __builtin_amdgcn_sched_barrier(0);
    uint4 hdr0[R], qs0[R], hdr1[R], qs1[R], qh[1];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint8_t* rp = W + (size_t)min(row0 + r, od - 1) * row_bytes;
        hdr0[r] = *reinterpret_cast<const uint4*>(rp + oh0);
        qs0[r] = *reinterpret_cast<const uint4*>(rp + oq0);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint8_t* rp = W + (size_t)min(row0 + r, od - 1) * row_bytes;
        hdr1[r] = *reinterpret_cast<const uint4*>(rp + oh1);
        qs1[r] = *reinterpret_cast<const uint4*>(rp + oq1);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    float acc0[R], acc1[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        acc0[i] = acc1[i] = 0.f;
    k4_tokens<1, 0, 1, R, false, false>(A0, bv0, half, p, selx, selz, plt2, hdr0, qs0, qh, acc0, nullptr, row0, od,
                                        nsb, b0);
    k4_tokens<1, 0, 1, R, false, false>(A1, bv1, half, p, selx, selz, plt2, hdr1, qs1, qh, acc1, nullptr, row0, od,
                                        nsb, b1);
    const float v0 = wave_reduce_spread<R>(acc0, lane);
    const float v1 = wave_reduce_spread<R>(acc1, lane);
    if (lane < R && row0 + lane < od)
        out[row0 + lane] = v0 + v1;
}

template <int NT, int R, bool DUMP>
__global__ __launch_bounds__(64 * kMaxWaves) void mmvq_q4k_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    const float* __restrict__ sx, float* __restrict__ out, int od, int id, int32_t* __restrict__ S,
    int wpr, int gpw)
{
    mmvq_k4_body<NT, R, DUMP, false>(W, q, dx, sx, out, od, id, S, wpr, gpw);
}

// Token batches of the 4-row Q4_K / Q5_K kernels: loading the activations of TB
// tokens at a time frees registers for more resident waves (Q5_K at 8 tokens: 166
// instead of 256 registers plus a spill; Q5_K at 4 tokens: 123 instead of 171, four
// waves per SIMD instead of two) and costs a round of load latency per batch.  The
// table is measured on 4096-, 8192- and 12288-row matrices of 4096 and 12288 columns
// (Q5_K at 8 tokens: 30.5 -> 18.0 us at 12288 x 4096; Q4_K at 7 tokens: 16.9 -> 14.9
// us); k4_batch_many marks a batch that pays only when the launch holds at least four
// waves per SIMD (4096 waves), i.e. when occupancy rather than latency is the limit.
constexpr int k4_batch(int nt, bool q5)
{
    return q5 ? (nt == 3 || nt == 4 ? 2 : nt >= 6 ? 4 : nt) : (nt == 3 || nt == 5 || nt == 7 ? 2 : nt == 8 ? 4 : nt);
}
constexpr bool k4_batch_many(int nt, bool q5) { return q5 ? nt == 4 : nt == 8; }
// Q6_K (both layouts) at 7 and 8 tokens, with at least 4096 waves: tokens 0..4, then
// the rest (32000 x 4096 at 8 tokens: 45.2 -> 39.5 us; 12288 x 4096: 19.2 -> 17.2).
constexpr int q6k_batch(int nt) { return nt >= 7 ? 5 : nt; }

template <int NT, int R, bool Q5, int TB>
__global__ __launch_bounds__(64 * kMaxWaves) void mmvq_k4_tb_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    const float* __restrict__ sx, float* __restrict__ out, int od, int id, int32_t* __restrict__ S,
    int wpr, int gpw)
{
    mmvq_k4_body<NT, R, false, Q5, TB>(W, q, dx, sx, out, od, id, S, wpr, gpw);
}

template <int NT, int R, bool DUMP>
__global__ __launch_bounds__(64 * kMaxWaves) void mmvq_q5k_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    const float* __restrict__ sx, float* __restrict__ out, int od, int id, int32_t* __restrict__ S,
    int wpr, int gpw)
{
    mmvq_k4_body<NT, R, DUMP, true>(W, q, dx, sx, out, od, id, S, wpr, gpw);
}

// ------------------------------------------------------------------ Q6_K
// Reading of the element map (the pages leave it open; public GGUF arrangement):
// half h of 128 elements uses low bytes 64h.., high bytes 32h..; quarter k of the
// half takes low nibbles (k < 2) or high nibbles (k >= 2) of low bytes 64h+32(k%2)+l
// and bits 2k..2k+1 of high byte 32h+l.  Lane chunk c: h = c/4, jq = (c/2)%2,
// half = c%2 -> 16 positions of quarter jq (low nibbles) and of quarter jq+2 (high
// nibbles) read from one 16-byte low chunk and one 16-byte high chunk.  Blocks
// are 210 bytes, so a block can start 2 bytes off a dword: chunks are read as
// five aligned dwords inside the block and funnel-shifted.  The raw 6-bit codes
// (0..63) enter the integer dot and the offset 32 comes off afterwards as
// 32 * sum(qx) of the group ([GEMM, "Weights: 8 rows per register"]: the offset
// folds out through the activation sum), the sum being computed once per window.
// PAD: blocks padded to 224 bytes ([GEMM, "The GPU path"]: every 16-byte piece
// aligned), so each chunk is one 16-byte load.
// Tokens T0 .. T0 + TN - 1 of one Q6_K window: the activation loads and sums, then
// the products with each of the R rows' chunks (ql, qh, scales and d loaded),
// added into acc.
// The activation loads of tokens T0 .. T0 + TN - 1 of one window for the Q6_K
// body: the lane's two 16-byte code pieces and the d of their two 32-blocks.
template <int TN>
struct Q6Act {
    int4 xa[TN], xb[TN];
    float da[TN], db[TN];
};

template <int TN, int T0>
__device__ __forceinline__ void q6k_act_load(Q6Act<TN>& A, const int8_t* __restrict__ q, const float* __restrict__ dx,
                                             int id, int nblk, uint32_t ox, uint32_t od2)
{
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int8_t* qt = q + (size_t)(T0 + t) * id;
        A.xa[t] = *reinterpret_cast<const int4*>(qt + ox);
        A.xb[t] = *reinterpret_cast<const int4*>(qt + ox + 64);
        A.da[t] = dx[(size_t)(T0 + t) * nblk + od2];
        A.db[t] = dx[(size_t)(T0 + t) * nblk + od2 + 2];
    }
}

template <int TN, int T0, int NTP, int R, bool DUMP>
__device__ __forceinline__ void q6k_tokens(
    const Q6Act<TN>& A, bool bv, uint32_t hs, int g1, int g2, const uint4 (&ql)[R], const uint4 (&qh)[R],
    const int (&sc1)[R], const int (&sc2)[R], const uint32_t (&dbits)[R], float (&acc)[R * NTP],
    int32_t* __restrict__ S, int row0, int od, int nsb, int b)
{
    const int4 (&xa)[TN] = A.xa;
    const int4 (&xb)[TN] = A.xb;
    float da[TN], db[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        da[t] = A.da[t];
        db[t] = A.db[t];
    }
    // 32 * sum of the activation codes of each of the lane's two groups
    int ca[TN], cb[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        da[t] = bv ? da[t] : 0.f;
        db[t] = bv ? db[t] : 0.f;
        int u = sdot4(0x01010101, xa[t].x, 0);
        u = sdot4(0x01010101, xa[t].y, u);
        u = sdot4(0x01010101, xa[t].z, u);
        ca[t] = 32 * sdot4(0x01010101, xa[t].w, u);
        int v = sdot4(0x01010101, xb[t].x, 0);
        v = sdot4(0x01010101, xb[t].y, v);
        v = sdot4(0x01010101, xb[t].z, v);
        cb[t] = 32 * sdot4(0x01010101, xb[t].w, v);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint4 L = ql[r], H = qh[r];
        // quarter jq: low nibbles with bits hs..hs+1 of the high bytes above them;
        // quarter jq+2: high nibbles with bits hs+4..hs+5
        const uint32_t h0 = H.x >> hs, h1 = H.y >> hs, h2 = H.z >> hs, h3 = H.w >> hs;
        const int a0 = (int)(((h0 << 4) & 0x30303030u) | (L.x & 0x0F0F0F0Fu));
        const int a1 = (int)(((h1 << 4) & 0x30303030u) | (L.y & 0x0F0F0F0Fu));
        const int a2 = (int)(((h2 << 4) & 0x30303030u) | (L.z & 0x0F0F0F0Fu));
        const int a3 = (int)(((h3 << 4) & 0x30303030u) | (L.w & 0x0F0F0F0Fu));
        const int b0 = (int)((h0 & 0x30303030u) | ((L.x >> 4) & 0x0F0F0F0Fu));
        const int b1 = (int)((h1 & 0x30303030u) | ((L.y >> 4) & 0x0F0F0F0Fu));
        const int b2 = (int)((h2 & 0x30303030u) | ((L.z >> 4) & 0x0F0F0F0Fu));
        const int b3 = (int)((h3 & 0x30303030u) | ((L.w >> 4) & 0x0F0F0F0Fu));
        const float dw = f16_bits_to_f32(dbits[r]);
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            int s1 = sdot4(a0, xa[t].x, 0);
            s1 = sdot4(a1, xa[t].y, s1);
            s1 = sdot4(a2, xa[t].z, s1);
            s1 = sdot4(a3, xa[t].w, s1) - ca[t];
            int s2 = sdot4(b0, xb[t].x, 0);
            s2 = sdot4(b1, xb[t].y, s2);
            s2 = sdot4(b2, xb[t].z, s2);
            s2 = sdot4(b3, xb[t].w, s2) - cb[t];
            if constexpr (DUMP) {
                if (bv && row0 + r < od) {
                    int32_t* dst = S + (((size_t)(T0 + t) * od + row0 + r) * nsb + b) * 16;
                    dst[g1] = s1;
                    dst[g2] = s2;
                }
            } else {
                // sc * S in integers (|sc * S| < 2^22, exact in f32)
                const float x1 = (float)__mul24(sc1[r], s1), x2 = (float)__mul24(sc2[r], s2);
                acc[r * NTP + T0 + t] = fmaf(dw, fmaf(da[t], x1, db[t] * x2), acc[r * NTP + T0 + t]);
            }
        }
    }
}

// TB < NT: token batches as in the Q4_K kernel.
template <int NT, int R, bool DUMP, bool PAD, int TB = NT>
__device__ __forceinline__ void mmvq_q6k_body(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    float* __restrict__ out, int od, int id, int32_t* __restrict__ S, int wpr, int gpw)
{
    constexpr int NTP = pow2_ceil<NT>::value;
    constexpr int V = R * NTP;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / wpr, wk = wave - grp * wpr;
    const int row0 = (blockIdx.x * gpw + grp) * R;
    const int g = lane >> 3, c = lane & 7;
    const int h = c >> 2, jq = (c >> 1) & 1, half = c & 1;
    const int g1 = 8 * h + 2 * jq + half;  // scale group of the low-nibble quarter
    const int g2 = g1 + 4;                 // scale group of the high-nibble quarter
    const uint32_t hs = 2u * (uint32_t)jq;
    const uint32_t f1 = 64 * h + 32 * jq + 16 * half, f2 = 128 + 32 * h + 16 * half;
    const int nsb = id >> 8;
    const int nblk = id >> 5;
    const int nwin = (nsb + 7) >> 3;
    constexpr uint32_t BB = PAD ? kQ6KP224Bytes : kQ6KBytes;
    const size_t row_bytes = (size_t)nsb * BB;
    const bool live = row0 < od;

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc[i] = 0.f;

    for (int w = wk; live && w < nwin; w += wpr) {
        const int b = 8 * w + g;
        const bool bv = b < nsb;
        const uint32_t bc = (uint32_t)(bv ? b : nsb - 1);
        const uint32_t ob = bc * BB;
        const uint32_t ox = 256 * bc + 128 * h + 32 * jq + 16 * half, od2 = 8 * bc + 4 * h + jq;
        // all tokens at once: the activations (cache hits) first, then the rows'
        // blocks in row order, so the compute of row r waits only for rows <= r
        Q6Act<TB> A;
        if constexpr (TB == NT)
            q6k_act_load<TB, 0>(A, q, dx, id, nblk, ox, od2);
        __builtin_amdgcn_sched_barrier(0);
        uint4 ql[R], qh[R];
        int sc1[R], sc2[R];
        uint32_t dbits[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint8_t* rp = W + (size_t)min(row0 + r, od - 1) * row_bytes;
            if constexpr (PAD || NT >= 2) {
                // 210-byte blocks leave these pieces 2-byte aligned; the GPU reads them
                // directly (user queues run with unaligned access enabled).  From 2
                // tokens on that is 10-25 % faster than assembling them from dwords
                // (fewer registers); at 1 token the dword form below is kept (32000 x
                // 4096: 22.4 against 22.9 us; 12288 x 4096: 10.6 against 10.1)
                ql[r] = *reinterpret_cast<const uint4*>(rp + ob + f1);
                qh[r] = *reinterpret_cast<const uint4*>(rp + ob + f2);
            } else {
                // rp's offset from a dword is uniform; the lane adds its block offset
                const uint32_t res = (uint32_t)(reinterpret_cast<uintptr_t>(rp) & 3);
                const uint8_t* rp4 = rp - res;
                const uint32_t o = ob + res, o4 = o & ~3u, sh = o & 3u;
                const uint32_t* pl = reinterpret_cast<const uint32_t*>(rp4 + o4 + f1);
                const uint32_t* ph = reinterpret_cast<const uint32_t*>(rp4 + o4 + f2);
                const uint32_t l0 = pl[0], l1 = pl[1], l2 = pl[2], l3 = pl[3], l4 = pl[4];
                const uint32_t m0 = ph[0], m1 = ph[1], m2 = ph[2], m3 = ph[3], m4 = ph[4];
                ql[r] = make_uint4(__builtin_amdgcn_alignbyte(l1, l0, sh), __builtin_amdgcn_alignbyte(l2, l1, sh),
                                   __builtin_amdgcn_alignbyte(l3, l2, sh), __builtin_amdgcn_alignbyte(l4, l3, sh));
                qh[r] = make_uint4(__builtin_amdgcn_alignbyte(m1, m0, sh), __builtin_amdgcn_alignbyte(m2, m1, sh),
                                   __builtin_amdgcn_alignbyte(m3, m2, sh), __builtin_amdgcn_alignbyte(m4, m3, sh));
            }
            sc1[r] = (int)reinterpret_cast<const int8_t*>(rp)[ob + 192 + g1];
            sc2[r] = (int)reinterpret_cast<const int8_t*>(rp)[ob + 192 + g2];
            dbits[r] = *reinterpret_cast<const uint16_t*>(rp + ob + 208);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (TB < NT)
            q6k_act_load<TB, 0>(A, q, dx, id, nblk, ox, od2);
        // keep every load above this point
        __builtin_amdgcn_sched_barrier(0);
        q6k_tokens<TB, 0, NTP, R, DUMP>(A, bv, hs, g1, g2, ql, qh, sc1, sc2, dbits, acc, S, row0, od, nsb, b);
        if constexpr (TB < NT) {
            Q6Act<NT - TB> B;
            q6k_act_load<NT - TB, TB>(B, q, dx, id, nblk, ox, od2);
            __builtin_amdgcn_sched_barrier(0);
            q6k_tokens<NT - TB, TB, NTP, R, DUMP>(B, bv, hs, g1, g2, ql, qh, sc1, sc2, dbits, acc, S, row0, od, nsb,
                                                  b);
        }
    }
    if constexpr (!DUMP) {
        const float v = wave_reduce_spread<V>(acc, lane);
        group_store<NT, R, NTP>(v, lane, wave, grp, wk, wpr, row0, od, out);
    }
}

template <int NT, int R, bool DUMP, bool PAD>
__global__ __launch_bounds__(64 * kMaxWaves) void mmvq_q6k_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    float* __restrict__ out, int od, int id, int32_t* __restrict__ S, int wpr, int gpw)
{
    mmvq_q6k_body<NT, R, DUMP, PAD>(W, q, dx, out, od, id, S, wpr, gpw);
}

template <int NT, int R, bool PAD, int TB>
__global__ __launch_bounds__(64 * kMaxWaves) void mmvq_q6k_tb_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    float* __restrict__ out, int od, int id, int32_t* __restrict__ S, int wpr, int gpw)
{
    mmvq_q6k_body<NT, R, false, PAD, TB>(W, q, dx, out, od, id, S, wpr, gpw);
}

// ------------------------------------------------------------------ Q4_0 / Q8_0
// 32-weight blocks ([CH03, section 3.2] Q4_0: f16 d, 16 bytes, byte l holding
// element l in the low and element l + 16 in the high nibble, w = d (nibble - 8);
// Q8_0: f16 d, 32 int8 codes, w = d q).  [CH04, section 3.4]: one integer 4-way
// dot per 4 code bytes, both scales folded once per block, the Q4_0 offset taken
// off through the activation sum: d4 * (dx * dot - 8 * s), s = dx * sum(qx) as
// stored by the quantizer.  A window is 64 blocks (2048 weights, as for the
// K-quants); lane L takes block 64 w + L.  Rows are 16-byte aligned (eight blocks
// are 144 or 272 bytes), so a block starts 0 or 2 bytes past a dword: the lane
// loads exactly the dwords the block covers (5 or 9) and funnel-shifts them.
template <int NT, int R, bool DUMP, bool Q8>
__global__ __launch_bounds__(64 * kMaxWaves) void mmvq_b32_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    const float* __restrict__ sx, float* __restrict__ out, int od, int id, int32_t* __restrict__ S,
    int wpr, int gpw)
{
    constexpr int NTP = pow2_ceil<NT>::value;
    constexpr int V = R * NTP;
    constexpr uint32_t BB = Q8 ? 34 : 18;  // bytes per block
    constexpr int ND = Q8 ? 9 : 5;         // dwords covering one block
    constexpr int NC = Q8 ? 8 : 4;         // code dwords
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / wpr, wk = wave - grp * wpr;
    const int row0 = (blockIdx.x * gpw + grp) * R;
    const int nblk = id >> 5;
    const int nsb = id >> 8;
    const int nwin = (nblk + 63) >> 6;
    const size_t row_bytes = (size_t)nblk * BB;
    const bool live = row0 < od;

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc[i] = 0.f;

    for (int w = wk; live && w < nwin; w += wpr) {
        const int u = 64 * w + lane;
        const bool bv = u < nblk;
        const uint32_t uc = (uint32_t)(bv ? u : nblk - 1);
        int4 xa[NT], xb[NT];
        float da[NT], sa[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int8_t* qt = q + (size_t)t * id + 32 * uc;
            xa[t] = *reinterpret_cast<const int4*>(qt);
            xb[t] = *reinterpret_cast<const int4*>(qt + 16);
            // lanes past the row's last block add nothing: both scale terms zero
            da[t] = bv ? dx[(size_t)t * nblk + uc] : 0.f;
            sa[t] = (Q8 || !bv) ? 0.f : sx[(size_t)t * nblk + uc];
        }
        uint32_t wd[R][ND];
        uint32_t shf[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint8_t* rp = W + (size_t)min(row0 + r, od - 1) * row_bytes;
            const uint32_t off = uc * BB;
            const uint32_t* pw = reinterpret_cast<const uint32_t*>(rp + (off & ~3u));
            shf[r] = off & 3u;
#pragma unroll
            for (int i = 0; i < ND; ++i)
                wd[r][i] = pw[i];
        }
        __builtin_amdgcn_sched_barrier(0);
        int sxi[NT];
        if constexpr (DUMP && !Q8) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                int v = sdot4(0x01010101, xa[t].x, 0);
                v = sdot4(0x01010101, xa[t].y, v);
                v = sdot4(0x01010101, xa[t].z, v);
                v = sdot4(0x01010101, xa[t].w, v);
                v = sdot4(0x01010101, xb[t].x, v);
                v = sdot4(0x01010101, xb[t].y, v);
                v = sdot4(0x01010101, xb[t].z, v);
                sxi[t] = sdot4(0x01010101, xb[t].w, v);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // block bytes from byte 0: bb[i] = bytes 4i .. 4i+3 of the block
            uint32_t bb[ND];
#pragma unroll
            for (int i = 0; i + 1 < ND; ++i)
                bb[i] = __builtin_amdgcn_alignbyte(wd[r][i + 1], wd[r][i], shf[r]);
            bb[ND - 1] = wd[r][ND - 1] >> (8 * shf[r]);
            const float dw = f16_bits_to_f32(bb[0] & 0xFFFF);
            uint32_t cd[NC];  // code bytes 2 .. of the block
#pragma unroll
            for (int i = 0; i < NC; ++i)
                cd[i] = __builtin_amdgcn_alignbyte(bb[i + 1], bb[i], 2);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                int dot;
                if constexpr (Q8) {
                    dot = sdot4((int)cd[0], xa[t].x, 0);
                    dot = sdot4((int)cd[1], xa[t].y, dot);
                    dot = sdot4((int)cd[2], xa[t].z, dot);
                    dot = sdot4((int)cd[3], xa[t].w, dot);
                    dot = sdot4((int)cd[4], xb[t].x, dot);
                    dot = sdot4((int)cd[5], xb[t].y, dot);
                    dot = sdot4((int)cd[6], xb[t].z, dot);
                    dot = sdot4((int)cd[7], xb[t].w, dot);
                } else {
                    // elements 4i.. in low nibbles (against xa), 16 + 4i.. in high (xb)
                    dot = sdot4((int)(cd[0] & 0x0F0F0F0Fu), xa[t].x, 0);
                    dot = sdot4((int)(cd[1] & 0x0F0F0F0Fu), xa[t].y, dot);
                    dot = sdot4((int)(cd[2] & 0x0F0F0F0Fu), xa[t].z, dot);
                    dot = sdot4((int)(cd[3] & 0x0F0F0F0Fu), xa[t].w, dot);
                    dot = sdot4((int)((cd[0] >> 4) & 0x0F0F0F0Fu), xb[t].x, dot);
                    dot = sdot4((int)((cd[1] >> 4) & 0x0F0F0F0Fu), xb[t].y, dot);
                    dot = sdot4((int)((cd[2] >> 4) & 0x0F0F0F0Fu), xb[t].z, dot);
                    dot = sdot4((int)((cd[3] >> 4) & 0x0F0F0F0Fu), xb[t].w, dot);
                }
                if constexpr (DUMP) {
                    if (bv && row0 + r < od) {
                        // centred integer dot of the block (Q4_0: dot - 8 sum(qx))
                        const int sc = Q8 ? dot : dot - 8 * sxi[t];
                        S[(((size_t)t * od + row0 + r) * nsb + (uc >> 3)) * 8 + (uc & 7)] = sc;
                    }
                } else if constexpr (Q8) {
                    acc[r * NTP + t] = fmaf(dw * da[t], (float)dot, acc[r * NTP + t]);
                } else {
                    acc[r * NTP + t] = fmaf(dw, fmaf(da[t], (float)dot, -8.0f * sa[t]), acc[r * NTP + t]);
                }
            }
        }
    }
    if constexpr (!DUMP) {
        const float v = wave_reduce_spread<V>(acc, lane);
        group_store<NT, R, NTP>(v, lane, wave, grp, wk, wpr, row0, od, out);
    }
}

// ------------------------------------------------------------------ launch

// Waves per row group: one per K window up to kMaxWaves (more windows are
// strided over the waves); row groups per workgroup fill up to four waves.
template <int NT, int R, bool DUMP>
static hipError_t launch_one(int type, const uint8_t* W, const int8_t* q, const float* d,
                             const float* s, int od, int id, float* out, int32_t* S, hipStream_t st)
{
    const int nwin = (id / 256 + 7) / 8;
    const int wpr = nwin < kMaxWaves ? nwin : kMaxWaves;
    const int gpw = wpr >= 4 ? 1 : 4 / wpr;
    const int groups = (od + R - 1) / R;
    const int grid = (groups + gpw - 1) / gpw;
    const dim3 block(64 * wpr * gpw);
    // one token, two K windows, at most 2 rows per group (matrices under 8192 rows):
    // the single-wave form (4096 x 4096: 4.40 -> 4.05 us in one process); from 4
    // rows on, the two-wave form's doubled wave count is worth more (12288 x 4096:
    // 6.93 against 7.23 us)
    if constexpr (!DUMP && NT == 1 && R <= 2) {
        if (type == 1 && nwin == 2) {
            hipLaunchKernelGGL((mmvq_q4k_w2_kernel<R>), dim3((groups + 3) / 4), dim3(256), 0, st, W, q, d, s, out, od,
                               id);
            return hipGetLastError();
        }
    }
    if constexpr (!DUMP && R == 4) {
        const bool many = (int64_t)grid * wpr * gpw >= 4096;
        if constexpr (k4_batch(NT, false) < NT) {
            if (type == 1 && (many || !k4_batch_many(NT, false))) {
                hipLaunchKernelGGL((mmvq_k4_tb_kernel<NT, R, false, k4_batch(NT, false)>), dim3(grid), block, 0, st,
                                   W, q, d, s, out, od, id, S, wpr, gpw);
                return hipGetLastError();
            }
        }
        if constexpr (k4_batch(NT, true) < NT) {
            if (type == 6 && (many || !k4_batch_many(NT, true))) {
                hipLaunchKernelGGL((mmvq_k4_tb_kernel<NT, R, true, k4_batch(NT, true)>), dim3(grid), block, 0, st,
                                   W, q, d, s, out, od, id, S, wpr, gpw);
                return hipGetLastError();
            }
        }
        if constexpr (q6k_batch(NT) < NT) {
            if (type == 2 && many) {
                hipLaunchKernelGGL((mmvq_q6k_tb_kernel<NT, R, false, q6k_batch(NT)>), dim3(grid), block, 0, st, W, q,
                                   d, out, od, id, S, wpr, gpw);
                return hipGetLastError();
            }
            if (type == 3 && many) {
                hipLaunchKernelGGL((mmvq_q6k_tb_kernel<NT, R, true, q6k_batch(NT)>), dim3(grid), block, 0, st, W, q,
                                   d, out, od, id, S, wpr, gpw);
                return hipGetLastError();
            }
        }
    }
    if (type == 1)
        hipLaunchKernelGGL((mmvq_q4k_kernel<NT, R, DUMP>), dim3(grid), block, 0, st, W, q, d, s, out, od, id,
                           S, wpr, gpw);
    else if (type == 2)
        hipLaunchKernelGGL((mmvq_q6k_kernel<NT, R, DUMP, false>), dim3(grid), block, 0, st, W, q, d, out, od, id, S,
                           wpr, gpw);
    else if (type == 3)
        hipLaunchKernelGGL((mmvq_q6k_kernel<NT, R, DUMP, true>), dim3(grid), block, 0, st, W, q, d, out, od, id, S,
                           wpr, gpw);
    else if (type == 4)
        hipLaunchKernelGGL((mmvq_b32_kernel<NT, R, DUMP, false>), dim3(grid), block, 0, st, W, q, d, s, out, od, id,
                           S, wpr, gpw);
    else if (type == 5)
        hipLaunchKernelGGL((mmvq_b32_kernel<NT, R, DUMP, true>), dim3(grid), block, 0, st, W, q, d, s, out, od, id,
                           S, wpr, gpw);
    else
        hipLaunchKernelGGL((mmvq_q5k_kernel<NT, R, DUMP>), dim3(grid), block, 0, st, W, q, d, s, out, od, id, S, wpr,
                           gpw);
    return hipGetLastError();
}

// Rows per row group R.  K of up to two windows (id <= 4096): one token, the
// largest of 4, 2, 1 that leaves at least 2048 row groups (eight per CU on 256
// CUs); several tokens: every lane's activation loads (NT tokens) are shared by R
// rows, so 4 rows from od = 4096 up (measured on 4096- and 12288-row Q4_K at nt = 4
// and 8: 7-9 % faster than 2).  Longer K: by the wave count (below).
// QMM_MMVQ_ROWS (1, 2, 4, or 8 for nt <= 2) overrides it, read once, for tuning
// sweeps.
static int rows_override()
{
    static int v = -1;
    int cur = __atomic_load_n(&v, __ATOMIC_ACQUIRE);
    if (cur >= 0)
        return cur;
    const char* e = getenv("QMM_MMVQ_ROWS");
    int val = e ? atoi(e) : 0;
    if (val != 1 && val != 2 && val != 4 && val != 8)
        val = 0;
    __atomic_store_n(&v, val, __ATOMIC_RELEASE);
    return val;
}

template <int NT>
static hipError_t launch_nt(int type, const uint8_t* W, const int8_t* q, const float* d,
                            const float* s, int od, int id, float* out, int32_t* S, hipStream_t st)
{
    if (S)
        return launch_one<NT, 1, true>(type, W, q, d, s, od, id, out, S, st);
    int R = rows_override();
    if (R == 0) {
        const int nwin = (id / 256 + 7) / 8;
        const bool q6_one = NT == 1 && (type == 2 || type == 3);
        if (nwin >= 3 && !q6_one) {
            // a K of three or more windows multiplies the waves of a row group, so
            // fewer row groups keep the chip busy and each wave's activation loads
            // serve more rows: 4 rows while there are at least 2048 waves (1024 for
            // several tokens), else 2 (Q4_K 4096 x 12288 nt = 1: 7.98 -> 7.15 us;
            // 2048 x 12288: 6.48 -> 5.47; 1024 x 12288 nt = 8: 13.5 -> 7.4; Q4_0, Q5_K
            // alike).  Q6_K at one token keeps the rule below (more rows per wave
            // were 4-6 % slower on 1024 and 2048 rows: its rows take more registers)
            const long need = NT >= 2 ? 1024 : 2048;
            R = (long)((od + 3) / 4) * nwin >= need ? 4 : (long)((od + 1) / 2) * nwin >= need ? 2 : 1;
        } else if constexpr (NT >= 2) {
            R = od >= 4096 ? 4 : od >= 2048 ? 2 : 1;
        } else {
            R = od >= 4 * 2048 ? 4 : od >= 2 * 2048 ? 2 : 1;
        }
    }
    if constexpr (NT <= 2) {
        if (R == 8)
            return launch_one<NT, 8, false>(type, W, q, d, s, od, id, out, S, st);
    } else if (R == 8) {
        R = 4;
    }
    if (R == 4)
        return launch_one<NT, 4, false>(type, W, q, d, s, od, id, out, S, st);
    if (R == 2)
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
