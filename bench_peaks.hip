// Microbenchmarks of the MI355X limits that the matmul kernels are measured
// against (bench.py --workload peaks):
//   * the streaming-read rate of HBM at the byte counts of the decode weight
//     matrices (a plain kernel that reads every byte once with 16-byte loads),
//   * the issue rate of the int8 MFMA the matrix kernels use
//     (v_mfma_i32_32x32x32_i8) and of the f32 MFMA outer product,
//   * the issue rate of the VALU instructions of the f32 epilogue (v_cvt_f32_i32,
//     v_fma_f32),
//   * whether MFMA and VALU work overlap: in one wave (independent instructions
//     interleaved) and across the two waves sharing a SIMD (one issuing MFMAs, the
//     other VALU instructions).
// [CH04, section 4.2] sets a documented peak beside a measured one; these kernels
// give the measured side.  Every kernel is a bounded loop over registers (or one
// read of a caller buffer whose size the host checked), and writes one dword per
// wave to a sink only when a result takes a value it never takes, so nothing is
// optimised away and nothing is stored in practice.
//
// C ABI: every call enqueues one launch on `stream` and returns the hipError_t of
// the launch; the caller times launches with events.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

namespace {

constexpr uint32_t kNever = 0x7FC00001u;  // a NaN bit pattern no sum below produces from its inputs

// Reads n16 16-byte words once: workgroup g reads U consecutive 4 KiB pieces, each
// lane one 16-byte word per piece (consecutive lanes, consecutive words).  n16 is
// a multiple of 256 * U (the host checks).
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, uint32_t* __restrict__ sink)
{
    const size_t base = (size_t)blockIdx.x * U * 256 + threadIdx.x;
    uint4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k)
        v[k] = p[base + (size_t)k * 256];
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < U; ++k)
        x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    if (x == kNever)
        sink[blockIdx.x] = x;
}

// Load shapes of a Q4_K matrix (rows of 16 blocks of 144 bytes), every byte read
// once, no arithmetic.  SHAPE 0, the vector kernel's: a workgroup of two waves (K
// windows 0 and 1) over 4 rows, lane l taking block 8w + l/8 of the window and per
// row one load of its 16-byte header and one of its 16-byte code chunk l%8.  SHAPE
// 1: one wave per 2 rows, each row read as its 144 consecutive 16-byte pieces (lane
// l: pieces l, 64 + l and 128 + l, the last clamped to piece 143).
template <int SHAPE>
__global__ __launch_bounds__(128) void load_shape_kernel(const uint8_t* __restrict__ w, uint32_t* __restrict__ sink)
{
    constexpr int kRow = 16 * 144;
    uint32_t x = 0;
    if constexpr (SHAPE == 0) {
        const int lane = threadIdx.x & 63, win = threadIdx.x >> 6;
        const int blk = 8 * win + (lane >> 3), c = lane & 7;
        uint4 h[4], q[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint8_t* rp = w + ((size_t)blockIdx.x * 4 + r) * kRow + blk * 144;
            h[r] = *reinterpret_cast<const uint4*>(rp);
            q[r] = *reinterpret_cast<const uint4*>(rp + 16 + 16 * c);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            x ^= h[r].x ^ h[r].y ^ h[r].z ^ h[r].w ^ q[r].x ^ q[r].y ^ q[r].z ^ q[r].w;
    } else {
        const int lane = threadIdx.x & 63;
        const size_t row0 = ((size_t)blockIdx.x * 2 + (threadIdx.x >> 6)) * 2;
        uint4 v[2][3];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const uint8_t* rp = w + (row0 + r) * kRow;
            v[r][0] = *reinterpret_cast<const uint4*>(rp + 16 * lane);
            v[r][1] = *reinterpret_cast<const uint4*>(rp + 16 * (64 + lane));
            v[r][2] = *reinterpret_cast<const uint4*>(rp + 16 * min(128 + lane, 143));
        }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int k = 0; k < 3; ++k)
                x ^= v[r][k].x ^ v[r][k].y ^ v[r][k].z ^ v[r][k].w;
    }
    if (x == kNever)
        sink[blockIdx.x] = x;
}

// Thread 0 of workgroup 0 records the shader-clock and 100 MHz reference-clock
// ticks its loop took into clk[0], clk[1] (clk may be null): the ratio gives the
// clock the chip ran at under this load.
__device__ __forceinline__ void clock_mark(uint64_t& c0, uint64_t& r0)
{
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ void clock_store(uint64_t c0, uint64_t r0, uint64_t* clk)
{
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (clk && blockIdx.x == 0 && threadIdx.x == 0) {
        clk[0] = c1 - c0;
        clk[1] = r1 - r0;
    }
}

// NACC independent accumulator chains of v_mfma_i32_32x32x32_i8, iters rounds.
template <int NACC>
__global__ __launch_bounds__(256) void mfma_i8_rate_kernel(int iters, uint32_t* __restrict__ sink, uint64_t* clk)
{
    const int lane = threadIdx.x & 63;
    uint64_t c0, r0;
    clock_mark(c0, r0);
    const v4i a = {lane, lane + 1, lane + 2, lane + 3}, b = {3 - lane, 2, 1, lane};
    v16i c[NACC];
#pragma unroll
    for (int m = 0; m < NACC; ++m)
        c[m] = (v16i){};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int m = 0; m < NACC; ++m)
            c[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[m], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int m = 0; m < NACC; ++m)
        for (int k = 0; k < 16; ++k)
            s += c[m][k];
    clock_store(c0, r0, clk);
    if ((uint32_t)s == kNever)
        sink[blockIdx.x] = s;
}

// NACC independent f32 outer-product pairs (v_mfma_f32_32x32x1_2b_f32), iters rounds.
template <int NACC>
__global__ __launch_bounds__(256) void mfma_outer_rate_kernel(int iters, float f, uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const float a = f * (float)lane, b = f - (float)lane;
    v32f c[NACC];
#pragma unroll
    for (int m = 0; m < NACC; ++m)
        c[m] = (v32f){};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int m = 0; m < NACC; ++m)
            c[m] = __builtin_amdgcn_mfma_f32_32x32x1f32(a, b, c[m], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < NACC; ++m)
        for (int k = 0; k < 32; ++k)
            s += c[m][k];
    if (__float_as_uint(s) == kNever)
        sink[blockIdx.x] = 1;
}

// VALU issue rate.  MODE 0: 16 independent v_fma_f32 chains.  MODE 1: the epilogue
// pair, 16 independent chains of acc = fma(cvt_f32_i32(c), p, acc) with c an
// integer register advanced by an add every 8 rounds (so the conversions are not
// hoisted; 1/8 extra op per pair, counted).
template <int MODE>
__global__ __launch_bounds__(256) void valu_rate_kernel(int iters, float f, uint32_t* __restrict__ sink,
                                                        uint64_t* clk)
{
    const int lane = threadIdx.x & 63;
    uint64_t c0, r0;
    clock_mark(c0, r0);
    float acc[16];
    int c[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        acc[k] = f * (float)(lane + k);
        c[k] = lane * 7 + k;
    }
    const float p = f * 0.5f;
    for (int i = 0; i < iters; ++i) {
        if constexpr (MODE == 0) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    acc[k] = fmaf(acc[k], p, f);
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    acc[k] = fmaf((float)c[k], p, acc[k]);
#pragma unroll
            for (int k = 0; k < 16; ++k)
                c[k] += 1 + k;
        }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        s += acc[k];
    clock_store(c0, r0, clk);
    if (__float_as_uint(s) == kNever)
        sink[blockIdx.x] = 1;
}

// Issue rate of one VALU instruction form, written as inline assembly so the
// exact encoding is timed: 16 independent registers, 8 rounds of 16 per loop
// iteration.  OP 0 v_fmac_f32 (VOP2), 1 v_fma_f32 (VOP3, VGPR operands), 2
// v_fma_f32 with an SGPR operand, 3 v_cvt_f32_i32 (VOP1), 4 v_mul_f32, 5 v_and_b32,
// 6 v_lshrrev_b32, 7 v_add_u32, 8 the epilogue pair v_cvt_f32_i32 + v_fmac_f32
// (the fmac reads the conversion: 2 instructions per unit), 9 v_mad_u32_u24.
template <int OP>
__global__ __launch_bounds__(256) void valu_instr_kernel(int iters, float f, uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    float acc[16];
    int iv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        acc[k] = f * (float)(lane + k);
        iv[k] = lane * 7 + k;
    }
    const float p = f * 0.5f;
    float pv = p + (float)lane;  // a VGPR operand
    const int m = 0x0F0F0F0F;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                if constexpr (OP == 0)
                    asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(acc[k]) : "v"(pv), "v"(acc[(k + 1) & 15]));
                else if constexpr (OP == 1)
                    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(acc[k]) : "v"(pv), "v"(acc[(k + 1) & 15]));
                else if constexpr (OP == 2)
                    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(acc[k]) : "v"(pv), "s"(p));
                else if constexpr (OP == 3)
                    asm volatile("v_cvt_f32_i32 %0, %1" : "=v"(acc[k]) : "v"(iv[k]));
                else if constexpr (OP == 4)
                    asm volatile("v_mul_f32 %0, %0, %1" : "+v"(acc[k]) : "v"(pv));
                else if constexpr (OP == 5)
                    asm volatile("v_and_b32 %0, %1, %0" : "+v"(iv[k]) : "s"(m));
                else if constexpr (OP == 6)
                    asm volatile("v_lshrrev_b32 %0, 4, %0" : "+v"(iv[k]));
                else if constexpr (OP == 7)
                    asm volatile("v_add_u32 %0, %0, %1" : "+v"(iv[k]) : "v"(iv[(k + 1) & 15]));
                else if constexpr (OP == 8) {
                    float t;
                    asm volatile("v_cvt_f32_i32 %0, %1" : "=v"(t) : "v"(iv[k]));
                    asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(acc[k]) : "v"(t), "v"(pv));
                } else
                    asm volatile("v_mad_u32_u24 %0, %0, %1, %2" : "+v"(iv[k]) : "v"(iv[(k + 1) & 15]), "v"(lane));
            }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        s += acc[k] + (float)iv[k];
    if (__float_as_uint(s) == kNever)
        sink[blockIdx.x] = 1;
}

// Shadow of an MFMA: per step one v_mfma_i32_32x32x32_i8 (accumulator input a fixed
// register block, result to fresh registers, as in the matrix kernels) followed by
// NV independent v_fmac_f32 (VOP2, VGPR operands) that do not read it; one element
// of every result is folded in one step later.  Time against the MFMA-only and the
// VALU-only forms gives how much VALU work a wave hides behind its own MFMAs.
template <int NV, bool DO_M, bool DO_V>
__global__ __launch_bounds__(256) void shadow_kernel(int iters, float f, uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    v4i a = {lane, lane + 1, lane + 2, lane + 3};
    const v4i b = {3 - lane, 2, 1, lane};
    v16i k;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        k[i] = 0x4B400000 + lane + i;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
        acc[i] = f * (float)(lane + i);
    const float pv = f * 0.5f + (float)lane, qv = f - (float)lane;
    uint32_t x = 0;
    v16i prev = k;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (DO_M) {
                const v16i C = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, k, 0, 0, 0);
                x ^= (uint32_t)prev[r];
                prev = C;
            }
            if (DO_V) {
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(acc[(r * NV + v) & 31]) : "v"(pv), "v"(qv));
            }
            a.x += 1;
        }
    }
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i)
        t += acc[i];
    if (x == kNever || __float_as_uint(t) == kNever)
        sink[blockIdx.x] = 1;
}

// Ping-pong of MFMA and VALU phases between the two waves of each SIMD, the step
// of a per-32 matrix kernel: per phase a wave either issues the MFMAs of two
// sub-blocks (2 x two int8 MFMAs with a fixed accumulator input, 2 f32 outer-product
// pairs: 128 result registers) or runs the epilogue of the results it issued in its
// previous MFMA phase (128 v_sub_f32 + 128 v_fma: acc += (C - bias) * P).  PP 1:
// 512-thread workgroups, waves 0-3 in one phase and 4-7 in the other, an s_barrier
// between phases; PP 0: every wave does its MFMA phase then its epilogue, no
// barriers (the same work per wave).
template <int PP>
__global__ __launch_bounds__(512) void pingpong_kernel(int iters, float f, uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v4i a = {lane, lane + 1, lane + 2, lane + 3};
    const v4i b = {3 - lane, 2, 1, lane};
    v16i k;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        k[i] = 0x4B400000 + lane + i;
    const float fk = __int_as_float(k[0]);
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
        acc[i] = f * (float)(lane + i);
    v16i C[4];
    v32f P[2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        C[m] = k;
#pragma unroll
    for (int m = 0; m < 2; ++m)
        P[m] = (v32f){};
    const float fa = f * (float)lane, fb = f - (float)lane;
    const bool second = PP && wave >= 4;
    auto mfma_phase = [&](int r) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            P[m] = __builtin_amdgcn_mfma_f32_32x32x1f32(fa + (float)(r + m), fb, (v32f){}, 0, 0, 0);
            C[2 * m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, k, 0, 0, 0);
            C[2 * m + 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, k, 0, 0, 0);
        }
        a.x += 1;
    };
    auto valu_phase = [&]() {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const v16f S0 = __builtin_bit_cast(v16f, C[2 * m]) - fk;
            const v16f S1 = __builtin_bit_cast(v16f, C[2 * m + 1]) - fk;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc[i] = fmaf(S0[i], P[m][i], acc[i]);
                acc[16 + i] = fmaf(S1[i], P[m][16 + i], acc[16 + i]);
            }
        }
    };
    for (int r = 0; r < iters; ++r) {
        if (PP) {
            if (second)
                valu_phase();
            else
                mfma_phase(r);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (second)
                mfma_phase(r);
            else
                valu_phase();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        } else {
            mfma_phase(r);
            __builtin_amdgcn_sched_barrier(0);
            valu_phase();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i)
        t += acc[i];
    if (__float_as_uint(t) == kNever)
        sink[blockIdx.x] = 1;
}

// Burst length of the per-32 step: per burst, NB sub-blocks over NN 32-token blocks
// (NN int8 MFMAs per sub-block with a fixed accumulator input; f32 outer-product
// pairs: one per sub-block for NN = 2, one per two sub-blocks for NN = 1), then the
// epilogue of all of them (acc += (C - bias) * P).  One wave does both in turn; 2
// waves per SIMD.
template <int NB, int NN>
__global__ __launch_bounds__(256) void burst_kernel(int iters, float f, uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    v4i a = {lane, lane + 1, lane + 2, lane + 3};
    const v4i b = {3 - lane, 2, 1, lane};
    v16i k;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        k[i] = 0x4B400000 + lane + i;
    const float fk = __int_as_float(k[0]);
    float acc[16 * NN];
#pragma unroll
    for (int i = 0; i < 16 * NN; ++i)
        acc[i] = f * (float)(lane + i);
    const float fb = f - (float)lane;
    constexpr int NP = NN == 2 ? NB : NB / 2;   // outer-product pairs per burst
    // distinct operands per MFMA (identical MFMAs would be computed once)
    v4i av[NB];
    float fav[NP];
#pragma unroll
    for (int m = 0; m < NB; ++m)
        av[m] = (v4i){lane + m, lane + 1, lane + 2 * m, lane + 3};
#pragma unroll
    for (int m = 0; m < NP; ++m)
        fav[m] = f * (float)(lane + m);
    v4i bv[NN];
#pragma unroll
    for (int n = 0; n < NN; ++n)
        bv[n] = (v4i){3 - lane, 2 + n, 1, lane};
    for (int r = 0; r < iters; ++r) {
        v16i C[NB * NN];
        v32f P[NP];
#pragma unroll
        for (int m = 0; m < NP; ++m)
            P[m] = __builtin_amdgcn_mfma_f32_32x32x1f32(fav[m], fb, (v32f){}, 0, 0, 0);
#pragma unroll
        for (int m = 0; m < NB * NN; ++m)
            C[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[m / NN], bv[m % NN], k, 0, 0, 0);
#pragma unroll
        for (int n = 0; n < NN; ++n)
            bv[n].x += 1;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sbk = 0; sbk < NB; ++sbk) {
#pragma unroll
            for (int n = 0; n < NN; ++n) {
                const v16f S = __builtin_bit_cast(v16f, C[sbk * NN + n]) - fk;
                // the scale products of (sub-block sbk, block n): pair NN == 2: P[sbk] half n;
                // NN == 1: P[sbk / 2] half sbk % 2
                const int pm = NN == 2 ? sbk : sbk / 2, ph = NN == 2 ? n : sbk % 2;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[16 * n + i] = fmaf(S[i], P[pm][16 * ph + i], acc[16 * n + i]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16 * NN; ++i)
        t += acc[i];
    if (__float_as_uint(t) == kNever)
        sink[blockIdx.x] = 1;
}

// The MFMA mix of a per-32 matrix step, MFMAs only: per round MODE 0: two
// v_mfma_i32_32x32x32_i8 whose accumulator input is a fixed register block
// (results to fresh registers) and one v_mfma_f32_32x32x1_2b_f32; MODE 1: the two
// int8 MFMAs alone; MODE 2: the outer product alone; MODE 3: two int8 MFMAs
// accumulating in place.  One element of every result is folded into a running
// xor (one VALU op per MFMA) so no MFMA is dead.
template <int MODE>
__global__ __launch_bounds__(256) void mfma_mix_kernel(int iters, float f, uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    v4i a = {lane, lane + 1, lane + 2, lane + 3}, b = {3 - lane, 2, 1, lane};
    v16i k;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        k[i] = 0x4B400000 + lane + i;
    v16i acc0 = k, acc1 = k;
    uint32_t x = 0;
    const float fa = f * (float)lane, fb = f - (float)lane;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (MODE == 0 || MODE == 2) {
                const v32f P = __builtin_amdgcn_mfma_f32_32x32x1f32(fa + (float)r, fb, (v32f){}, 0, 0, 0);
                x ^= __float_as_uint(P[r]);
            }
            if constexpr (MODE == 0 || MODE == 1) {
                const v16i C0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, k, 0, 0, 0);
                const v16i C1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, k, 0, 0, 0);
                x ^= (uint32_t)(C0[r] + C1[15 - r]);
            }
            if constexpr (MODE == 3) {
                acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, acc1, 0, 0, 0);
            }
            a.x += 1;
        }
    }
    if constexpr (MODE == 3)
        x ^= (uint32_t)(acc0[lane & 15] + acc1[3]);
    if (x == kNever)
        sink[blockIdx.x] = x;
}

// LDS read bandwidth: every wave reads 16 bytes per lane per ds_read_b128 from
// addresses spread over a 64 KiB LDS buffer (consecutive lanes, consecutive 16-byte
// words: no bank conflicts), 16 reads in flight per round.
__global__ __launch_bounds__(512) void lds_read_kernel(int iters, uint32_t* __restrict__ sink)
{
    __shared__ uint4 buf[4096];
    for (int i = threadIdx.x; i < 4096; i += blockDim.x)
        buf[i] = make_uint4(i, i * 3, i * 5, i * 7);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = 0;
    for (int i = 0; i < iters; ++i) {
        uint4 v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            v[k] = buf[((wave * 16 + k + i) & 63) * 64 + lane];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    if (x == kNever)
        sink[blockIdx.x] = x;
}

// Overlap of MFMA and VALU work.  Per round: 8 int8 MFMAs on 8 independent
// accumulators and NV * 8 v_fmac_f32 (VOP2, the epilogue's form) on 16 independent
// chains that never read an MFMA result.
//   SPLIT 0: every wave issues both, one MFMA then NV VALU instructions, in that
//            order (sched_group_barrier);
//   SPLIT 1: workgroups of 8 waves; waves 0..3 issue only the MFMAs, waves 4..7
//            only the VALU instructions (the two waves of a SIMD: one of each);
//   DO_M / DO_V switch a part off (the same kernel with one side removed).
template <int NV, int SPLIT, bool DO_M, bool DO_V>
__global__ __launch_bounds__(512) void overlap_kernel(int iters, float f, uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool do_m = DO_M && (SPLIT == 0 || wave < 4);
    const bool do_v = DO_V && (SPLIT == 0 || wave >= 4);
    const v4i a = {lane, lane + 1, lane + 2, lane + 3}, b = {3 - lane, 2, 1, lane};
    v16i c[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
        c[m] = (v16i){};
    float acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
        acc[k] = f * (float)(lane + k);
    const float pv = f * 0.5f + (float)lane, qv = f - (float)lane;
    if (SPLIT == 0) {
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                if (DO_M)
                    c[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[m], 0, 0, 0);
                if (DO_V) {
#pragma unroll
                    for (int v = 0; v < NV; ++v)
                        asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(acc[(m * NV + v) & 15]) : "v"(pv), "v"(qv));
                }
            }
            if (DO_M && DO_V) {
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
                }
            }
        }
    } else {
        if (do_m) {
            for (int i = 0; i < iters; ++i) {
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    c[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[m], 0, 0, 0);
            }
        }
        if (do_v) {
            for (int i = 0; i < iters; ++i) {
#pragma unroll
                for (int m = 0; m < 8; ++m)
#pragma unroll
                    for (int v = 0; v < NV; ++v)
                        asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(acc[(m * NV + v) & 15]) : "v"(pv), "v"(qv));
            }
        }
    }
    int s = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m)
        for (int k = 0; k < 16; ++k)
            s += c[m][k];
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        t += acc[k];
    if ((uint32_t)s == kNever || __float_as_uint(t) == kNever)
        sink[blockIdx.x] = 1;
}

}  // namespace

extern "C" {

// Streaming read of `bytes` bytes at `p` (device, 16-byte aligned; bytes a
// multiple of 256 * 16 * u, u = 1, 2, 4 or 8 words per lane).  sink: device buffer
// of bytes / (4096 * u) dwords.  Returns hipErrorInvalidValue on a bad argument.
int peaks_stream_read(const void* p, size_t bytes, int u, uint32_t* sink, hipStream_t stream)
{
    if (!p || !sink || (reinterpret_cast<uintptr_t>(p) & 15) || (u != 1 && u != 2 && u != 4 && u != 8))
        return hipErrorInvalidValue;
    const size_t per_wg = (size_t)4096 * u;
    if (bytes == 0 || bytes % per_wg != 0 || bytes / per_wg > 0x7FFFFFFFu)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(bytes / per_wg)), block(256);
    const uint4* q = static_cast<const uint4*>(p);
    switch (u) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, grid, block, 0, stream, q, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, stream, q, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, stream, q, sink); break;
    default: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, stream, q, sink); break;
    }
    return hipGetLastError();
}

// Load shape `shape` (0 or 1, see load_shape_kernel) over `rows` rows of a Q4_K
// matrix of 4096 columns at `w` (device, 16-byte aligned; rows a multiple of 4).
// sink: rows / 4 dwords.  Returns hipErrorInvalidValue on a bad argument.
int peaks_load_shape(const void* w, int rows, int shape, uint32_t* sink, hipStream_t stream)
{
    if (!w || !sink || (reinterpret_cast<uintptr_t>(w) & 15) || rows < 4 || rows % 4 || (shape != 0 && shape != 1))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(rows / 4)), block(128);
    const uint8_t* p = static_cast<const uint8_t*>(w);
    if (shape == 0)
        hipLaunchKernelGGL(load_shape_kernel<0>, grid, block, 0, stream, p, sink);
    else
        hipLaunchKernelGGL(load_shape_kernel<1>, grid, block, 0, stream, p, sink);
    return hipGetLastError();
}

// kind 0: int8 MFMA, 8 accumulators; kind 1: f32 outer-product pair MFMA, 4
// accumulators; kind 2: VALU v_fma_f32; kind 3: VALU cvt + fma pairs.  blocks
// workgroups of 256 threads, iters rounds each.  sink: blocks dwords.  clk: null,
// or 2 device uint64 receiving the shader-clock and 100 MHz reference ticks of
// workgroup 0's loop (kinds 0, 2, 3).
int peaks_rate(int kind, int blocks, int iters, uint32_t* sink, uint64_t* clk, hipStream_t stream)
{
    if (!sink || blocks < 1 || iters < 1)
        return hipErrorInvalidValue;
    const dim3 grid(blocks), block(256);
    switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_i8_rate_kernel<8>, grid, block, 0, stream, iters, sink, clk); break;
    case 1: hipLaunchKernelGGL(mfma_outer_rate_kernel<4>, grid, block, 0, stream, iters, 0.5f, sink); break;
    case 2: hipLaunchKernelGGL(valu_rate_kernel<0>, grid, block, 0, stream, iters, 0.5f, sink, clk); break;
    case 3: hipLaunchKernelGGL(valu_rate_kernel<1>, grid, block, 0, stream, iters, 0.5f, sink, clk); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// One VALU instruction form (op 0..9 of valu_instr_kernel), blocks workgroups of
// 256 threads, iters rounds of 128 instructions (op 8: 128 pairs).
int peaks_valu_instr(int op, int blocks, int iters, uint32_t* sink, hipStream_t stream)
{
    if (!sink || blocks < 1 || iters < 1)
        return hipErrorInvalidValue;
    const dim3 grid(blocks), block(256);
    switch (op) {
#define QMM_VI(N) \
    case N: hipLaunchKernelGGL(valu_instr_kernel<N>, grid, block, 0, stream, iters, 0.5f, sink); break;
    QMM_VI(0) QMM_VI(1) QMM_VI(2) QMM_VI(3) QMM_VI(4) QMM_VI(5) QMM_VI(6) QMM_VI(7) QMM_VI(8) QMM_VI(9)
#undef QMM_VI
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// MFMA shadow: nv in {0, 4, 8, 12, 16, 24, 32} VALU per MFMA; parts 3 both, 1 MFMA
// only, 2 VALU only.  blocks workgroups of 256 threads, iters rounds of 8 steps.
int peaks_shadow(int nv, int parts, int blocks, int iters, uint32_t* sink, hipStream_t stream)
{
    if (!sink || blocks < 1 || iters < 1 || parts < 1 || parts > 3)
        return hipErrorInvalidValue;
    const dim3 grid(blocks), block(256);
#define QMM_SH(N)                                                                                            \
    do {                                                                                                     \
        if (parts == 3)                                                                                      \
            hipLaunchKernelGGL((shadow_kernel<N, true, true>), grid, block, 0, stream, iters, 0.5f, sink);   \
        else if (parts == 1)                                                                                 \
            hipLaunchKernelGGL((shadow_kernel<N, true, false>), grid, block, 0, stream, iters, 0.5f, sink);  \
        else                                                                                                 \
            hipLaunchKernelGGL((shadow_kernel<N, false, true>), grid, block, 0, stream, iters, 0.5f, sink);  \
    } while (0)
    switch (nv) {
    case 4: QMM_SH(4); break;
    case 8: QMM_SH(8); break;
    case 12: QMM_SH(12); break;
    case 16: QMM_SH(16); break;
    case 24: QMM_SH(24); break;
    case 32: QMM_SH(32); break;
    default: return hipErrorInvalidValue;
    }
#undef QMM_SH
    return hipGetLastError();
}

// Ping-pong probe: pp 1 (phases alternate between the wave halves) or 0 (serial).
// blocks workgroups of 512 threads, iters rounds (each: one MFMA phase and one
// epilogue phase per wave).
int peaks_pingpong(int pp, int blocks, int iters, uint32_t* sink, hipStream_t stream)
{
    if (!sink || blocks < 1 || iters < 1 || pp < 0 || pp > 1)
        return hipErrorInvalidValue;
    if (pp)
        hipLaunchKernelGGL(pingpong_kernel<1>, dim3(blocks), dim3(512), 0, stream, iters, 0.5f, sink);
    else
        hipLaunchKernelGGL(pingpong_kernel<0>, dim3(blocks), dim3(512), 0, stream, iters, 0.5f, sink);
    return hipGetLastError();
}

// Burst probe: mode 0..5 = (NB, NN) of (1,2) (2,2) (2,1) (4,1) (8,1) (1,1)... see
// peaks_burst_modes; blocks workgroups of 256 threads, iters bursts.
int peaks_burst(int mode, int blocks, int iters, uint32_t* sink, hipStream_t stream)
{
    if (!sink || blocks < 1 || iters < 1)
        return hipErrorInvalidValue;
    const dim3 grid(blocks), block(256);
    switch (mode) {
    case 0: hipLaunchKernelGGL((burst_kernel<1, 2>), grid, block, 0, stream, iters, 0.5f, sink); break;
    case 1: hipLaunchKernelGGL((burst_kernel<2, 2>), grid, block, 0, stream, iters, 0.5f, sink); break;
    case 2: hipLaunchKernelGGL((burst_kernel<2, 1>), grid, block, 0, stream, iters, 0.5f, sink); break;
    case 3: hipLaunchKernelGGL((burst_kernel<4, 1>), grid, block, 0, stream, iters, 0.5f, sink); break;
    case 4: hipLaunchKernelGGL((burst_kernel<8, 1>), grid, block, 0, stream, iters, 0.5f, sink); break;
    case 5: hipLaunchKernelGGL((burst_kernel<4, 2>), grid, block, 0, stream, iters, 0.5f, sink); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// MFMA mix (mode 0..3 of mfma_mix_kernel), blocks workgroups of 256 threads, iters
// rounds of 8 steps.
int peaks_mfma_mix(int mode, int blocks, int iters, uint32_t* sink, hipStream_t stream)
{
    if (!sink || blocks < 1 || iters < 1)
        return hipErrorInvalidValue;
    const dim3 grid(blocks), block(256);
    switch (mode) {
    case 0: hipLaunchKernelGGL(mfma_mix_kernel<0>, grid, block, 0, stream, iters, 0.5f, sink); break;
    case 1: hipLaunchKernelGGL(mfma_mix_kernel<1>, grid, block, 0, stream, iters, 0.5f, sink); break;
    case 2: hipLaunchKernelGGL(mfma_mix_kernel<2>, grid, block, 0, stream, iters, 0.5f, sink); break;
    case 3: hipLaunchKernelGGL(mfma_mix_kernel<3>, grid, block, 0, stream, iters, 0.5f, sink); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// LDS read bandwidth: blocks workgroups of 512 threads (8 waves), iters rounds of 16
// ds_read_b128 per lane.
int peaks_lds_read(int blocks, int iters, uint32_t* sink, hipStream_t stream)
{
    if (!sink || blocks < 1 || iters < 1)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(lds_read_kernel, dim3(blocks), dim3(512), 0, stream, iters, sink);
    return hipGetLastError();
}

// Overlap kernel: nv VALU instructions per MFMA (4, 8 or 16), split 0 or 1, parts
// = 3 (both), 1 (MFMA only) or 2 (VALU only).  blocks workgroups of 512 threads.
int peaks_overlap(int nv, int split, int parts, int blocks, int iters, uint32_t* sink, hipStream_t stream)
{
    if (!sink || blocks < 1 || iters < 1 || parts < 1 || parts > 3 || split < 0 || split > 1)
        return hipErrorInvalidValue;
    const dim3 grid(blocks), block(512);
#define QMM_OVL(NV, S)                                                                                        \
    do {                                                                                                      \
        if (parts == 3)                                                                                       \
            hipLaunchKernelGGL((overlap_kernel<NV, S, true, true>), grid, block, 0, stream, iters, 0.5f, sink);  \
        else if (parts == 1)                                                                                  \
            hipLaunchKernelGGL((overlap_kernel<NV, S, true, false>), grid, block, 0, stream, iters, 0.5f, sink); \
        else                                                                                                  \
            hipLaunchKernelGGL((overlap_kernel<NV, S, false, true>), grid, block, 0, stream, iters, 0.5f, sink); \
    } while (0)
    if (nv == 4) {
        if (split) QMM_OVL(4, 1); else QMM_OVL(4, 0);
    } else if (nv == 8) {
        if (split) QMM_OVL(8, 1); else QMM_OVL(8, 0);
    } else if (nv == 16) {
        if (split) QMM_OVL(16, 1); else QMM_OVL(16, 0);
    } else {
        return hipErrorInvalidValue;
    }
#undef QMM_OVL
    return hipGetLastError();
}

}  // extern "C"
