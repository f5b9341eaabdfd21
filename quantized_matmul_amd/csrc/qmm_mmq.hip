// MMQ: the prefill-side quantized matmul for nt > 8 tokens, on int8 MFMA.
//
// [GEMM, "The GPU path"]: stage each row's raw super-block and the matching
// activation codes in on-chip memory, unpack codes in registers, run one int8
// matrix op per scale group (32 weights for Q4_K, 16 for Q6_K), and take the
// int32 result to f32 with the two scales and, for Q4_K, the min term.
// [MMQ, section 6]: rescale per 32-k chunk as acc += (d*sc)*dx*C - (dmin*m)*s with
// f32 accumulation and a plain f32 store; [MMQ, section 11.4]: codes 0..15 enter
// the integer op uncentred.  [GEMM, "Q4_K: packed in shared memory"]: one LDS
// read of a 16-byte code piece feeds two sub-blocks (low and high nibbles).
// [GEMM, "Prefetching the next super-block"]: the next super-block is read into
// registers while the current one computes, and stored to LDS after the barrier.
//
// MI355X mapping:
//  * Workgroup tile BM = 32*WR rows x BN = 32*WC tokens, one wave per 32 x 32
//    output block.  Workgroups are numbered so that the tiles of one row block
//    land on one XCD (workgroups go round-robin over the 8 XCDs), which keeps a
//    weight tile in one L2.
//  * v_mfma_i32_32x32x32_i8: K = 32 is exactly one Q4_K sub-block.  Operand A =
//    32 weight rows x 32 codes, B = 32 codes x 32 tokens; lane l supplies row/token
//    l%32 and K positions 16*(l/32) .. +15 for both operands (any common K order
//    gives the same dot).  Result lane l: token l%32, rows 8*(i/4)+4*(l/32)+i%4 for
//    accumulator i.  Q6_K groups of 16 use v_mfma_i32_32x32x16_i8 (8 K bytes per lane).
//  * The f32 epilogue is the bottleneck on this chip (one rescale per 32 int8
//    MACs).  Only the per-element work stays on VALU: cvt(C) and one fma with the
//    scale product.  The scale product P = (d*sc)[row] x dx[token] of two
//    sub-blocks comes from one v_mfma_f32_32x32x1_2b_f32 (two outer products), and
//    the min term sum_j (-dmin*m_j)[row] * s_j[token] accumulates in its own
//    accumulator, once per super-block on three bf16 MFMAs over exact three-part
//    splits of both factors (q4_min_term).  Measured on this GPU, MFMA
//    and VALU time of the waves on one SIMD add up rather than overlap (a
//    register-only probe: 4 int8 MFMAs ~130 clocks, 64 independent f32 FMAs
//    ~160, both ~260-285), so the f32 outer products (64 clocks each) are not
//    free: they are cheaper than the 16 VALU multiplies per lane and sub-block
//    they replace.
//    The compute steps are software pipelined (MFMAs, and where registers allow
//    LDS reads, issued a step ahead of the epilogue).
//  * Per super-block: raw code bytes (rows padded so 16-byte LDS reads are
//    conflict-free), decoded per-(row, group) f32 scales, activation codes and
//    activation scales are staged in LDS; the next super-block's global loads are
//    issued before the compute of the current one.
#include <stdlib.h>

#include "qmm_mmq_common.h"

namespace qmm {

// ------------------------------------------------------------------ Q4_K

// v as three bf16 parts p[0] + p[1] + p[2] (bit patterns): each part is the next 8
// significant bits, cut by truncation, and both subtractions are exact, so the sum
// is v exactly for a normal v (a remainder below the normal range loses its bits).
struct Bf16x3 {
    uint16_t p[3];
};

__device__ __forceinline__ Bf16x3 split3_bf16(float v)
{
    const uint32_t u0 = __float_as_uint(v);
    const float r1 = v - __uint_as_float(u0 & 0xFFFF0000u);
    const uint32_t u1 = __float_as_uint(r1);
    const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);
    return {{(uint16_t)(u0 >> 16), (uint16_t)(u1 >> 16), (uint16_t)(__float_as_uint(r2) >> 16)}};
}

// Q5 (Q5_K): also the 32 high-bit bytes of each row (stride 48).
template <int BM, int BN, bool Q5 = false>
struct __attribute__((aligned(16))) Q4Smem {
    static constexpr int QS_STRIDE = 144;   // 128 code bytes + 16 pad
    static constexpr int X_STRIDE = 272;    // 256 activation codes + 16 pad
    static constexpr int H_STRIDE = 48;     // 32 high-bit bytes + 16 pad
    uint8_t qs[BM * QS_STRIDE];
    float wsc[8 * BM];                      // d * sc_j, [j][row]
    uint16_t wmn3[3 * BM * 8];              // -dmin * m_j as three bf16 parts, [part][row][j]
    uint8_t xq[BN * X_STRIDE];
    float xd[8 * BN];                       // activation d, [j][token]
    uint16_t xs3[3 * BN * 8];               // activation s as three bf16 parts, [part][token][j]
    uint8_t qh[Q5 ? BM * H_STRIDE : 0];  // empty without Q5 (a clang extension): the Q4_K layout is unchanged
};

template <int QC, int HC, int XC, int SC, int BC = 1>
struct Q4Offs {
    uint32_t q[QC], h[HC], x[XC], s[SC], b5[BC];
};

// BC: high-bit chunk tasks (Q5_K only; two 16-byte chunks per row)
template <int BM, int BN, int NTH, int QC, int HC, int XC, int SC, bool Q5 = false, int BC = 1>
__device__ __forceinline__ void q4_offsets(Q4Offs<QC, HC, XC, SC, BC>& o, int tid, int row0, int tok0, int nt,
                                           int od, int id, int nblk, uint32_t row_bytes)
{
#pragma unroll
    for (int k = 0; k < QC; ++k) {
        const int e = task<BM * 8, NTH, QC>(tid + k * NTH);
        const uint32_t r = (uint32_t)(min(row0 + (e >> 3), od - 1) - row0);
        o.q[k] = r * row_bytes + (Q5 ? 48 : 16) + 16 * (e & 7);
    }
    if constexpr (Q5) {
#pragma unroll
        for (int k = 0; k < BC; ++k) {
            const int e = task<BM * 2, NTH, BC>(tid + k * NTH);
            o.b5[k] = (uint32_t)(min(row0 + (e >> 1), od - 1) - row0) * row_bytes + 16 + 16 * (e & 1);
        }
    }
#pragma unroll
    for (int k = 0; k < HC; ++k) {
        const int e = task<BM * 4, NTH, HC>(tid + k * NTH);
        o.h[k] = (uint32_t)(min(row0 + (e >> 2), od - 1) - row0) * row_bytes;
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {
        const int e = task<BN * 16, NTH, XC>(tid + k * NTH);
        o.x[k] = (uint32_t)(min(tok0 + (e >> 4), nt - 1) - tok0) * (uint32_t)id + 16 * (e & 15);
    }
#pragma unroll
    for (int k = 0; k < SC; ++k) {
        const int e = task<BN * 2, NTH, SC>(tid + k * NTH);
        const uint32_t t = (uint32_t)(min(tok0 + (e >> 1), nt - 1) - tok0);
        o.s[k] = (t * (uint32_t)nblk + 4 * (e & 1)) * 4;
    }
}

// Resources of one tile: weights from row0, activation codes / d / s from tok0.
struct Q4Rsrc {
    __amdgpu_buffer_rsrc_t w, x, d, s;
};

template <int QC, int HC, int XC, int SC, bool Q5 = false, int BC = 1>
__device__ __forceinline__ void q4_prefetch(v4i (&pq)[QC], v4i (&ph)[HC], v4i (&px)[XC], v4i (&pd)[SC], v4i (&ps)[SC],
                                            const Q4Offs<QC, HC, XC, SC, BC>& o, const Q4Rsrc& rs, int sb,
                                            v4i* pb5 = nullptr)
{
    const uint32_t ow = (uint32_t)sb * (Q5 ? kQ5KBytes : kQ4KBytes), ox = 256u * (uint32_t)sb,
                   os = 32u * (uint32_t)sb;
    if constexpr (Q5) {
#pragma unroll
        for (int k = 0; k < BC; ++k)
            pb5[k] = bload16(rs.w, o.b5[k], ow);
    }
#pragma unroll
    for (int k = 0; k < QC; ++k)
        pq[k] = bload16(rs.w, o.q[k], ow);
#pragma unroll
    for (int k = 0; k < HC; ++k)
        ph[k] = bload16(rs.w, o.h[k], ow);
#pragma unroll
    for (int k = 0; k < XC; ++k)
        px[k] = bload16(rs.x, o.x[k], ox);
#pragma unroll
    for (int k = 0; k < SC; ++k) {
        pd[k] = bload16(rs.d, o.s[k], os);
        ps[k] = bload16(rs.s, o.s[k], os);
    }
}

// valid == false (a super-block index past the end, in a split over K) stages
// zero scales: that super-block then adds nothing, with no branch.
template <int BM, int BN, int NTH, int QC, int HC, int XC, int SC, bool Q5 = false, int BC = 1>
__device__ __forceinline__ void q4_stage(Q4Smem<BM, BN, Q5>& sm, const v4i (&pq)[QC], const v4i (&ph)[HC],
                                         const v4i (&px)[XC], const v4i (&pd)[SC], const v4i (&ps)[SC], int tid,
                                         bool valid, const v4i* pb5 = nullptr)
{
    using SM = Q4Smem<BM, BN, Q5>;
    if constexpr (Q5) {
#pragma unroll
        for (int k = 0; k < BC; ++k) {
            const int e = task<BM * 2, NTH, BC>(tid + k * NTH);
            *reinterpret_cast<v4i*>(&sm.qh[(e >> 1) * SM::H_STRIDE + 16 * (e & 1)]) = pb5[k];
        }
    }
#pragma unroll
    for (int k = 0; k < QC; ++k) {
        const int e = task<BM * 8, NTH, QC>(tid + k * NTH);
        *reinterpret_cast<v4i*>(&sm.qs[(e >> 3) * SM::QS_STRIDE + 16 * (e & 7)]) = pq[k];
    }
#pragma unroll
    for (int k = 0; k < HC; ++k) {
        const int e = task<BM * 4, NTH, HC>(tid + k * NTH);
        // task (r, jj) decodes sub-blocks jj and jj + 4 of row r
        const int r = e >> 2, jj = e & 3;
        const v4i h = ph[k];
        const float dw = f16_bits_to_f32((uint32_t)h.x & 0xFFFF);
        const float dm = f16_bits_to_f32((uint32_t)h.x >> 16);
        int sc0, m0, sc1, m1;
        q4k_scale_min_pair((uint32_t)h.y, (uint32_t)h.z, (uint32_t)h.w, jj, sc0, m0, sc1, m1);
        sm.wsc[jj * BM + r] = valid ? dw * (float)sc0 : 0.f;
        sm.wsc[(jj + 4) * BM + r] = valid ? dw * (float)sc1 : 0.f;
        const Bf16x3 mn0 = split3_bf16(valid ? -(dm * (float)m0) : 0.f);
        const Bf16x3 mn1 = split3_bf16(valid ? -(dm * (float)m1) : 0.f);
#pragma unroll
        for (int pt = 0; pt < 3; ++pt) {
            sm.wmn3[(pt * BM + r) * 8 + jj] = mn0.p[pt];
            sm.wmn3[(pt * BM + r) * 8 + jj + 4] = mn1.p[pt];
        }
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {
        const int e = task<BN * 16, NTH, XC>(tid + k * NTH);
        *reinterpret_cast<v4i*>(&sm.xq[(e >> 4) * SM::X_STRIDE + 16 * (e & 15)]) = px[k];
    }
#pragma unroll
    for (int k = 0; k < SC; ++k) {
        const int e = task<BN * 2, NTH, SC>(tid + k * NTH);
        const int t = e >> 1, hf = e & 1;
        // __int_as_float per element: __builtin_bit_cast of an ext-vector
        // element is lowered as a cast of element 0 by this compiler.
        sm.xd[(4 * hf + 0) * BN + t] = __int_as_float(pd[k].x);
        sm.xd[(4 * hf + 1) * BN + t] = __int_as_float(pd[k].y);
        sm.xd[(4 * hf + 2) * BN + t] = __int_as_float(pd[k].z);
        sm.xd[(4 * hf + 3) * BN + t] = __int_as_float(pd[k].w);
        const Bf16x3 s0 = split3_bf16(__int_as_float(ps[k].x)), s1 = split3_bf16(__int_as_float(ps[k].y));
        const Bf16x3 s2 = split3_bf16(__int_as_float(ps[k].z)), s3 = split3_bf16(__int_as_float(ps[k].w));
#pragma unroll
        for (int pt = 0; pt < 3; ++pt) {
            // sub-blocks 4 hf .. 4 hf + 3 of token t: 8 contiguous bytes per part
            const uint2 v = make_uint2((uint32_t)s0.p[pt] | ((uint32_t)s1.p[pt] << 16),
                                       (uint32_t)s2.p[pt] | ((uint32_t)s3.p[pt] << 16));
            *reinterpret_cast<uint2*>(&sm.xs3[(pt * BN + t) * 8 + 4 * hf]) = v;
        }
    }

}

// The LDS operands of one compute step (sub-blocks 2p and 2p + 1): this lane's 16
// code bytes (row arow), its two 16-byte activation pieces (token btok), and the
// scale factors of sub-block 2p + lh for the outer products.
struct Q4Ops {
    v4i a16, b0, b1;
    float wsc, xd;
};

// The same for the kernels whose two steps' codes come as separate pieces (Q6_K:
// 8 bytes per lane and group; Q4_0 / Q8_0: 16 bytes) with one scale product.
template <typename T>
struct StepOps {
    T a0, a1, b0, b1;
    float ws, xd;
};
using Ops8 = StepOps<long>;
using Ops16 = StepOps<v4i>;

template <int BM, int BN, bool Q5>
__device__ __forceinline__ Q4Ops q4_load(const Q4Smem<BM, BN, Q5>& sm, int p, int arow, int btok, int lh)
{
    using SM = Q4Smem<BM, BN, Q5>;
    Q4Ops o;
    o.a16 = *reinterpret_cast<const v4i*>(&sm.qs[arow * SM::QS_STRIDE + 32 * p + 16 * lh]);
    o.b0 = *reinterpret_cast<const v4i*>(&sm.xq[btok * SM::X_STRIDE + 64 * p + 16 * lh]);
    o.b1 = *reinterpret_cast<const v4i*>(&sm.xq[btok * SM::X_STRIDE + 64 * p + 32 + 16 * lh]);
    const int j = 2 * p + lh;
    o.wsc = sm.wsc[j * BM + arow];
    o.xd = sm.xd[j * BN + btok];
    return o;
}

// The A operands of sub-blocks 2p and 2p + 1 from one 16-byte code piece (low and
// high nibbles); Q5_K adds bit 2p / 2p + 1 of the row's high-bit bytes h16 as the
// fifth code bit.
template <bool Q5>
__device__ __forceinline__ void q4_unpack(const v4i& a16, const v4i& h16, int p, v4i& a0, v4i& a1)
{
    a0 = a16 & 0x0F0F0F0F;
    a1 = (a16 >> 4) & 0x0F0F0F0F;
    if constexpr (Q5) {
        a0 |= ((h16 >> (2 * p)) & 0x01010101) << 4;
        a1 |= ((h16 >> (2 * p + 1)) & 0x01010101) << 4;
    }
}

// One compute step from loaded operands: C0 / C1 the two int8 tile products, P
// their scale products (d*sc)[row] x dx[token] from one outer-product pair.  h16:
// the row's high-bit bytes (Q5_K).
template <bool Q5>
__device__ __forceinline__ void q4_mma(const Q4Ops& o, int p, const v4i& h16, v16i& C0, v16i& C1, v32f& P)
{
    v4i a0, a1;
    q4_unpack<Q5>(o.a16, h16, p, a0, a1);
    C0 = mfma_i8_k32(a0, o.b0);
    C1 = mfma_i8_k32(a1, o.b1);
    P = mfma_outer2(o.wsc, o.xd);
}

// NS compute steps of one staged super-block: load(p) reads a step's operands from
// LDS, mma(ops, p, C0, C1, P) issues its MFMAs, and the f32 epilogue adds
// cvt(C) * P into accv (two scale groups per step: P registers 0..15 and 16..31).
// PIPE 0: each step in turn.  PIPE 1: the MFMAs of step p + 1 are issued before the
// epilogue of step p (one more step of results, 64 registers).  PIPE 2: the LDS
// reads of step p + 2 are issued there too, so their latency is covered by a step
// of work instead of stalling the next MFMA (one more step of operands; measured
// 4-6 % faster than PIPE 1 on 512-token Q4_K shapes).  Each kernel takes the
// highest mode that does not spill.
enum { kPipeNone = 0, kPipeMfma = 1, kPipeLds = 2 };

template <int NS, int PIPE, typename Ops, typename Load, typename Mma>
__device__ __forceinline__ void pipelined_steps(const Load& load, const Mma& mma, v16f& accv)
{
    const auto epilogue = [&](const v16i& C0, const v16i& C1, const v32f& P) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            accv[i] = fmaf((float)C0[i], P[i], accv[i]);
            accv[i] = fmaf((float)C1[i], P[16 + i], accv[i]);
        }
    };
    if constexpr (PIPE == kPipeNone) {
#pragma unroll 2
        for (int p = 0; p < NS; ++p) {
            v16i C0, C1;
            v32f P;
            mma(load(p), p, C0, C1, P);
            epilogue(C0, C1, P);
            // one step's results at a time
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        constexpr bool AHEAD = PIPE == kPipeLds;
        Ops o2 = load(0);
        v16i Ca0, Ca1;
        v32f Pa;
        mma(o2, 0, Ca0, Ca1, Pa);
        if constexpr (AHEAD)
            o2 = load(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < NS; ++p) {
            // with AHEAD, o2 holds step p + 1's operands and step p + 2's are loaded here
            Ops o3 = o2;
            if (AHEAD && p + 2 < NS)
                o3 = load(p + 2);
            if (!AHEAD && p + 1 < NS)
                o2 = load(p + 1);
            v16i Cb0, Cb1;
            v32f Pb;
            if (p + 1 < NS)
                mma(o2, p + 1, Cb0, Cb1, Pb);
            __builtin_amdgcn_sched_barrier(0);
            epilogue(Ca0, Ca1, Pa);
            __builtin_amdgcn_sched_barrier(0);
            if (p + 1 < NS) {
                Ca0 = Cb0;
                Ca1 = Cb1;
                Pa = Pb;
                if constexpr (AHEAD)
                    o2 = o3;
            }
        }
    }
}

// The min term of one staged super-block, sum_j (-dmin*m_j)[row] * s_j[token] over
// its 8 sub-blocks, added into accm on the bf16 MFMA: both factors are staged as
// three bf16 parts (a = a1 + a2 + a3 exactly), and the six part products whose
// size is above 2^-24 of a*s, (1,1) (1,2) (2,1) (1,3) (2,2) (3,1), are the K = 48
// entries of three v_mfma_f32_32x32x16_bf16 (K index 8 q + j for part pair q and
// sub-block j; a lane's 8 entries are one part of one row or token across the 8
// sub-blocks: one 16-byte LDS read).  Each part product is exact in f32; the f32
// MFMA it replaces cost 64 clocks per two sub-blocks, these three about 100 per
// eight.
template <int BM, int BN, bool Q5>
__device__ __forceinline__ void q4_min_term(const Q4Smem<BM, BN, Q5>& sm, int arow, int btok, int lh, v16f& accm)
{
    // part of the row / token factor for part pair q = 2 m + lh
    constexpr int kRowPart[6] = {0, 0, 1, 0, 1, 2};
    constexpr int kTokPart[6] = {0, 1, 0, 2, 1, 0};
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int q = 2 * m + lh;
        const v8bf a = *reinterpret_cast<const v8bf*>(&sm.wmn3[(kRowPart[q] * BM + arow) * 8]);
        const v8bf b = *reinterpret_cast<const v8bf*>(&sm.xs3[(kTokPart[q] * BN + btok) * 8]);
        accm = mfma_bf16_k16(a, b, accm);
    }
}

// The four steps (sub-blocks 2p, 2p + 1) of one staged Q4_K / Q5_K super-block.
template <int BM, int BN, bool Q5, int PIPE>
__device__ __forceinline__ void q4_superblock(const Q4Smem<BM, BN, Q5>& sm, int arow, int btok, int lh, v16f& accv,
                                              v16f& accm)
{
    using SM = Q4Smem<BM, BN, Q5>;
    v4i h16 = {};
    if constexpr (Q5)
        h16 = *reinterpret_cast<const v4i*>(&sm.qh[arow * SM::H_STRIDE + 16 * lh]);
    q4_min_term<BM, BN, Q5>(sm, arow, btok, lh, accm);
    pipelined_steps<4, PIPE, Q4Ops>(
        [&](int p) { return q4_load<BM, BN, Q5>(sm, p, arow, btok, lh); },
        [&](const Q4Ops& o, int p, v16i& C0, v16i& C1, v32f& P) { q4_mma<Q5>(o, p, h16, C0, C1, P); }, accv);
}

// KS > 1 splits K inside the workgroup: KS groups of WR x WC waves, each with its
// own double-buffered LDS tiles, take super-blocks kg, kg + KS, kg + 2 KS, ...;
// at the end groups 1 .. KS-1 hand their 32 x 32 partial sums to group 0 through
// LDS, which adds them in group order (a fixed order: the result does not
// depend on timing).  It gives a tile grid with few tiles more waves.
template <int WR, int WC, int KS, bool DUMP, bool Q5>
__device__ __forceinline__ void mmq_k4_body(const uint8_t* __restrict__ W, const int8_t* __restrict__ q,
                                            const float* __restrict__ dx, const float* __restrict__ sx,
                                            float* __restrict__ out, int nt, int od, int id,
                                            int32_t* __restrict__ S)
{
    constexpr int BM = 32 * WR, BN = 32 * WC, NTH = 64 * WR * WC;   // NTH: threads of one K group
    constexpr int QC = (BM * 8 + NTH - 1) / NTH;   // code chunks per thread
    constexpr int HC = (BM * 4 + NTH - 1) / NTH;   // header tasks per thread
    constexpr int XC = (BN * 16 + NTH - 1) / NTH;  // activation chunks per thread
    constexpr int SC = (BN * 2 + NTH - 1) / NTH;   // activation (d, s) float4 pairs per thread
    constexpr int BC = (BM * 2 + NTH - 1) / NTH;   // high-bit chunks per thread (Q5_K)
    using SM = Q4Smem<BM, BN, Q5>;
    __shared__ SM smb[KS][2];
    static_assert(!DUMP || KS == 1, "the debug dump runs unsplit");
    static_assert((KS - 1) * WR * WC * 1024 * sizeof(float) <= sizeof(smb), "reduction scratch fits the tiles");

    const int ntb = (nt + BN - 1) / BN;
    const int tile = xcd_tile(ntb * ((od + BM - 1) / BM));
    if (tile < 0)
        return;  // whole workgroup
    const int row0 = (tile / ntb) * BM, tok0 = (tile % ntb) * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // K group and wave in group (a compile-time 0 without a split)
    const int kg = KS > 1 ? wave / (WR * WC) : 0, gw = wave - kg * (WR * WC);
    const int tid = threadIdx.x - kg * NTH;                           // thread in group
    const int wr = gw / WC, wc = gw % WC;
    const int li = lane & 31, lh = lane >> 5;
    const int nsb = id >> 8;
    const int nblk = id >> 5;
    const int niter = (nsb + KS - 1) / KS;
    const uint32_t row_bytes = (uint32_t)nsb * (Q5 ? kQ5KBytes : kQ4KBytes);

    // ---- prefetch registers (one super-block), per-thread offsets, resources
    v4i pq[QC], ph[HC], px[XC], pd[SC], ps[SC], pb5[BC];
    Q4Offs<QC, HC, XC, SC, BC> offs;
    q4_offsets<BM, BN, NTH, QC, HC, XC, SC, Q5, BC>(offs, tid, row0, tok0, nt, od, id, nblk, row_bytes);
    Q4Rsrc rs;
    rs.w = buffer_rsrc(W + (size_t)row0 * row_bytes, (size_t)(od - row0) * row_bytes);
    rs.x = buffer_rsrc(q + (size_t)tok0 * id, (size_t)(nt - tok0) * id);
    rs.d = buffer_rsrc(dx + (size_t)tok0 * nblk, (size_t)(nt - tok0) * nblk * 4);
    rs.s = buffer_rsrc(sx + (size_t)tok0 * nblk, (size_t)(nt - tok0) * nblk * 4);
    auto prefetch = [&](int sbi) { q4_prefetch<QC, HC, XC, SC, Q5, BC>(pq, ph, px, pd, ps, offs, rs, sbi, pb5); };
    v16f accv = {}, accm = {};
    const int arow = wr * 32 + li;   // this lane's row as an A operand
    const int btok = wc * 32 + li;   // this lane's token as a B operand

    // Two LDS buffers per K group: iteration i computes from smb[kg][i & 1] while
    // the next super-block, already in registers, is stored into the other buffer
    // and the loads of the one after are issued; one barrier per iteration.
    // Prefetches are unconditional (index clamped to the last super-block, an L2
    // re-read at the end): a prefetch under a branch merges register values and
    // costs spills.
    prefetch(min(kg, nsb - 1));
    q4_stage<BM, BN, NTH, QC, HC, XC, SC, Q5, BC>(smb[kg][0], pq, ph, px, pd, ps, tid, kg < nsb, pb5);
    prefetch(min(KS + kg, nsb - 1));
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
        const SM& sm = smb[kg][it & 1];
        const int sb = it * KS + kg;
        if constexpr (DUMP) {
            // integer products only, written out per sub-block
            v4i h16 = {};
            if constexpr (Q5)
                h16 = *reinterpret_cast<const v4i*>(&sm.qh[arow * SM::H_STRIDE + 16 * lh]);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const Q4Ops o = q4_load<BM, BN, Q5>(sm, p, arow, btok, lh);
                v4i a0, a1;
                q4_unpack<Q5>(o.a16, h16, p, a0, a1);
                const v16i C0 = mfma_i8_k32(a0, o.b0);
                const v16i C1 = mfma_i8_k32(a1, o.b1);
                const int tg = tok0 + btok;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rg = row0 + wr * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                    if (tg < nt && rg < od) {
                        int32_t* dst = S + (((size_t)tg * od + rg) * nsb + sb) * 8 + 2 * p;
                        dst[0] = C0[i];
                        dst[1] = C1[i];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            q4_superblock<BM, BN, Q5, (Q5 && KS > 1) ? kPipeMfma : kPipeLds>(sm, arow, btok, lh, accv, accm);
        }
        // keep the staging of the next super-block after the compute (moved into
        // it, its values would be live across the whole compute phase)
        __builtin_amdgcn_sched_barrier(0);
        // smb[kg][(it + 1) & 1] was last read in iteration it - 1, before the
        // barrier; after the last iteration this fills a buffer nobody reads
        q4_stage<BM, BN, NTH, QC, HC, XC, SC, Q5, BC>(smb[kg][(it + 1) & 1], pq, ph, px, pd, ps, tid, sb + KS < nsb,
                                                      pb5);
        prefetch(min(sb + 2 * KS, nsb - 1));
        __syncthreads();
    }

    if constexpr (!DUMP) {
        v16f v = accv + accm;
        if (!combine_k_groups<WR * WC, KS>(v, reinterpret_cast<float*>(&smb[0][0]), kg, gw, lane))
            return;
        store_tile(v, out, nt, od, tok0 + btok, row0 + wr * 32, lh);
    }
}

template <int WR, int WC, int KS, bool DUMP>
__global__ __launch_bounds__(64 * WR * WC * KS, 2) void mmq_q4k_kernel(const uint8_t* __restrict__ W,
                                                                    const int8_t* __restrict__ q,
                                                                    const float* __restrict__ dx,
                                                                    const float* __restrict__ sx,
                                                                    float* __restrict__ out, int nt, int od,
                                                                    int id, int32_t* __restrict__ S)
{
    mmq_k4_body<WR, WC, KS, DUMP, false>(W, q, dx, sx, out, nt, od, id, S);
}

// Q5_K (176-byte blocks): the Q4_K kernel with the fifth code bit from the staged
// high-bit bytes.
template <int WR, int WC, int KS, bool DUMP>
__global__ __launch_bounds__(64 * WR * WC * KS, 2) void mmq_q5k_kernel(const uint8_t* __restrict__ W,
                                                                    const int8_t* __restrict__ q,
                                                                    const float* __restrict__ dx,
                                                                    const float* __restrict__ sx,
                                                                    float* __restrict__ out, int nt, int od,
                                                                    int id, int32_t* __restrict__ S)
{
    mmq_k4_body<WR, WC, KS, DUMP, true>(W, q, dx, sx, out, nt, od, id, S);
}

// ------------------------------------------------------------------ Q4_K stream-K
// The work of a launch is ntiles x nsb units (one tile, one super-block), numbered
// tile-major, and cut into G equal contiguous ranges, one per workgroup
// ([MMQ, section 12.3] on tile counts that do not fill the chip; the pages flag
// non-deterministic split reductions, so the combine here has a fixed order).  A
// workgroup walks its range tile segment by tile segment with the per-tile
// kernel's pipeline; a tile it covers whole is stored directly, a partial tile goes
// to its slot in the workspace (slot 0: the first tile of its range, 1: the last).
// The fixup kernel then adds, for every split tile, the partials of the
// workgroups covering it in workgroup order and stores the sum.  Workgroups are
// numbered so that those on one XCD take consecutive ranges (one row block's tiles
// stay in one L2).  G is a multiple of 8.
__host__ __device__ inline long sk_first_unit(int g, long units, int G) { return (long)g * units / G; }

template <int WR, int WC>
__global__ __launch_bounds__(64 * WR * WC, 2) void mmq_q4k_streamk_kernel(const uint8_t* __restrict__ W,
                                                                         const int8_t* __restrict__ q,
                                                                         const float* __restrict__ dx,
                                                                         const float* __restrict__ sx,
                                                                         float* __restrict__ out, int nt, int od,
                                                                         int id, float* __restrict__ ws, int G)
{
    constexpr int BM = 32 * WR, BN = 32 * WC, NTH = 64 * WR * WC, NW = WR * WC;
    constexpr int QC = (BM * 8 + NTH - 1) / NTH;
    constexpr int HC = (BM * 4 + NTH - 1) / NTH;
    constexpr int XC = (BN * 16 + NTH - 1) / NTH;
    constexpr int SC = (BN * 2 + NTH - 1) / NTH;
    using SM = Q4Smem<BM, BN>;
    __shared__ SM smb[2];

    const int ntb = (nt + BN - 1) / BN;
    const int ntiles = ntb * ((od + BM - 1) / BM);
    const int nsb = id >> 8, nblk = id >> 5;
    const long units = (long)ntiles * nsb;
    const int g = (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
    const long u0 = sk_first_unit(g, units, G), u1 = sk_first_unit(g + 1, units, G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / WC, wc = wave % WC;
    const int li = lane & 31, lh = lane >> 5;
    const uint32_t row_bytes = (uint32_t)nsb * kQ4KBytes;
    const int arow = wr * 32 + li, btok = wc * 32 + li;
    const int first_tile = (int)(u0 / nsb);

    for (long u = u0; u < u1;) {
        const int tile = (int)(u / nsb);
        const int k0 = (int)(u - (long)tile * nsb);
        const int k1 = (int)min((long)nsb, k0 + (u1 - u));
        const int row0 = (tile / ntb) * BM, tok0 = (tile % ntb) * BN;

        v4i pq[QC], ph[HC], px[XC], pd[SC], ps[SC];
        Q4Offs<QC, HC, XC, SC> offs;
        q4_offsets<BM, BN, NTH, QC, HC, XC, SC>(offs, tid, row0, tok0, nt, od, id, nblk, row_bytes);
        Q4Rsrc rs;
        rs.w = buffer_rsrc(W + (size_t)row0 * row_bytes, (size_t)(od - row0) * row_bytes);
        rs.x = buffer_rsrc(q + (size_t)tok0 * id, (size_t)(nt - tok0) * id);
        rs.d = buffer_rsrc(dx + (size_t)tok0 * nblk, (size_t)(nt - tok0) * nblk * 4);
        rs.s = buffer_rsrc(sx + (size_t)tok0 * nblk, (size_t)(nt - tok0) * nblk * 4);
        auto prefetch = [&](int sbi) { q4_prefetch<QC, HC, XC, SC>(pq, ph, px, pd, ps, offs, rs, sbi); };
        v16f accv = {}, accm = {};

        prefetch(k0);
        q4_stage<BM, BN, NTH, QC, HC, XC, SC>(smb[0], pq, ph, px, pd, ps, tid, true);
        prefetch(min(k0 + 1, k1 - 1));
        __syncthreads();
        for (int sb = k0; sb < k1; ++sb) {
            const SM& sm = smb[(sb - k0) & 1];
            q4_superblock<BM, BN, false, kPipeMfma>(sm, arow, btok, lh, accv, accm);
            __builtin_amdgcn_sched_barrier(0);
            q4_stage<BM, BN, NTH, QC, HC, XC, SC>(smb[(sb - k0 + 1) & 1], pq, ph, px, pd, ps, tid, sb + 1 < k1);
            prefetch(min(sb + 2, k1 - 1));
            __syncthreads();
        }
        const v16f v = accv + accm;
        if (k0 == 0 && k1 == nsb) {
            store_tile(v, out, nt, od, tok0 + btok, row0 + wr * 32, lh);
        } else {
            float* slot = ws + ((size_t)(2 * g + (tile == first_tile ? 0 : 1)) * NW + wave) * 1024;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                slot[i * 64 + lane] = v[i];
        }
        u += k1 - k0;
    }
}

// One single-wave workgroup per (range boundary b = 1 .. G-1, 32 x 32 block of the
// tile): a boundary inside a tile splits it; the first boundary inside a tile adds,
// block by block, the partials of the workgroups covering the tile in workgroup
// order and stores the sum (a tile one workgroup covered whole was stored by that
// workgroup).  Single waves spread the sums over all CUs; up to four partials per
// wave are in flight at once.  G is a compile-time constant, so the range
// boundaries cost a shift, not a 64-bit division.
template <int WR, int WC, int G>
__global__ __launch_bounds__(64) void mmq_streamk_fixup_kernel(const float* __restrict__ ws, float* __restrict__ out,
                                                               int nt, int od, int nsb)
{
    constexpr int BM = 32 * WR, BN = 32 * WC, NW = WR * WC, PF = 4;
    const int ntb = (nt + BN - 1) / BN;
    const int ntiles = ntb * ((od + BM - 1) / BM);
    const long units = (long)ntiles * nsb;
    const int b = (int)(blockIdx.x / NW) + 1, wave = (int)(blockIdx.x % NW);
    const long ub = sk_first_unit(b, units, G);
    if (b >= G || ub >= units || ub % nsb == 0)
        return;  // not a boundary inside a tile
    const int tile = (int)(ub / nsb);
    const long t0 = (long)tile * nsb, t1 = t0 + nsb;
    long f = sk_first_unit(b - 1, units, G);
    if (f > t0)
        return;  // an earlier boundary inside this tile does the sum
    // workgroups b-1, b, ... cover the tile (b-1 holds its first unit); a covering
    // workgroup keeps the tile in slot 0 when its range starts inside the tile (its
    // first tile), else in slot 1 (its last)
    const int lane = threadIdx.x;
    v16f v = {};
    for (int gg = b - 1; gg < G && f < t1; gg += PF) {
        long fs[PF + 1];
        fs[0] = f;
#pragma unroll
        for (int k = 1; k <= PF; ++k)
            fs[k] = gg + k <= G ? sk_first_unit(gg + k, units, G) : units;
        float a[PF][16];
        bool used[PF];
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            // gg + k covers part of the tile with a non-empty range; an unused read
            // takes workgroup b-1's slot (inside the workspace) and is not added
            used[k] = gg + k < G && fs[k] < t1 && fs[k + 1] > fs[k];
            const float* src =
                ws + ((size_t)(2 * (used[k] ? gg + k : b - 1) + (used[k] && fs[k] < t0 ? 1 : 0)) * NW + wave) * 1024;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                a[k][i] = src[i * 64 + lane];
        }
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            if (used[k]) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    v[i] += a[k][i];
            }
        }
        f = fs[PF];
    }
    const int wr = wave / WC, wc = wave % WC;
    store_tile(v, out, nt, od, (tile % ntb) * BN + wc * 32 + (lane & 31), (tile / ntb) * BM + wr * 32, lane >> 5);
}

// ------------------------------------------------------------------ Q6_K
// Groups of 16 weights: v_mfma_i32_32x32x16_i8 (lane l: row/token l%32, K bytes
// 8*(l/32) .. +7).  Codes are rebuilt and centred at staging time into signed
// bytes in LDS ([MMQ, section 4, Q6_K specialization]: centre at load), so the
// MFMA operands are plain 8-byte LDS reads.  Rescale per group:
// acc += (d*sc_g) * dx * C, dx the scale of the 32-block holding group g; the two
// groups of a 32-block share dx, so one outer-product MFMA gives both products.
template <int BM, int BN>
struct __attribute__((aligned(16))) Q6Smem {
    static constexpr int W_STRIDE = 272;    // 256 centred codes + 16 pad
    static constexpr int X_STRIDE = 272;
    int8_t wq[BM * W_STRIDE];
    float wsc[16 * BM];                     // d * sc_g, [g][row]
    uint8_t xq[BN * X_STRIDE];
    float xd[8 * BN];
};

template <int BM, int BN, int NTH, int WC8, int XC, int SC, bool PAD>
__device__ __forceinline__ void q6_prefetch(uint32_t (&pl)[WC8][5], uint32_t (&phh)[WC8][5], uint32_t (&pshift)[WC8],
                                            v4i (&px)[XC], v4i (&ps)[SC], uint32_t (&psd)[WC8],
                                            const uint8_t* __restrict__ W, const int8_t* __restrict__ q,
                                            const float* __restrict__ dx, int sb, int tid, int row0, int tok0, int nt,
                                            int od, int id, int nblk, size_t row_bytes)
{
    // unconditional loads, as for Q4_K: clamped task, row and token indices.  The
    // weight part is q6_prefetch_task (and q6_stage's code part q6_stage_codes)
    // written out: calling the shared helpers here moves these kernels' register
    // allocation into spills at 256 VGPRs.
#pragma unroll
    for (int k = 0; k < WC8; ++k) {
        const int e = task<BM * 8, NTH, WC8>(tid + k * NTH);
        const int r = e >> 3, c = e & 7;
        const int h = c >> 2, jq = (c >> 1) & 1, half = c & 1;
        const uint8_t* blk =
            W + (size_t)min(row0 + r, od - 1) * row_bytes + (size_t)sb * (PAD ? kQ6KP224Bytes : kQ6KBytes);
        const uintptr_t al = reinterpret_cast<uintptr_t>(blk + 64 * h + 32 * jq + 16 * half);
        const uintptr_t ah = reinterpret_cast<uintptr_t>(blk + 128 + 32 * h + 16 * half);
        if constexpr (PAD) {
            // 224-byte blocks: both chunks are 16-byte aligned, one load each
            const uint4 l4 = *reinterpret_cast<const uint4*>(al), h4 = *reinterpret_cast<const uint4*>(ah);
            pl[k][0] = l4.x, pl[k][1] = l4.y, pl[k][2] = l4.z, pl[k][3] = l4.w, pl[k][4] = 0;
            phh[k][0] = h4.x, phh[k][1] = h4.y, phh[k][2] = h4.z, phh[k][3] = h4.w, phh[k][4] = 0;
            pshift[k] = 0;
        } else {
            const uint32_t* wl = reinterpret_cast<const uint32_t*>(al & ~(uintptr_t)3);
            const uint32_t* wh = reinterpret_cast<const uint32_t*>(ah & ~(uintptr_t)3);
            pshift[k] = (uint32_t)(al & 3);  // same for both chunks
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                pl[k][i] = wl[i];
                phh[k][i] = wh[i];
            }
        }
        // task c also stages group scales 2c and 2c+1 (two bytes, 2-byte aligned)
        // and reads d: low half the two int8 scales, high half the f16 d
        const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(blk + 192 + 2 * c);
        const uint32_t d16 = *reinterpret_cast<const uint16_t*>(blk + 208);
        psd[k] = sc2 | (d16 << 16);
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {
        const int e = task<BN * 16, NTH, XC>(tid + k * NTH);
        const int t = min(tok0 + (e >> 4), nt - 1), ch = e & 15;
        px[k] = *reinterpret_cast<const v4i*>(q + (size_t)t * id + 256 * sb + 16 * ch);
    }
#pragma unroll
    for (int k = 0; k < SC; ++k) {
        const int e = task<BN * 2, NTH, SC>(tid + k * NTH);
        const int t = min(tok0 + (e >> 1), nt - 1), hf = e & 1;
        ps[k] = *reinterpret_cast<const v4i*>(dx + (size_t)t * nblk + 8 * sb + 4 * hf);
    }
}

template <int BM, int BN, int NTH, int WC8, int XC, int SC>
__device__ __forceinline__ void q6_stage(Q6Smem<BM, BN>& sm, const uint32_t (&pl)[WC8][5], const uint32_t (&phh)[WC8][5],
                                         const uint32_t (&pshift)[WC8], const v4i (&px)[XC], const v4i (&ps)[SC],
                                         const uint32_t (&psd)[WC8], int tid, bool valid)
{
    using SM = Q6Smem<BM, BN>;
#pragma unroll
    for (int k = 0; k < WC8; ++k) {
        const int e = task<BM * 8, NTH, WC8>(tid + k * NTH);
        const int r = e >> 3, c = e & 7;
        const int h = c >> 2, jq = (c >> 1) & 1, half = c & 1;
        const uint32_t sh = pshift[k];
        uint32_t L[4], H[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            L[i] = __builtin_amdgcn_alignbyte(pl[k][i + 1], pl[k][i], sh);
            H[i] = __builtin_amdgcn_alignbyte(phh[k][i + 1], phh[k][i], sh);
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
        // element index of the low-nibble piece: 128h + 32jq + 16half; high: +64
        const int e1 = 128 * h + 32 * jq + 16 * half;
        *reinterpret_cast<int4*>(&sm.wq[r * SM::W_STRIDE + e1]) = ca;
        *reinterpret_cast<int4*>(&sm.wq[r * SM::W_STRIDE + e1 + 64]) = cb;
        // group scales 2c and 2c+1
        // a super-block past the end (split over K) stages zero scales
        const float dw = valid ? f16_bits_to_f32(psd[k] >> 16) : 0.f;
        sm.wsc[(2 * c) * BM + r] = dw * (float)(int8_t)(psd[k] & 0xFF);
        sm.wsc[(2 * c + 1) * BM + r] = dw * (float)(int8_t)((psd[k] >> 8) & 0xFF);
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {
        const int e = task<BN * 16, NTH, XC>(tid + k * NTH);
        *reinterpret_cast<v4i*>(&sm.xq[(e >> 4) * SM::X_STRIDE + 16 * (e & 15)]) = px[k];
    }
#pragma unroll
    for (int k = 0; k < SC; ++k) {
        const int e = task<BN * 2, NTH, SC>(tid + k * NTH);
        const int t = e >> 1, hf = e & 1;
        sm.xd[(4 * hf + 0) * BN + t] = __int_as_float(ps[k].x);
        sm.xd[(4 * hf + 1) * BN + t] = __int_as_float(ps[k].y);
        sm.xd[(4 * hf + 2) * BN + t] = __int_as_float(ps[k].z);
        sm.xd[(4 * hf + 3) * BN + t] = __int_as_float(ps[k].w);
    }
}

// Step m of a staged Q6_K super-block: groups 2m and 2m + 1 (they share activation
// block m): this lane's 8 code bytes of each group (row arow), the matching 8
// activation bytes (token btok), and the scale factors of group 2m + lh.
template <int BM, int BN>
__device__ __forceinline__ Ops8 q6_load(const Q6Smem<BM, BN>& sm, int m, int arow, int btok, int lh)
{
    using SM = Q6Smem<BM, BN>;
    Ops8 o;
    o.a0 = *reinterpret_cast<const long*>(&sm.wq[arow * SM::W_STRIDE + 32 * m + 8 * lh]);
    o.a1 = *reinterpret_cast<const long*>(&sm.wq[arow * SM::W_STRIDE + 32 * m + 16 + 8 * lh]);
    o.b0 = *reinterpret_cast<const long*>(&sm.xq[btok * SM::X_STRIDE + 32 * m + 8 * lh]);
    o.b1 = *reinterpret_cast<const long*>(&sm.xq[btok * SM::X_STRIDE + 32 * m + 16 + 8 * lh]);
    o.ws = sm.wsc[(2 * m + lh) * BM + arow];
    o.xd = sm.xd[m * BN + btok];
    return o;
}

// The eight steps of one staged Q6_K super-block, added into accv (the stream-K
// kernel; the per-tile kernel keeps its own copy of the step code, which the
// compiler fits in registers without spilling at 128 x 64).
template <int BM, int BN, int PIPE>
__device__ __forceinline__ void q6_superblock(const Q6Smem<BM, BN>& sm, int arow, int btok, int lh, v16f& accv)
{
    pipelined_steps<8, PIPE, Ops8>(
        [&](int m) { return q6_load<BM, BN>(sm, m, arow, btok, lh); },
        [&](const Ops8& o, int, v16i& C0, v16i& C1, v32f& P) {
            C0 = mfma_i8_k16(o.a0, o.b0);
            C1 = mfma_i8_k16(o.a1, o.b1);
            P = mfma_outer2(o.ws, o.xd);
        },
        accv);
}

template <int WR, int WC, int KS, bool DUMP, bool PAD>
__global__ __launch_bounds__(64 * WR * WC * KS, 2) void mmq_q6k_kernel(const uint8_t* __restrict__ W,
                                                                    const int8_t* __restrict__ q,
                                                                    const float* __restrict__ dx,
                                                                    float* __restrict__ out, int nt, int od,
                                                                    int id, int32_t* __restrict__ S)
{
    constexpr int BM = 32 * WR, BN = 32 * WC, NTH = 64 * WR * WC;   // NTH: threads of one K group
    constexpr int WC8 = (BM * 8 + NTH - 1) / NTH;  // (row, 32-code piece) tasks per thread
    constexpr int XC = (BN * 16 + NTH - 1) / NTH;
    constexpr int SC = (BN * 2 + NTH - 1) / NTH;
    using SM = Q6Smem<BM, BN>;
    __shared__ SM smb[KS][2];   // K groups as in the Q4_K kernel
    static_assert(!DUMP || KS == 1, "the debug dump runs unsplit");
    static_assert((KS - 1) * WR * WC * 1024 * sizeof(float) <= sizeof(smb), "reduction scratch fits the tiles");

    const int ntb = (nt + BN - 1) / BN;
    const int tile = xcd_tile(ntb * ((od + BM - 1) / BM));
    if (tile < 0)
        return;
    const int row0 = (tile / ntb) * BM, tok0 = (tile % ntb) * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = KS > 1 ? wave / (WR * WC) : 0, gw = wave - kg * (WR * WC);
    const int tid = threadIdx.x - kg * NTH;
    const int wr = gw / WC, wc = gw % WC;
    const int li = lane & 31, lh = lane >> 5;
    const int nsb = id >> 8;
    const int nblk = id >> 5;
    const int niter = (nsb + KS - 1) / KS;
    const size_t row_bytes = (size_t)nsb * (PAD ? kQ6KP224Bytes : kQ6KBytes);

    // prefetch registers: per task the five-dword windows of a low and a high
    // chunk (2-byte aligned blocks), the two scale dwords and d
    uint32_t pl[WC8][5], phh[WC8][5];
    uint32_t pshift[WC8];
    v4i px[XC], ps[SC];
    uint32_t psd[WC8];
    v16f accv = {};
    const int arow = wr * 32 + li;
    const int btok = wc * 32 + li;

    // double-buffered LDS per K group, one barrier per iteration (as in the Q4_K kernel)
    q6_prefetch<BM, BN, NTH, WC8, XC, SC, PAD>(pl, phh, pshift, px, ps, psd, W, q, dx, min(kg, nsb - 1), tid, row0, tok0,
                                          nt, od, id, nblk, row_bytes);
    q6_stage<BM, BN, NTH, WC8, XC, SC>(smb[kg][0], pl, phh, pshift, px, ps, psd, tid, kg < nsb);
    q6_prefetch<BM, BN, NTH, WC8, XC, SC, PAD>(pl, phh, pshift, px, ps, psd, W, q, dx, min(KS + kg, nsb - 1), tid, row0,
                                          tok0, nt, od, id, nblk, row_bytes);
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
        const SM& sm = smb[kg][it & 1];
        const int sb = it * KS + kg;
        // step m: groups 2m and 2m+1 (they share activation block m)
        const auto load = [&](int m) {
            Ops8 o;
            o.a0 = *reinterpret_cast<const long*>(&sm.wq[arow * SM::W_STRIDE + 32 * m + 8 * lh]);
            o.a1 = *reinterpret_cast<const long*>(&sm.wq[arow * SM::W_STRIDE + 32 * m + 16 + 8 * lh]);
            o.b0 = *reinterpret_cast<const long*>(&sm.xq[btok * SM::X_STRIDE + 32 * m + 8 * lh]);
            o.b1 = *reinterpret_cast<const long*>(&sm.xq[btok * SM::X_STRIDE + 32 * m + 16 + 8 * lh]);
            o.ws = sm.wsc[(2 * m + lh) * BM + arow];
            o.xd = sm.xd[m * BN + btok];
            return o;
        };
        if constexpr (DUMP) {
#pragma unroll 2
            for (int m = 0; m < 8; ++m) {
                const Ops8 o = load(m);
                const v16i C0 = mfma_i8_k16(o.a0, o.b0);
                const v16i C1 = mfma_i8_k16(o.a1, o.b1);
                const int tg = tok0 + btok;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rg = row0 + wr * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                    if (tg < nt && rg < od) {
                        int32_t* dst = S + (((size_t)tg * od + rg) * nsb + sb) * 16 + 2 * m;
                        dst[0] = C0[i];
                        dst[1] = C1[i];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            pipelined_steps<8, (KS == 1 ? kPipeLds : PAD ? kPipeMfma : kPipeNone), Ops8>(load, [&](const Ops8& o, int, v16i& C0, v16i& C1, v32f& P) {
                C0 = mfma_i8_k16(o.a0, o.b0);
                C1 = mfma_i8_k16(o.a1, o.b1);
                P = mfma_outer2(o.ws, o.xd);
            }, accv);
        }
        __builtin_amdgcn_sched_barrier(0);
        q6_stage<BM, BN, NTH, WC8, XC, SC>(smb[kg][(it + 1) & 1], pl, phh, pshift, px, ps, psd, tid, sb + KS < nsb);
        q6_prefetch<BM, BN, NTH, WC8, XC, SC, PAD>(pl, phh, pshift, px, ps, psd, W, q, dx, min(sb + 2 * KS, nsb - 1), tid,
                                              row0, tok0, nt, od, id, nblk, row_bytes);
        __syncthreads();
    }

    if constexpr (!DUMP) {
        v16f v = accv;
        if (!combine_k_groups<WR * WC, KS>(v, reinterpret_cast<float*>(&smb[0][0]), kg, gw, lane))
            return;
        store_tile(v, out, nt, od, tok0 + btok, row0 + wr * 32, lh);
    }
}

// ------------------------------------------------------------------ Q4_0 / Q8_0
// 32-weight blocks (Q4_0: f16 d, 16 bytes, element l in the low and l + 16 in the
// high nibble of byte l, w = d (nibble - 8); Q8_0: f16 d, 32 int8, w = d q), read
// in groups of eight (a super-block step is 256 weights).  [MMQ, section 4]:
// codes are centred at staging (Q4_0: nibble - 8 as a signed byte) so the int8
// MFMA gives the centred dot and no min term is needed; one
// v_mfma_i32_32x32x32_i8 per block, rescale acc += (d_w * dx) * C with the scale
// products of two blocks from one outer-product pair.  A staging task (row, block)
// loads the dwords the block covers (blocks start 0 or 2 bytes past a dword; rows
// are 16-byte aligned) and funnel-shifts them.
template <int BM, int BN>
struct __attribute__((aligned(16))) B32Smem {
    static constexpr int W_STRIDE = 272;    // 256 centred codes + 16 pad
    static constexpr int X_STRIDE = 272;
    int8_t wq[BM * W_STRIDE];
    float wsc[8 * BM];                      // d of block j, [j][row]
    uint8_t xq[BN * X_STRIDE];
    float xd[8 * BN];
};

// byte-wise n - 8 for nibbles n in 0..15 held one per byte: t = n ^ 8 is n - 8
// when bit 3 of t is clear; when it is set, filling the top four bits gives t - 16
__device__ __forceinline__ uint32_t b32_center(uint32_t nib)
{
    const uint32_t t = nib ^ 0x08080808u;
    return t | ((t & 0x08080808u) * 30u);
}

template <int BM, int BN, int NTH, int WC8, int XC, int SC, bool Q8>
__device__ __forceinline__ void b32_prefetch(uint32_t (&pw)[WC8][Q8 ? 9 : 5], uint32_t (&psh)[WC8], v4i (&px)[XC],
                                             v4i (&ps)[SC], const uint8_t* __restrict__ W,
                                             const int8_t* __restrict__ q, const float* __restrict__ dx, int sb,
                                             int tid, int row0, int tok0, int nt, int od, int id, int nblk,
                                             size_t row_bytes)
{
    constexpr uint32_t BB = Q8 ? 34 : 18;
    constexpr int ND = Q8 ? 9 : 5;
#pragma unroll
    for (int k = 0; k < WC8; ++k) {
        const int e = task<BM * 8, NTH, WC8>(tid + k * NTH);
        const int r = e >> 3, j = e & 7;
        const uint8_t* rp = W + (size_t)min(row0 + r, od - 1) * row_bytes;
        const uint32_t off = ((uint32_t)sb * 8 + (uint32_t)j) * BB;
        const uint32_t* p4 = reinterpret_cast<const uint32_t*>(rp + (off & ~3u));
        psh[k] = off & 3u;
#pragma unroll
        for (int i = 0; i < ND; ++i)
            pw[k][i] = p4[i];
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {
        const int e = task<BN * 16, NTH, XC>(tid + k * NTH);
        const int t = min(tok0 + (e >> 4), nt - 1), ch = e & 15;
        px[k] = *reinterpret_cast<const v4i*>(q + (size_t)t * id + 256 * sb + 16 * ch);
    }
#pragma unroll
    for (int k = 0; k < SC; ++k) {
        const int e = task<BN * 2, NTH, SC>(tid + k * NTH);
        const int t = min(tok0 + (e >> 1), nt - 1), hf = e & 1;
        ps[k] = *reinterpret_cast<const v4i*>(dx + (size_t)t * nblk + 8 * sb + 4 * hf);
    }
}

template <int BM, int BN, int NTH, int WC8, int XC, int SC, bool Q8>
__device__ __forceinline__ void b32_stage(B32Smem<BM, BN>& sm, const uint32_t (&pw)[WC8][Q8 ? 9 : 5],
                                          const uint32_t (&psh)[WC8], const v4i (&px)[XC], const v4i (&ps)[SC],
                                          int tid, bool valid)
{
    using SM = B32Smem<BM, BN>;
    constexpr int ND = Q8 ? 9 : 5;
#pragma unroll
    for (int k = 0; k < WC8; ++k) {
        const int e = task<BM * 8, NTH, WC8>(tid + k * NTH);
        const int r = e >> 3, j = e & 7;
        uint32_t bb[ND];  // block bytes from byte 0
#pragma unroll
        for (int i = 0; i + 1 < ND; ++i)
            bb[i] = __builtin_amdgcn_alignbyte(pw[k][i + 1], pw[k][i], psh[k]);
        bb[ND - 1] = pw[k][ND - 1] >> (8 * psh[k]);
        uint32_t cd[ND - 1];  // code bytes from byte 2
#pragma unroll
        for (int i = 0; i + 1 < ND; ++i)
            cd[i] = __builtin_amdgcn_alignbyte(bb[i + 1], bb[i], 2);
        int8_t* dst = &sm.wq[r * SM::W_STRIDE + 32 * j];
        if constexpr (Q8) {
            *reinterpret_cast<uint4*>(dst) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
            *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
        } else {
            *reinterpret_cast<uint4*>(dst) =
                make_uint4(b32_center(cd[0] & 0x0F0F0F0Fu), b32_center(cd[1] & 0x0F0F0F0Fu),
                           b32_center(cd[2] & 0x0F0F0F0Fu), b32_center(cd[3] & 0x0F0F0F0Fu));
            *reinterpret_cast<uint4*>(dst + 16) =
                make_uint4(b32_center((cd[0] >> 4) & 0x0F0F0F0Fu), b32_center((cd[1] >> 4) & 0x0F0F0F0Fu),
                           b32_center((cd[2] >> 4) & 0x0F0F0F0Fu), b32_center((cd[3] >> 4) & 0x0F0F0F0Fu));
        }
        sm.wsc[j * BM + r] = valid ? f16_bits_to_f32(bb[0] & 0xFFFF) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {
        const int e = task<BN * 16, NTH, XC>(tid + k * NTH);
        *reinterpret_cast<v4i*>(&sm.xq[(e >> 4) * SM::X_STRIDE + 16 * (e & 15)]) = px[k];
    }
#pragma unroll
    for (int k = 0; k < SC; ++k) {
        const int e = task<BN * 2, NTH, SC>(tid + k * NTH);
        const int t = e >> 1, hf = e & 1;
        sm.xd[(4 * hf + 0) * BN + t] = __int_as_float(ps[k].x);
        sm.xd[(4 * hf + 1) * BN + t] = __int_as_float(ps[k].y);
        sm.xd[(4 * hf + 2) * BN + t] = __int_as_float(ps[k].z);
        sm.xd[(4 * hf + 3) * BN + t] = __int_as_float(ps[k].w);
    }
}

template <int WR, int WC, int KS, bool DUMP, bool Q8>
__global__ __launch_bounds__(64 * WR * WC * KS, 2) void mmq_b32_kernel(const uint8_t* __restrict__ W,
                                                                    const int8_t* __restrict__ q,
                                                                    const float* __restrict__ dx,
                                                                    float* __restrict__ out, int nt, int od,
                                                                    int id, int32_t* __restrict__ S)
{
    constexpr int BM = 32 * WR, BN = 32 * WC, NTH = 64 * WR * WC;
    constexpr int WC8 = (BM * 8 + NTH - 1) / NTH;  // (row, block) tasks per thread
    constexpr int XC = (BN * 16 + NTH - 1) / NTH;
    constexpr int SC = (BN * 2 + NTH - 1) / NTH;
    constexpr int ND = Q8 ? 9 : 5;
    using SM = B32Smem<BM, BN>;
    __shared__ SM smb[KS][2];
    static_assert(!DUMP || KS == 1, "the debug dump runs unsplit");
    static_assert((KS - 1) * WR * WC * 1024 * sizeof(float) <= sizeof(smb), "reduction scratch fits the tiles");

    const int ntb = (nt + BN - 1) / BN;
    const int tile = xcd_tile(ntb * ((od + BM - 1) / BM));
    if (tile < 0)
        return;
    const int row0 = (tile / ntb) * BM, tok0 = (tile % ntb) * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = KS > 1 ? wave / (WR * WC) : 0, gw = wave - kg * (WR * WC);
    const int tid = threadIdx.x - kg * NTH;
    const int wr = gw / WC, wc = gw % WC;
    const int li = lane & 31, lh = lane >> 5;
    const int nsb = id >> 8;
    const int nblk = id >> 5;
    const int niter = (nsb + KS - 1) / KS;
    const size_t row_bytes = (size_t)nblk * (Q8 ? 34 : 18);

    uint32_t pw[WC8][ND], psh[WC8];
    v4i px[XC], ps[SC];
    v16f accv = {};
    const int arow = wr * 32 + li;
    const int btok = wc * 32 + li;

    b32_prefetch<BM, BN, NTH, WC8, XC, SC, Q8>(pw, psh, px, ps, W, q, dx, min(kg, nsb - 1), tid, row0, tok0, nt, od,
                                               id, nblk, row_bytes);
    b32_stage<BM, BN, NTH, WC8, XC, SC, Q8>(smb[kg][0], pw, psh, px, ps, tid, kg < nsb);
    b32_prefetch<BM, BN, NTH, WC8, XC, SC, Q8>(pw, psh, px, ps, W, q, dx, min(KS + kg, nsb - 1), tid, row0, tok0,
                                               nt, od, id, nblk, row_bytes);
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
        const SM& sm = smb[kg][it & 1];
        const int sb = it * KS + kg;
        // step p: blocks 2p and 2p + 1
        const auto load = [&](int p) {
            Ops16 o;
            o.a0 = *reinterpret_cast<const v4i*>(&sm.wq[arow * SM::W_STRIDE + 64 * p + 16 * lh]);
            o.a1 = *reinterpret_cast<const v4i*>(&sm.wq[arow * SM::W_STRIDE + 64 * p + 32 + 16 * lh]);
            o.b0 = *reinterpret_cast<const v4i*>(&sm.xq[btok * SM::X_STRIDE + 64 * p + 16 * lh]);
            o.b1 = *reinterpret_cast<const v4i*>(&sm.xq[btok * SM::X_STRIDE + 64 * p + 32 + 16 * lh]);
            o.ws = sm.wsc[(2 * p + lh) * BM + arow];
            o.xd = sm.xd[(2 * p + lh) * BN + btok];
            return o;
        };
        if constexpr (DUMP) {
#pragma unroll 2
            for (int p = 0; p < 4; ++p) {
                const Ops16 o = load(p);
                const v16i C0 = mfma_i8_k32(o.a0, o.b0);
                const v16i C1 = mfma_i8_k32(o.a1, o.b1);
                const int tg = tok0 + btok;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rg = row0 + wr * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                    if (tg < nt && rg < od) {
                        int32_t* dst = S + (((size_t)tg * od + rg) * nsb + sb) * 8 + 2 * p;
                        dst[0] = C0[i];
                        dst[1] = C1[i];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            pipelined_steps<4, kPipeLds, Ops16>(load, [&](const Ops16& o, int, v16i& C0, v16i& C1, v32f& P) {
                C0 = mfma_i8_k32(o.a0, o.b0);
                C1 = mfma_i8_k32(o.a1, o.b1);
                P = mfma_outer2(o.ws, o.xd);
            }, accv);
        }
        __builtin_amdgcn_sched_barrier(0);
        b32_stage<BM, BN, NTH, WC8, XC, SC, Q8>(smb[kg][(it + 1) & 1], pw, psh, px, ps, tid, sb + KS < nsb);
        b32_prefetch<BM, BN, NTH, WC8, XC, SC, Q8>(pw, psh, px, ps, W, q, dx, min(sb + 2 * KS, nsb - 1), tid, row0,
                                                   tok0, nt, od, id, nblk, row_bytes);
        __syncthreads();
    }

    if constexpr (!DUMP) {
        v16f v = accv;
        if (!combine_k_groups<WR * WC, KS>(v, reinterpret_cast<float*>(&smb[0][0]), kg, gw, lane))
            return;
        store_tile(v, out, nt, od, tok0 + btok, row0 + wr * 32, lh);
    }
}

// ------------------------------------------------------------------ probes
// One MFMA tile with the operand and result mapping the MMQ kernels rely on,
// written out in a fixed layout (C[.][token][row]) for a test:
//  kind 1: v_mfma_i32_32x32x32_i8; A [32 rows][32 K] int8, B [32 tokens][32 K]
//          int8 -> C [32 tokens][32 rows] int32 = B . A^T
//  kind 2: v_mfma_f32_32x32x1_2b_f32; A [2][32 rows], B [2][32 tokens] f32 ->
//          C [2][32 tokens][32 rows] f32 = outer products per block
//  kind 3: v_mfma_f32_32x32x2_f32; A [2 K][32 rows], B [2 K][32 tokens] f32 ->
//          C [32 tokens][32 rows] f32 = sum over K
__global__ __launch_bounds__(64) void mfma_tile_probe_kernel(int kind, const void* __restrict__ A,
                                                             const void* __restrict__ B,
                                                             void* __restrict__ C)
{
    const int lane = threadIdx.x, li = lane & 31, lh = lane >> 5;
    if (kind == 1) {
        const int8_t* a8 = static_cast<const int8_t*>(A);
        const int8_t* b8 = static_cast<const int8_t*>(B);
        const int4 a = *reinterpret_cast<const int4*>(a8 + 32 * li + 16 * lh);
        const int4 b = *reinterpret_cast<const int4*>(b8 + 32 * li + 16 * lh);
        const v16i r = mfma_i8_k32(v4i{a.x, a.y, a.z, a.w}, v4i{b.x, b.y, b.z, b.w});
        int32_t* c = static_cast<int32_t*>(C);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            c[32 * li + 8 * (i >> 2) + 4 * lh + (i & 3)] = r[i];
    } else if (kind == 2) {
        const v32f r = mfma_outer2(static_cast<const float*>(A)[lane], static_cast<const float*>(B)[lane]);
        float* c = static_cast<float*>(C);
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                c[1024 * k + 32 * li + 8 * (i >> 2) + 4 * lh + (i & 3)] = r[16 * k + i];
    } else {
        const v16f z = {};
        const v16f r = mfma_k2(static_cast<const float*>(A)[lane], static_cast<const float*>(B)[lane], z);
        float* c = static_cast<float*>(C);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            c[32 * li + 8 * (i >> 2) + 4 * lh + (i & 3)] = r[i];
    }
}

hipError_t launch_mfma_tile_probe(int kind, const void* A, const void* B, void* C, hipStream_t st)
{
    hipLaunchKernelGGL(mfma_tile_probe_kernel, dim3(1), dim3(64), 0, st, kind, A, B, C);
    return hipGetLastError();
}

// ------------------------------------------------------------------ launch

template <int WR, int WC, int KS, bool DUMP>
static hipError_t launch_tile(int type, const uint8_t* W, const int8_t* q, const float* d,
                              const float* s, int nt, int od, int id, float* out, int32_t* S,
                              hipStream_t st)
{
    const int ntiles = ((nt + 32 * WC - 1) / (32 * WC)) * ((od + 32 * WR - 1) / (32 * WR));
    const int grid = 8 * ((ntiles + 7) / 8);
    if (type == 1)
        hipLaunchKernelGGL((mmq_q4k_kernel<WR, WC, KS, DUMP>), dim3(grid), dim3(64 * WR * WC * KS), 0, st, W, q,
                           d, s, out, nt, od, id, S);
    else if (type == 2)
        hipLaunchKernelGGL((mmq_q6k_kernel<WR, WC, KS, DUMP, false>), dim3(grid), dim3(64 * WR * WC * KS), 0, st,
                           W, q, d, out, nt, od, id, S);
    else if (type == 3)
        hipLaunchKernelGGL((mmq_q6k_kernel<WR, WC, KS, DUMP, true>), dim3(grid), dim3(64 * WR * WC * KS), 0, st,
                           W, q, d, out, nt, od, id, S);
    else if (type == 4)
        hipLaunchKernelGGL((mmq_b32_kernel<WR, WC, KS, DUMP, false>), dim3(grid), dim3(64 * WR * WC * KS), 0, st,
                           W, q, d, out, nt, od, id, S);
    else if (type == 5)
        hipLaunchKernelGGL((mmq_b32_kernel<WR, WC, KS, DUMP, true>), dim3(grid), dim3(64 * WR * WC * KS), 0, st,
                           W, q, d, out, nt, od, id, S);
    else
        hipLaunchKernelGGL((mmq_q5k_kernel<WR, WC, KS, DUMP>), dim3(grid), dim3(64 * WR * WC * KS), 0, st, W, q,
                           d, s, out, nt, od, id, S);
    return hipGetLastError();
}

// Shape of the launch, by a cost model: the time of a configuration is taken as
// (rounds of workgroups over the 256 CUs) x (super-blocks each wave walks), all
// configurations running two waves per SIMD when the chip is full:
//   128 x 64 tile, 8 waves, 1 workgroup per CU (LDS);
//   64 x 64 tile, 4 waves, 2 workgroups per CU;
//   64 x 64 tile split over K in 2 groups, 8 waves, 1 workgroup per CU.
// Ties go to the larger tile (fewer re-reads of weights and activations).
// QMM_MMQ_TILE (1, 2 or 3 for the three shapes above) overrides it, for tuning.
static int tile_override()
{
    static int v = -1;
    int cur = __atomic_load_n(&v, __ATOMIC_ACQUIRE);
    if (cur >= 0)
        return cur;
    const char* e = getenv("QMM_MMQ_TILE");
    int val = e ? atoi(e) : 0;
    if (val < 1 || val > 3)
        val = 0;
    __atomic_store_n(&v, val, __ATOMIC_RELEASE);
    return val;
}

int mmq_tile_choice(int nt, int od, int id)
{
    const int o = tile_override();
    if (o)
        return o;
    const long nsb = id / 256;
    const long t42 = (long)((nt + 63) / 64) * ((od + 127) / 128);
    const long t22 = (long)((nt + 63) / 64) * ((od + 63) / 64);
    const long c1 = ((t42 + 255) / 256) * nsb;
    const long c2 = ((t22 + 511) / 512) * nsb;
    const long c3 = ((t22 + 255) / 256) * ((nsb + 1) / 2);
    if (c1 <= c2 && c1 <= c3)
        return 1;
    return c2 <= c3 ? 2 : 3;
}

// Q6_K stream-K: the Q4_K stream-K walk (unit ranges, direct stores of whole tiles,
// workspace slots for partial ones) over the Q6_K staging and steps.
template <int WR, int WC, bool PAD>
__global__ __launch_bounds__(64 * WR * WC, 2) void mmq_q6k_streamk_kernel(const uint8_t* __restrict__ W,
                                                                         const int8_t* __restrict__ q,
                                                                         const float* __restrict__ dx,
                                                                         float* __restrict__ out, int nt, int od,
                                                                         int id, float* __restrict__ ws, int G)
{
    constexpr int BM = 32 * WR, BN = 32 * WC, NTH = 64 * WR * WC, NW = WR * WC;
    constexpr int WC8 = (BM * 8 + NTH - 1) / NTH;
    constexpr int XC = (BN * 16 + NTH - 1) / NTH;
    constexpr int SC = (BN * 2 + NTH - 1) / NTH;
    using SM = Q6Smem<BM, BN>;
    __shared__ SM smb[2];

    const int ntb = (nt + BN - 1) / BN;
    const int ntiles = ntb * ((od + BM - 1) / BM);
    const int nsb = id >> 8, nblk = id >> 5;
    const long units = (long)ntiles * nsb;
    const int g = (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
    const long u0 = sk_first_unit(g, units, G), u1 = sk_first_unit(g + 1, units, G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / WC, wc = wave % WC;
    const int li = lane & 31, lh = lane >> 5;
    const size_t row_bytes = (size_t)nsb * (PAD ? kQ6KP224Bytes : kQ6KBytes);
    const int arow = wr * 32 + li, btok = wc * 32 + li;
    const int first_tile = (int)(u0 / nsb);

    for (long u = u0; u < u1;) {
        const int tile = (int)(u / nsb);
        const int k0 = (int)(u - (long)tile * nsb);
        const int k1 = (int)min((long)nsb, k0 + (u1 - u));
        const int row0 = (tile / ntb) * BM, tok0 = (tile % ntb) * BN;

        uint32_t pl[WC8][5], phh[WC8][5];
        uint32_t pshift[WC8];
        v4i px[XC], ps[SC];
        uint32_t psd[WC8];
        v16f accv = {};
        q6_prefetch<BM, BN, NTH, WC8, XC, SC, PAD>(pl, phh, pshift, px, ps, psd, W, q, dx, k0, tid, row0, tok0, nt, od,
                                                  id, nblk, row_bytes);
        q6_stage<BM, BN, NTH, WC8, XC, SC>(smb[0], pl, phh, pshift, px, ps, psd, tid, true);
        q6_prefetch<BM, BN, NTH, WC8, XC, SC, PAD>(pl, phh, pshift, px, ps, psd, W, q, dx, min(k0 + 1, k1 - 1), tid,
                                                  row0, tok0, nt, od, id, nblk, row_bytes);
        __syncthreads();
        for (int sb = k0; sb < k1; ++sb) {
            const SM& sm = smb[(sb - k0) & 1];
            // the unpadded layout's five-dword prefetch windows leave no room for a step of results
            q6_superblock<BM, BN, PAD ? kPipeMfma : kPipeNone>(sm, arow, btok, lh, accv);
            __builtin_amdgcn_sched_barrier(0);
            q6_stage<BM, BN, NTH, WC8, XC, SC>(smb[(sb - k0 + 1) & 1], pl, phh, pshift, px, ps, psd, tid, sb + 1 < k1);
            q6_prefetch<BM, BN, NTH, WC8, XC, SC, PAD>(pl, phh, pshift, px, ps, psd, W, q, dx, min(sb + 2, k1 - 1), tid,
                                                      row0, tok0, nt, od, id, nblk, row_bytes);
            __syncthreads();
        }
        if (k0 == 0 && k1 == nsb) {
            store_tile(accv, out, nt, od, tok0 + btok, row0 + wr * 32, lh);
        } else {
            float* slot = ws + ((size_t)(2 * g + (tile == first_tile ? 0 : 1)) * NW + wave) * 1024;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                slot[i * 64 + lane] = accv[i];
        }
        u += k1 - k0;
    }
}

// Stream-K launch (Q4_K, Q6_K in both layouts): 128 x 64 tiles, 256 workgroups (one
// per CU at this tile's LDS size).  Workspace: 2 partial tiles per workgroup.
constexpr int kStreamKGroups = 256;

size_t mmq_streamk_ws_bytes() { return (size_t)kStreamKGroups * 2 * 128 * 64 * sizeof(float); }

hipError_t launch_mmq_streamk(int type, const uint8_t* W, const int8_t* q, const float* d, const float* s, int nt,
                              int od, int id, float* out, float* ws, hipStream_t st)
{
    const int G = kStreamKGroups;
    if (type == 1)
        hipLaunchKernelGGL((mmq_q4k_streamk_kernel<4, 2>), dim3(G), dim3(512), 0, st, W, q, d, s, out, nt, od, id, ws,
                           G);
    else if (type == 2)
        hipLaunchKernelGGL((mmq_q6k_streamk_kernel<4, 2, false>), dim3(G), dim3(512), 0, st, W, q, d, out, nt, od, id,
                           ws, G);
    else if (type == 3)
        hipLaunchKernelGGL((mmq_q6k_streamk_kernel<4, 2, true>), dim3(G), dim3(512), 0, st, W, q, d, out, nt, od, id,
                           ws, G);
    else
        return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // the fixup only where a range boundary falls inside a tile
    const long nsb = id / 256, units = (long)((nt + 63) / 64) * ((od + 127) / 128) * nsb;
    bool split = false;
    for (int g = 1; g < G && !split; ++g) {
        const long u = sk_first_unit(g, units, G);
        split = u < units && u % nsb != 0;
    }
    if (!split)
        return hipSuccess;
    hipLaunchKernelGGL((mmq_streamk_fixup_kernel<4, 2, kStreamKGroups>), dim3((G - 1) * 8), dim3(64), 0, st, ws, out, nt,
                       od, (int)nsb);
    return hipGetLastError();
}

// Two of the 4-wave kernel's workgroups share a CU, so one round holds 512 tiles.
// Measured (Q4_K, 4096 and 8192 columns, same process): where the cost model names
// 128 x 64 tiles and there are more than 256, it is 3-10 % faster than this file's
// 8-wave tiles and 12-31 % faster than stream-K (448-768 tiles); where it names the
// 64 x 64 split, it wins from 384 tiles up to one full round (12288 x 4096 at 256
// tokens: 62.1 against 67.1 us stream-K and 73.4 us split; 12288 x 8192: 113.0
// against 119.5 and 128.8), and loses to stream-K at 288-320 tiles (by 3-4 %) and
// past one round (576 tiles: 100.8 against 95.6 us).  On at most 256 tiles it holds
// one wave per SIMD; there its split over K (8 waves, one workgroup per CU, two
// waves per SIMD) beats the 8-wave 128 x 64 tiles by 1-4 % where the cost model
// names them (4096 x 8192 at 512 tokens: 70.7 against 72.4 us; 4096 x 12288 at 384,
// 448 and 512 tokens: 100.6 / 101.0 / 101.7-103.1 against 103.0 / 103.0 /
// 104.1-106.2 us).
int mmq_q4k_wave_form(int nt, int od, int id)
{
    const long t128 = (long)((nt + 63) / 64) * ((od + 127) / 128);
    const int choice = mmq_tile_choice(nt, od, id);
    if (t128 > 256 && (choice == 1 || (t128 >= 384 && t128 <= 512)))
        return 1;
    return (choice == 1 && t128 >= 192) ? 2 : 0;
}

hipError_t launch_mmq(int type, const uint8_t* W, const int8_t* q, const float* d, const float* s,
                      int nt, int od, int id, float* out, int32_t* S, hipStream_t st, int tile)
{
    // Q4_K: the kernel of 4 waves of 32 rows x 64 tokens (qmm_mmq2.hip) and its
    // split over K by mmq_q4k_wave_form, or when asked for
    const int wf = (type == 1 && tile == 0 && !S) ? mmq_q4k_wave_form(nt, od, id) : 0;
    if (type == 1 && (tile == 4 || (tile == 0 && S) || wf == 1))
        return launch_mmq_q4k_v2(W, q, d, s, nt, od, id, out, S, st);
    if (type == 1 && !S && (tile == 5 || wf == 2))
        return launch_mmq_q4k_v2(W, q, d, s, nt, od, id, out, nullptr, st, 2);
    if (tile == 4 || tile == 5)
        return hipErrorInvalidValue;
    if (S)
        return launch_tile<2, 2, 1, true>(type, W, q, d, s, nt, od, id, out, S, st);
    switch (tile ? tile : mmq_tile_choice(nt, od, id)) {
    case 1: return launch_tile<4, 2, 1, false>(type, W, q, d, s, nt, od, id, out, S, st);
    case 2: return launch_tile<2, 2, 1, false>(type, W, q, d, s, nt, od, id, out, S, st);
    default: return launch_tile<2, 2, 2, false>(type, W, q, d, s, nt, od, id, out, S, st);
    }
}

}  // namespace qmm
