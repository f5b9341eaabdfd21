// MMQ on Q8_K activations (one scale per 256 values): Q4_K / Q5_K and Q6_K weights,
// int8 MFMA, the group products combined in integer inside each super-block.
//
// [GEMM, "Activations: int8 with a scale per 256"]: the activations carry one f32
// scale per 256 values and the code sum of every 16-value group.  [GEMM, "The zero
// points do not touch the inner loop"]: the Q4_K min term is dmin * m times the
// sub-block's activation sum, from those stored sums.  With one activation scale
// per super-block, a super-block's contribution to out[t][r] is
//   d[r] * dx[t] * S1 - dmin[r] * dx[t] * S2,
//   S1 = sum_j sc_j[r] * sum(q * qx)  (integer),  S2 = sum_j m_j[r] * (bsum_2j + bsum_2j+1)
// so the per-sub-block scaling of the per-32 path becomes integer arithmetic and
// the float work is once per super-block.
//
// MI355X mapping:
//  * Workgroup tile BM = 32*WR weight rows x BN = 32*WC tokens, one wave per
//    32 x 32 block, tiles ordered so one row block stays on one XCD.
//  * v_mfma_i32_32x32x32_i8 with the roles of the per-32 kernel swapped: operand A
//    is the activation codes (token = lane % 32), operand B the weight codes
//    (row = lane % 32).  A result lane then holds one weight row and 16 tokens, so
//    the row's scale sc_j is one register per lane and the integer combine is one
//    v_mad_i32_i24 per value per sub-block (|sum(q*qx)| <= 60960, sc <= 63).
//  * S2 on v_mfma_f32_32x32x16_f16: the 16 group sums (|bsum| <= 2032) and the
//    mins m_{g/2} (<= 63) are exact in f16 and every partial sum is an integer
//    below 2^24, so the f32 result is exact.
//  * d[r]*dx[t] and -dmin[r]*dx[t] in the result layout from one pair of outer
//    products (v_mfma_f32_32x32x1_2b_f32); per value and super-block: one
//    conversion of S1 and two FMAs.
//  * LDS per super-block (double buffered): raw code bytes, sc as int32 [row][8],
//    m as f16 [row][16 groups], d and -dmin, activation codes, group sums as f16,
//    dx; the next super-block's loads are issued before the compute.
#include "qmm_mmq_common.h"

namespace qmm {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v16f mfma_f16_k16(v8h a, v8h b)
{
    const v16f z = {};
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, z, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

template <int BM, int BN>
struct __attribute__((aligned(16))) Q8KSmemK4 {
    static constexpr int QS_STRIDE = 144;   // 128 code bytes + 16 pad
    static constexpr int X_STRIDE = 272;    // 256 activation codes + 16 pad
    uint8_t qs[BM * QS_STRIDE];
    int32_t sc[BM * 8];                     // [row][j]
    _Float16 mn[BM * 16];                   // [row][g] = m_{g/2}
    float dd[2 * BM];                       // [0][row] = d, [1][row] = -dmin
    uint8_t xq[BN * X_STRIDE];
    _Float16 bs[BN * 16];                   // [token][g] group code sums
    float dx[BN];                           // [token] activation scale
};

template <int BM, int BN, bool Q5>
struct __attribute__((aligned(16))) Q8KSmem : Q8KSmemK4<BM, BN> {};

// Q5_K: also the 32 high-bit bytes of each row
template <int BM, int BN>
struct __attribute__((aligned(16))) Q8KSmem<BM, BN, true> : Q8KSmemK4<BM, BN> {
    uint8_t qh[BM * 32];
};

// Per-thread prefetch slots: code chunks, row headers, activation chunks, group
// sum chunks (four per token), activation scales.
template <int QC, int HC, int XC, int BC, int DC, int HBC>
struct Q8KRegs {
    v4i q[QC], h[HC], x[XC], b[BC], hb[HBC];
    uint32_t d[DC];
};

template <int QC, int HC, int XC, int BC, int DC, int HBC>
struct Q8KOffs {
    uint32_t q[QC], h[HC], x[XC], b[BC], d[DC], hb[HBC];
};

struct Q8KRsrc {
    __amdgpu_buffer_rsrc_t w, x, d, b;
};

// Q5 (Q5_K, 176-byte blocks): the codes start at byte 48, after the 32 high-bit
// bytes at 16 (task HBC: one 16-byte half of a row's high-bit bytes).
template <int BM, int BN, int NTH, int QC, int HC, int XC, int BC, int DC, int HBC, bool Q5>
__device__ __forceinline__ void q8k_offsets(Q8KOffs<QC, HC, XC, BC, DC, HBC>& o, int tid, int row0, int tok0,
                                            int nt, int od, int id, int nsb, uint32_t row_bytes)
{
#pragma unroll
    for (int k = 0; k < QC; ++k) {
        const int e = task<BM * 8, NTH, QC>(tid + k * NTH);
        o.q[k] = (uint32_t)(min(row0 + (e >> 3), od - 1) - row0) * row_bytes + (Q5 ? 48 : 16) + 16 * (e & 7);
    }
    if constexpr (Q5) {
#pragma unroll
        for (int k = 0; k < HBC; ++k) {
            const int e = task<BM * 2, NTH, HBC>(tid + k * NTH);
            o.hb[k] = (uint32_t)(min(row0 + (e >> 1), od - 1) - row0) * row_bytes + 16 + 16 * (e & 1);
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
    for (int k = 0; k < BC; ++k) {
        const int e = task<BN * 4, NTH, BC>(tid + k * NTH);
        o.b[k] = ((uint32_t)(min(tok0 + (e >> 2), nt - 1) - tok0) * (uint32_t)(id / 16) + 4 * (e & 3)) * 4;
    }
#pragma unroll
    for (int k = 0; k < DC; ++k) {
        const int e = task<BN, NTH, DC>(tid + k * NTH);
        o.d[k] = (uint32_t)(min(tok0 + e, nt - 1) - tok0) * (uint32_t)nsb * 4;
    }
}

template <int QC, int HC, int XC, int BC, int DC, int HBC, bool Q5>
__device__ __forceinline__ void q8k_prefetch(Q8KRegs<QC, HC, XC, BC, DC, HBC>& r,
                                             const Q8KOffs<QC, HC, XC, BC, DC, HBC>& o, const Q8KRsrc& rs, int sb)
{
    const uint32_t ow = (uint32_t)sb * (Q5 ? kQ5KBytes : kQ4KBytes), ox = 256u * (uint32_t)sb,
                   ob = 64u * (uint32_t)sb, odx = 4u * (uint32_t)sb;
#pragma unroll
    for (int k = 0; k < QC; ++k)
        r.q[k] = bload16(rs.w, o.q[k], ow);
    if constexpr (Q5) {
#pragma unroll
        for (int k = 0; k < HBC; ++k)
            r.hb[k] = bload16(rs.w, o.hb[k], ow);
    }
#pragma unroll
    for (int k = 0; k < HC; ++k)
        r.h[k] = bload16(rs.w, o.h[k], ow);
#pragma unroll
    for (int k = 0; k < XC; ++k)
        r.x[k] = bload16(rs.x, o.x[k], ox);
#pragma unroll
    for (int k = 0; k < BC; ++k)
        r.b[k] = bload16(rs.b, o.b[k], ob);
#pragma unroll
    for (int k = 0; k < DC; ++k)
        r.d[k] = bload4(rs.d, o.d[k], odx);
}

// valid == false (a super-block index past the end) stages d = dmin = 0: that
// super-block then adds nothing.
template <int BM, int BN, int NTH, int QC, int HC, int XC, int BC, int DC, int HBC, bool Q5>
__device__ __forceinline__ void q8k_stage(Q8KSmem<BM, BN, Q5>& sm, const Q8KRegs<QC, HC, XC, BC, DC, HBC>& r,
                                          int tid, bool valid)
{
    using SM = Q8KSmem<BM, BN, Q5>;
#pragma unroll
    for (int k = 0; k < QC; ++k) {
        const int e = task<BM * 8, NTH, QC>(tid + k * NTH);
        *reinterpret_cast<v4i*>(&sm.qs[(e >> 3) * SM::QS_STRIDE + 16 * (e & 7)]) = r.q[k];
    }
    if constexpr (Q5) {
#pragma unroll
        for (int k = 0; k < HBC; ++k) {
            const int e = task<BM * 2, NTH, HBC>(tid + k * NTH);
            *reinterpret_cast<v4i*>(&sm.qh[(e >> 1) * 32 + 16 * (e & 1)]) = r.hb[k];
        }
    }
#pragma unroll
    for (int k = 0; k < HC; ++k) {
        // task (row, jj) decodes sub-blocks jj and jj + 4; every task of a row
        // writes the same d and -dmin
        const int e = task<BM * 4, NTH, HC>(tid + k * NTH);
        const int row = e >> 2, jj = e & 3;
        const v4i h = r.h[k];
        int sc0, m0, sc1, m1;
        q4k_scale_min_pair((uint32_t)h.y, (uint32_t)h.z, (uint32_t)h.w, jj, sc0, m0, sc1, m1);
        sm.sc[row * 8 + jj] = sc0;
        sm.sc[row * 8 + jj + 4] = sc1;
        const v2h mh0 = {(_Float16)m0, (_Float16)m0}, mh1 = {(_Float16)m1, (_Float16)m1};
        *reinterpret_cast<v2h*>(&sm.mn[row * 16 + 2 * jj]) = mh0;
        *reinterpret_cast<v2h*>(&sm.mn[row * 16 + 2 * (jj + 4)]) = mh1;
        sm.dd[row] = valid ? f16_bits_to_f32((uint32_t)h.x & 0xFFFF) : 0.f;
        sm.dd[BM + row] = valid ? -f16_bits_to_f32((uint32_t)h.x >> 16) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {
        const int e = task<BN * 16, NTH, XC>(tid + k * NTH);
        *reinterpret_cast<v4i*>(&sm.xq[(e >> 4) * SM::X_STRIDE + 16 * (e & 15)]) = r.x[k];
    }
#pragma unroll
    for (int k = 0; k < BC; ++k) {
        // four group sums (exact small integers) to f16
        const int e = task<BN * 4, NTH, BC>(tid + k * NTH);
        const v2h lo = {(_Float16)__int_as_float(r.b[k].x), (_Float16)__int_as_float(r.b[k].y)};
        const v2h hi = {(_Float16)__int_as_float(r.b[k].z), (_Float16)__int_as_float(r.b[k].w)};
        *reinterpret_cast<v2h*>(&sm.bs[(e >> 2) * 16 + 4 * (e & 3)]) = lo;
        *reinterpret_cast<v2h*>(&sm.bs[(e >> 2) * 16 + 4 * (e & 3) + 2]) = hi;
    }
#pragma unroll
    for (int k = 0; k < DC; ++k) {
        const int e = task<BN, NTH, DC>(tid + k * NTH);
        sm.dx[e] = __uint_as_float(r.d[k]);
    }
}

// Sub-blocks 2p and 2p + 1 of the staged super-block: the two int8 products,
// token-major (A = activation codes of token atok, B = weight codes of row brow).
// Q5: bits 2p and 2p + 1 of the row's high-bit bytes 16 lh .. + 15 are the fifth
// code bits of the two sub-blocks at those positions (codes 0..31).
template <int BM, int BN, bool Q5>
__device__ __forceinline__ void q8k_step(const Q8KSmem<BM, BN, Q5>& sm, int p, int atok, int brow, int lh, v16i& C0,
                                         v16i& C1)
{
    using SM = Q8KSmem<BM, BN, Q5>;
    const v4i w16 = *reinterpret_cast<const v4i*>(&sm.qs[brow * SM::QS_STRIDE + 32 * p + 16 * lh]);
    v4i b0 = w16 & 0x0F0F0F0F, b1 = (w16 >> 4) & 0x0F0F0F0F;
    if constexpr (Q5) {
        const v4i hb = *reinterpret_cast<const v4i*>(&sm.qh[brow * 32 + 16 * lh]);
        b0 |= ((hb >> (2 * p)) & 0x01010101) << 4;
        b1 |= ((hb >> (2 * p + 1)) & 0x01010101) << 4;
    }
    const v4i x0 = *reinterpret_cast<const v4i*>(&sm.xq[atok * SM::X_STRIDE + 64 * p + 16 * lh]);
    const v4i x1 = *reinterpret_cast<const v4i*>(&sm.xq[atok * SM::X_STRIDE + 64 * p + 32 + 16 * lh]);
    C0 = mfma_i8_k32(x0, b0);
    C1 = mfma_i8_k32(x1, b1);
}

// Result tile of one wave: lane holds weight row r and tokens t0 + 8k + 4 lh + i
// (k = 0..3, i = 0..3) in v[4k + i]; store into out [nt][od], masked.
__device__ __forceinline__ void store_tile_rowmajor(const v16f& v, float* __restrict__ out, int nt, int od, int t0,
                                                    int r, int lh)
{
    if (r >= od)
        return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = t0 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (t < nt)
            out[(size_t)t * od + r] = v[i];
    }
}

// Q4_K (Q5 false) and Q5_K (Q5 true, 176-byte blocks: the fifth code bit from the
// staged high-bit bytes; |sum(q * qx)| <= 32 * 31 * 127 per sub-block, sc <= 63,
// so the integer combine stays in range).  One kernel rather than a shared body
// under two wrappers: the wrapped body took 15 more VGPRs.
// KS = 2: two groups of WR x WC waves in one workgroup split K (alternate
// super-blocks, each group with its own LDS buffers), their 32 x 32 partial sums
// added at the end in group order (combine_k_groups), as in the per-32 kernels.
template <int WR, int WC, int KS, bool DUMP, bool Q5>
__global__ __launch_bounds__(64 * WR * WC * KS) void mmq_k4_q8k_kernel(const uint8_t* __restrict__ W,
                                                                       const int8_t* __restrict__ q,
                                                                       const float* __restrict__ dx,
                                                                       const float* __restrict__ bsum,
                                                                       float* __restrict__ out, int nt, int od,
                                                                       int id, int32_t* __restrict__ S)
{
    constexpr int BM = 32 * WR, BN = 32 * WC, NTH = 64 * WR * WC;   // NTH: threads of one K group
    constexpr int QC = (BM * 8 + NTH - 1) / NTH;
    constexpr int HC = (BM * 4 + NTH - 1) / NTH;
    constexpr int XC = (BN * 16 + NTH - 1) / NTH;
    constexpr int BC = (BN * 4 + NTH - 1) / NTH;
    constexpr int DC = (BN + NTH - 1) / NTH;
    constexpr int HBC = Q5 ? (BM * 2 + NTH - 1) / NTH : 1;
    using SM = Q8KSmem<BM, BN, Q5>;
    __shared__ SM smb[KS][2];
    static_assert(!DUMP || KS == 1, "the integer-stage dump runs unsplit");
    static_assert((KS - 1) * WR * WC * 1024 * sizeof(float) <= sizeof(smb), "reduction scratch fits the tiles");

    const int ntb = (nt + BN - 1) / BN;
    const int tile = xcd_tile(ntb * ((od + BM - 1) / BM));
    if (tile < 0)
        return;  // whole workgroup
    const int row0 = (tile / ntb) * BM, tok0 = (tile % ntb) * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = KS > 1 ? wave / (WR * WC) : 0, gw = wave - kg * (WR * WC);
    const int tid = threadIdx.x - kg * NTH;
    const int wr = gw / WC, wc = gw % WC;
    const int li = lane & 31, lh = lane >> 5;
    const int nsb = id >> 8;
    const int niter = (nsb + KS - 1) / KS;
    const uint32_t row_bytes = (uint32_t)nsb * (Q5 ? kQ5KBytes : kQ4KBytes);

    Q8KRegs<QC, HC, XC, BC, DC, HBC> pr;
    Q8KOffs<QC, HC, XC, BC, DC, HBC> offs;
    q8k_offsets<BM, BN, NTH, QC, HC, XC, BC, DC, HBC, Q5>(offs, tid, row0, tok0, nt, od, id, nsb, row_bytes);
    Q8KRsrc rs;
    rs.w = buffer_rsrc(W + (size_t)row0 * row_bytes, (size_t)(od - row0) * row_bytes);
    rs.x = buffer_rsrc(q + (size_t)tok0 * id, (size_t)(nt - tok0) * id);
    rs.d = buffer_rsrc(dx + (size_t)tok0 * nsb, (size_t)(nt - tok0) * nsb * 4);
    rs.b = buffer_rsrc(bsum + (size_t)tok0 * (id / 16), (size_t)(nt - tok0) * (id / 16) * 4);
    v16f acc = {};
    const int atok = wc * 32 + li;   // this lane's token as an A operand
    const int brow = wr * 32 + li;   // this lane's weight row as a B operand

    // double-buffered LDS as in the per-32 kernel: compute from smb[it & 1] while
    // the next super-block (in registers) goes to the other buffer and the loads
    // of the one after are issued; unconditional prefetches with clamped indices
    q8k_prefetch<QC, HC, XC, BC, DC, HBC, Q5>(pr, offs, rs, min(kg, nsb - 1));
    q8k_stage<BM, BN, NTH, QC, HC, XC, BC, DC, HBC, Q5>(smb[kg][0], pr, tid, kg < nsb);
    q8k_prefetch<QC, HC, XC, BC, DC, HBC, Q5>(pr, offs, rs, min(KS + kg, nsb - 1));
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
        const SM& sm = smb[kg][it & 1];
        const int sb = it * KS + kg;
        // operands that do not depend on the codes first: the exact min sums and
        // the scale products d*dx (registers 0..15) and -dmin*dx (16..31)
        const v8h bsv = *reinterpret_cast<const v8h*>(&sm.bs[atok * 16 + 8 * lh]);
        const v8h mnv = *reinterpret_cast<const v8h*>(&sm.mn[brow * 16 + 8 * lh]);
        const v16f cmin = mfma_f16_k16(bsv, mnv);
        const v32f pp = mfma_outer2(sm.dx[atok], sm.dd[lh * BM + brow]);
        const v4i s03 = *reinterpret_cast<const v4i*>(&sm.sc[brow * 8]);
        const v4i s47 = *reinterpret_cast<const v4i*>(&sm.sc[brow * 8 + 4]);
        const int scv[8] = {s03.x, s03.y, s03.z, s03.w, s47.x, s47.y, s47.z, s47.w};

        v16i acci = {}, acco = {};
        v16i Ca0, Ca1;
        q8k_step<BM, BN, Q5>(sm, 0, atok, brow, lh, Ca0, Ca1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            v16i Cb0, Cb1;
            if (p < 3)
                q8k_step<BM, BN, Q5>(sm, p + 1, atok, brow, lh, Cb0, Cb1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                // even and odd sub-blocks in separate sums: each update is one
                // v_mad_i32_i24 (a shared sum is reassociated into two multiplies
                // and a three-input add)
                acci[i] = __mul24(Ca0[i], scv[2 * p]) + acci[i];
                acco[i] = __mul24(Ca1[i], scv[2 * p + 1]) + acco[i];
            }
            __builtin_amdgcn_sched_barrier(0);
            if (p < 3) {
                Ca0 = Cb0;
                Ca1 = Cb1;
            }
        }
        acci += acco;
        if constexpr (DUMP) {
            const int r = row0 + brow;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = tok0 + wc * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                if (t < nt && r < od) {
                    int32_t* dst = S + (((size_t)t * od + r) * nsb + sb) * 2;
                    dst[0] = acci[i];
                    dst[1] = (int32_t)cmin[i];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc[i] = fmaf(pp[i], (float)acci[i], acc[i]);
                acc[i] = fmaf(pp[16 + i], cmin[i], acc[i]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        q8k_stage<BM, BN, NTH, QC, HC, XC, BC, DC, HBC, Q5>(smb[kg][(it + 1) & 1], pr, tid, sb + KS < nsb);
        q8k_prefetch<QC, HC, XC, BC, DC, HBC, Q5>(pr, offs, rs, min(sb + 2 * KS, nsb - 1));
        __syncthreads();
    }
    if constexpr (!DUMP) {
        if (!combine_k_groups<WR * WC, KS>(acc, reinterpret_cast<float*>(&smb[0][0]), kg, gw, lane))
            return;
        store_tile_rowmajor(acc, out, nt, od, tok0 + wc * 32, row0 + brow, lh);
    }
}

// ------------------------------------------------------------------ Q6_K on Q8_K
// [GEMM, "Activations: int8 with a scale per 256"] with Q6_K weights: the sixteen
// 16-weight groups of a super-block share one activation scale, so its contribution
// to out[t][r] is d[r] * dx[t] * S, S = sum_g sc_g[r] * sum((q6 - 32) * qx) an exact
// integer (|sum((q6 - 32) * qx)| <= 16 * 32 * 127, |sc_g| <= 128, |S| < 2^28).  No
// min term (the codes are centred).  Same swapped MFMA roles as the Q4_K kernel
// (A = activation codes, B = weight codes, a result lane holds one weight row and
// 16 tokens), so sc_g is one register per lane and the combine is one
// v_mad_i32_i24 per value and group on v_mfma_i32_32x32x16_i8 results (the per-32
// path: a conversion and an FMA per value and group).  Codes are centred at
// staging as in the per-32 Q6_K kernel; PAD reads the 224-byte layout.
template <int BM, int BN>
struct __attribute__((aligned(16))) Q6Q8KSmem {
    static constexpr int W_STRIDE = 272;    // 256 centred codes + 16 pad
    static constexpr int X_STRIDE = 272;    // 256 activation codes + 16 pad
    int8_t wq[BM * W_STRIDE];
    int32_t sc[BM * 16];                    // [row][g]
    float dd[BM];                           // [row] d
    uint8_t xq[BN * X_STRIDE];
    float dx[BN];                           // [token] activation scale
};

// Groups 2m and 2m + 1 of the staged super-block: the two int8 products,
// token-major (A = activation codes of token atok, B = weight codes of row brow).
template <int BM, int BN>
__device__ __forceinline__ void q6q8k_step(const Q6Q8KSmem<BM, BN>& sm, int m, int atok, int brow, int lh, v16i& C0,
                                           v16i& C1)
{
    using SM = Q6Q8KSmem<BM, BN>;
    const long x0 = *reinterpret_cast<const long*>(&sm.xq[atok * SM::X_STRIDE + 32 * m + 8 * lh]);
    const long x1 = *reinterpret_cast<const long*>(&sm.xq[atok * SM::X_STRIDE + 32 * m + 16 + 8 * lh]);
    const long w0 = *reinterpret_cast<const long*>(&sm.wq[brow * SM::W_STRIDE + 32 * m + 8 * lh]);
    const long w1 = *reinterpret_cast<const long*>(&sm.wq[brow * SM::W_STRIDE + 32 * m + 16 + 8 * lh]);
    C0 = mfma_i8_k16(x0, w0);
    C1 = mfma_i8_k16(x1, w1);
}

template <int WR, int WC, int KS, bool DUMP, bool PAD>
__global__ __launch_bounds__(64 * WR * WC * KS) void mmq_q6k_q8k_kernel(const uint8_t* __restrict__ W,
                                                                        const int8_t* __restrict__ q,
                                                                        const float* __restrict__ dx,
                                                                        float* __restrict__ out, int nt, int od,
                                                                        int id, int32_t* __restrict__ S)
{
    constexpr int BM = 32 * WR, BN = 32 * WC, NTH = 64 * WR * WC;   // NTH: threads of one K group
    constexpr int WC8 = (BM * 8 + NTH - 1) / NTH;  // (row, 32-code piece) tasks per thread
    constexpr int XC = (BN * 16 + NTH - 1) / NTH;
    constexpr int DC = (BN + NTH - 1) / NTH;
    using SM = Q6Q8KSmem<BM, BN>;
    __shared__ SM smb[KS][2];
    static_assert(!DUMP || KS == 1, "the integer-stage dump runs unsplit");
    static_assert((KS - 1) * WR * WC * 1024 * sizeof(float) <= sizeof(smb), "reduction scratch fits the tiles");

    const int ntb = (nt + BN - 1) / BN;
    const int tile = xcd_tile(ntb * ((od + BM - 1) / BM));
    if (tile < 0)
        return;  // whole workgroup
    const int row0 = (tile / ntb) * BM, tok0 = (tile % ntb) * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = KS > 1 ? wave / (WR * WC) : 0, gw = wave - kg * (WR * WC);
    const int tid = threadIdx.x - kg * NTH;
    const int wr = gw / WC, wc = gw % WC;
    const int li = lane & 31, lh = lane >> 5;
    const int nsb = id >> 8;
    const int niter = (nsb + KS - 1) / KS;
    const size_t row_bytes = (size_t)nsb * (PAD ? kQ6KP224Bytes : kQ6KBytes);

    uint32_t pl[WC8][5], phh[WC8][5], pshift[WC8], psd[WC8];
    v4i px[XC];
    uint32_t pdx[DC];
    // unconditional loads with clamped task, row and token indices
    const auto prefetch = [&](int sb) {
#pragma unroll
        for (int k = 0; k < WC8; ++k)
            q6_prefetch_task<PAD>(pl[k], phh[k], pshift[k], psd[k], W, task<BM * 8, NTH, WC8>(tid + k * NTH), sb,
                                  row0, od, row_bytes);
#pragma unroll
        for (int k = 0; k < XC; ++k) {
            const int e = task<BN * 16, NTH, XC>(tid + k * NTH);
            const int t = min(tok0 + (e >> 4), nt - 1);
            px[k] = *reinterpret_cast<const v4i*>(q + (size_t)t * id + 256 * sb + 16 * (e & 15));
        }
#pragma unroll
        for (int k = 0; k < DC; ++k) {
            const int t = min(tok0 + task<BN, NTH, DC>(tid + k * NTH), nt - 1);
            pdx[k] = __float_as_uint(dx[(size_t)t * nsb + sb]);
        }
    };
    // valid == false (a super-block past the end) stages d = 0: it adds nothing
    const auto stage = [&](SM& sm, bool valid) {
#pragma unroll
        for (int k = 0; k < WC8; ++k) {
            const int e = task<BM * 8, NTH, WC8>(tid + k * NTH);
            const int r = e >> 3, c = e & 7;
            q6_stage_codes(&sm.wq[r * SM::W_STRIDE], pl[k], phh[k], pshift[k], c);
            sm.sc[r * 16 + 2 * c] = (int)(int8_t)(psd[k] & 0xFF);
            sm.sc[r * 16 + 2 * c + 1] = (int)(int8_t)((psd[k] >> 8) & 0xFF);
            sm.dd[r] = valid ? f16_bits_to_f32(psd[k] >> 16) : 0.f;  // every task of a row writes the same d
        }
#pragma unroll
        for (int k = 0; k < XC; ++k) {
            const int e = task<BN * 16, NTH, XC>(tid + k * NTH);
            *reinterpret_cast<v4i*>(&sm.xq[(e >> 4) * SM::X_STRIDE + 16 * (e & 15)]) = px[k];
        }
#pragma unroll
        for (int k = 0; k < DC; ++k)
            sm.dx[task<BN, NTH, DC>(tid + k * NTH)] = __uint_as_float(pdx[k]);
    };

    v16f acc = {};
    const int atok = wc * 32 + li;   // this lane's token as an A operand
    const int brow = wr * 32 + li;   // this lane's weight row as a B operand

    prefetch(min(kg, nsb - 1));
    stage(smb[kg][0], kg < nsb);
    prefetch(min(KS + kg, nsb - 1));
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
        const SM& sm = smb[kg][it & 1];
        const int sb = it * KS + kg;
        // the scale product d[r] * dx[t] in the result layout (one outer product on
        // the k = 0 lanes), and this row's sixteen group scales
        const float oa = lh == 0 ? sm.dx[atok] : 0.f, ob = lh == 0 ? sm.dd[brow] : 0.f;
        const v16f pp = mfma_k2(oa, ob, v16f{});
        const v4i s0 = *reinterpret_cast<const v4i*>(&sm.sc[brow * 16]);
        const v4i s1 = *reinterpret_cast<const v4i*>(&sm.sc[brow * 16 + 4]);
        const v4i s2 = *reinterpret_cast<const v4i*>(&sm.sc[brow * 16 + 8]);
        const v4i s3 = *reinterpret_cast<const v4i*>(&sm.sc[brow * 16 + 12]);
        const int scv[16] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w,
                             s2.x, s2.y, s2.z, s2.w, s3.x, s3.y, s3.z, s3.w};

        // step m: groups 2m, 2m + 1; the MFMAs of step m + 1 are issued before the
        // combine of step m
        v16i acci = {}, acco = {};
        v16i Ca0, Ca1;
        q6q8k_step<BM, BN>(sm, 0, atok, brow, lh, Ca0, Ca1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            v16i Cb0, Cb1;
            if (m < 7)
                q6q8k_step<BM, BN>(sm, m + 1, atok, brow, lh, Cb0, Cb1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                // even and odd groups in separate sums, one v_mad_i32_i24 each
                acci[i] = __mul24(Ca0[i], scv[2 * m]) + acci[i];
                acco[i] = __mul24(Ca1[i], scv[2 * m + 1]) + acco[i];
            }
            __builtin_amdgcn_sched_barrier(0);
            if (m < 7) {
                Ca0 = Cb0;
                Ca1 = Cb1;
            }
        }
        acci += acco;
        if constexpr (DUMP) {
            const int r = row0 + brow;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = tok0 + wc * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                if (t < nt && r < od) {
                    int32_t* dst = S + (((size_t)t * od + r) * nsb + sb) * 2;
                    dst[0] = acci[i];
                    dst[1] = 0;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc[i] = fmaf(pp[i], (float)acci[i], acc[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
        stage(smb[kg][(it + 1) & 1], sb + KS < nsb);
        prefetch(min(sb + 2 * KS, nsb - 1));
        __syncthreads();
    }
    if constexpr (!DUMP) {
        if (!combine_k_groups<WR * WC, KS>(acc, reinterpret_cast<float*>(&smb[0][0]), kg, gw, lane))
            return;
        store_tile_rowmajor(acc, out, nt, od, tok0 + wc * 32, row0 + brow, lh);
    }
}

// The shape with the fewest (rounds of workgroups over the 256 CUs) x (super-blocks
// each wave walks): 1 = 128 x 64 (8 waves, one workgroup per CU), 2 = 64 x 64 (4
// waves, two per CU), 3 = 64 x 64 split over K (8 waves in two groups, one
// workgroup per CU by LDS); ties go to the lower number.  The per-32 kernels'
// rule.
int q8k_tile_choice(int nt, int od, int id)
{
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

// type 1: Q4_K, 2: Q6_K, 3: Q6_K padded, 6: Q5_K (checked by the caller)
template <int WR, int WC, int KS, bool DUMP>
static hipError_t launch_q8k_tile(int type, const uint8_t* W, const int8_t* q, const float* d, const float* bsum,
                                  int nt, int od, int id, float* out, int32_t* S, hipStream_t st)
{
    const long tiles = (long)((nt + 32 * WC - 1) / (32 * WC)) * ((od + 32 * WR - 1) / (32 * WR));
    const long grid = (tiles + 7) / 8 * 8;  // a multiple of the 8 XCDs (xcd_tile drops the padding)
    const dim3 g((unsigned)grid), b(64 * WR * WC * KS);
    if (type == 1)
        hipLaunchKernelGGL((mmq_k4_q8k_kernel<WR, WC, KS, DUMP, false>), g, b, 0, st, W, q, d, bsum, out, nt, od, id,
                           S);
    else if (type == 6)
        hipLaunchKernelGGL((mmq_k4_q8k_kernel<WR, WC, KS, DUMP, true>), g, b, 0, st, W, q, d, bsum, out, nt, od, id,
                           S);
    else if (type == 2)
        hipLaunchKernelGGL((mmq_q6k_q8k_kernel<WR, WC, KS, DUMP, false>), g, b, 0, st, W, q, d, out, nt, od, id, S);
    else if (type == 3)
        hipLaunchKernelGGL((mmq_q6k_q8k_kernel<WR, WC, KS, DUMP, true>), g, b, 0, st, W, q, d, out, nt, od, id, S);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mmq_q8k(int type, const uint8_t* W, const int8_t* q, const float* d, const float* bsum, int nt,
                          int od, int id, float* out, int32_t* S, hipStream_t st, int tile)
{
    // Q4_K on the wave kernel with the scales in the int8 operand wherever there
    // are more than 256 of its 128 x 64 tiles (measured 6-9 % faster than the tile
    // the cost model picks there, the 64 x 64 split included; on fewer tiles it
    // holds one wave per SIMD and the staged kernels win)
    const long t128 = (long)((nt + 63) / 64) * ((od + 127) / 128);
    if (type == 1 && (tile == 4 || tile == 5 || (tile == 0 && t128 > 256)))
        return launch_mmq_k4_q8k_v2(W, q, d, bsum, nt, od, id, out, S, st, tile == 5 ? 2 : 1);
    if (S)
        return launch_q8k_tile<2, 2, 1, true>(type, W, q, d, bsum, nt, od, id, out, S, st);
    switch (tile ? tile : q8k_tile_choice(nt, od, id)) {
    case 1: return launch_q8k_tile<4, 2, 1, false>(type, W, q, d, bsum, nt, od, id, out, nullptr, st);
    case 2: return launch_q8k_tile<2, 2, 1, false>(type, W, q, d, bsum, nt, od, id, out, nullptr, st);
    default: return launch_q8k_tile<2, 2, 2, false>(type, W, q, d, bsum, nt, od, id, out, nullptr, st);
    }
}

}  // namespace qmm
