// MMQ for Q4_K weights on Q8_K activations (one activation scale per 256 values):
// the kernel of 4 waves x (32 rows x 64 tokens) per workgroup.
//
// [GEMM, "Activations: int8 with a scale per 256"] and [GEMM, "The zero points do
// not touch the inner loop"]: with one activation scale per super-block, the
// super-block's contribution to out[t][r] is
//   d[r] * dx[t] * S1 - dmin[r] * dx[t] * S2,
//   S1 = sum_j sc_j[r] * sum(q * qx),  S2 = sum_j m_j[r] * (bsum_2j + bsum_2j+1),
// both exact integers.
//
// MI355X mapping:
//  * The sub-block scale moves into the int8 operand.  sc_j = 8 a_j + b_j with
//    a_j, b_j in 0..7, so a_j * q and b_j * q are at most 15 * 7 = 105: int8.  Two
//    int32 accumulators chained through the MFMA over the eight sub-blocks,
//    Ca = sum_j sum((a_j q) qx) and Cb = sum_j sum((b_j q) qx), give
//    S1 = 8 Ca + Cb exactly (|S1| <= 63 * 256 * 15 * 127 < 2^31).  Per value and
//    sub-block nothing runs on the VALU; per sub-block each operand dword takes one
//    packed 16-bit multiply (four codes at once: no product reaches the next
//    byte).  The int8 MFMA count doubles and the kernel is bound by the MFMA pipe,
//    not by a VALU combine per value and sub-block.
//  * Workgroup of 4 waves = 128 rows x 64 tokens; wave w owns rows 32w .. 32w+31
//    and both 32-token blocks.  MFMA roles: A = activation codes (token =
//    lane % 32), B = weight codes (row = lane % 32), so a result lane holds one
//    weight row and 16 tokens.  A lane's weight codes never leave its wave: they go
//    from global memory straight into registers, two super-blocks ahead.
//  * Activation codes, group sums (f16), dx and the decoded per-row factors are
//    staged in LDS, double buffered, one barrier per super-block; the next
//    super-block's global loads are in flight meanwhile.
//  * Per super-block and token block: S2 on one f16 MFMA (exact: |bsum| <= 2032,
//    m <= 63, every partial sum an integer below 2^24), d*dx and -dmin*dx from one
//    pair of outer products, then per value one conversion and two FMAs.
//  * One workgroup per tile, tiles of one row block numbered onto one XCD.
#include "qmm_mmq_common.h"

namespace qmm {

namespace {

constexpr int kQ2BM = 128, kQ2BN = 64, kQ2NTH = 256;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

struct __attribute__((aligned(16))) Q2Stage {
    static constexpr int X_STRIDE = 272;   // 256 codes + 16 pad: 16-byte reads of 16 tokens hit 16 bank groups
    uint8_t xq[kQ2BN * X_STRIDE];          // activation codes [token][256]
    uint32_t sca[kQ2BM * 8];               // sc_j >> 3 [row][j]
    uint32_t scb[kQ2BM * 8];               // sc_j & 7 [row][j]
    _Float16 mn[kQ2BM * 16];               // m_{g/2} [row][g]
    _Float16 bs[kQ2BN * 16];               // group code sums [token][g]
    float dd[2 * kQ2BM];                   // [0][row] d, [1][row] -dmin
    float dx[kQ2BN];                       // activation scale [token]
};

// One thread's global loads of one super-block's staged data: 4 activation code
// pieces (token e/16, piece e%16, e = tid + 256k), 4 group sums (token tid/4,
// quarter tid%4), the activation scale of token min(tid, 63), and the 16-byte
// header of row tid/2.
struct Q2Pref {
    v4i x[4];
    v4i b;
    v4i h;
    uint32_t d;
};

struct Q2Offs {
    uint32_t x[4], b, h, d;
};

struct Q2Rsrc {
    __amdgpu_buffer_rsrc_t w, x, b, d;
};

__device__ __forceinline__ void q2_prefetch(Q2Pref& pf, const Q2Offs& o, const Q2Rsrc& rs, int sb)
{
#pragma unroll
    for (int k = 0; k < 4; ++k)
        pf.x[k] = bload16(rs.x, o.x[k], 256u * (uint32_t)sb);
    pf.b = bload16(rs.b, o.b, 64u * (uint32_t)sb);
    pf.h = bload16(rs.w, o.h, (uint32_t)sb * kQ4KBytes);
    pf.d = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs.d, (int)o.d, (int)(4u * (uint32_t)sb), 0);
}

// Store one super-block's prefetched data into a stage: codes as they are, group
// sums as f16 (exact small integers), dx as it is, and the header decoded to the
// per-row factors.  Thread (row r = tid/2, half h = tid%2) decodes sub-blocks 2h,
// 2h+1, 2h+4, 2h+5 and writes d (h = 0) or -dmin (h = 1).  valid == false (a
// super-block index past the end, in the split over K) stages d = dmin = 0: that
// super-block then adds nothing.
__device__ __forceinline__ void q2_stage(Q2Stage& st, const Q2Pref& pf, int tid, bool valid)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = tid + 256 * k;
        *reinterpret_cast<v4i*>(&st.xq[(e >> 4) * Q2Stage::X_STRIDE + 16 * (e & 15)]) = pf.x[k];
    }
    const h4 bh = {(_Float16)__int_as_float(pf.b.x), (_Float16)__int_as_float(pf.b.y),
                   (_Float16)__int_as_float(pf.b.z), (_Float16)__int_as_float(pf.b.w)};
    *reinterpret_cast<h4*>(&st.bs[(tid >> 2) * 16 + 4 * (tid & 3)]) = bh;
    st.dx[min(tid, kQ2BN - 1)] = __uint_as_float(pf.d);
    const int r = tid >> 1, hf = tid & 1;
    const uint32_t dbits = hf ? ((uint32_t)pf.h.x >> 16) : ((uint32_t)pf.h.x & 0xFFFF);
    const float dv = valid ? f16_bits_to_f32(dbits) : 0.f;
    st.dd[hf * kQ2BM + r] = hf ? -dv : dv;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int jj = 2 * hf + u;  // sub-blocks jj and jj + 4
        int sc0, m0, sc1, m1;
        q4k_scale_min_pair((uint32_t)pf.h.y, (uint32_t)pf.h.z, (uint32_t)pf.h.w, jj, sc0, m0, sc1, m1);
        st.sca[r * 8 + jj] = (uint32_t)(sc0 >> 3);
        st.scb[r * 8 + jj] = (uint32_t)(sc0 & 7);
        st.sca[r * 8 + jj + 4] = (uint32_t)(sc1 >> 3);
        st.scb[r * 8 + jj + 4] = (uint32_t)(sc1 & 7);
        const _Float16 f0 = (_Float16)m0, f1 = (_Float16)m1;
        const unsigned short b0 = __builtin_bit_cast(unsigned short, f0), b1 = __builtin_bit_cast(unsigned short, f1);
        *reinterpret_cast<uint32_t*>(&st.mn[r * 16 + 2 * jj]) = (uint32_t)b0 * 0x10001u;
        *reinterpret_cast<uint32_t*>(&st.mn[r * 16 + 2 * (jj + 4)]) = (uint32_t)b1 * 0x10001u;
    }
}

// The four 16-byte code pieces of this lane's weight row for super-block sb.
__device__ __forceinline__ void q2_load_w(v4i (&w)[4], __amdgpu_buffer_rsrc_t rw, uint32_t off, int sb)
{
#pragma unroll
    for (int p = 0; p < 4; ++p)
        w[p] = bload16(rw, off + 32u * (uint32_t)p, (uint32_t)sb * kQ4KBytes);
}

// Each byte of x times the small factor in the low half of s (products <= 105, so
// no byte carries into the next): one packed 16-bit multiply per dword.  The
// whole vector is reinterpreted at once (a bit cast of a single vector element
// reads element 0 with this compiler).
__device__ __forceinline__ v4i scale_codes(const v4i& x, uint32_t s)
{
    return __builtin_bit_cast(v4i, __builtin_bit_cast(u16x8, x) * (u16x8)(unsigned short)s);
}

// A VGPR holding v (kept out of constant operands: VALU instructions with a
// scalar or literal operand issue at half rate on this chip).
__device__ __forceinline__ uint32_t vgpr_u32_q2(uint32_t bits)
{
    uint32_t v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(bits));
    return v;
}

// The integer stage of one staged super-block for wave w: per sub-block pair p,
// the four scaled weight operands and eight int8 MFMAs into the chained
// accumulators ca[tb], cb[tb] (started at zero).
__device__ __forceinline__ void q2_products(const Q2Stage& st, const v4i (&w16)[4], uint32_t mask, int brow, int li,
                                            int lh, v16i (&ca)[2], v16i (&cb)[2])
{
    const v4i a03 = *reinterpret_cast<const v4i*>(&st.sca[brow * 8]);
    const v4i a47 = *reinterpret_cast<const v4i*>(&st.sca[brow * 8 + 4]);
    const v4i b03 = *reinterpret_cast<const v4i*>(&st.scb[brow * 8]);
    const v4i b47 = *reinterpret_cast<const v4i*>(&st.scb[brow * 8 + 4]);
    const int fa[8] = {a03.x, a03.y, a03.z, a03.w, a47.x, a47.y, a47.z, a47.w};
    const int fb[8] = {b03.x, b03.y, b03.z, b03.w, b47.x, b47.y, b47.z, b47.w};
    const uint8_t* x0p = &st.xq[li * Q2Stage::X_STRIDE + 16 * lh];
    const uint8_t* x1p = &st.xq[(32 + li) * Q2Stage::X_STRIDE + 16 * lh];
    const v16i z = {};
    // activation operands of sub-block j at bytes 32 j (token blocks 0 and 1),
    // read one sub-block ahead of their MFMAs
    v4i c0 = *reinterpret_cast<const v4i*>(x0p), c1 = *reinterpret_cast<const v4i*>(x1p);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const v4i x0 = c0, x1 = c1;
        if (j < 7) {
            c0 = *reinterpret_cast<const v4i*>(x0p + 32 * (j + 1));
            c1 = *reinterpret_cast<const v4i*>(x1p + 32 * (j + 1));
        }
        // sub-block j: low nibbles of piece j/2 for even j, high for odd j
        const v4i cw = (j & 1) ? ((w16[j >> 1] >> 4) & (int)mask) : (w16[j >> 1] & (int)mask);
        const v4i wa = scale_codes(cw, (uint32_t)fa[j]), wb = scale_codes(cw, (uint32_t)fb[j]);
        // four independent chains, each step four MFMAs after the last one
        ca[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x0, wa, j ? ca[0] : z, 0, 0, 0);
        cb[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x0, wb, j ? cb[0] : z, 0, 0, 0);
        ca[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x1, wa, j ? ca[1] : z, 0, 0, 0);
        cb[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x1, wb, j ? cb[1] : z, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One staged super-block for wave w: the integer stage, then S2 and the scale
// products per token block and the f32 update.  DUMP: write S1 and S2 instead
// (S [nt][od][nsb][2]).
template <bool DUMP>
__device__ __forceinline__ void q2_superblock(const Q2Stage& st, const v4i (&w16)[4], uint32_t mask, int w, int li,
                                              int lh, v16f (&acc)[2], int32_t* S, int nt, int od, int nsb, int sb,
                                              int row0, int tok0)
{
    const int brow = 32 * w + li;
    v16i ca[2], cb[2];
    q2_products(st, w16, mask, brow, li, lh, ca, cb);
    // S1 = 8 Ca + Cb for both token blocks first (frees the four accumulators)
    const v16i s1v[2] = {(ca[0] << 3) + cb[0], (ca[1] << 3) + cb[1]};
    __builtin_amdgcn_sched_barrier(0);
    const h8 mnv = *reinterpret_cast<const h8*>(&st.mn[brow * 16 + 8 * lh]);
    const float ddv = st.dd[lh * kQ2BM + brow];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const h8 bsv = *reinterpret_cast<const h8*>(&st.bs[(32 * tb + li) * 16 + 8 * lh]);
        const v16f zf = {};
        const v16f cmin = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsv, mnv, zf, 0, 0, 0);
        const v16i& s1 = s1v[tb];
        if constexpr (DUMP) {
            const int r = row0 + brow;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = tok0 + 32 * tb + 8 * (i >> 2) + 4 * lh + (i & 3);
                if (t < nt && r < od && sb < nsb) {
                    int32_t* dst = S + (((size_t)t * od + r) * nsb + sb) * 2;
                    dst[0] = s1[i];
                    dst[1] = (int32_t)cmin[i];
                }
            }
        } else {
            // registers 0..15: d * dx, 16..31: -dmin * dx (this lane's row, its tokens)
            const v32f pp = mfma_outer2(st.dx[32 * tb + li], ddv);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc[tb][i] = fmaf(pp[i], (float)s1[i], acc[tb][i]);
                acc[tb][i] = fmaf(pp[16 + i], cmin[i], acc[tb][i]);
            }
        }
    }
}

// Result tile of one wave and token block: lane holds weight row r and tokens
// t0 + 8k + 4 lh + i (k = 0..3, i = 0..3) in v[4k + i]; store into out [nt][od].
__device__ __forceinline__ void q2_store(const v16f& v, float* __restrict__ out, int nt, int od, int t0, int r, int lh)
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

// KS = 2: two groups of 4 waves in one workgroup split K (group g takes
// super-blocks g, g + 2, ...; each group has its own LDS stages); at the end the
// second group's partial tiles are added to the first's in a fixed order.
template <int KS, bool DUMP>
__global__ __launch_bounds__(kQ2NTH * KS, KS == 1 ? 2 : 1) void mmq_k4_q8k_v2_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    const float* __restrict__ bsum, float* __restrict__ out, int nt, int od, int id, int32_t* __restrict__ S)
{
    static_assert(!DUMP || KS == 1, "the integer-stage dump runs unsplit");
    __shared__ Q2Stage stg[KS][2];
    static_assert(KS == 1 || sizeof(stg) >= 4 * 2 * 1024 * sizeof(float), "the combine fits the stages");
    const int ntb = (nt + kQ2BN - 1) / kQ2BN;
    const int ntiles = ntb * ((od + kQ2BM - 1) / kQ2BM);
    const int tile = xcd_tile(ntiles);
    if (tile < 0)
        return;  // whole workgroup
    const int nsb = id >> 8, ngs = id >> 4;
    const int kg = KS > 1 ? (int)(threadIdx.x >> 8) : 0;
    const int tid = threadIdx.x & 255, lane = tid & 63, w = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int niter = (nsb + KS - 1) / KS;   // the same count for every group (barriers)
    const uint32_t row_bytes = (uint32_t)nsb * kQ4KBytes;
    const uint32_t mask = vgpr_u32_q2(0x0F0F0F0Fu);
    const int row0 = (tile / ntb) * kQ2BM, tok0 = (tile % ntb) * kQ2BN;

    // per-thread offsets (rows past od / tokens past nt read the last valid one)
    Q2Offs o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = tid + 256 * k;
        o.x[k] = (uint32_t)(min(tok0 + (e >> 4), nt - 1) - tok0) * (uint32_t)id + 16u * (uint32_t)(e & 15);
    }
    o.b = ((uint32_t)(min(tok0 + (tid >> 2), nt - 1) - tok0) * (uint32_t)ngs + 4u * (uint32_t)(tid & 3)) * 4u;
    o.d = (uint32_t)(min(tok0 + min(tid, kQ2BN - 1), nt - 1) - tok0) * (uint32_t)nsb * 4u;
    o.h = (uint32_t)(min(row0 + (tid >> 1), od - 1) - row0) * row_bytes;
    Q2Rsrc rs;
    rs.w = buffer_rsrc(W + (size_t)row0 * row_bytes, (size_t)(od - row0) * row_bytes);
    rs.x = buffer_rsrc(q + (size_t)tok0 * id, (size_t)(nt - tok0) * id);
    rs.b = buffer_rsrc(bsum + (size_t)tok0 * ngs, (size_t)(nt - tok0) * ngs * 4);
    rs.d = buffer_rsrc(dx + (size_t)tok0 * nsb, (size_t)(nt - tok0) * nsb * 4);
    const uint32_t ow = (uint32_t)(min(row0 + 32 * w + li, od - 1) - row0) * row_bytes + 16u + 16u * (uint32_t)lh;
    Q2Stage* sg = stg[kg];
    // this group's super-block of local iteration it, and its clamped load index
    auto sbi = [&](int it) { return it * KS + kg; };
    auto ld = [&](int it) { return min(sbi(it), nsb - 1); };

    Q2Pref pf;
    v4i wA[4], wB[4];
    v16f acc[2] = {{}, {}};
    q2_prefetch(pf, o, rs, ld(0));
    q2_load_w(wA, rs.w, ow, ld(0));
    q2_stage(sg[0], pf, tid, sbi(0) < nsb);
    q2_prefetch(pf, o, rs, ld(1));
    q2_load_w(wB, rs.w, ow, ld(1));
    __syncthreads();
    // two iterations per trip so the weight registers alternate without copies;
    // the prefetch indices are clamped to the last super-block (no load under a
    // branch)
    for (int it = 0; it < niter; it += 2) {
        q2_superblock<DUMP>(sg[0], wA, mask, w, li, lh, acc, S, nt, od, nsb, sbi(it), row0, tok0);
        __builtin_amdgcn_sched_barrier(0);
        q2_stage(sg[1], pf, tid, sbi(it + 1) < nsb);
        q2_prefetch(pf, o, rs, ld(it + 2));
        q2_load_w(wA, rs.w, ow, ld(it + 2));
        __syncthreads();
        if (it + 1 >= niter)
            break;
        q2_superblock<DUMP>(sg[1], wB, mask, w, li, lh, acc, S, nt, od, nsb, sbi(it + 1), row0, tok0);
        __builtin_amdgcn_sched_barrier(0);
        q2_stage(sg[0], pf, tid, sbi(it + 2) < nsb);
        q2_prefetch(pf, o, rs, ld(it + 3));
        q2_load_w(wB, rs.w, ow, ld(it + 3));
        __syncthreads();
    }
    if constexpr (!DUMP) {
        if constexpr (KS == 2) {
            // every wave is past the last barrier of the loop: the stages are free
            float* red = reinterpret_cast<float*>(&stg[0][0]);
            if (kg == 1) {
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        red[((w * 2 + tb) * 16 + i) * 64 + lane] = acc[tb][i];
            }
            __syncthreads();
            if (kg == 1)
                return;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[tb][i] += red[((w * 2 + tb) * 16 + i) * 64 + lane];
        }
        q2_store(acc[0], out, nt, od, tok0, row0 + 32 * w + li, lh);
        q2_store(acc[1], out, nt, od, tok0 + 32, row0 + 32 * w + li, lh);
    }
}

}  // namespace

hipError_t launch_mmq_k4_q8k_v2(const uint8_t* W, const int8_t* q, const float* d, const float* bsum, int nt, int od,
                                int id, float* out, int32_t* S, hipStream_t st, int ks)
{
    const int ntiles = ((nt + kQ2BN - 1) / kQ2BN) * ((od + kQ2BM - 1) / kQ2BM);
    const dim3 grid((unsigned)(8 * ((ntiles + 7) / 8)));
    if (S)
        hipLaunchKernelGGL((mmq_k4_q8k_v2_kernel<1, true>), grid, dim3(kQ2NTH), 0, st, W, q, d, bsum, out, nt, od, id,
                           S);
    else if (ks == 2)
        hipLaunchKernelGGL((mmq_k4_q8k_v2_kernel<2, false>), grid, dim3(2 * kQ2NTH), 0, st, W, q, d, bsum, out, nt,
                           od, id, S);
    else
        hipLaunchKernelGGL((mmq_k4_q8k_v2_kernel<1, false>), grid, dim3(kQ2NTH), 0, st, W, q, d, bsum, out, nt, od,
                           id, S);
    return hipGetLastError();
}

}  // namespace qmm
