// MMQ for Q4_K weights on per-32 activations, nt > 8 tokens: the int8-MFMA matrix
// kernel the dispatcher runs for Q4_K prefill shapes.
//
// [GEMM, "The GPU path", "One mma per scale group"]: one int8 matrix op per
// 32-weight sub-block, the int32 result taken to f32 with the two scales, and the
// min term; [GEMM, "Q4_K: packed in shared memory, unpacked in registers"]: the
// 16-byte code piece of a sub-block pair feeds two matrix ops (low and high
// nibbles); [GEMM, "Prefetching the next super-block"]: the next super-block is
// read into registers while the current one computes; [MMQ, section 6]: per-32
// rescale acc += (d*sc)*dx*C - (dmin*m)*s in f32; [MMQ, section 11.4]: codes 0..15
// enter the integer op uncentred.
//
// MI355X mapping (measured on this chip: v_cvt_f32_i32 issues at a quarter of the
// rate of an f32 fma with VGPR operands, MFMA and VALU work of the two waves on a
// SIMD overlap, and the per-32 epilogue -- one rescale per 32 int8 MACs -- bounds
// the kernel):
//  * Workgroup of 4 waves = a tile of 128 rows x 64 tokens; wave w owns rows
//    32w .. 32w+31 and both 32-token blocks, so one unpacked A operand (the wave's
//    own weight rows) feeds two int8 MFMAs (v_mfma_i32_32x32x32_i8, K = 32 = one
//    sub-block).  A lane's codes never leave its wave, so they go from global
//    memory straight into registers (no LDS): lane (row li, half lh) loads the four
//    16-byte pieces 16*lh of the super-block's 32-byte code chunks.
//  * The activation codes, activation d and s, and the decoded per-row factors
//    (d*sc_j and -dmin*m_j) are staged in LDS, double buffered, one barrier per
//    super-block; the next super-block's global loads are in flight meanwhile.
//  * The int8 accumulator starts at the bit pattern of 1.5 * 2^23, so the int32
//    result C = S + 0x4B400000 read as f32 is exactly 12582912 + S (|S| <= 60960):
//    one exact v_sub_f32 recovers S as f32 instead of a quarter-rate conversion.
//    Per output element and sub-block the VALU then does one subtraction and one
//    fma with the scale product P = (d*sc_j)[row] * dx_j[token], which one
//    v_mfma_f32_32x32x1_2b_f32 forms for both token blocks.
//  * The min term sum_j (-dmin*m_j)[row] * s_j[token] goes straight into the
//    accumulators once per super-block on three bf16 MFMAs over exact three-part
//    splits of both factors (the six part products above 2^-24 of the product).
//  * One workgroup per tile, tiles of one row block numbered onto one XCD.
#include "qmm_mmq_common.h"

namespace qmm {

namespace {

constexpr int kK4BM = 128, kK4BN = 64, kK4NTH = 256;
constexpr uint32_t kMagicBits = 0x4B400000u;  // 1.5 * 2^23 as f32: integer steps of 1 in its mantissa

struct __attribute__((aligned(16))) K4Stage {
    static constexpr int X_STRIDE = 272;   // 256 codes + 16 pad: 16-byte reads of 16 rows hit 16 bank groups
    uint8_t xq[kK4BN * X_STRIDE];          // activation codes [token][256]
    float xd[8 * kK4BN];                   // activation d [j][token]
    uint16_t xs3[3 * kK4BN * 8];           // activation s, three bf16 parts [part][token][j]
    float wsc[kK4BM * 8];                  // d * sc_j [row][j]
    uint16_t wmn3[3 * kK4BM * 8];          // -dmin * m_j, three bf16 parts [part][row][j]
};

// v as three bf16 parts (bit patterns) whose sum is v exactly for a normal v:
// each part is the next 8 significant bits, cut by truncation.
struct Split3 {
    uint32_t p[3];
};

__device__ __forceinline__ Split3 split3(float v)
{
    const uint32_t u0 = __float_as_uint(v);
    const float r1 = v - __uint_as_float(u0 & 0xFFFF0000u);
    const uint32_t u1 = __float_as_uint(r1);
    const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);
    return {{u0 >> 16, u1 >> 16, __float_as_uint(r2) >> 16}};
}

// One thread's global loads of one super-block's staged data: 4 activation code
// pieces (token e/16, piece e%16, e = tid + 256k), one 16-byte piece of activation
// d (waves 0-1) or s (waves 2-3) of token t/2, half t%2 (t = tid % 128), and the
// 16-byte header of row tid/2.
struct K4Pref {
    v4i x[4];
    v4i ds;
    v4i h;
};

struct K4Offs {
    uint32_t x[4], ds, h;
};

struct K4Rsrc {
    __amdgpu_buffer_rsrc_t w, x, ds;
};

__device__ __forceinline__ void k4_prefetch(K4Pref& pf, const K4Offs& o, const K4Rsrc& rs, int sb, int nblk)
{
    (void)nblk;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        pf.x[k] = bload16(rs.x, o.x[k], 256u * (uint32_t)sb);
    pf.ds = bload16(rs.ds, o.ds, 32u * (uint32_t)sb);
    pf.h = bload16(rs.w, o.h, (uint32_t)sb * kQ4KBytes);
}

// Store one super-block's prefetched data into a stage: codes as they are, d as it
// is, s split in three bf16 parts, and the header decoded to the per-row factors.
// Thread (row r = tid/2, half h = tid%2) decodes sub-blocks 2h, 2h+1, 2h+4, 2h+5.
__device__ __forceinline__ void k4_stage(K4Stage& st, const K4Pref& pf, int tid, bool valid)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = tid + 256 * k;
        *reinterpret_cast<v4i*>(&st.xq[(e >> 4) * K4Stage::X_STRIDE + 16 * (e & 15)]) = pf.x[k];
    }
    const int t = (tid & 127) >> 1, hf = tid & 1;
    if (tid < 128) {
        st.xd[(4 * hf + 0) * kK4BN + t] = __int_as_float(pf.ds.x);
        st.xd[(4 * hf + 1) * kK4BN + t] = __int_as_float(pf.ds.y);
        st.xd[(4 * hf + 2) * kK4BN + t] = __int_as_float(pf.ds.z);
        st.xd[(4 * hf + 3) * kK4BN + t] = __int_as_float(pf.ds.w);
    } else {
        const Split3 s0 = split3(__int_as_float(pf.ds.x)), s1 = split3(__int_as_float(pf.ds.y));
        const Split3 s2 = split3(__int_as_float(pf.ds.z)), s3 = split3(__int_as_float(pf.ds.w));
#pragma unroll
        for (int pt = 0; pt < 3; ++pt)
            *reinterpret_cast<uint2*>(&st.xs3[(pt * kK4BN + t) * 8 + 4 * hf]) =
                make_uint2(s0.p[pt] | (s1.p[pt] << 16), s2.p[pt] | (s3.p[pt] << 16));
    }
    const int r = tid >> 1;
    // valid == false (a super-block past the end in the split over K): zero row
    // factors, so that super-block adds nothing
    const float dw = valid ? f16_bits_to_f32((uint32_t)pf.h.x & 0xFFFF) : 0.f;
    const float dm = valid ? f16_bits_to_f32((uint32_t)pf.h.x >> 16) : 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int jj = 2 * hf + u;  // sub-blocks jj and jj + 4
        int sc0, m0, sc1, m1;
        q4k_scale_min_pair((uint32_t)pf.h.y, (uint32_t)pf.h.z, (uint32_t)pf.h.w, jj, sc0, m0, sc1, m1);
        st.wsc[r * 8 + jj] = dw * (float)sc0;
        st.wsc[r * 8 + jj + 4] = dw * (float)sc1;
        const Split3 a = split3(-(dm * (float)m0)), b = split3(-(dm * (float)m1));
#pragma unroll
        for (int pt = 0; pt < 3; ++pt) {
            st.wmn3[(pt * kK4BM + r) * 8 + jj] = (uint16_t)a.p[pt];
            st.wmn3[(pt * kK4BM + r) * 8 + jj + 4] = (uint16_t)b.p[pt];
        }
    }
}

// The four 16-byte code pieces of this lane's weight row for super-block sb.
__device__ __forceinline__ void k4_load_a(v4i (&a)[4], __amdgpu_buffer_rsrc_t w, uint32_t off, int sb)
{
#pragma unroll
    for (int p = 0; p < 4; ++p)
        a[p] = bload16(w, off + 32u * (uint32_t)p, (uint32_t)sb * kQ4KBytes);
}

// A VGPR holding v (the compiler cannot fold it back into a constant operand: VALU
// instructions with a constant or scalar operand issue at half rate on this chip).
__device__ __forceinline__ float vgpr_f32(uint32_t bits)
{
    float v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(bits));
    return v;
}

__device__ __forceinline__ uint32_t vgpr_u32(uint32_t bits)
{
    uint32_t v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(bits));
    return v;
}

// The compute of one staged super-block for wave w: 8 sub-blocks x 2 token blocks of
// int8 MFMAs, their epilogue, then the min term.  DUMP: write the integer dots
// instead (S [nt][od][nsb][8]).
template <bool DUMP>
__device__ __forceinline__ void k4_superblock(const K4Stage& st, const v4i (&a16)[4], const v16i& magic, float Mv,
                                              uint32_t mask, int w, int li, int lh, v16f& acc0, v16f& acc1,
                                              int32_t* S, int nt, int od, int nsb, int sb, int row0, int tok0)
{
    const int arow = 32 * w + li;
    const float4 aw0 = *reinterpret_cast<const float4*>(&st.wsc[arow * 8]);
    const float4 aw1 = *reinterpret_cast<const float4*>(&st.wsc[arow * 8 + 4]);
    const float aw[8] = {aw0.x, aw0.y, aw0.z, aw0.w, aw1.x, aw1.y, aw1.z, aw1.w};
    const uint8_t* xb0 = &st.xq[li * K4Stage::X_STRIDE + 16 * lh];
    const uint8_t* xb1 = &st.xq[(32 + li) * K4Stage::X_STRIDE + 16 * lh];
    const float* xdl = &st.xd[32 * lh + li];
    // the LDS operands of sub-block j + 1 are read while sub-block j computes
    v4i nb0 = *reinterpret_cast<const v4i*>(xb0), nb1 = *reinterpret_cast<const v4i*>(xb1);
    float ndx = xdl[0];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const v4i& c = a16[j >> 1];
        const v4i a = (j & 1) ? ((c >> 4) & (int)mask) : (c & (int)mask);
        const v4i b0 = nb0, b1 = nb1;
        const float dxv = ndx;
        if (j < 7) {
            nb0 = *reinterpret_cast<const v4i*>(xb0 + 32 * (j + 1));
            nb1 = *reinterpret_cast<const v4i*>(xb1 + 32 * (j + 1));
            ndx = xdl[(j + 1) * kK4BN];
        }
        if constexpr (DUMP) {
            const v16i C0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, magic, 0, 0, 0);
            const v16i C1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, magic, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int rg = row0 + arow - li + 8 * (i >> 2) + 4 * lh + (i & 3);
                const int t0 = tok0 + li, t1 = tok0 + 32 + li;
                if (rg < od && t0 < nt)
                    S[(((size_t)t0 * od + rg) * nsb + sb) * 8 + j] = C0[i] - (int)kMagicBits;
                if (rg < od && t1 < nt)
                    S[(((size_t)t1 * od + rg) * nsb + sb) * 8 + j] = C1[i] - (int)kMagicBits;
            }
        } else {
            const v32f P = mfma_outer2(aw[j], dxv);
            const v16i C0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, magic, 0, 0, 0);
            const v16i C1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, magic, 0, 0, 0);
            // S = C - 12582912 in f32 (exact), as whole-vector subtractions so the
            // 32 of them are independent of each other, then 32 independent fmas
            const v16f S0 = __builtin_bit_cast(v16f, C0) - Mv;
            const v16f S1 = __builtin_bit_cast(v16f, C1) - Mv;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc0[i] = fmaf(S0[i], P[i], acc0[i]);
                acc1[i] = fmaf(S1[i], P[16 + i], acc1[i]);
            }
        }
        // one sub-block's results live at a time
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!DUMP) {
        // min term: part pair q = 2 m + lh pairs row part kRowPart[q] with token part kTokPart[q]
        constexpr int kRowPart[6] = {0, 0, 1, 0, 1, 2};
        constexpr int kTokPart[6] = {0, 1, 0, 2, 1, 0};
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int q = 2 * m + lh;
            const v8bf A = *reinterpret_cast<const v8bf*>(&st.wmn3[(kRowPart[q] * kK4BM + arow) * 8]);
            const v8bf B0 = *reinterpret_cast<const v8bf*>(&st.xs3[(kTokPart[q] * kK4BN + li) * 8]);
            const v8bf B1 = *reinterpret_cast<const v8bf*>(&st.xs3[(kTokPart[q] * kK4BN + 32 + li) * 8]);
            acc0 = mfma_bf16_k16(A, B0, acc0);
            acc1 = mfma_bf16_k16(A, B1, acc1);
        }
    }
}

// The kernel body for one whole tile: rows row0 .. row0 + 127 and tokens tok0 ..
// tok0 + 63 over all super-blocks.  KS = 2: two groups of 4 waves split K (group g
// takes super-blocks g, g + 2, ..., each group with its own stages); the second
// group's partial tiles are added to the first's in a fixed order at the end.
template <int KS, bool DUMP>
__device__ __forceinline__ void k4_tile(const uint8_t* __restrict__ W, const int8_t* __restrict__ q,
                                        const float* __restrict__ dx, const float* __restrict__ sx,
                                        float* __restrict__ out, int nt, int od, int id, int tile,
                                        int32_t* __restrict__ S)
{
    __shared__ K4Stage stg[KS][2];
    static_assert(KS == 1 || sizeof(stg) >= 4 * 2 * 1024 * sizeof(float), "the combine fits the stages");
    const int ntb = (nt + kK4BN - 1) / kK4BN;
    const int nsb = id >> 8, nblk = id >> 5;
    const int kg = KS > 1 ? (int)(threadIdx.x >> 8) : 0;
    const int tid = threadIdx.x & 255, lane = tid & 63, w = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int niter = (nsb + KS - 1) / KS;   // the same count for every group (barriers)
    const uint32_t row_bytes = (uint32_t)nsb * kQ4KBytes;
    const float Mv = vgpr_f32(kMagicBits);
    const uint32_t mask = vgpr_u32(0x0F0F0F0Fu);
    v16i magic;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        magic[i] = (int)__float_as_uint(Mv);
    const int row0 = (tile / ntb) * kK4BM, tok0 = (tile % ntb) * kK4BN;

    // per-thread offsets (rows past od / tokens past nt read the last valid one)
    K4Offs o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = tid + 256 * k;
        o.x[k] = (uint32_t)(min(tok0 + (e >> 4), nt - 1) - tok0) * (uint32_t)id + 16u * (uint32_t)(e & 15);
    }
    const int tds = (tid & 127) >> 1;
    o.ds = ((uint32_t)(min(tok0 + tds, nt - 1) - tok0) * (uint32_t)nblk + 4u * (uint32_t)(tid & 1)) * 4u;
    o.h = (uint32_t)(min(row0 + (tid >> 1), od - 1) - row0) * row_bytes;
    K4Rsrc rs;
    rs.w = buffer_rsrc(W + (size_t)row0 * row_bytes, (size_t)(od - row0) * row_bytes);
    rs.x = buffer_rsrc(q + (size_t)tok0 * id, (size_t)(nt - tok0) * id);
    // waves 0-1 of a group stage d, waves 2-3 stage s: a wave-uniform choice, made
    // scalar so the buffer resource stays in scalar registers
    const uintptr_t pds = reinterpret_cast<uintptr_t>(tid < 128 ? dx : sx);
    const uintptr_t pdsu = ((uintptr_t)__builtin_amdgcn_readfirstlane((uint32_t)(pds >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)pds);
    rs.ds = buffer_rsrc(reinterpret_cast<const float*>(pdsu) + (size_t)tok0 * nblk, (size_t)(nt - tok0) * nblk * 4);
    const uint32_t oa = (uint32_t)(min(row0 + 32 * w + li, od - 1) - row0) * row_bytes + 16u + 16u * (uint32_t)lh;
    K4Stage* sg = stg[kg];
    // this group's super-block of local iteration it, and its clamped load index
    auto sbi = [&](int it) { return it * KS + kg; };
    auto ld = [&](int it) { return min(sbi(it), nsb - 1); };

    K4Pref pf;
    v4i aA[4], aB[4];
    v16f acc0 = {}, acc1 = {};
    k4_prefetch(pf, o, rs, ld(0), nblk);
    k4_load_a(aA, rs.w, oa, ld(0));
    k4_stage(sg[0], pf, tid, sbi(0) < nsb);
    k4_prefetch(pf, o, rs, ld(1), nblk);
    k4_load_a(aB, rs.w, oa, ld(1));
    __syncthreads();
    // two iterations per trip so the A registers alternate without copies; the
    // prefetch indices are clamped to the last super-block (no load under a branch)
    for (int it = 0; it < niter; it += 2) {
        k4_superblock<DUMP>(sg[0], aA, magic, Mv, mask, w, li, lh, acc0, acc1, S, nt, od, nsb, sbi(it), row0, tok0);
        __builtin_amdgcn_sched_barrier(0);
        k4_stage(sg[1], pf, tid, sbi(it + 1) < nsb);
        k4_prefetch(pf, o, rs, ld(it + 2), nblk);
        k4_load_a(aA, rs.w, oa, ld(it + 2));
        __syncthreads();
        if (it + 1 >= niter)
            break;
        k4_superblock<DUMP>(sg[1], aB, magic, Mv, mask, w, li, lh, acc0, acc1, S, nt, od, nsb, sbi(it + 1), row0,
                            tok0);
        __builtin_amdgcn_sched_barrier(0);
        k4_stage(sg[0], pf, tid, sbi(it + 2) < nsb);
        k4_prefetch(pf, o, rs, ld(it + 3), nblk);
        k4_load_a(aB, rs.w, oa, ld(it + 3));
        __syncthreads();
    }
    if constexpr (!DUMP) {
        if constexpr (KS == 2) {
            // every wave is past the last barrier of the loop: the stages are free
            float* red = reinterpret_cast<float*>(&stg[0][0]);
            if (kg == 1) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    red[((w * 2 + 0) * 16 + i) * 64 + lane] = acc0[i];
                    red[((w * 2 + 1) * 16 + i) * 64 + lane] = acc1[i];
                }
            }
            __syncthreads();
            if (kg == 1)
                return;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc0[i] += red[((w * 2 + 0) * 16 + i) * 64 + lane];
                acc1[i] += red[((w * 2 + 1) * 16 + i) * 64 + lane];
            }
        }
        store_tile(acc0, out, nt, od, tok0 + li, row0 + 32 * w, lh);
        store_tile(acc1, out, nt, od, tok0 + 32 + li, row0 + 32 * w, lh);
    }
}

// One tile per workgroup (tiles of one row block on one XCD).
template <int KS, bool DUMP>
__global__ __launch_bounds__(kK4NTH * KS, KS == 1 ? 2 : 1) void mmq_q4k_v2_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ q, const float* __restrict__ dx,
    const float* __restrict__ sx, float* __restrict__ out, int nt, int od, int id, int32_t* __restrict__ S)
{
    static_assert(!DUMP || KS == 1, "the integer dump runs unsplit");
    const int ntiles = ((nt + kK4BN - 1) / kK4BN) * ((od + kK4BM - 1) / kK4BM);
    const int tile = xcd_tile(ntiles);
    if (tile < 0)
        return;  // whole workgroup
    k4_tile<KS, DUMP>(W, q, dx, sx, out, nt, od, id, tile, S);
}

}  // namespace

hipError_t launch_mmq_q4k_v2(const uint8_t* W, const int8_t* q, const float* d, const float* s, int nt, int od,
                             int id, float* out, int32_t* S, hipStream_t st, int ks)
{
    const int ntiles = ((nt + kK4BN - 1) / kK4BN) * ((od + kK4BM - 1) / kK4BM);
    const dim3 grid((unsigned)(8 * ((ntiles + 7) / 8)));
    if (S)
        hipLaunchKernelGGL((mmq_q4k_v2_kernel<1, true>), grid, dim3(kK4NTH), 0, st, W, q, d, s, out, nt, od, id, S);
    else if (ks == 2)
        hipLaunchKernelGGL((mmq_q4k_v2_kernel<2, false>), grid, dim3(2 * kK4NTH), 0, st, W, q, d, s, out, nt, od, id,
                           S);
    else
        hipLaunchKernelGGL((mmq_q4k_v2_kernel<1, false>), grid, dim3(kK4NTH), 0, st, W, q, d, s, out, nt, od, id, S);
    return hipGetLastError();
}

}  // namespace qmm
