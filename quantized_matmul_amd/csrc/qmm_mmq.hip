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
//
// MI355X mapping:
//  * Workgroup tile BM rows x BN tokens, 256 threads = 4 waves in a 2 x 2 grid,
//    each wave (BM/2) x (BN/2) in 32 x 32 MFMA blocks.
//  * v_mfma_i32_32x32x32_i8: K = 32 is exactly one Q4_K sub-block.  Operand A =
//    32 weight rows x 32 codes, B = 32 codes x 32 tokens; lane l supplies row/token
//    l%32 and K positions 16*(l/32) .. +15 for both operands (any common K order
//    gives the same dot).  Result lane l: token l%32, rows 8*(i/4)+4*(l/32)+i%4 for
//    accumulator i.  Q6_K groups of 16 use v_mfma_i32_32x32x16_i8 (8 K bytes per lane).
//  * Per super-block: stage raw code bytes (rows padded to keep 16-byte LDS reads
//    conflict-free), decoded per-(row, group) f32 scales, activation codes and
//    activation scales into LDS with 16-byte global loads; barrier; MFMA + f32
//    epilogue; barrier.
#include "qmm_internal.h"

namespace qmm {

typedef long v1l;

template <int BM, int BN>
struct __attribute__((aligned(16))) Q4Smem {
    static constexpr int QS_STRIDE = 144;   // 128 code bytes + 16 pad
    static constexpr int X_STRIDE = 272;    // 256 activation codes + 16 pad
    uint8_t qs[BM * QS_STRIDE];
    float wsc[8 * BM];                      // d * sc_j, [j][row]
    float wmn[8 * BM];                      // dmin * m_j, [j][row]
    uint8_t xq[BN * X_STRIDE];
    float xd[8 * BN];                       // activation d, [j][token]
    float xs[8 * BN];                       // activation s, [j][token]
};

template <int BM, int BN, bool DUMP>
__global__ __launch_bounds__(256) void mmq_q4k_kernel(const uint8_t* __restrict__ W,
                                                      const int8_t* __restrict__ q,
                                                      const float* __restrict__ dx,
                                                      const float* __restrict__ sx,
                                                      float* __restrict__ out, int nt, int od,
                                                      int id, int32_t* __restrict__ S)
{
    using SM = Q4Smem<BM, BN>;
    __shared__ SM sm;
    constexpr int MR = BM / 64;   // 32-row blocks per wave
    constexpr int NC = BN / 64;   // 32-token blocks per wave
    static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int li = lane & 31, lh = lane >> 5;
    const int row0 = blockIdx.y * BM;
    const int tok0 = blockIdx.x * BN;
    const int nsb = id >> 8;
    const int nblk = id >> 5;

    float acc[MR][NC][16];
#pragma unroll
    for (int a = 0; a < MR; ++a)
#pragma unroll
        for (int b = 0; b < NC; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc[a][b][i] = 0.f;

    for (int sb = 0; sb < nsb; ++sb) {
        // ---- stage weights: BM rows, 4 threads per row per pass
        for (int e = tid; e < BM * 4; e += 256) {
            const int r = e >> 2, part = e & 3;
            const int rg = min(row0 + r, od - 1);
            const uint8_t* blk = W + ((size_t)rg * nsb + sb) * kQ4KBytes;
            const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
            const uint4 c0 = *reinterpret_cast<const uint4*>(blk + 16 + 16 * part);
            const uint4 c1 = *reinterpret_cast<const uint4*>(blk + 16 + 16 * (part + 4));
            *reinterpret_cast<uint4*>(&sm.qs[r * SM::QS_STRIDE + 16 * part]) = c0;
            *reinterpret_cast<uint4*>(&sm.qs[r * SM::QS_STRIDE + 16 * (part + 4)]) = c1;
            const float dw = f16_bits_to_f32(hdr.x & 0xFFFF);
            const float dm = f16_bits_to_f32(hdr.x >> 16);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int j = 2 * part + u;
                int sc, m;
                q4k_scale_min(hdr.y, hdr.z, hdr.w, j, sc, m);
                sm.wsc[j * BM + r] = dw * (float)sc;
                sm.wmn[j * BM + r] = dm * (float)m;
            }
        }
        // ---- stage activations: BN tokens x 16 pieces of 16 bytes
        for (int e = tid; e < BN * 16; e += 256) {
            const int t = e >> 4, part = e & 15;
            const int tg = tok0 + t;
            int4 v = make_int4(0, 0, 0, 0);
            if (tg < nt)
                v = *reinterpret_cast<const int4*>(q + (size_t)tg * id + 256 * sb + 16 * part);
            *reinterpret_cast<int4*>(&sm.xq[t * SM::X_STRIDE + 16 * part]) = v;
        }
        for (int e = tid; e < BN * 2; e += 256) {
            const int t = e >> 1, hf = e & 1;
            const int tg = tok0 + t;
            float4 vd = make_float4(0.f, 0.f, 0.f, 0.f), vs = vd;
            if (tg < nt) {
                vd = *reinterpret_cast<const float4*>(dx + (size_t)tg * nblk + 8 * sb + 4 * hf);
                vs = *reinterpret_cast<const float4*>(sx + (size_t)tg * nblk + 8 * sb + 4 * hf);
            }
            sm.xd[(4 * hf + 0) * BN + t] = vd.x;
            sm.xd[(4 * hf + 1) * BN + t] = vd.y;
            sm.xd[(4 * hf + 2) * BN + t] = vd.z;
            sm.xd[(4 * hf + 3) * BN + t] = vd.w;
            sm.xs[(4 * hf + 0) * BN + t] = vs.x;
            sm.xs[(4 * hf + 1) * BN + t] = vs.y;
            sm.xs[(4 * hf + 2) * BN + t] = vs.z;
            sm.xs[(4 * hf + 3) * BN + t] = vs.w;
        }
        __syncthreads();

        // ---- compute
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint4 A16[MR];
#pragma unroll
            for (int a = 0; a < MR; ++a) {
                const int r = wr * (BM / 2) + 32 * a + li;
                A16[a] = *reinterpret_cast<const uint4*>(&sm.qs[r * SM::QS_STRIDE + 32 * p + 16 * lh]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int j = 2 * p + u;
                v4i Bv[NC];
#pragma unroll
                for (int b = 0; b < NC; ++b) {
                    const int t = wc * (BN / 2) + 32 * b + li;
                    const int4 bq = *reinterpret_cast<const int4*>(&sm.xq[t * SM::X_STRIDE + 32 * j + 16 * lh]);
                    Bv[b] = v4i{bq.x, bq.y, bq.z, bq.w};
                }
#pragma unroll
                for (int a = 0; a < MR; ++a) {
                    const uint32_t sh = 4 * u;
                    const v4i Av = v4i{(int)((A16[a].x >> sh) & 0x0F0F0F0Fu), (int)((A16[a].y >> sh) & 0x0F0F0F0Fu),
                                       (int)((A16[a].z >> sh) & 0x0F0F0F0Fu), (int)((A16[a].w >> sh) & 0x0F0F0F0Fu)};
                    // weight scales of this lane's 16 rows
                    const int rbase = wr * (BM / 2) + 32 * a + 4 * lh;
                    float ws[16], wm[16];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float4 w4 = *reinterpret_cast<const float4*>(&sm.wsc[j * BM + rbase + 8 * k]);
                        const float4 m4 = *reinterpret_cast<const float4*>(&sm.wmn[j * BM + rbase + 8 * k]);
                        ws[4 * k + 0] = w4.x; ws[4 * k + 1] = w4.y; ws[4 * k + 2] = w4.z; ws[4 * k + 3] = w4.w;
                        wm[4 * k + 0] = m4.x; wm[4 * k + 1] = m4.y; wm[4 * k + 2] = m4.z; wm[4 * k + 3] = m4.w;
                    }
#pragma unroll
                    for (int b = 0; b < NC; ++b) {
                        const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                        const v16i C = __builtin_amdgcn_mfma_i32_32x32x32_i8(Av, Bv[b], zero, 0, 0, 0);
                        const int t = wc * (BN / 2) + 32 * b + li;
                        if constexpr (DUMP) {
                            const int tg = tok0 + t;
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const int rg = row0 + rbase + 8 * (i >> 2) + (i & 3);
                                if (tg < nt && rg < od)
                                    S[(((size_t)tg * od + rg) * nsb + sb) * 8 + j] = C[i];
                            }
                        } else {
                            const float dxv = sm.xd[j * BN + t];
                            const float sxv = sm.xs[j * BN + t];
#pragma unroll
                            for (int i = 0; i < 16; ++i)
                                acc[a][b][i] += ws[i] * (dxv * (float)C[i]) - wm[i] * sxv;
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    if constexpr (!DUMP) {
#pragma unroll
        for (int a = 0; a < MR; ++a)
#pragma unroll
            for (int b = 0; b < NC; ++b) {
                const int tg = tok0 + wc * (BN / 2) + 32 * b + li;
                if (tg >= nt)
                    continue;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int rg = row0 + wr * (BM / 2) + 32 * a + 4 * lh + 8 * k;
                    float* o = out + (size_t)tg * od + rg;
                    if (rg + 3 < od && ((od & 3) == 0)) {
                        *reinterpret_cast<float4*>(o) =
                            make_float4(acc[a][b][4 * k], acc[a][b][4 * k + 1], acc[a][b][4 * k + 2], acc[a][b][4 * k + 3]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (rg + i < od)
                                o[i] = acc[a][b][4 * k + i];
                    }
                }
            }
    }
}

// ------------------------------------------------------------------ Q6_K
// Groups of 16 weights: v_mfma_i32_32x32x16_i8 (lane l: row/token l%32, K bytes
// 8*(l/32) .. +7).  Codes are rebuilt and centred at staging time into signed
// bytes in LDS ([MMQ, section 4, Q6_K specialization]: centre at load), so the
// MFMA operands are plain 8-byte LDS reads.  Rescale per group:
// acc += (d*sc_g) * dx * C, dx the scale of the 32-block holding group g.
template <int BM, int BN>
struct __attribute__((aligned(16))) Q6Smem {
    static constexpr int W_STRIDE = 272;    // 256 centred codes + 16 pad
    static constexpr int X_STRIDE = 272;
    int8_t wq[BM * W_STRIDE];
    float wsc[16 * BM];                     // d * sc_g, [g][row]
    uint8_t xq[BN * X_STRIDE];
    float xd[8 * BN];
};

template <int BM, int BN, bool DUMP>
__global__ __launch_bounds__(256) void mmq_q6k_kernel(const uint8_t* __restrict__ W,
                                                      const int8_t* __restrict__ q,
                                                      const float* __restrict__ dx,
                                                      float* __restrict__ out, int nt, int od,
                                                      int id, int32_t* __restrict__ S)
{
    using SM = Q6Smem<BM, BN>;
    __shared__ SM sm;
    constexpr int MR = BM / 64;
    constexpr int NC = BN / 64;
    static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int li = lane & 31, lh = lane >> 5;
    const int row0 = blockIdx.y * BM;
    const int tok0 = blockIdx.x * BN;
    const int nsb = id >> 8;
    const int nblk = id >> 5;

    float acc[MR][NC][16];
#pragma unroll
    for (int a = 0; a < MR; ++a)
#pragma unroll
        for (int b = 0; b < NC; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc[a][b][i] = 0.f;

    for (int sb = 0; sb < nsb; ++sb) {
        // ---- stage weights: 8 threads per row, thread c rebuilds 32 codes
        for (int e = tid; e < BM * 8; e += 256) {
            const int r = e >> 3, c = e & 7;
            const int h = c >> 2, jq = (c >> 1) & 1, half = c & 1;
            const int rg = min(row0 + r, od - 1);
            const uint8_t* blk = W + ((size_t)rg * nsb + sb) * kQ6KBytes;
            // low bytes 64h+32jq+16half.., high bytes 32h+16half.. (2-byte aligned block)
            const uintptr_t al = reinterpret_cast<uintptr_t>(blk + 64 * h + 32 * jq + 16 * half);
            const uintptr_t ah = reinterpret_cast<uintptr_t>(blk + 128 + 32 * h + 16 * half);
            const uint32_t* pl = reinterpret_cast<const uint32_t*>(al & ~(uintptr_t)3);
            const uint32_t* ph = reinterpret_cast<const uint32_t*>(ah & ~(uintptr_t)3);
            const uint32_t shl = (uint32_t)(al & 3), shh = (uint32_t)(ah & 3);
            uint32_t L[4], H[4];
            {
                const uint32_t l0 = pl[0], l1 = pl[1], l2 = pl[2], l3 = pl[3], l4 = pl[4];
                L[0] = __builtin_amdgcn_alignbyte(l1, l0, shl);
                L[1] = __builtin_amdgcn_alignbyte(l2, l1, shl);
                L[2] = __builtin_amdgcn_alignbyte(l3, l2, shl);
                L[3] = __builtin_amdgcn_alignbyte(l4, l3, shl);
                const uint32_t h0 = ph[0], h1 = ph[1], h2 = ph[2], h3 = ph[3], h4 = ph[4];
                H[0] = __builtin_amdgcn_alignbyte(h1, h0, shh);
                H[1] = __builtin_amdgcn_alignbyte(h2, h1, shh);
                H[2] = __builtin_amdgcn_alignbyte(h3, h2, shh);
                H[3] = __builtin_amdgcn_alignbyte(h4, h3, shh);
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
            if (c < 2) {
                // scales: thread c = 0 takes groups 0..7, c = 1 groups 8..15
                const float dw = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(blk + 208));
                const int8_t* scp = reinterpret_cast<const int8_t*>(blk + 192 + 8 * c);
#pragma unroll
                for (int gg = 0; gg < 8; ++gg)
                    sm.wsc[(8 * c + gg) * BM + r] = dw * (float)scp[gg];
            }
        }
        for (int e = tid; e < BN * 16; e += 256) {
            const int t = e >> 4, part = e & 15;
            const int tg = tok0 + t;
            int4 v = make_int4(0, 0, 0, 0);
            if (tg < nt)
                v = *reinterpret_cast<const int4*>(q + (size_t)tg * id + 256 * sb + 16 * part);
            *reinterpret_cast<int4*>(&sm.xq[t * SM::X_STRIDE + 16 * part]) = v;
        }
        for (int e = tid; e < BN * 2; e += 256) {
            const int t = e >> 1, hf = e & 1;
            const int tg = tok0 + t;
            float4 vd = make_float4(0.f, 0.f, 0.f, 0.f);
            if (tg < nt)
                vd = *reinterpret_cast<const float4*>(dx + (size_t)tg * nblk + 8 * sb + 4 * hf);
            sm.xd[(4 * hf + 0) * BN + t] = vd.x;
            sm.xd[(4 * hf + 1) * BN + t] = vd.y;
            sm.xd[(4 * hf + 2) * BN + t] = vd.z;
            sm.xd[(4 * hf + 3) * BN + t] = vd.w;
        }
        __syncthreads();

#pragma unroll 4
        for (int gq = 0; gq < 16; ++gq) {
            long Bv[NC];
#pragma unroll
            for (int b = 0; b < NC; ++b) {
                const int t = wc * (BN / 2) + 32 * b + li;
                Bv[b] = *reinterpret_cast<const long*>(&sm.xq[t * SM::X_STRIDE + 16 * gq + 8 * lh]);
            }
#pragma unroll
            for (int a = 0; a < MR; ++a) {
                const int r = wr * (BM / 2) + 32 * a + li;
                const long Av = *reinterpret_cast<const long*>(&sm.wq[r * SM::W_STRIDE + 16 * gq + 8 * lh]);
                const int rbase = wr * (BM / 2) + 32 * a + 4 * lh;
                float ws[16];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float4 w4 = *reinterpret_cast<const float4*>(&sm.wsc[gq * BM + rbase + 8 * k]);
                    ws[4 * k + 0] = w4.x; ws[4 * k + 1] = w4.y; ws[4 * k + 2] = w4.z; ws[4 * k + 3] = w4.w;
                }
#pragma unroll
                for (int b = 0; b < NC; ++b) {
                    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                    const v16i C = __builtin_amdgcn_mfma_i32_32x32x16_i8(Av, Bv[b], zero, 0, 0, 0);
                    const int t = wc * (BN / 2) + 32 * b + li;
                    if constexpr (DUMP) {
                        const int tg = tok0 + t;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int rg = row0 + rbase + 8 * (i >> 2) + (i & 3);
                            if (tg < nt && rg < od)
                                S[(((size_t)tg * od + rg) * nsb + sb) * 16 + gq] = C[i];
                        }
                    } else {
                        const float dxv = sm.xd[(gq >> 1) * BN + t];
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            acc[a][b][i] += ws[i] * (dxv * (float)C[i]);
                    }
                }
            }
        }
        __syncthreads();
    }

    if constexpr (!DUMP) {
#pragma unroll
        for (int a = 0; a < MR; ++a)
#pragma unroll
            for (int b = 0; b < NC; ++b) {
                const int tg = tok0 + wc * (BN / 2) + 32 * b + li;
                if (tg >= nt)
                    continue;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int rg = row0 + wr * (BM / 2) + 32 * a + 4 * lh + 8 * k;
                    float* o = out + (size_t)tg * od + rg;
                    if (rg + 3 < od && ((od & 3) == 0)) {
                        *reinterpret_cast<float4*>(o) =
                            make_float4(acc[a][b][4 * k], acc[a][b][4 * k + 1], acc[a][b][4 * k + 2], acc[a][b][4 * k + 3]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (rg + i < od)
                                o[i] = acc[a][b][4 * k + i];
                    }
                }
            }
    }
}

// ------------------------------------------------------------------ probe
// One 32 x 32 x 32 int8 MFMA with the operand and result mapping the MMQ kernel
// assumes: A [32 rows][32 K] and B [32 tokens][32 K] row-major int8, C [32 tokens]
// [32 rows] int32 = B . A^T.  Used by a test to pin the lane layout.
__global__ __launch_bounds__(64) void mfma_tile_probe_kernel(const int8_t* __restrict__ A,
                                                             const int8_t* __restrict__ B,
                                                             int32_t* __restrict__ C)
{
    const int lane = threadIdx.x, li = lane & 31, lh = lane >> 5;
    const int4 a = *reinterpret_cast<const int4*>(A + 32 * li + 16 * lh);
    const int4 b = *reinterpret_cast<const int4*>(B + 32 * li + 16 * lh);
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const v16i r = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{a.x, a.y, a.z, a.w}, v4i{b.x, b.y, b.z, b.w}, zero, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * lh + (i & 3);
        C[32 * li + row] = r[i];
    }
}

hipError_t launch_mfma_tile_probe(const int8_t* A, const int8_t* B, int32_t* C, hipStream_t st)
{
    hipLaunchKernelGGL(mfma_tile_probe_kernel, dim3(1), dim3(64), 0, st, A, B, C);
    return hipGetLastError();
}

// ------------------------------------------------------------------ launch

template <int BM, int BN, bool DUMP>
static hipError_t launch_tile(int type, const uint8_t* W, const int8_t* q, const float* d,
                              const float* s, int nt, int od, int id, float* out, int32_t* S,
                              hipStream_t st)
{
    const dim3 grid((nt + BN - 1) / BN, (od + BM - 1) / BM);
    if (type == 1)
        hipLaunchKernelGGL((mmq_q4k_kernel<BM, BN, DUMP>), grid, dim3(256), 0, st, W, q, d, s, out, nt,
                           od, id, S);
    else
        hipLaunchKernelGGL((mmq_q6k_kernel<BM, BN, DUMP>), grid, dim3(256), 0, st, W, q, d, out, nt, od,
                           id, S);
    return hipGetLastError();
}

hipError_t launch_mmq(int type, const uint8_t* W, const int8_t* q, const float* d, const float* s,
                      int nt, int od, int id, float* out, int32_t* S, hipStream_t st)
{
    if (S)
        return launch_tile<64, 64, true>(type, W, q, d, s, nt, od, id, out, S, st);
    return launch_tile<64, 64, false>(type, W, q, d, s, nt, od, id, out, S, st);
}

}  // namespace qmm
