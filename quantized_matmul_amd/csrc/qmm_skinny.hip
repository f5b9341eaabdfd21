// Small-batch Q4_K matmul on int8 MFMA: 1..16 tokens, the decode and short-prefill
// shapes where the 64-token MMQ tiles are mostly padding and the v_dot4 MMVQ
// kernel re-reads every token's activations once per four weight rows.
//
// [MMQ, section 12.2]: the tokens live in registers and every weight block is
// streamed once for all of them.  [GEMM, "One mma per scale group"]: one int8
// matrix op per 32-weight sub-block, its int32 result taken to f32 with the two
// scales; [MMQ, section 6]: per-32 rescale acc += (d*sc_j)*dx*S - (dmin*m_j)*s in
// f32; [MMQ, section 11.4]: codes 0..15 enter the integer op uncentred.
//
// MI355X mapping:
//  * v_mfma_i32_16x16x32_i8 with the activations as operand A (16 tokens x 32
//    values: lane l gives token l%16, values 8*(l/16) .. +7 of the sub-block) and
//    the weights as operand B (32 values x 16 rows: lane l gives row l%16, the
//    same 8 values).  Result lane l holds weight row l%16 for tokens 4*(l/16) ..
//    +3, so the row's d*sc_j is one register per lane and sub-block, and every
//    lane decodes the header of its own row.  A Q4_K code chunk (32 bytes) holds
//    sub-blocks 2c (low nibbles) and 2c+1 (high nibbles) at the same byte
//    positions: lane group p reads bytes 8p .. 8p+7 of each chunk, which feed two
//    MFMAs.
//  * Per output and sub-block the VALU does two operations: the exact subtraction
//    below and one fma with the scale product (d*sc_j)[row] * dx_j[token].  The int8
//    accumulator starts at the bit pattern of 1.5 * 2^23, so the result read as f32
//    is 12582912 + S exactly (|S| <= 60960).  The scale products of four sub-blocks
//    come from one four-block v_mfma_f32_16x16x1_f32 (block b: the outer product of
//    lanes 16b .. 16b+15's dx and d*sc_j), already in the result layout; a lane
//    loads dx and s of its own token for two sub-blocks and decodes d*sc_j and
//    dmin*m_j of its own row for the same two.
//  * The min term sum_j (-dmin*m_j)[row] * s_j[token] is a product over the 8
//    sub-blocks: two v_mfma_f32_16x16x4_f32 per super-block add it into the same
//    accumulators (same result layout).
//  * Every weight and code load is a 16-byte piece of a contiguous run -- a row's
//    144-byte block, a token's 256 codes -- so a load instruction
//    touches few cache lines; the pieces go through a wave-private LDS area into
//    the MFMA operand layout (no barrier: one wave's LDS operations complete in
//    order).  The next super-block's loads are issued before the current one is
//    staged and computed.
//  * A wave takes RT tiles of 16 rows (RT = 1 is launched); their MFMAs share the
//    activation operand.  The KS waves of a workgroup split K (super-blocks w,
//    w + KS, ...); the partial sums are kept per virtual wave of a 16-way split and
//    added through LDS in a fixed order, so the result does not depend on KS.
//  * Tokens past nt read the last token (their results are not stored); rows past
//    od read the last row.
#include "qmm_mmq_common.h"

namespace qmm {

namespace {

constexpr uint32_t kSkMagic = 0x4B400000u;  // 1.5 * 2^23 as f32

typedef long v1l;

// One super-block's loads for one lane, all contiguous 16-byte pieces: the RT*16
// rows' 144-byte blocks (piece e: row e/9, bytes 16*(e%9) ..), the activation codes
// of NTB tokens (piece e: token e/16, bytes 16*(e%16) ..), and the activation d and
// s of token l%16 for blocks p = l/16 and 4 + p of the super-block.  Buffer loads: a wave-uniform
// resource per operand, a per-lane offset fixed for the kernel, the super-block
// step as the scalar offset (plain loads from read-only memory may be sunk by the
// compiler to their first use, which would undo the prefetch).
template <int RT, int NTB>
struct SkLoad {
    static constexpr int NW = (RT * 144 + 63) / 64, NX = (NTB * 16 + 63) / 64;
    v4i w[NW];
    v4i x[NX];
    float d[2], s[2];   // activation d and s of token l%16, blocks p and 4 + p
};

template <int RT, int NTB>
struct SkAddr {
    __amdgpu_buffer_rsrc_t rw, rx, rd, rs;
    uint32_t w[SkLoad<RT, NTB>::NW], x[SkLoad<RT, NTB>::NX], ds;
};

template <int RT, int NTB>
__device__ __forceinline__ void sk_load(SkLoad<RT, NTB>& L, const SkAddr<RT, NTB>& a, int sb)
{
#pragma unroll
    for (int k = 0; k < SkLoad<RT, NTB>::NW; ++k)
        L.w[k] = bload16(a.rw, a.w[k], (uint32_t)sb * kQ4KBytes);
#pragma unroll
    for (int k = 0; k < SkLoad<RT, NTB>::NX; ++k)
        L.x[k] = bload16(a.rx, a.x[k], (uint32_t)sb * 256u);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        L.d[h] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(a.rd, (int)a.ds, sb * 32 + 16 * h, 0));
        L.s[h] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(a.rs, (int)a.ds, sb * 32 + 16 * h, 0));
    }
}

// Scale products of a Q4_K header for this lane's row and sub-blocks j = 4h + p
// (h = 0, 1): a[h] = d * sc_j, b[h] = -dmin * m_j ([MMQ, section 6,
// get_scale_min_k4 semantics]: sub-blocks 0-3 take the low six bits of scale bytes
// j and j+4; 4-7 take the nibbles of bytes j+4 with the top two bits of bytes j-4
// and j as bits 4-5).
__device__ __forceinline__ void sk_scales(const uint4& h, int p, float (&a)[2], float (&b)[2])
{
    const float d = f16_bits_to_f32(h.x & 0xFFFFu), dm = f16_bits_to_f32(h.x >> 16);
    const uint32_t sh = 8u * (uint32_t)p;
    const uint32_t sc_lo = (h.y >> sh) & 0x3Fu, m_lo = (h.z >> sh) & 0x3Fu;
    const uint32_t sc_hi = ((h.w >> sh) & 0x0Fu) | (((h.y >> sh) >> 2) & 0x30u);
    const uint32_t m_hi = (((h.w >> sh) >> 4) & 0x0Fu) | (((h.z >> sh) >> 2) & 0x30u);
    a[0] = d * (float)sc_lo;
    a[1] = d * (float)sc_hi;
    b[0] = -(dm * (float)m_lo);
    b[1] = -(dm * (float)m_hi);
}

// Wave-private LDS area for one super-block: the rows' blocks [row][144] and the
// activation codes [token][272] (16 bytes of padding: the 16 tokens' reads of one
// sub-block piece fall in 16 different bank groups).
template <int RT, int NTB>
struct __attribute__((aligned(16))) SkStage {
    static constexpr int X_STRIDE = 272;
    uint8_t w[RT * 16 * 144];
    uint8_t x[NTB * X_STRIDE];
};

template <int RT, int NTB>
__device__ __forceinline__ void sk_stage(SkStage<RT, NTB>& sl, const SkLoad<RT, NTB>& L, int lane)
{
#pragma unroll
    for (int k = 0; k < SkLoad<RT, NTB>::NW; ++k) {
        const int e = min(64 * k + lane, RT * 144 - 1);   // lanes past the end repeat the last piece
        *reinterpret_cast<v4i*>(&sl.w[16 * e]) = L.w[k];
    }
#pragma unroll
    for (int k = 0; k < SkLoad<RT, NTB>::NX; ++k) {
        const int e = min(64 * k + lane, NTB * 16 - 1);
        *reinterpret_cast<v4i*>(&sl.x[(e >> 4) * SkStage<RT, NTB>::X_STRIDE + 16 * (e & 15)]) = L.x[k];
    }
}

typedef float v4f __attribute__((ext_vector_type(4)));

// The compute of one staged super-block: decode the headers, 8 sub-blocks x RT
// tiles of MFMA and rescale.  The wave's own LDS writes are visible to its later
// reads: one wave's LDS operations complete in the order it issues them.
template <int RT, int NTB>
__device__ __forceinline__ void sk_superblock(const SkStage<RT, NTB>& sl, const SkLoad<RT, NTB>& L, v4f (&acc)[RT],
                                              int lane, uint32_t mask, float Mv, const v4i& magic)
{
    const int p = lane >> 4, r16 = lane & 15;
    const int tx = min(r16, NTB - 1);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        float a[2], b[2];
        sk_scales(*reinterpret_cast<const uint4*>(&sl.w[(16 * r + r16) * 144]), p, a, b);
        // the min term sum_j (-dmin*m_j)[row] * s_j[token] of the super-block: two
        // f32 16 x 16 x 4 MFMAs over its 8 sub-blocks (operand A: token lane%16,
        // sub-block 4h + lane/16; operand B: this lane's row, the same sub-block)
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(L.s[0], b[0], acc[r], 0, 0, 0);
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(L.s[1], b[1], acc[r], 0, 0, 0);
        // the scale products (d*sc_j)[row] * dx_j[token] of sub-blocks 4h .. 4h+3 in
        // the result layout: one four-block 16 x 16 x 1 f32 outer product (block b
        // from the lanes b*16 .. b*16+15: token / row lane%16, sub-block 4h + b);
        // P[h][4b + i] is sub-block 4h + b, token 4p + i, this lane's row
        const v16f z = {};
        const v16f P0 = __builtin_amdgcn_mfma_f32_16x16x1f32(L.d[0], a[0], z, 0, 0, 0);
        const v16f P1 = __builtin_amdgcn_mfma_f32_16x16x1f32(L.d[1], a[1], z, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint2 wc = *reinterpret_cast<const uint2*>(&sl.w[(16 * r + r16) * 144 + 16 + 32 * c + 8 * p]);
#pragma unroll
            for (int hn = 0; hn < 2; ++hn) {
                const int j = 2 * c + hn;
                const v1l xa =
                    *reinterpret_cast<const v1l*>(&sl.x[tx * SkStage<RT, NTB>::X_STRIDE + 32 * j + 8 * p]);
                const uint2 wv = hn ? make_uint2((wc.x >> 4) & mask, (wc.y >> 4) & mask)
                                    : make_uint2(wc.x & mask, wc.y & mask);
                const v4i C = __builtin_amdgcn_mfma_i32_16x16x32_i8(xa, __builtin_bit_cast(v1l, wv), magic, 0, 0, 0);
                const v16f& P = j < 4 ? P0 : P1;
                const int b4 = 4 * (j & 3);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[r][i] = fmaf(__int_as_float(C[i]) - Mv, P[b4 + i], acc[r][i]);
            }
        }
    }
}

// Compiler-only ordering point between the staging writes and the reads of the
// staged data (a memory fence here would also make the wave wait for its
// prefetch loads still in flight).
__device__ __forceinline__ void sk_handover()
{
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// A VGPR holding the bit pattern (not folded back into a constant operand).
__device__ __forceinline__ uint32_t sk_vgpr(uint32_t bits)
{
    uint32_t v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(bits));
    return v;
}

// Workgroup: KS waves (KS = 1, 2, 4, 8 or 16) splitting K, wave w taking super-blocks
// w, w + KS, ...; all over the same RT*16 rows.  N > 0: every wave has exactly N
// super-blocks (KS * N == nsb); N = 0: any share.  NTB >= nt tokens are staged
// (the 16-token tile's other lanes repeat token NTB-1 or nt-1; their results are
// not stored).
//
// The sum does not depend on KS: super-block sb belongs to virtual wave sb % 16 of
// a 16-way split, each wave keeps one accumulator per virtual wave it covers (16 /
// KS of them: super-blocks v, v + 16, v + 32, ... in order), and the 16 virtual
// partial tiles are added in the order 0, 1, .., 15.  So every KS gives the same
// bits, a token's result does not depend on the other tokens of the call, and KS is
// chosen per shape for speed alone.  Dynamic LDS: KS stage areas, then the 16
// partial tiles.
constexpr int kSkVirt = 16;   // the virtual split (KS divides it)

template <int RT, int NTB, int N, int KS>
__global__ __launch_bounds__(64 * KS) void mmq_skinny_q4k_kernel(const uint8_t* __restrict__ W,
                                                                 const int8_t* __restrict__ q,
                                                                 const float* __restrict__ dx,
                                                                 const float* __restrict__ sx,
                                                                 float* __restrict__ out, int nt, int od, int id)
{
    constexpr int NV = kSkVirt / KS;   // virtual waves per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t sk_lds[];
    auto* stage = reinterpret_cast<SkStage<RT, NTB>*>(sk_lds);
    auto* red = reinterpret_cast<float*>(sk_lds + (size_t)KS * sizeof(SkStage<RT, NTB>));
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = lane >> 4;
    const int nsb = id >> 8, nblk = id >> 5;
    const int row0 = blockIdx.x * 16 * RT;
    const size_t row_bytes = (size_t)nsb * kQ4KBytes;
    SkAddr<RT, NTB> ad;
    ad.rw = buffer_rsrc(W + (size_t)row0 * row_bytes, (size_t)(od - row0) * row_bytes);
    ad.rx = buffer_rsrc(q, (size_t)nt * id);
    ad.rd = buffer_rsrc(dx, (size_t)nt * nblk * 4);
    ad.rs = buffer_rsrc(sx, (size_t)nt * nblk * 4);
#pragma unroll
    for (int k = 0; k < SkLoad<RT, NTB>::NW; ++k) {
        const int e = min(64 * k + lane, RT * 144 - 1);
        ad.w[k] = (uint32_t)(min(row0 + e / 9, od - 1) - row0) * (uint32_t)row_bytes + 16u * (uint32_t)(e % 9);
    }
#pragma unroll
    for (int k = 0; k < SkLoad<RT, NTB>::NX; ++k) {
        const int e = min(64 * k + lane, NTB * 16 - 1);
        ad.x[k] = (uint32_t)min(e >> 4, nt - 1) * (uint32_t)id + 16u * (uint32_t)(e & 15);
    }
    ad.ds = ((uint32_t)min(lane & 15, nt - 1) * (uint32_t)nblk + (uint32_t)p) * 4u;
    const float Mv = __uint_as_float(sk_vgpr(kSkMagic));
    const uint32_t mask = sk_vgpr(0x0F0F0F0Fu);
    const int mg = (int)__float_as_uint(Mv);
    const v4i magic = {mg, mg, mg, mg};
    SkStage<RT, NTB>& my = stage[w];

    // acc[j]: virtual wave w + j * KS (super-blocks w + j * KS, + 16, + 32, ...)
    v4f acc[NV][RT];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int r = 0; r < RT; ++r)
            acc[j][r] = (v4f){0.f, 0.f, 0.f, 0.f};
    int rot = 0;   // the loop form rotates acc: acc[j] then holds virtual wave w + ((rot + j) % NV) * KS

    if constexpr (N > 0) {
        // exactly N super-blocks per wave (KS * N == nsb): every load first, then
        // stage and compute in order -- straight-line code, so the compiler waits
        // for one set at a time (one memory latency per wave); the k-th
        // super-block (w + k * KS) belongs to virtual wave w + (k % NV) * KS
        SkLoad<RT, NTB> L[N];
#pragma unroll
        for (int k = 0; k < N; ++k) {
            sk_load<RT, NTB>(L[k], ad, w + k * KS);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = 0; k < N; ++k) {
            sk_handover();
            sk_stage<RT, NTB>(my, L[k], lane);
            sk_handover();
            sk_superblock<RT, NTB>(my, L[k], acc[k % NV], lane, mask, Mv, magic);
        }
    } else {
        // super-blocks w, w + KS, ...: two per trip so the load sets alternate, the
        // odd last one after the loop (no exit between a prefetch and its use: the
        // compiler keeps the loads where they are issued).  Each super-block adds
        // into acc[0], then the accumulators rotate by one, so acc[0] always holds
        // the virtual wave of the next super-block.
        const int n = (nsb - w + KS - 1) / KS;  // >= 1: the launch has KS <= nsb
        auto rotate = [&]() {
            if constexpr (NV > 1) {
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    const v4f t = acc[0][r];
#pragma unroll
                    for (int j = 0; j + 1 < NV; ++j)
                        acc[j][r] = acc[j + 1][r];
                    acc[NV - 1][r] = t;
                }
            }
        };
        SkLoad<RT, NTB> A, B;
        sk_load<RT, NTB>(A, ad, w);
        for (int i = 0; i + 1 < n; i += 2) {
            const int sb = w + i * KS;
            sk_load<RT, NTB>(B, ad, sb + KS);
            __builtin_amdgcn_sched_barrier(0);
            sk_handover();
            sk_stage<RT, NTB>(my, A, lane);
            sk_handover();
            sk_superblock<RT, NTB>(my, A, acc[0], lane, mask, Mv, magic);
            rotate();
            sk_load<RT, NTB>(A, ad, min(sb + 2 * KS, nsb - 1));
            __builtin_amdgcn_sched_barrier(0);
            sk_handover();
            sk_stage<RT, NTB>(my, B, lane);
            sk_handover();
            sk_superblock<RT, NTB>(my, B, acc[0], lane, mask, Mv, magic);
            rotate();
        }
        if (n & 1) {
            sk_handover();
            sk_stage<RT, NTB>(my, A, lane);
            sk_handover();
            sk_superblock<RT, NTB>(my, A, acc[0], lane, mask, Mv, magic);
            rotate();
        }
        rot = n % NV;
    }
    // every wave's virtual partial tiles to LDS (tile v at red[v][r][i][lane]); then
    // wave w adds value e = w, w + KS, ... (value e: row tile e / 4, token slot
    // 4p + e % 4) over the virtual waves in the order 0, 1, .., 15 and stores it
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int v = w + ((rot + j) % NV) * KS;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[((v * RT + r) * 4 + i) * 64 + lane] = acc[j][r][i];
    }
    __syncthreads();
    for (int e = w; e < RT * 4; e += KS) {
        float sum = red[e * 64 + lane];
#pragma unroll
        for (int v = 1; v < kSkVirt; ++v)
            sum += red[(v * RT * 4 + e) * 64 + lane];
        const int row = row0 + 16 * (e >> 2) + (lane & 15), t = 4 * p + (e & 3);
        if (row < od && t < nt)
            out[(size_t)t * od + row] = sum;
    }
}

template <int NTB, int N, int KS>
hipError_t launch_rk(const uint8_t* W, const int8_t* q, const float* d, const float* s, int nt, int od, int id,
                     float* out, hipStream_t st)
{
    constexpr int RT = 1;
    const int grid = (od + 16 * RT - 1) / (16 * RT);
    const size_t lds = (size_t)KS * sizeof(SkStage<RT, NTB>) + (size_t)kSkVirt * RT * 4 * 64 * sizeof(float);
    hipLaunchKernelGGL((mmq_skinny_q4k_kernel<RT, NTB, N, KS>), dim3(grid), dim3(64 * KS), lds, st, W, q, d, s, out,
                       nt, od, id);
    return hipGetLastError();
}

// Straight-line form when the waves share K evenly in at most 4 super-blocks each.
template <int NTB, int KS>
hipError_t launch_rkk(const uint8_t* W, const int8_t* q, const float* d, const float* s, int nt, int od, int id,
                      float* out, hipStream_t st)
{
    const int nsb = id / 256;
    switch (nsb % KS ? 0 : nsb / KS) {
    case 1: return launch_rk<NTB, 1, KS>(W, q, d, s, nt, od, id, out, st);
    case 2: return launch_rk<NTB, 2, KS>(W, q, d, s, nt, od, id, out, st);
    case 3: return launch_rk<NTB, 3, KS>(W, q, d, s, nt, od, id, out, st);
    case 4: return launch_rk<NTB, 4, KS>(W, q, d, s, nt, od, id, out, st);
    default: return launch_rk<NTB, 0, KS>(W, q, d, s, nt, od, id, out, st);
    }
}

template <int NTB>
hipError_t launch_rkn(const uint8_t* W, const int8_t* q, const float* d, const float* s, int nt, int od, int id,
                      float* out, int ks, hipStream_t st)
{
    switch (ks) {
    case 1: return launch_rkk<NTB, 1>(W, q, d, s, nt, od, id, out, st);
    case 2: return launch_rkk<NTB, 2>(W, q, d, s, nt, od, id, out, st);
    case 4: return launch_rkk<NTB, 4>(W, q, d, s, nt, od, id, out, st);
    case 8: return launch_rkk<NTB, 8>(W, q, d, s, nt, od, id, out, st);
    default: return launch_rkk<NTB, 16>(W, q, d, s, nt, od, id, out, st);
    }
}

}  // namespace

// Waves per workgroup (ks, splitting K; 1, 2, 4, 8 or 16, never more than the
// super-blocks): 8, or 16 on a matrix of at most 256 row tiles with 32 or 48
// super-blocks per row (2 or 3 per wave; 16 waves of 4 or more would spill).  ks
// does not change the results (see the kernel), so the choice is by speed alone.
// Measured (us): 8 waves as fast as 4 or faster at every token count on 8192..16384
// x 4096 (alternating processes: 12288 x 4096 nt = 4 9.2 -> 8.6, nt = 8 10.3 ->
// 10.0, nt = 16 13.0 -> 12.1; 8192 x 4096 nt = 8 8.1 -> 7.2); 16 against 8 in one
// process: 4096 x 12288 nt = 4 9.4 -> 8.7, nt = 8 10.9 -> 9.9, but 12288 x 4096 nt = 4
// 8.2 -> 9.0, nt = 8 9.6 -> 12.6 (many row tiles) and 4096 x 4096 within 2 %.
// cfg != 0 forces 100 + ks (ks 1, 2, 4, 8 or 16) for tests and tuning.
hipError_t launch_skinny(const uint8_t* W, const int8_t* q, const float* d, const float* s, int nt, int od, int id,
                         float* out, hipStream_t st, int cfg)
{
    if (nt < 1 || nt > 16)
        return hipErrorInvalidValue;
    const int nsb = id / 256;
    int ks;
    if (cfg) {
        ks = cfg - 100;
        if (ks != 1 && ks != 2 && ks != 4 && ks != 8 && ks != 16)
            return hipErrorInvalidValue;
    } else {
        const int grid = (od + 15) / 16;
        ks = grid <= 256 && (nsb == 32 || nsb == 48) ? 16 : 8;
    }
    while (ks > nsb)
        ks >>= 1;
    if (nt <= 4)
        return launch_rkn<4>(W, q, d, s, nt, od, id, out, ks, st);
    if (nt <= 8)
        return launch_rkn<8>(W, q, d, s, nt, od, id, out, ks, st);
    return launch_rkn<16>(W, q, d, s, nt, od, id, out, ks, st);
}

}  // namespace qmm
