// Internal declarations and device helpers of libqmm (HIP, gfx950 only).
//
// Pages cited (by title, section in brackets):
//   [GEMM] "The quantized GEMM" (mojo-dllm kernels page)
//   [MMQ]  "llama.cpp MMQ -- quantized-weight int8 tensor-core matmul: structure,
//          numerics, SASS census, and minfer contrast"
//   [CH04] "04 - Reading minfer's kernels II -- from GEMV to tiled GEMM"
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmm {

constexpr int kQK = 256;          // weights per super-block
constexpr int kQ4KBytes = 144;    // Q4_K super-block
constexpr int kQ6KBytes = 210;    // Q6_K super-block
constexpr int kQ6KP224Bytes = 224;  // Q6_K super-block padded to 16-byte alignment (weight type 3)
constexpr int kQ5KBytes = 176;    // Q5_K super-block (weight type 6)
constexpr int kActBlock = 32;     // activation values per scale

// Launchers (return hipError_t of the launch).  All pointers are device
// pointers validated by the C ABI layer; shapes satisfy id % 256 == 0.
hipError_t launch_quantize(const float* x, int nt, int id, int8_t* q, float* d, float* s,
                           hipStream_t st);
hipError_t launch_mmvq(int type, const uint8_t* W, const int8_t* q, const float* d, const float* s,
                       int nt, int od, int id, float* out, int32_t* S, hipStream_t st);
// tile: 0 = by the cost model (mmq_tile_choice), 1 = 128 x 64, 2 = 64 x 64,
// 3 = 64 x 64 split over K in two groups.  S != null (the debug dump) runs 64 x 64.
hipError_t launch_mmq(int type, const uint8_t* W, const int8_t* q, const float* d, const float* s,
                      int nt, int od, int id, float* out, int32_t* S, hipStream_t st, int tile = 0);
int mmq_tile_choice(int nt, int od, int id);
// Which form of the 4-wave kernel (launch_mmq_q4k_v2) a Q4_K matrix call runs:
// 1 (4 waves) on more than 256 of its 128 x 64 tiles where the cost model names
// 128 x 64 or the tiles fill 384..512 of one round of 512 workgroup slots (two per
// CU); 2 (8 waves in two groups splitting K, one workgroup per CU) on 192..256
// tiles where the cost model names 128 x 64; 0 otherwise (the 8-wave tiles).
int mmq_q4k_wave_form(int nt, int od, int id);
// Q4_K matrix kernel of 4 waves x (32 rows x 64 tokens) per workgroup (qmm_mmq2.hip);
// S != null writes the integer dots instead (S [nt][od][nsb][8]); ks = 2: 8 waves in
// two groups splitting K.
hipError_t launch_mmq_q4k_v2(const uint8_t* W, const int8_t* q, const float* d, const float* s, int nt, int od,
                             int id, float* out, int32_t* S, hipStream_t st, int ks = 1);
// Small-batch Q4_K kernel on 16 x 16 x 32 int8 MFMA tiles, 1..16 tokens
// (qmm_skinny.hip).  cfg 0: rows per wave and waves per workgroup by the shape;
// else RT * 100 + KS (RT 1 or 2 tiles of 16 rows per wave, KS <= 8 waves).
hipError_t launch_skinny(const uint8_t* W, const int8_t* q, const float* d, const float* s, int nt, int od, int id,
                         float* out, hipStream_t st, int cfg = 0);
// Stream-K (Q4_K and Q6_K in both layouts): workspace of mmq_streamk_ws_bytes() bytes, 16-byte aligned.
size_t mmq_streamk_ws_bytes();
hipError_t launch_mmq_streamk(int type, const uint8_t* W, const int8_t* q, const float* d, const float* s, int nt,
                              int od, int id, float* out, float* ws, hipStream_t st);

// Q8_K activations: q [nt][id] int8, d [nt][id/256] f32, bsum [nt][id/16] f32
// (id % 256 == 0), and the Q4_K / Q6_K matmul on them (qmm_mmq_q8k.hip; type 1
// Q4_K, 2 Q6_K, 3 Q6_K padded).  S != null: the integer stage only, S
// [nt][od][id/256][2] int32.  tile: 0 = q8k_tile_choice, else 1 = 128 x 64, 2 =
// 64 x 64, 3 = 64 x 64 split over K, 4 = Q4_K on launch_mmq_k4_q8k_v2.
hipError_t launch_quantize_q8k(const float* x, int nt, int id, int8_t* q, float* d, float* bsum, hipStream_t st);
int q8k_tile_choice(int nt, int od, int id);
hipError_t launch_mmq_q8k(int type, const uint8_t* W, const int8_t* q, const float* d, const float* bsum, int nt,
                          int od, int id, float* out, int32_t* S, hipStream_t st, int tile);
// Q4_K on Q8_K activations, 4 waves x (32 rows x 64 tokens) per workgroup, the
// sub-block scales inside the int8 operands (qmm_mmq_q8k2.hip); S != null writes
// the integer stage instead (S [nt][od][nsb][2]).  ks = 2: 8 waves in two groups
// splitting K.
hipError_t launch_mmq_k4_q8k_v2(const uint8_t* W, const int8_t* q, const float* d, const float* bsum, int nt, int od,
                                int id, float* out, int32_t* S, hipStream_t st, int ks);

// Producer-side steps that feed the quantizer (qmm_fused.hip).  Rows are [nt][id]
// f32, id % 32 == 0; q/d/s as for launch_quantize.  With q == null the kernels
// store the f32 values y instead of quantizing them (the unfused chain's steps).
// q8k: quantize to Q8_K instead (id % 256 == 0; d [nt][id/256], s = the group
// sums bsum [nt][id/16], as launch_quantize_q8k).
hipError_t launch_rmsnorm(const float* x, const float* o, float* h, const float* w, float eps, int nt,
                          int id, int8_t* q, float* d, float* s, float* y, hipStream_t st, bool q8k = false);
hipError_t launch_residual_add(float* h, const float* o, long n, hipStream_t st);
hipError_t launch_silu_mul(const float* g, const float* u, int nt, int id, int8_t* q, float* d, float* s,
                           float* y, hipStream_t st, bool q8k = false);
hipError_t launch_mfma_tile_probe(int kind, const void* A, const void* B, void* C, hipStream_t st);

// ---------------------------------------------------------------- device helpers

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
    return (float)v;
}

// DPP lane moves inside one wave64 (all lanes active).
__device__ __forceinline__ int dpp_quad_xor1(int v) { return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_quad_xor2(int v) { return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_half_mirror(int v) { return __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_row_mirror(int v) { return __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false); }

__device__ __forceinline__ int sdot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

// One lane's share of the activation quantizer.  Eight consecutive lanes (an
// aligned group of eight) hold one 32-value block, four consecutive values each,
// and all eight must make the call together.  [GEMM, "The GPU path",
// "Activations get one scale per 32"]: d = amax / 127 (IEEE division), codes
// round(v / d) half away from zero, s = d * (float)sum(q); a zero block gives
// d = q = s = 0.  Returns the four codes packed low byte first; every lane gets
// the block's d and s.  The plain quantizer and the producer-fused kernels both
// quantize through this function, so a fused result equals the plain quantizer
// applied to the same f32 values.
__device__ __forceinline__ uint32_t quantize_lane4(float4 v, float& dk, float& sk)
{
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    int ai = __builtin_bit_cast(int, a);  // non-negative floats order like their bits
    ai = max(ai, dpp_quad_xor1(ai));
    ai = max(ai, dpp_quad_xor2(ai));
    ai = max(ai, dpp_half_mirror(ai));
    const float amax = __builtin_bit_cast(float, ai);

    dk = amax / 127.0f;
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (dk != 0.0f) {
        q0 = (int)roundf(v.x / dk);
        q1 = (int)roundf(v.y / dk);
        q2 = (int)roundf(v.z / dk);
        q3 = (int)roundf(v.w / dk);
    }
    int sum = q0 + q1 + q2 + q3;
    sum += dpp_quad_xor1(sum);
    sum += dpp_quad_xor2(sum);
    sum += dpp_half_mirror(sum);
    sk = dk * (float)sum;
    return (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
           ((uint32_t)(q3 & 0xFF) << 24);
}

// One lane's share of the Q8_K activation quantizer ([GEMM, "Activations: int8
// with a scale per 256"]): the 64 lanes of a wave hold one 256-value block, four
// consecutive values each, and all make the call together.  Same rules as
// quantize_lane4 over 256 values: d = amax / 127, codes round(v / d) half away
// from zero, a zero block gives d = q = 0.  gsum: the sum of the codes of this
// lane's 16-value group (its quad).  The plain Q8_K quantizer and the
// producer-fused kernels both quantize through this function.
__device__ __forceinline__ uint32_t quantize_lane4_q8k(float4 v, float& dk, int& gsum)
{
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    int ai = __builtin_bit_cast(int, a);  // non-negative floats order like their bits
    ai = max(ai, dpp_quad_xor1(ai));
    ai = max(ai, dpp_quad_xor2(ai));
    ai = max(ai, dpp_half_mirror(ai));
    ai = max(ai, dpp_row_mirror(ai));
    ai = max(ai, __shfl_xor(ai, 16));
    ai = max(ai, __shfl_xor(ai, 32));
    dk = __builtin_bit_cast(float, ai) / 127.0f;
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (dk != 0.0f) {
        q0 = (int)roundf(v.x / dk);
        q1 = (int)roundf(v.y / dk);
        q2 = (int)roundf(v.z / dk);
        q3 = (int)roundf(v.w / dk);
    }
    int sum = q0 + q1 + q2 + q3;
    sum += dpp_quad_xor1(sum);
    sum += dpp_quad_xor2(sum);
    gsum = sum;
    return (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
           ((uint32_t)(q3 & 0xFF) << 24);
}

// Q4_K (scale, min) of sub-block j from header dwords h1 = bytes 4..7, h2 = 8..11,
// h3 = 12..15.  [MMQ, section 6, get_scale_min_k4 semantics]: j < 4 takes the low
// six bits of byte j (scale) and of byte j+4 (min); j >= 4 takes a nibble of byte
// j+4 for the low four bits and the top two bits of byte j-4 (scale) or byte j
// (min) for the high two.
__device__ __forceinline__ void q4k_scale_min(uint32_t h1, uint32_t h2, uint32_t h3, int j, int& sc,
                                              int& m)
{
    const int jj = j & 3;
    const int sh = 8 * jj;
    const uint32_t b1 = (h1 >> sh) & 0xFF, b2 = (h2 >> sh) & 0xFF, b3 = (h3 >> sh) & 0xFF;
    if (j < 4) {
        sc = (int)(b1 & 63);
        m = (int)(b2 & 63);
    } else {
        sc = (int)((b3 & 0xF) | ((b1 >> 6) << 4));
        m = (int)((b3 >> 4) | ((b2 >> 6) << 4));
    }
}

// The same for the pair of sub-blocks jj and jj + 4 (jj < 4), which share their
// three source bytes; no data-dependent branch.
__device__ __forceinline__ void q4k_scale_min_pair(uint32_t h1, uint32_t h2, uint32_t h3, int jj, int& sc_lo,
                                                   int& m_lo, int& sc_hi, int& m_hi)
{
    const int sh = 8 * jj;
    const uint32_t b1 = (h1 >> sh) & 0xFF, b2 = (h2 >> sh) & 0xFF, b3 = (h3 >> sh) & 0xFF;
    sc_lo = (int)(b1 & 63);
    m_lo = (int)(b2 & 63);
    sc_hi = (int)((b3 & 0xF) | ((b1 >> 6) << 4));
    m_hi = (int)((b3 >> 4) | ((b2 >> 6) << 4));
}

// Q6_K: build four signed codes (q6 - 32) from a dword of low fields and a dword
// of high 2-bit fields.  [GEMM, "Q6_K: the same layout and prefetch"]: the code is
// the nibble plus the two high bits, and the offset 32 comes off by flipping the
// bias into a sign: (q | 0x80) - 0x20 never borrows across bytes, ^ 0x80 then
// gives q - 32 as int8.
__device__ __forceinline__ int q6_center4(uint32_t low4, uint32_t high2)
{
    const uint32_t q = low4 | (high2 << 4);
    return (int)(((q | 0x80808080u) - 0x20202020u) ^ 0x80808080u);
}

}  // namespace qmm
