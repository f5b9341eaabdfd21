// C ABI of libqmm: argument validation, workspace layout, nt dispatch.
// Declarations and their contracts are in include/qmm.h.
//
// [CH04, section 3.3]: one entry point takes raw pointers, the weight type and the
// shape and decides the kernel from nt; shapes it cannot serve are errors, never a
// silent fallback.  [MMQ, section 12.1]: nt <= 8 runs the vector kernel, larger nt
// the matrix kernel, so every nt has a dedicated kernel.
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "qmm.h"
#include "qmm_internal.h"

namespace {

// Fixed device scratch of qmm_matmul_noalloc: the quantized activations (at most
// QMM_NOALLOC_ACT_BYTES) followed by the stream-K partial tiles.  A file-scope
// device array: every device the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: host code uses only the address that hipGetSymbolAddress returns
// for the current device (noalloc_scratch below).
constexpr size_t kNoallocBytes = (size_t)QMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoallocBytes];

constexpr int kMaxDevices = 64;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return QMM_ERR_DEVICE;
    if (dev >= kMaxDevices)
        return QMM_ERR_DEVICE;
    int st = __atomic_load_n(&g_dev_state[dev], __ATOMIC_ACQUIRE);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return QMM_ERR_DEVICE;
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        __atomic_store_n(&g_dev_state[dev], st, __ATOMIC_RELEASE);
    }
    return st == 1 ? QMM_OK : QMM_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int noalloc_scratch(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QMM_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return QMM_ERR_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QMM_OK;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

int check_type(int type)
{
    return (type >= QMM_TYPE_Q4_K && type <= QMM_TYPE_Q5_K) ? QMM_OK : QMM_ERR_TYPE;
}

// bytes per 256 weights
size_t block_bytes(int type)
{
    switch (type) {
    case QMM_TYPE_Q4_K: return qmm::kQ4KBytes;
    case QMM_TYPE_Q6_K: return qmm::kQ6KBytes;
    case QMM_TYPE_Q6_K_P224: return qmm::kQ6KP224Bytes;
    case QMM_TYPE_Q4_0: return 8 * 18;
    case QMM_TYPE_Q5_K: return qmm::kQ5KBytes;
    default: return 8 * 34;
    }
}

// One thread per 16-byte piece of a padded block (14 per block): bytes of the
// 210-byte source block, zero past byte 209.
__global__ __launch_bounds__(256) void pad_q6k_kernel(const uint8_t* __restrict__ src, uint4* __restrict__ dst,
                                                      long long npieces)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= npieces)
        return;
    const long long b = i / 14;
    const int p = (int)(i - b * 14);
    const uint8_t* s = src + b * qmm::kQ6KBytes + 16 * p;
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (16 * p + k < qmm::kQ6KBytes)
            w[k >> 2] |= (uint32_t)s[k] << (8 * (k & 3));
    dst[i] = make_uint4(w[0], w[1], w[2], w[3]);
}

// Shape rule shared by the matmul entry points.
int check_shape(int nt, int od, int id)
{
    if (nt < 1 || od < 1)
        return QMM_ERR_ARG;
    if (id < 256 || id % 256 != 0)
        return QMM_ERR_SHAPE;
    if ((long long)nt * id > 0x7FFFFFFFLL || (long long)od * (id / 256) > 0x7FFFFFFFLL ||
        (long long)nt * od > 0x7FFFFFFFLL)
        return QMM_ERR_SHAPE;
    return QMM_OK;
}

int nt_switch_value()
{
    static int v = -1;
    int cur = __atomic_load_n(&v, __ATOMIC_ACQUIRE);
    if (cur >= 0)
        return cur;
    int val = 8;
    const char* e = getenv("QMM_NT_SWITCH");
    if (e && *e) {
        val = atoi(e);
        if (val < 0)
            val = 0;
        if (val > 8)
            val = 8;
    }
    __atomic_store_n(&v, val, __ATOMIC_RELEASE);
    return val;
}

int launched(hipError_t e) { return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH; }

// The small-batch kernel's K split: 100 + KS (KS = 1, 2, 4, 8 or 16 waves per workgroup)
// forced, 0 = by shape; set by qmm_set_skinny_split, else read once from
// QMM_SKINNY_CFG (the same encoding), for tests and tuning sweeps (the results do
// not depend on it).
int g_skinny_cfg = -1;

int skinny_cfg_override()
{
    int cur = __atomic_load_n(&g_skinny_cfg, __ATOMIC_ACQUIRE);
    if (cur >= 0)
        return cur;
    const char* e = getenv("QMM_SKINNY_CFG");
    int val = e ? atoi(e) : 0;
    if (val != 101 && val != 102 && val != 104 && val != 108 && val != 116)
        val = 0;
    int expect = -1;
    __atomic_compare_exchange_n(&g_skinny_cfg, &expect, val, false, __ATOMIC_ACQ_REL, __ATOMIC_ACQUIRE);
    return __atomic_load_n(&g_skinny_cfg, __ATOMIC_ACQUIRE);
}

// The kernel a call runs.  With the default switch (8): Q4_K runs the small-batch
// MFMA kernel on 9..16 tokens of any matrix, on 3..8 tokens of a matrix of at least
// 3072 rows, on 5..8 tokens of at least 2048 rows, and on 6..8 tokens of at least
// 1024 rows of at most 4096 columns (measured, us, small-batch against MMVQ, one
// process: nt = 3: 3072 x 3072 4.0 / 4.6, 4096 x 4096 4.8 / 5.2, 12288 x 4096 8.3 /
// 9.8, 3072 x 12288 8.5 / 9.5; 2048 x 4096 nt = 3: 4.0 / 3.8; 2048 x 12288 nt = 4:
// 8.5 / 7.6, nt = 5: 9.0 / 10.4; 1024 x 4096 nt = 5: 4.1 / 4.0, nt = 6: 4.1 / 4.3,
// nt = 8: 4.3 / 4.9; 1024 x 12288 nt = 8: 10.1 / 7.6; 12288 x 4096 nt = 8: 10.0 /
// 16.8; at 2 tokens within a few per cent either way, so MMVQ; 9..16 tokens: 6-15 us
// against 21-58 for MMQ); on 17..32 tokens of at most 12288 rows and on 33..48
// tokens of at most 8192 rows and 4096 columns, as launches on token slices of 16
// (the MMQ tile grids of these calls fill a fraction of the GPU; us, slices against
// per-tile MMQ and stream-K: 4096 x 4096 nt = 32 10.4 / 22.0 / 20.6, 12288 x 4096
// nt = 32 22.0 / 24.7 / 29.1, 4096 x 12288 nt = 32 25.3 / 59.6 / 28.4, 8192 x 4096
// nt = 48 24.1 / 24.3 / 24.0; 14336 x 4096 nt = 32 27.1 / 24.6, 4096 x 12288 nt = 40
// 34.4 / 28.7 (stream-K)); MMVQ up to the switch otherwise; other types also on
// 9..16 tokens of a matrix of at most 4096 rows, as launches on token slices of 8
// (such a matrix gives MMQ at most 64 tiles of 64 rows, a quarter of the 256 CUs;
// 4096 x 4096: MMQ 22 us, two MMVQ launches 13.7-14.7 us); MMQ beyond.
int dispatch_kind(int type, int nt, int od, int id)
{
    const int sw = nt_switch_value();
    if (sw == 8 && type == QMM_TYPE_Q4_K &&
        ((nt <= 16 &&
          (nt >= 9 || (nt >= 3 && od >= 3072) || (nt >= 5 && od >= 2048) || (nt >= 6 && od >= 1024 && id <= 4096))) ||
         (nt >= 17 && nt <= 32 && od <= 12288) || (nt >= 33 && nt <= 48 && od <= 8192 && id <= 4096)))
        return QMM_KIND_SKINNY;
    if (nt <= sw || (sw == 8 && nt <= 16 && od <= 4096))
        return QMM_KIND_MMVQ;
    return QMM_KIND_MMQ;
}

// Whether the stream-K kernel is expected to beat the per-tile MMQ on this call
// (Q4_K and Q6_K, measured over 1024..32000-row, 4096..14336-column matrices at
// 17..512 tokens).  With T tiles of 128 x 64 and R = ceil(T / 256) rounds of the
// 256 CUs:
//  * T a whole number of rounds: no tail to balance; per tile (within 5 % either
//    way, and stream-K re-reads more from HBM);
//  * T > 256: stream-K when the last round leaves at least 10 % of the R * 256
//    workgroup slots idle (6-22 % faster there; equal below);
//  * T < 256: stream-K for a long K (>= 32 super-blocks: the few tiles each walk a
//    long chain; up to 2x faster for Q4_K, 2.5x for Q6_K), except at T = 128, where
//    the per-tile dispatch's 64 x 64 split over K is exactly 256 workgroups (one
//    full round; stream-K equal or up to 5 % slower, also in a whole-model graph);
//    and for Q6_K grids of at most 64 tiles (1.2-1.4x); otherwise per tile
//    (stream-K up to 25 % slower).
// Where Q4_K runs the 4-wave kernel within one of its rounds (qmm::mmq_q4k_wave_form
// 1 on 257-512 tiles: two of its workgroups per CU, so a round holds 512 tiles) the
// per-tile launch stays: stream-K was 5-31 % slower at every such shape measured.
bool streamk_preferred(int type, int nt, int od, int id)
{
    const bool q6 = type == QMM_TYPE_Q6_K || type == QMM_TYPE_Q6_K_P224;
    if ((type != QMM_TYPE_Q4_K && !q6) || dispatch_kind(type, nt, od, id) != QMM_KIND_MMQ)
        return false;
    const long tiles = (long)((nt + 63) / 64) * ((od + 127) / 128);
    if (type == QMM_TYPE_Q4_K && tiles <= 512 && qmm::mmq_q4k_wave_form(nt, od, id) == 1)
        return false;
    if (tiles % 256 == 0)
        return false;
    if (tiles > 256) {
        const long slots = 256 * ((tiles + 255) / 256);
        return (slots - tiles) * 10 >= slots;
    }
    return (id / 256 >= 32 && tiles != 128) || (q6 && tiles <= 64);
}

int matmul_q8_checked(int kind, int type, const void* W, const int8_t* q, const float* d,
                      const float* s, int nt, int od, int id, float* out, int32_t* S, void* stream)
{
    const auto st = reinterpret_cast<hipStream_t>(stream);
    const auto w = reinterpret_cast<const uint8_t*>(W);
    if (kind == QMM_KIND_SKINNY) {
        if (type != QMM_TYPE_Q4_K)
            return QMM_ERR_TYPE;
        if (S)
            return QMM_ERR_ARG;  // no integer dump from this kernel
        // up to 16 tokens per launch; more as token slices of 16 (rows t0.. of q, d,
        // s and out), each a complete call on its own
        const size_t nblk = (size_t)id / 32;
        for (int t0 = 0; t0 < nt; t0 += 16) {
            const int rc = launched(qmm::launch_skinny(w, q + (size_t)t0 * id, d + (size_t)t0 * nblk,
                                                       s + (size_t)t0 * nblk, min(16, nt - t0), od, id,
                                                       out + (size_t)t0 * od, st, skinny_cfg_override()));
            if (rc)
                return rc;
        }
        return QMM_OK;
    }
    if (kind == QMM_KIND_MMVQ) {
        if (nt <= 8)
            return launched(qmm::launch_mmvq(type, w, q, d, s, nt, od, id, out, S, st));
        if (S)
            return QMM_ERR_ARG;  // the integer dump runs on up to 8 tokens
        // tokens t0 .. t0 + 7 are rows t0.. of q, d, s and out: each slice is a
        // complete call on its own (a token's outputs do not depend on the others)
        const size_t nblk = (size_t)id / 32;
        for (int t0 = 0; t0 < nt; t0 += 8) {
            const int rc = launched(qmm::launch_mmvq(type, w, q + (size_t)t0 * id, d + (size_t)t0 * nblk,
                                                     s + (size_t)t0 * nblk, min(8, nt - t0), od, id,
                                                     out + (size_t)t0 * od, nullptr, st));
            if (rc)
                return rc;
        }
        return QMM_OK;
    }
    const int tile = kind == QMM_KIND_MMQ_WAVE32X64_SPLITK ? 5
                     : kind >= QMM_KIND_MMQ_128X64     ? kind - QMM_KIND_MMQ_128X64 + 1
                                                       : 0;
    return launched(qmm::launch_mmq(type, w, q, d, s, nt, od, id, out, S, st, tile));
}

int validate_q8(int type, const void* W, const int8_t* q, const float* d, const float* s, int nt,
                int od, int id, const void* out)
{
    if (!W || !q || !d || !s || !out)
        return QMM_ERR_ARG;
    int rc = check_type(type);
    if (rc)
        return rc;
    rc = check_shape(nt, od, id);
    if (rc)
        return rc;
    if (!aligned16(W) || !aligned16(q) || !aligned16(d) || !aligned16(s) || !aligned16(out))
        return QMM_ERR_ALIGN;
    return QMM_OK;
}

// Shape and argument rules shared by the producer-side steps.
int check_rows(int nt, int id)
{
    if (nt < 1)
        return QMM_ERR_ARG;
    if (id < 32 || id % 32 || (long long)nt * id > 0x7FFFFFFFLL)
        return QMM_ERR_SHAPE;
    return QMM_OK;
}

bool eps_ok(float eps) { return eps >= 0.0f && eps <= 3.4028234663852886e38f; }  // rejects NaN, inf

bool all_aligned(std::initializer_list<const void*> ps)
{
    for (const void* p : ps)
        if (!aligned16(p))
            return false;
    return true;
}

}  // namespace

extern "C" {

size_t qmm_weight_bytes(int type, int od, int id)
{
    if (check_type(type) || od < 1 || id < 256 || id % 256)
        return 0;
    return (size_t)od * (size_t)(id / 256) * block_bytes(type);
}

size_t qmm_act_bytes(int nt, int id)
{
    if (nt < 1 || id < 32 || id % 32)
        return 0;
    const size_t n = (size_t)nt * (size_t)id;
    return round256(n) + 2 * round256(n / 32 * sizeof(float));
}

int qmm_quantize_act(const float* x, int nt, int id, int8_t* q, float* d, float* s, void* stream)
{
    if (!x || !q || !d || !s || nt < 1)
        return QMM_ERR_ARG;
    if (id < 32 || id % 32 || (long long)nt * id > 0x7FFFFFFFLL)
        return QMM_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned16(d) || !aligned16(s))
        return QMM_ERR_ALIGN;
    int rc = check_device();
    if (rc)
        return rc;
    return launched(qmm::launch_quantize(x, nt, id, q, d, s, reinterpret_cast<hipStream_t>(stream)));
}

// The fused producers, per-32 (q8k false) or Q8_K (q8k true: whole 256-value
// blocks, d [nt][id/256], s = the group sums [nt][id/16]).
static int add_rmsnorm_quantize(float* h, const float* o, const float* w, float eps, int nt, int id, int8_t* q,
                                float* d, float* s, void* stream, bool q8k)
{
    if (!h || !o || !w || !q || !d || !s || !eps_ok(eps))
        return QMM_ERR_ARG;
    int rc = check_rows(nt, id);
    if (rc)
        return rc;
    if (q8k && id % 256)
        return QMM_ERR_SHAPE;
    if (!all_aligned({h, o, w, q, d, s}))
        return QMM_ERR_ALIGN;
    if ((rc = check_device()))
        return rc;
    return launched(qmm::launch_rmsnorm(h, o, h, w, eps, nt, id, q, d, s, nullptr,
                                        reinterpret_cast<hipStream_t>(stream), q8k));
}

static int rmsnorm_quantize(const float* x, const float* w, float eps, int nt, int id, int8_t* q, float* d,
                            float* s, void* stream, bool q8k)
{
    if (!x || !w || !q || !d || !s || !eps_ok(eps))
        return QMM_ERR_ARG;
    int rc = check_rows(nt, id);
    if (rc)
        return rc;
    if (q8k && id % 256)
        return QMM_ERR_SHAPE;
    if (!all_aligned({x, w, q, d, s}))
        return QMM_ERR_ALIGN;
    if ((rc = check_device()))
        return rc;
    return launched(qmm::launch_rmsnorm(x, nullptr, nullptr, w, eps, nt, id, q, d, s, nullptr,
                                        reinterpret_cast<hipStream_t>(stream), q8k));
}

static int silu_mul_quantize(const float* g, const float* u, int nt, int id, int8_t* q, float* d, float* s,
                             void* stream, bool q8k)
{
    if (!g || !u || !q || !d || !s)
        return QMM_ERR_ARG;
    int rc = check_rows(nt, id);
    if (rc)
        return rc;
    if (q8k && id % 256)
        return QMM_ERR_SHAPE;
    if (!all_aligned({g, u, q, d, s}))
        return QMM_ERR_ALIGN;
    if ((rc = check_device()))
        return rc;
    return launched(qmm::launch_silu_mul(g, u, nt, id, q, d, s, nullptr, reinterpret_cast<hipStream_t>(stream),
                                         q8k));
}

int qmm_add_rmsnorm_quantize(float* h, const float* o, const float* w, float eps, int nt, int id, int8_t* q,
                             float* d, float* s, void* stream)
{
    return add_rmsnorm_quantize(h, o, w, eps, nt, id, q, d, s, stream, false);
}

int qmm_rmsnorm_quantize(const float* x, const float* w, float eps, int nt, int id, int8_t* q, float* d, float* s,
                         void* stream)
{
    return rmsnorm_quantize(x, w, eps, nt, id, q, d, s, stream, false);
}

int qmm_silu_mul_quantize(const float* g, const float* u, int nt, int id, int8_t* q, float* d, float* s,
                          void* stream)
{
    return silu_mul_quantize(g, u, nt, id, q, d, s, stream, false);
}

int qmm_add_rmsnorm_quantize_q8k(float* h, const float* o, const float* w, float eps, int nt, int id, int8_t* q,
                                 float* d, float* bsum, void* stream)
{
    return add_rmsnorm_quantize(h, o, w, eps, nt, id, q, d, bsum, stream, true);
}

int qmm_rmsnorm_quantize_q8k(const float* x, const float* w, float eps, int nt, int id, int8_t* q, float* d,
                             float* bsum, void* stream)
{
    return rmsnorm_quantize(x, w, eps, nt, id, q, d, bsum, stream, true);
}

int qmm_silu_mul_quantize_q8k(const float* g, const float* u, int nt, int id, int8_t* q, float* d, float* bsum,
                              void* stream)
{
    return silu_mul_quantize(g, u, nt, id, q, d, bsum, stream, true);
}

int qmm_residual_add(float* h, const float* o, int nt, int id, void* stream)
{
    if (!h || !o)
        return QMM_ERR_ARG;
    int rc = check_rows(nt, id);
    if (rc)
        return rc;
    if (!all_aligned({h, o}))
        return QMM_ERR_ALIGN;
    if ((rc = check_device()))
        return rc;
    return launched(qmm::launch_residual_add(h, o, (long)nt * id, reinterpret_cast<hipStream_t>(stream)));
}

int qmm_rmsnorm(const float* x, const float* w, float eps, int nt, int id, float* y, void* stream)
{
    if (!x || !w || !y || !eps_ok(eps))
        return QMM_ERR_ARG;
    int rc = check_rows(nt, id);
    if (rc)
        return rc;
    if (!all_aligned({x, w, y}))
        return QMM_ERR_ALIGN;
    if ((rc = check_device()))
        return rc;
    return launched(qmm::launch_rmsnorm(x, nullptr, nullptr, w, eps, nt, id, nullptr, nullptr, nullptr, y,
                                        reinterpret_cast<hipStream_t>(stream)));
}

int qmm_silu_mul(const float* g, const float* u, int nt, int id, float* y, void* stream)
{
    if (!g || !u || !y)
        return QMM_ERR_ARG;
    int rc = check_rows(nt, id);
    if (rc)
        return rc;
    if (!all_aligned({g, u, y}))
        return QMM_ERR_ALIGN;
    if ((rc = check_device()))
        return rc;
    return launched(qmm::launch_silu_mul(g, u, nt, id, nullptr, nullptr, nullptr, y,
                                         reinterpret_cast<hipStream_t>(stream)));
}

int qmm_quantize_act_q8k(const float* x, int nt, int id, int8_t* q, float* d, float* bsum, void* stream)
{
    if (!x || !q || !d || !bsum || nt < 1)
        return QMM_ERR_ARG;
    if (id < 256 || id % 256 || (long long)nt * id > 0x7FFFFFFFLL)
        return QMM_ERR_SHAPE;
    if (!all_aligned({x, q, d, bsum}))
        return QMM_ERR_ALIGN;
    int rc = check_device();
    if (rc)
        return rc;
    return launched(qmm::launch_quantize_q8k(x, nt, id, q, d, bsum, reinterpret_cast<hipStream_t>(stream)));
}

static int q8k_checked(int type, const void* W, const int8_t* q, const float* d, const float* bsum, int nt, int od,
                       int id, float* out, int32_t* S, void* stream, int tile = 0)
{
    if (!W || !q || !d || !bsum || (!out && !S))
        return QMM_ERR_ARG;
    int rc = check_type(type);
    if (rc)
        return rc;
    if (type != QMM_TYPE_Q4_K && type != QMM_TYPE_Q5_K && type != QMM_TYPE_Q6_K && type != QMM_TYPE_Q6_K_P224)
        return QMM_ERR_TYPE;
    if ((rc = check_shape(nt, od, id)))
        return rc;
    if (S && (long long)nt * od * (id / 256) * 2 > 0x7FFFFFFFLL)
        return QMM_ERR_SHAPE;
    if (!all_aligned({W, q, d, bsum, out ? (const void*)out : (const void*)S}))
        return QMM_ERR_ALIGN;
    if ((rc = check_device()))
        return rc;
    return launched(qmm::launch_mmq_q8k(type, reinterpret_cast<const uint8_t*>(W), q, d, bsum, nt, od, id, out, S,
                                        reinterpret_cast<hipStream_t>(stream), tile));
}

int qmm_matmul_q8k(int type, const void* W, const int8_t* q, const float* d, const float* bsum, int nt, int od,
                   int id, float* out, void* stream)
{
    if (!out)
        return QMM_ERR_ARG;
    return q8k_checked(type, W, q, d, bsum, nt, od, id, out, nullptr, stream);
}

int qmm_matmul_q8k_kind(int kind, int type, const void* W, const int8_t* q, const float* d, const float* bsum,
                        int nt, int od, int id, float* out, void* stream)
{
    const bool wave = kind == QMM_KIND_MMQ_WAVE32X64 || kind == QMM_KIND_MMQ_WAVE32X64_SPLITK;
    if (kind != QMM_KIND_MMQ && !wave && (kind < QMM_KIND_MMQ_128X64 || kind > QMM_KIND_MMQ_64X64_SPLITK))
        return QMM_ERR_ARG;
    if (!out)
        return QMM_ERR_ARG;
    if (wave && type != QMM_TYPE_Q4_K)
        return QMM_ERR_TYPE;
    const int tile = kind == QMM_KIND_MMQ ? 0 : kind == QMM_KIND_MMQ_WAVE32X64_SPLITK ? 5 : kind - QMM_KIND_MMQ_128X64 + 1;
    return q8k_checked(type, W, q, d, bsum, nt, od, id, out, nullptr, stream, tile);
}

int qmm_q8k_tile(int nt, int od, int id)
{
    const int rc = check_shape(nt, od, id);
    if (rc)
        return rc;
    return QMM_KIND_MMQ_128X64 - 1 + qmm::q8k_tile_choice(nt, od, id);
}

int qmm_q8k_superblock_sums(int type, const void* W, const int8_t* q, const float* d, const float* bsum, int nt,
                            int od, int id, int32_t* S, void* stream)
{
    if (!S)
        return QMM_ERR_ARG;
    return q8k_checked(type, W, q, d, bsum, nt, od, id, nullptr, S, stream);
}

int qmm_pad_q6k(const void* src, void* dst, long long nblocks, void* stream)
{
    if (!src || !dst)
        return QMM_ERR_ARG;
    if (nblocks < 1 || nblocks > (1LL << 40) / qmm::kQ6KP224Bytes)
        return QMM_ERR_SHAPE;
    if (!aligned16(dst))
        return QMM_ERR_ALIGN;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + (uintptr_t)nblocks * qmm::kQ6KP224Bytes && d0 < s0 + (uintptr_t)nblocks * qmm::kQ6KBytes)
        return QMM_ERR_ARG;  // overlap
    int rc = check_device();
    if (rc)
        return rc;
    const long long np = nblocks * 14;
    hipLaunchKernelGGL(pad_q6k_kernel, dim3((unsigned)((np + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint8_t*>(src),
                       reinterpret_cast<uint4*>(dst), np);
    return launched(hipGetLastError());
}

size_t qmm_streamk_ws_bytes(void) { return qmm::mmq_streamk_ws_bytes(); }

int qmm_matmul_q8_streamk(int type, const void* W, const int8_t* q, const float* d, const float* s, int nt, int od,
                          int id, float* out, void* workspace, size_t ws_bytes, void* stream)
{
    int rc = validate_q8(type, W, q, d, s, nt, od, id, out);
    if (rc)
        return rc;
    if (type != QMM_TYPE_Q4_K && type != QMM_TYPE_Q6_K && type != QMM_TYPE_Q6_K_P224)
        return QMM_ERR_TYPE;
    if (!workspace)
        return QMM_ERR_ARG;
    if (!aligned16(workspace))
        return QMM_ERR_ALIGN;
    if (ws_bytes < qmm::mmq_streamk_ws_bytes())
        return QMM_ERR_WORKSPACE;
    if ((rc = check_device()))
        return rc;
    return launched(qmm::launch_mmq_streamk(type, reinterpret_cast<const uint8_t*>(W), q, d, s, nt, od, id, out,
                                            reinterpret_cast<float*>(workspace),
                                            reinterpret_cast<hipStream_t>(stream)));
}

int qmm_nt_switch(void) { return nt_switch_value(); }

int qmm_set_skinny_split(int ks)
{
    if (ks != 0 && ks != 1 && ks != 2 && ks != 4 && ks != 8 && ks != 16)
        return QMM_ERR_ARG;
    __atomic_store_n(&g_skinny_cfg, ks ? 100 + ks : 0, __ATOMIC_RELEASE);
    return QMM_OK;
}

int qmm_streamk_preferred(int type, int nt, int od, int id)
{
    int rc = check_type(type);
    if (rc)
        return rc;
    rc = check_shape(nt, od, id);
    if (rc)
        return rc;
    return streamk_preferred(type, nt, od, id) ? 1 : 0;
}

int qmm_dispatch_kind(int type, int nt, int od, int id)
{
    int rc = check_type(type);
    if (rc)
        return rc;
    rc = check_shape(nt, od, id);
    if (rc)
        return rc;
    return dispatch_kind(type, nt, od, id);
}

int qmm_mmq_tile(int nt, int od, int id)
{
    const int rc = check_shape(nt, od, id);
    if (rc)
        return rc;
    return QMM_KIND_MMQ_128X64 - 1 + qmm::mmq_tile_choice(nt, od, id);
}

int qmm_matmul_q8(int type, const void* W, const int8_t* q, const float* d, const float* s, int nt,
                  int od, int id, float* out, void* stream)
{
    int rc = validate_q8(type, W, q, d, s, nt, od, id, out);
    if (rc)
        return rc;
    rc = check_device();
    if (rc)
        return rc;
    const int kind = dispatch_kind(type, nt, od, id);
    return matmul_q8_checked(kind, type, W, q, d, s, nt, od, id, out, nullptr, stream);
}

int qmm_matmul_q8_kind(int kind, int type, const void* W, const int8_t* q, const float* d,
                       const float* s, int nt, int od, int id, float* out, void* stream)
{
    if (kind < QMM_KIND_MMVQ || (kind > QMM_KIND_SKINNY && kind != QMM_KIND_MMQ_WAVE32X64_SPLITK))
        return QMM_ERR_ARG;
    if ((kind == QMM_KIND_MMQ_WAVE32X64 || kind == QMM_KIND_MMQ_WAVE32X64_SPLITK || kind == QMM_KIND_SKINNY) &&
        type != QMM_TYPE_Q4_K)
        return QMM_ERR_TYPE;
    int rc = validate_q8(type, W, q, d, s, nt, od, id, out);
    if (rc)
        return rc;
    rc = check_device();
    if (rc)
        return rc;
    return matmul_q8_checked(kind, type, W, q, d, s, nt, od, id, out, nullptr, stream);
}

int qmm_matmul(int type, const void* W, const float* x, int nt, int od, int id, float* out,
               void* workspace, size_t ws_bytes, void* stream)
{
    if (!W || !x || !out || !workspace)
        return QMM_ERR_ARG;
    int rc = check_type(type);
    if (rc)
        return rc;
    rc = check_shape(nt, od, id);
    if (rc)
        return rc;
    if (!aligned16(W) || !aligned16(x) || !aligned16(out) || !aligned16(workspace))
        return QMM_ERR_ALIGN;
    if (ws_bytes < qmm_act_bytes(nt, id))
        return QMM_ERR_WORKSPACE;
    rc = check_device();
    if (rc)
        return rc;
    const size_t n = (size_t)nt * (size_t)id;
    auto* base = static_cast<uint8_t*>(workspace);
    auto* q = reinterpret_cast<int8_t*>(base);
    auto* d = reinterpret_cast<float*>(base + round256(n));
    auto* s = reinterpret_cast<float*>(base + round256(n) + round256(n / 32 * sizeof(float)));
    const auto st = reinterpret_cast<hipStream_t>(stream);
    rc = launched(qmm::launch_quantize(x, nt, id, q, d, s, st));
    if (rc)
        return rc;
    // the stream-K kernel where it is faster and the workspace also holds its
    // partial tiles (after the q8 plane, at a 256-byte boundary)
    const size_t act = qmm_act_bytes(nt, id);
    if (streamk_preferred(type, nt, od, id) && ws_bytes >= act + qmm::mmq_streamk_ws_bytes())
        return launched(qmm::launch_mmq_streamk(type, static_cast<const uint8_t*>(W), q, d, s, nt, od, id, out,
                                                reinterpret_cast<float*>(base + act), st));
    const int kind = dispatch_kind(type, nt, od, id);
    return matmul_q8_checked(kind, type, W, q, d, s, nt, od, id, out, nullptr, stream);
}

int qmm_matmul_noalloc(int type, const void* W, const float* x, int nt, int od, int id, float* out, void* stream)
{
    if (!W || !x || !out)
        return QMM_ERR_ARG;
    int rc = check_type(type);
    if (rc)
        return rc;
    rc = check_shape(nt, od, id);
    if (rc)
        return rc;
    if (!aligned16(W) || !aligned16(x) || !aligned16(out))
        return QMM_ERR_ALIGN;
    if (qmm_act_bytes(nt, id) > (size_t)QMM_NOALLOC_ACT_BYTES)
        return QMM_ERR_SCRATCH;
    rc = check_device();
    if (rc)
        return rc;
    void* ws = nullptr;
    rc = noalloc_scratch(&ws);
    if (rc)
        return rc;
    static_assert(QMM_NOALLOC_SCRATCH_BYTES >= QMM_NOALLOC_ACT_BYTES, "the scratch holds the activation region");
    // the same launches as qmm_matmul with a workspace of the whole scratch: the q8
    // plane at its start, the stream-K partial tiles after it where they fit
    return qmm_matmul(type, W, x, nt, od, id, out, ws, kNoallocBytes, stream);
}

int qmm_group_dots(int kind, int type, const void* W, const int8_t* q, int nt, int od, int id,
                   int32_t* S, void* stream)
{
    if (!W || !q || !S)
        return QMM_ERR_ARG;
    if (kind != QMM_KIND_MMVQ && kind != QMM_KIND_MMQ)
        return QMM_ERR_ARG;
    int rc = check_type(type);
    if (rc)
        return rc;
    rc = check_shape(nt, od, id);
    if (rc)
        return rc;
    if (kind == QMM_KIND_MMVQ && nt > 8)
        return QMM_ERR_ARG;
    if (!aligned16(W) || !aligned16(q) || !aligned16(S))
        return QMM_ERR_ALIGN;
    rc = check_device();
    if (rc)
        return rc;
    // the integer stage does not use the activation scales; the code buffer (at
    // least 8x larger than a scale plane) stands in so any scale read stays in bounds
    const float* dummy = reinterpret_cast<const float*>(q);
    return matmul_q8_checked(kind, type, W, q, dummy, dummy, nt, od, id, nullptr, S, stream);
}

int qmm_mfma_tile_check(int kind, const void* A, const void* B, void* C, void* stream)
{
    if (!A || !B || !C || kind < 1 || kind > 3)
        return QMM_ERR_ARG;
    if (!aligned16(A) || !aligned16(B) || !aligned16(C))
        return QMM_ERR_ALIGN;
    int rc = check_device();
    if (rc)
        return rc;
    return launched(qmm::launch_mfma_tile_probe(kind, A, B, C, reinterpret_cast<hipStream_t>(stream)));
}

const char* qmm_strerror(int status)
{
    switch (status) {
    case QMM_OK: return "ok";
    case QMM_ERR_ARG: return "invalid argument (null pointer, nt or od < 1, or bad kind)";
    case QMM_ERR_TYPE: return "unknown weight type";
    case QMM_ERR_SHAPE: return "bad shape (id must be a positive multiple of 256; sizes must fit 31 bits)";
    case QMM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QMM_ERR_WORKSPACE: return "workspace too small (see qmm_act_bytes)";
    case QMM_ERR_DEVICE: return "current device is not gfx950";
    case QMM_ERR_LAUNCH: return "kernel launch failed";
    case QMM_ERR_SCRATCH:
        return "call too large for the fixed scratch of qmm_matmul_noalloc (qmm_act_bytes(nt, id) > "
               "QMM_NOALLOC_ACT_BYTES)";
    default: return "unknown status";
    }
}

}  // extern "C"
